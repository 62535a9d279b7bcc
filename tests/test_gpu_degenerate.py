"""Degenerate inputs through the GPU path, against the oracle.

The method's edge values, each on a small batch of both gates: zero keys
(the L2 norm's eps leaves k^ = 0, so the token updates nothing) and zero
queries (o = 0), beta at both saturations, gates that wipe the state in
one token (decay exp(g) underflows to 0 with the unbounded gate) or leave
it untouched (decay -> 1), a zero checkpoint, and values near the top of
the bf16 range for v. Outputs, records and committed states are compared
with the oracle at the tests' tolerances; the commit must still give the
recurrence's bits.
"""

import numpy as np
import pytest

from workloads import bf16_from_f32, make_batch

from .helpers import oracle_prefill_pool
from .test_gpu_parity import run_verify_commit, say

pytestmark = pytest.mark.gpu

K = 128


def _tokens_cols(batch, which):
    hk = batch.H * K
    j = {"q": 0, "k": 1, "v": 2}[which]
    return slice(j * hk, (j + 1) * hk)


def _rows_token(batch, t):
    """Token index t of every row that has it."""
    cu, T = batch.cu_seqlens, batch.seq_lens()
    return np.array([cu[i] + t for i in range(batch.num_rows) if T[i] > t], np.int64)


def _bf16(x):
    return bf16_from_f32(np.float32(x))


CASES = ("zero_k_q", "beta_saturated", "gate_extremes", "zero_state", "large_v")


def degenerate_batch(case, name):
    batch = make_batch(name, B=8, H=4)
    t = batch.tokens
    pool = oracle_prefill_pool(batch)
    if case == "zero_k_q":
        t.qkv[_rows_token(batch, 1), _tokens_cols(batch, "k")] = 0      # k = 0: k^ = 0
        t.qkv[_rows_token(batch, 2), _tokens_cols(batch, "q")] = 0      # q = 0: o = 0
        t.qkv[_rows_token(batch, 3), _tokens_cols(batch, "k")] = 0x8000  # -0.0
    elif case == "beta_saturated":
        t.beta[_rows_token(batch, 0)] = _bf16(-60.0)                    # beta ~ 0
        t.beta[_rows_token(batch, 2)] = _bf16(60.0)                     # beta ~ 1
    elif case == "gate_extremes":
        g = t.g.reshape(t.num_tokens, batch.H, K)
        g[_rows_token(batch, 1), :, :64] = _bf16(80.0)     # unbounded: decay 0; bounded: e^lb
        g[_rows_token(batch, 1), :, 64:] = _bf16(-80.0)    # decay -> 1
        g[_rows_token(batch, 3)] = _bf16(80.0)
    elif case == "zero_state":
        pool[:] = 0.0
    elif case == "large_v":
        v = t.qkv[:, _tokens_cols(batch, "v")]
        t.qkv[:, _tokens_cols(batch, "v")] = np.where(np.arange(v.shape[1]) % 2 == 0,
                                                      _bf16(3.0e4), _bf16(-3.0e4))
    else:
        raise ValueError(case)
    return batch, pool


@pytest.mark.parametrize("name", ["decode", "decode_bounded"])
@pytest.mark.parametrize("case", CASES)
def test_degenerate_inputs_against_oracle(case, name):
    batch, pool = degenerate_batch(case, name)
    say(f"case degenerate {case} {name}")
    run_verify_commit(batch, pool)
    run_verify_commit(batch, pool, bench_launch=True)
