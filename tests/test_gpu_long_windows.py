"""GPU parity for windows longer than one chunk of the chunked verify (more
than 4 tokens with a window Q <= 4, more than 8 otherwise): the verify runs
chunk after chunk, advancing the state in registers between them. Checked
against the oracle for kda_verify and for kda_verify_deferred (fold first,
then the long window), with records bitwise and the pool checked."""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_batch

from .helpers import (DevTokens, bits_host, check_o, check_state, dev_layer, dev_records,
                      oracle_layer, oracle_records, records_host, to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7E7E


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def long_rows(batch, Q, rng):
    """Re-partition the batch's tokens into rows of 1..5*Q + 3 tokens (the
    token values are i.i.d., so any partition is a valid workload); slots
    are distinct, two rows are skipped."""
    ntok = batch.tokens.num_tokens
    lens = []
    while sum(lens) < ntok:
        lens.append(int(rng.integers(1, 5 * Q + 4)))
    lens[-1] -= sum(lens) - ntok
    if lens[-1] == 0:
        lens.pop()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    B = len(lens)
    slots = rng.permutation(np.arange(1, batch.num_slots))[:B].astype(np.int32)
    slots[[1, B // 2]] = [0, -1]
    return cu, slots


def oracle_pool(batch, rng):
    pool = batch.initial_pool()
    if not pool.any():
        pool = (rng.standard_normal(pool.shape, dtype=np.float32) * np.float32(0.02))
        pool[0] = 0
    return pool


@pytest.mark.parametrize("Q", [4, 8])
def test_long_windows_verify(Q):
    batch = make_batch("ragged", B=64, H=4)
    rng = np.random.default_rng(31 + Q)
    cu, slots = long_rows(batch, Q, rng)
    B, H, ntok = len(slots), batch.H, batch.tokens.num_tokens
    say(f"case long windows verify Q={Q} rows={B} max T={int(np.diff(cu).max())}")
    pool_np = oracle_pool(batch, rng)
    pool = to_dev(pool_np)
    rec = dev_records(B, H, Q, fill=SENT)
    o = torch.zeros((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify(dev_layer(batch), *DevTokens(batch.tokens).args(), to_dev(cu), pool,
                   to_dev(slots), rec, o)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), pool_np), "verify wrote the pool"
    t = batch.tokens
    rec_ref = oracle_records(B, H, Q, fill=SENT)
    o_ref = np.zeros((ntok, H, 128), np.uint16)
    ref.kda_verify(oracle_layer(batch), t.q, t.k, t.v, t.g, t.beta, cu, pool_np.copy(), slots,
                   rec_ref, o_ref)
    check_o(bits_host(o), o_ref, what=f"o, Q={Q}")
    rg = records_host(rec)
    for f in ("k", "v", "g", "beta"):
        assert np.array_equal(getattr(rg, f), getattr(rec_ref, f)), f"records {f}"


@pytest.mark.parametrize("Q", [4, 8])
def test_long_windows_verify_deferred(Q):
    batch = make_batch("ragged", B=64, H=4)
    rng = np.random.default_rng(47 + Q)
    cu, slots = long_rows(batch, Q, rng)
    B, H, ntok = len(slots), batch.H, batch.tokens.num_tokens
    say(f"case long windows deferred Q={Q} rows={B} max T={int(np.diff(cu).max())}")
    pool_np = oracle_pool(batch, rng)
    lay_ref = oracle_layer(batch)
    t = batch.tokens
    # rec_prev: the records of a first verify of the same windows (written
    # by the oracle: records are bit copies of the inputs); pending counts
    # cover negative, zero, in-range and beyond-window values
    rec_prev = oracle_records(B, H, Q)
    ref.kda_verify(lay_ref, t.q, t.k, t.v, t.g, t.beta, cu, pool_np.copy(), slots, rec_prev,
                   np.zeros((ntok, H, 128), np.uint16))
    pending = rng.integers(-1, Q + 2, size=B).astype(np.int32)
    # ---- GPU
    pool = to_dev(pool_np)
    rp = dev_records(B, H, Q)
    for f in ("k", "v", "g", "beta"):
        getattr(rp, f).view(torch.int16).copy_(to_dev(getattr(rec_prev, f).view(np.int16)))
    rn = dev_records(B, H, Q, fill=SENT)
    o = torch.zeros((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify_deferred(dev_layer(batch), *DevTokens(batch.tokens).args(), to_dev(cu), pool,
                            to_dev(slots), rp, to_dev(pending), rn, o)
    torch.cuda.synchronize()
    # ---- oracle
    pool_ref = pool_np.copy()
    rec_next = oracle_records(B, H, Q, fill=SENT)
    o_ref = np.zeros((ntok, H, 128), np.uint16)
    ref.kda_verify_deferred(lay_ref, t.q, t.k, t.v, t.g, t.beta, cu, pool_ref, slots, rec_prev,
                            pending, rec_next, None, o_ref)
    check_o(bits_host(o), o_ref, what=f"o, Q={Q}")
    rg = records_host(rn)
    for f in ("k", "v", "g", "beta"):
        assert np.array_equal(getattr(rg, f), getattr(rec_next, f)), f"records {f}"
    got = pool.cpu().numpy()
    for i in range(B):
        s = int(slots[i])
        if s > 0:
            check_state(got[s], pool_ref[s], what=f"row {i} slot {s}")
    others = np.ones(batch.num_slots, bool)
    others[slots[slots > 0]] = False
    assert np.array_equal(got[others], pool_np[others]), "a slot of no row was written"
