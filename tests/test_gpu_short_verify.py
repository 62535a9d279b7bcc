"""GPU parity of kda_verify with the caller's window bound (kda_tokens.max_seqlen):
the short kernels, with token loads issued at a predicted uniform span,
give the bits of the general kernels for every row within the bound, match
the oracle, fall back correctly where the prediction fails, and mark the
rows longer than the bound (NaN outputs and beta records)."""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_batch

from .helpers import (DevTokens, bits_host, check_o, dev_layer, dev_records, oracle_layer,
                      oracle_records, records_host, to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7E57


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def random_pool(batch, seed=23):
    pool = batch.initial_pool()
    rng = np.random.default_rng(seed)
    for s in batch.state_indices[batch.state_indices > 0]:
        pool[s] = rng.standard_normal(pool.shape[1:], dtype=np.float32) * np.float32(0.02)
    return pool


def run_verify(batch, pool, cu_np, max_seqlen, Q=None):
    """o and records of one kda_verify call (sentinel-filled outputs)."""
    H = batch.H
    Q = Q or batch.Q
    ntok = batch.tokens.num_tokens
    rows = len(cu_np) - 1
    o = torch.full((ntok, H, 128), 0, dtype=torch.int16, device=DEV)
    o.fill_(np.int16(np.uint16(SENT).view(np.int16)))
    rec = dev_records(rows, H, Q, fill=SENT)
    kda.kda_verify(dev_layer(batch), *DevTokens(batch.tokens).args(), to_dev(cu_np), to_dev(pool),
                   to_dev(batch.state_indices[:rows]), rec, o.view(torch.bfloat16),
                   max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return bits_host(o), records_host(rec)


def same_records(a, b, what):
    for f in ("k", "v", "g", "beta"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f"{what}: records.{f}"


@pytest.mark.parametrize("name,B", [("tiny", None), ("decode", None), ("decode", 128),
                                    ("deep", None), ("ragged", None)])
def test_short_verify_same_bits_as_general(name, B):
    # decode at B=128 (4096 row-heads): the 128-row tiles of the 4-token kernels
    batch = make_batch(name, B=B)
    T = batch.seq_lens()
    bound = int(T.max())
    say(f"short verify vs general: {name} B={batch.num_rows} max_seqlen={bound}")
    pool = random_pool(batch)
    o_g, r_g = run_verify(batch, pool, batch.cu_seqlens, None)
    o_s, r_s = run_verify(batch, pool, batch.cu_seqlens, bound)
    assert np.array_equal(o_g, o_s), f"{name}: o"
    same_records(r_g, r_s, name)


def _oracle(batch, pool, cu_np, Q):
    t = batch.tokens
    rows = len(cu_np) - 1
    rec = oracle_records(rows, batch.H, Q, fill=SENT)
    o = np.full((t.num_tokens, batch.H, 128), SENT, np.uint16)
    ref.kda_verify(oracle_layer(batch), t.q, t.k, t.v, t.g, t.beta, cu_np, pool.copy(),
                   batch.state_indices[:rows], rec, o)
    return o, rec


def test_short_verify_mispredicted_spans():
    # 12 rows over 36 tokens: the predicted span is 3 tokens per row; the
    # lengths below put some rows on the prediction and some off it (row 4
    # is empty, rows 0..3 are off by their start or their length).
    batch = make_batch("ragged", B=16, H=4)
    lens = np.array([2, 4, 3, 3, 0, 4, 2, 3, 3, 4, 4, 4], np.int64)
    rows = len(lens)
    cu = np.zeros(rows + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    assert cu[-1] == 36 and cu[-1] <= batch.tokens.num_tokens
    say(f"short verify, mispredicted spans: lens={lens.tolist()}")
    pool = random_pool(batch)
    o_g, r_g = run_verify(batch, pool, cu, None, Q=4)
    o_s, r_s = run_verify(batch, pool, cu, 4, Q=4)
    assert np.array_equal(o_g, o_s), "o: short vs general"
    same_records(r_g, r_s, "short vs general")
    o_r, r_r = _oracle(batch, pool, cu, 4)
    valid = np.zeros(batch.tokens.num_tokens, bool)
    valid[:36] = True
    live = np.repeat(batch.state_indices[:rows] > 0, lens)
    mask = np.zeros(batch.tokens.num_tokens, bool)
    mask[:36] = live
    check_o(o_s[mask], o_r[mask], what="o vs oracle")
    same_records(r_s, r_r, "records vs oracle")
    assert np.all(o_s[~mask] == SENT), "o written outside the valid rows"


NAN = 0x7FC0


@pytest.mark.parametrize("bound", [2, 3, 4, 5, 7])
def test_short_verify_poisons_rows_longer_than_the_bound(bound):
    """Rows within the bound give the general kernel's bits; a row with a
    slot and T_i > bound gets NaN outputs and NaN beta records (its other
    records untouched), so that the commit after it stores NaN for that row
    and nothing plausible; skipped rows stay untouched."""
    batch = make_batch("ragged", B=16, H=4)
    batch.state_indices = batch.state_indices.copy()
    batch.state_indices[6] = -1     # a long row without a slot: skipped, untouched
    lens = np.array([bound, bound + 1, bound - 1, bound, bound + 1, 1, bound + 1, bound], np.int64)
    rows = len(lens)
    cu = np.zeros(rows + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    assert cu[-1] <= batch.tokens.num_tokens
    si = batch.state_indices[:rows]
    say(f"short verify, rows longer than the bound: lens={lens.tolist()} bound={bound} "
        f"slots={si.tolist()}")
    pool = random_pool(batch)
    Q = 8
    o_g, r_g = run_verify(batch, pool, cu, None, Q=Q)
    o_s, r_s = run_verify(batch, pool, cu, bound, Q=Q)
    starts = cu[:-1]
    long_rows = []
    for i in range(rows):
        span = slice(starts[i], starts[i] + lens[i])
        rr = i + 1
        if si[i] <= 0:
            assert np.all(o_s[span] == SENT), f"skipped row {i}: o written"
            for f in ("k", "v", "g", "beta"):
                assert np.all(getattr(r_s, f)[rr] == SENT), f"skipped row {i}: records.{f}"
        elif lens[i] > bound:
            long_rows.append(i)
            assert np.all(o_s[span] == NAN), f"row {i} (T={lens[i]} > {bound}): o not NaN"
            n = min(int(lens[i]), Q)
            assert np.all(r_s.beta[rr][:, :n] == NAN), f"row {i}: beta records not NaN"
            assert np.all(r_s.beta[rr][:, n:] == SENT), f"row {i}: beta written past the window"
            for f in ("k", "v", "g"):
                assert np.all(getattr(r_s, f)[rr] == SENT), f"row {i}: records.{f} written"
        else:
            assert np.array_equal(o_s[span], o_g[span]), f"row {i}: o"
            for f in ("k", "v", "g", "beta"):
                assert np.array_equal(getattr(r_s, f)[rr], getattr(r_g, f)[rr]), f"row {i}: {f}"
    assert long_rows, "no row above the bound has a slot"
    # the commit after the short verify: the long rows store NaN (every
    # element of every head), the others what the commit after the general
    # verify stores
    nacc = np.maximum(lens, 1).astype(np.int32)
    pools = []
    for bnd in (None, bound):
        p = to_dev(pool)
        rec = dev_records(rows, batch.H, Q, fill=SENT)
        L = dev_layer(batch)
        sid, cud = to_dev(si), to_dev(cu)
        o = torch.empty((batch.tokens.num_tokens, batch.H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_verify(L, *DevTokens(batch.tokens).args(), cud, p, sid, rec, o, max_seqlen=bnd)
        kda.kda_commit(L, cud, p, sid, rec, to_dev(nacc))
        torch.cuda.synchronize()
        pools.append(p.cpu().numpy())
    for i in range(rows):
        s = int(si[i])
        if s <= 0:
            continue
        if i in long_rows:
            assert np.all(np.isnan(pools[1][s])), f"row {i}: the commit stored a number"
        else:
            assert np.array_equal(pools[1][s], pools[0][s]), f"row {i}: committed state differs"


def test_short_verify_eight_token_kernel_on_short_windows():
    # a bound of 8 on 4-token windows: the 8-token short kernel (matrix-core
    # dot products at 64-row tiles) against the oracle
    batch = make_batch("decode", B=32, H=16)
    say("short verify, bound 8 on 4-token windows: decode B=32 H=16")
    pool = random_pool(batch)
    o_s, r_s = run_verify(batch, pool, batch.cu_seqlens, 8)
    o_r, r_r = _oracle(batch, pool, batch.cu_seqlens, batch.Q)
    check_o(o_s, o_r, what="o vs oracle")
    same_records(r_s, r_r, "records vs oracle")
