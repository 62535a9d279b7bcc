"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Small cases compare every element; full-size workloads (the launch
configurations the benchmark times) compare sampled rows against the oracle
and check the GPU-only identities (commit == recurrence over the accepted
prefix, bitwise; verify leaves the pool bitwise untouched) everywhere.
"""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_batch

from .helpers import (DevTokens, bits_host, bf16_dev, check_o, check_state, dev_layer,
                      dev_records, oracle_layer, oracle_prefill_pool, oracle_records,
                      records_host, to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7E7E   # sentinel bits for memory that must stay untouched


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_verify_commit(batch, pool_np, nacc=None, sample_rows=None, bench_launch=False):
    """Run verify + commit on the GPU and in the oracle; compare.

    sample_rows: oracle only on these rows (others are skipped on the oracle
    side and not compared). bench_launch: the calls as the benchmark makes
    them (the verify with the window bound, so the short kernels; the commit
    through the multi-layer kernel)."""
    B, H, Q = batch.num_rows, batch.H, batch.Q
    nacc = batch.num_accepted if nacc is None else nacc
    ntok = batch.tokens.num_tokens
    say(f"case {batch.name} B={B} H={H} Q={Q} tokens={ntok} sample={sample_rows is not None}")
    # ---- GPU
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    cu = to_dev(batch.cu_seqlens)
    si = to_dev(batch.state_indices)
    pool = to_dev(pool_np)
    pool_before = pool.clone()
    rec = dev_records(B, H, Q, fill=SENT)
    o = torch.full((ntok, H, 128), 0, dtype=torch.int16, device=DEV)
    o.fill_(np.int16(np.uint16(SENT).view(np.int16)))
    o = o.view(torch.bfloat16)
    bound = int(batch.seq_lens().max()) if bench_launch else None
    kda.kda_verify(L, *toks.args(), cu, pool, si, rec, o, max_seqlen=bound)
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int32), pool_before.view(torch.int32)), "verify wrote the pool"
    o_gpu = bits_host(o)
    rec_gpu = records_host(rec)
    if bench_launch:
        kda.kda_commit_layers([L], cu, [pool], si, [rec], to_dev(nacc.astype(np.int32)))
    else:
        kda.kda_commit(L, cu, pool, si, rec, to_dev(nacc.astype(np.int32)))
    torch.cuda.synchronize()
    pool_gpu = pool.cpu().numpy()
    # ---- oracle
    lay = oracle_layer(batch)
    t = batch.tokens
    si_ref = batch.state_indices.copy()
    if sample_rows is not None:
        keep = np.zeros(B, bool)
        keep[sample_rows] = True
        si_ref[~keep] = 0
    pool_ref = pool_np.copy()
    rec_ref = oracle_records(B, H, Q, fill=SENT)
    o_ref = np.full((ntok, H, 128), SENT, np.uint16)
    ref.kda_verify(lay, t.q, t.k, t.v, t.g, t.beta, batch.cu_seqlens, pool_ref, si_ref, rec_ref, o_ref)
    ref.kda_commit(lay, batch.cu_seqlens, ntok, pool_ref, si_ref, rec_ref, nacc)
    # ---- compare
    rows = range(B) if sample_rows is None else sample_rows
    tok_mask = np.zeros((ntok, 1, 1), bool)
    for i in rows:
        if batch.state_indices[i] > 0:
            bos, T = int(batch.cu_seqlens[i]), int(batch.seq_lens()[i])
            tok_mask[bos:bos + T] = True
    check_o(o_gpu, o_ref, mask=tok_mask,
            what=f"{batch.name}{'' if batch.lower_bound is None else ' bounded'} o, "
                 f"{len(rows)} rows{' (bench launch)' if bench_launch else ''}")
    for i in rows:
        assert np.array_equal(rec_gpu.k[i + 1], rec_ref.k[i + 1]), f"records k row {i}"
        assert np.array_equal(rec_gpu.v[i + 1], rec_ref.v[i + 1]), f"records v row {i}"
        assert np.array_equal(rec_gpu.g[i + 1], rec_ref.g[i + 1]), f"records g row {i}"
        assert np.array_equal(rec_gpu.beta[i + 1], rec_ref.beta[i + 1]), f"records beta row {i}"
        s = int(batch.state_indices[i])
        if 0 < s < batch.num_slots:
            check_state(pool_gpu[s], pool_ref[s], what=f"state row {i} slot {s}")
    # skipped rows: o untouched
    for i in range(B):
        if batch.state_indices[i] <= 0:
            bos, T = int(batch.cu_seqlens[i]), int(batch.seq_lens()[i])
            assert np.all(o_gpu[bos:bos + T] == SENT), f"skipped row {i} wrote o"
    # slots used by no row: untouched bitwise
    used = set(int(s) for s in batch.state_indices if s > 0)
    unused = [s for s in range(batch.num_slots) if s not in used]
    assert np.array_equal(pool_gpu[unused], pool_np[unused])
    return o_gpu, pool_gpu


# ------------------------------------------------------------- small ----

@pytest.mark.parametrize("name,B,H", [("tiny", None, None), ("decode", 8, 4),
                                      ("deep", 6, 4), ("ragged", 24, 4)])
def test_verify_commit_match_oracle_small(name, B, H):
    batch = make_batch(name, B=B, H=H)
    run_verify_commit(batch, oracle_prefill_pool(batch))


def test_recurrent_matches_oracle_prefill():
    # 64 prefill tokens per row from a zero state (the decode recipe), and the
    # tiny workload's window.
    batch = make_batch("decode", B=6, H=4)
    say("case recurrent prefill 64 tokens B=6 H=4")
    p = batch.prefill
    L = dev_layer(batch)
    toks = DevTokens(p)
    pool = torch.zeros((batch.num_slots, batch.H, 128, 128), dtype=torch.float32, device=DEV)
    o = torch.empty((p.num_tokens, batch.H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_recurrent(L, *toks.args(), to_dev(batch.prefill_cu), pool,
                      to_dev(batch.state_indices), o)
    torch.cuda.synchronize()
    pool_ref = oracle_prefill_pool(batch)
    o_ref = np.zeros((p.num_tokens, batch.H, 128), np.uint16)
    ref.kda_recurrent(oracle_layer(batch), p.q, p.k, p.v, p.g, p.beta, batch.prefill_cu,
                      batch.initial_pool(), batch.state_indices, o_ref)
    check_o(bits_host(o), o_ref, what="prefill o")
    check_state(pool.cpu().numpy()[1:batch.num_rows + 1], pool_ref[1:batch.num_rows + 1])


def _gather_prefix(batch, nacc):
    """Pack the first n' tokens of every row (for the recurrence over the
    accepted prefix)."""
    T = batch.seq_lens()
    n = np.minimum(np.maximum(nacc, 0), np.minimum(T, batch.Q))
    n = np.where(batch.state_indices > 0, n, 0)
    idx = np.concatenate([np.arange(batch.cu_seqlens[i], batch.cu_seqlens[i] + n[i])
                          for i in range(batch.num_rows)]).astype(np.int64)
    cu = np.zeros(batch.num_rows + 1, np.int32)
    cu[1:] = np.cumsum(n)
    t = batch.tokens
    from workloads.configs import Tokens
    return Tokens(qkv=t.qkv[idx], g=t.g[idx], beta=t.beta[idx], H=t.H), cu


def commit_bitexact_vs_recurrent(batch, pool_np, nacc):
    say(f"case bitexact {batch.name} B={batch.num_rows} H={batch.H}")
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    cu = to_dev(batch.cu_seqlens)
    si = to_dev(batch.state_indices)
    pool_a = to_dev(pool_np)
    pool_b = pool_a.clone()
    rec = dev_records(batch.num_rows, batch.H, batch.Q)
    o = torch.empty((batch.tokens.num_tokens, batch.H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify(L, *toks.args(), cu, pool_a, si, rec, o)
    kda.kda_commit(L, cu, pool_a, si, rec, to_dev(nacc.astype(np.int32)))
    ptoks, pcu = _gather_prefix(batch, nacc)
    dt = DevTokens(ptoks)
    po = torch.empty((max(ptoks.num_tokens, 1), batch.H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_recurrent(L, *dt.args(), to_dev(pcu), pool_b, si, po[:ptoks.num_tokens])
    torch.cuda.synchronize()
    assert torch.equal(pool_a.view(torch.int32), pool_b.view(torch.int32)), \
        "commit differs from the recurrence over the accepted prefix"


@pytest.mark.parametrize("name,B,H", [("tiny", None, None), ("ragged", 24, 4), ("deep", 6, 4)])
def test_commit_bitexact_vs_recurrent_small(name, B, H):
    batch = make_batch(name, B=B, H=H)
    commit_bitexact_vs_recurrent(batch, oracle_prefill_pool(batch), batch.num_accepted)


def test_commit_edge_counts():
    # negative, zero and too-large accepted counts clamp; n' = 0 leaves the
    # pool bitwise untouched.
    batch = make_batch("ragged", B=16, H=4)
    pool = batch.initial_pool()
    nacc = np.array([-5, 0, 1, 100, 3, 0, 8, 2, -1, 7, 4, 0, 9, 1, 2, 3], np.int32)
    run_verify_commit(batch, pool, nacc=nacc)
    commit_bitexact_vs_recurrent(batch, pool, nacc)
    zero = np.zeros(16, np.int32)
    L = dev_layer(batch)
    p = to_dev(pool)
    rec = dev_records(16, 4, 8)
    kda.kda_commit(L, to_dev(batch.cu_seqlens), p, to_dev(batch.state_indices), rec, to_dev(zero))
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), pool)


def test_bad_metadata_is_skipped_safely():
    # out-of-range slots, record rows and spans are skipped by the kernels'
    # own range checks: no access outside the buffers, nothing written.
    batch = make_batch("tiny", B=4, H=4)
    say("case bad metadata")
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    pool_np = batch.initial_pool()
    pool = to_dev(pool_np)
    si = to_dev(np.array([1, 99, -7, 3], np.int32))            # 99 >= num_slots
    cu = to_dev(np.array([0, 4, 8, 12, 400], np.int32))        # last span beyond the tokens
    rec = dev_records(4, 4, 4, fill=SENT)
    rr = to_dev(np.array([0, 1, 2, 50], np.int32))             # 50 >= rows: scratch
    o = torch.zeros((16, 4, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify(L, *toks.args(), cu, pool, si, rec, o, record_rows=rr)
    kda.kda_recurrent(L, *toks.args(), cu, pool, si, o)
    torch.cuda.synchronize()
    after = pool.cpu().numpy()
    assert not np.array_equal(after[1], pool_np[1])              # row 0 ran
    for s in (0, 2, 3, 4):
        assert np.array_equal(after[s], pool_np[s])
    oh = bits_host(o)
    assert np.all(oh[4:12] == 0)                                 # rows 1, 2 skipped
    assert np.all(oh[12:] == 0)                                  # row 3: span out of range


def test_empty_and_window_longer_than_records():
    # T_i > Q: o for every token, records for the first Q only.
    batch = make_batch("ragged", B=10, H=4)
    say("case window > records")
    Q = 4
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    pool_np = batch.initial_pool()
    pool = to_dev(pool_np)
    rec = dev_records(10, 4, Q, fill=SENT)
    ntok = batch.tokens.num_tokens
    o = torch.zeros((ntok, 4, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify(L, *toks.args(), to_dev(batch.cu_seqlens), pool, to_dev(batch.state_indices), rec, o)
    torch.cuda.synchronize()
    t = batch.tokens
    rec_ref = oracle_records(10, 4, Q, fill=SENT)
    o_ref = np.zeros((ntok, 4, 128), np.uint16)
    ref.kda_verify(oracle_layer(batch), t.q, t.k, t.v, t.g, t.beta, batch.cu_seqlens,
                   pool_np.copy(), batch.state_indices, rec_ref, o_ref)
    rg = records_host(rec)
    assert np.array_equal(rg.k, rec_ref.k) and np.array_equal(rg.v, rec_ref.v)
    assert np.array_equal(rg.g, rec_ref.g) and np.array_equal(rg.beta, rec_ref.beta)
    check_o(bits_host(o), o_ref)
    # an empty batch is a no-op
    kda.kda_verify(L, *toks.args(), to_dev(np.zeros(1, np.int32)), pool,
                   to_dev(np.zeros(0, np.int32)), rec, o)
    torch.cuda.synchronize()


# --------------------------------------------------------- full size ----

_POOL_CACHE = {}
FULL_SIZE = ["decode", "decode_bounded", "deep", "ragged"]


def full_pool(batch):
    key = (batch.name, batch.lower_bound)
    if key not in _POOL_CACHE:
        say(f"oracle checkpoints for {batch.name} (B={batch.num_rows}, H={batch.H})")
        _POOL_CACHE[key] = oracle_prefill_pool(batch)
    return _POOL_CACHE[key]


def sampled_rows(batch, seed, n=32):
    """At least n rows, always the first and the last (every row when there
    are no more than n)."""
    B = batch.num_rows
    if B <= n:
        return list(range(B))
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, B - 1), size=n - 2, replace=False)
    return sorted([0, B - 1, *inner.tolist()])


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_sampled_parity(name):
    batch = make_batch(name)
    run_verify_commit(batch, full_pool(batch), sample_rows=sampled_rows(batch, 99))


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_sampled_parity_bench_launch(name):
    """The benchmark's kernels against the oracle at full size: the verify
    with the window bound (short kernels, predicted spans) and the commit
    through the multi-layer kernel, on sampled rows."""
    batch = make_batch(name)
    run_verify_commit(batch, full_pool(batch), sample_rows=sampled_rows(batch, 98),
                      bench_launch=True)


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_commit_bitexact(name):
    batch = make_batch(name)
    commit_bitexact_vs_recurrent(batch, full_pool(batch), batch.num_accepted)


@pytest.mark.parametrize("name", FULL_SIZE)
def test_verify_outputs_match_recurrent_outputs(name):
    """kda_verify (the chunked form against the checkpoint) and kda_recurrent
    (the per-token loop) compute the same window from the same checkpoints:
    every output within the output tolerance (the sums run in different
    orders, so not bit for bit)."""
    batch = make_batch(name)
    say(f"verify vs recurrent outputs: {name}")
    B, H, Q = batch.num_rows, batch.H, batch.Q
    pool_np = batch.initial_pool()
    if not pool_np.any():   # checkpoints made by a prefill: use N(0, 0.02) states instead
        rng = np.random.default_rng(17)
        for s in batch.state_indices[batch.state_indices > 0]:
            pool_np[s] = rng.standard_normal(pool_np.shape[1:], dtype=np.float32) * np.float32(0.02)
    ntok = batch.tokens.num_tokens
    layer = dev_layer(batch)
    tok = DevTokens(batch.tokens)
    cu, si = to_dev(batch.cu_seqlens), to_dev(batch.state_indices)
    pool = to_dev(pool_np)
    o_v = torch.zeros((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
    o_r = torch.zeros_like(o_v)
    kda.kda_verify(layer, *tok.args(), cu, pool, si, dev_records(B, H, Q), o_v)
    kda.kda_recurrent(layer, *tok.args(), cu, pool.clone(), si, o_r)
    torch.cuda.synchronize()
    check_o(bits_host(o_v), bits_host(o_r), what=f"{name}: verify o vs recurrent o")


def test_debug_validation_checks_rows_before_the_launch(monkeypatch):
    """With the debug check on (KDA_DEBUG_VALIDATE=1 at import), a call whose
    rows break a precondition raises before anything is enqueued; good rows
    run as usual."""
    import linear_attention_speculative_kda_amd.kda as kda_mod
    monkeypatch.setattr(kda_mod, "_DEBUG_VALIDATE", True)
    batch = make_batch("tiny", B=4, H=4)
    say("case debug validation")
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    pool_np = batch.initial_pool()
    pool = to_dev(pool_np)
    cu = to_dev(batch.cu_seqlens)
    rec = dev_records(4, 4, 4, fill=SENT)
    o = torch.zeros((16, 4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kda.KdaError, match="row 3: slot shared"):
        kda.kda_verify(L, *toks.args(), cu, pool, to_dev(np.array([1, 2, 3, 1], np.int32)), rec, o)
    with pytest.raises(kda.KdaError, match="window longer"):
        kda.kda_verify(L, *toks.args(), cu, pool, to_dev(batch.state_indices), rec, o, max_seqlen=3)
    with pytest.raises(kda.KdaError, match="record row"):
        kda.kda_commit(L, cu, pool, to_dev(batch.state_indices), rec, to_dev(batch.num_accepted),
                       record_rows=to_dev(np.array([0, 1, 1, 2], np.int32)))
    torch.cuda.synchronize()
    assert np.all(bits_host(o) == 0), "a rejected call wrote o"
    assert np.array_equal(pool.cpu().numpy(), pool_np), "a rejected call wrote the pool"
    kda.kda_verify(L, *toks.args(), cu, pool, to_dev(batch.state_indices), rec, o, max_seqlen=4)
    kda.kda_commit(L, cu, pool, to_dev(batch.state_indices), rec, to_dev(batch.num_accepted))
    torch.cuda.synchronize()
