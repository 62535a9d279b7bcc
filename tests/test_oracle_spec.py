"""Pins of the oracle's stock speculative step (every verified token's state
stored) and of the align-mode deferred commit: a hand-worked table of the
stock step's column rules, the dense product form of the recurrence for the
stored states, and the already-pinned plain and align commits."""

import math
import os

import numpy as np
import pytest

from oracle import kda_ref as ref
from workloads import make_batch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(x):
    return ref.f64_to_bf16_bits(np.asarray(x, np.float64))


def _golden_columns():
    rows = []
    for line in open(os.path.join(GOLDEN, "spec_columns.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("|")
        l = [int(x) for x in left.split()]
        r = right.split()
        written = {} if r[1] == "-" else {int(a): int(b) for a, b in (w.split(":") for w in r[1:])}
        rows.append(dict(T=l[1], acc=l[2], table=l[3:7], src=int(r[0]), written=written))
    return rows


def _inputs(ntok, H, K, seed, lower_bound=None):
    rng = np.random.default_rng(seed)
    layer = ref.Layer(a_log=np.log(rng.uniform(1, 16, H)).astype(np.float32),
                      g_bias=(rng.standard_normal(H * K) * 0.1).astype(np.float32),
                      scale=float(np.float32(K ** -0.5)), lower_bound=lower_bound)
    q, k, v, g = (_bits(rng.standard_normal((ntok, H, K))) for _ in range(4))
    beta = _bits(rng.standard_normal((ntok, H)))
    return layer, (q, k, v, g, beta)


def test_spec_columns_golden():
    """Which block holds the state after how many tokens: the hand-worked
    table; each stored state equals the plain recurrence over that many of
    the row's tokens from the source block; nothing else is written."""
    rows = _golden_columns()
    N, H, K, nslots = len(rows), 2, 8, 40
    T = np.array([r["T"] for r in rows])
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(T)
    ntok = int(cu[-1])
    layer, toks = _inputs(ntok, H, K, 11)
    rng = np.random.default_rng(12)
    pool0 = (rng.standard_normal((nslots, H, K, K)) * 0.3).astype(np.float32)
    pool = pool0.copy()
    table = np.array([r["table"] for r in rows], np.int32)
    acc = np.array([r["acc"] for r in rows], np.int32)
    o = np.full((ntok, H, K), 0x7E7E, np.uint16)
    ref.kda_recurrent_spec(layer, *toks, cu, pool, table, acc, o)
    written = set()
    for i, r in enumerate(rows):
        assert ref.spec_source_column(acc, i, 4) in range(4)
        src = int(table[i, ref.spec_source_column(acc, i, 4)])
        assert src == r["src"] or not 0 < src < nslots, f"row {i}: source {src}"
        for blk, n in r["written"].items():
            # the recurrence over the row's first n tokens from the source
            sub = np.zeros((nslots, H, K, K), np.float32)
            sub[1] = pool0[r["src"]]
            oo = np.zeros((ntok, H, K), np.uint16)
            ref.kda_recurrent(layer, *toks, np.array([cu[i], cu[i] + n], np.int32), sub,
                              np.array([1], np.int32), oo)
            assert np.array_equal(pool[blk], sub[1]), f"row {i}: block {blk} after {n} tokens"
            written.add(blk)
        span = slice(cu[i], cu[i + 1])
        if r["written"] or (r["src"] > 0 and r["T"] > 0):
            assert np.all(o[span] != 0x7E7E), f"row {i}: outputs missing"
        else:
            assert np.all(o[span] == 0x7E7E), f"row {i}: outputs of a skipped row"
    for blk in range(nslots):
        if blk not in written:
            assert np.array_equal(pool[blk], pool0[blk]), f"block {blk} written"


@pytest.mark.parametrize("lower_bound", [None, -5.0])
def test_spec_states_and_outputs_match_product_form(lower_bound):
    """The stored states and the outputs against the dense product form of
    the recurrence, built from the page's definitions of q^, k^, g, beta."""
    K, H, T = 4, 2, 3
    layer, (q, k, v, g, beta) = _inputs(T, H, K, 21, lower_bound)
    rng = np.random.default_rng(22)
    pool0 = (rng.standard_normal((6, H, K, K)) * 0.3).astype(np.float32)
    pool = pool0.copy()
    table = np.array([[3, 2, 0, 5]], np.int32)      # source column 1 (two accepted): block 2
    o = np.zeros((T, H, K), np.uint16)
    ref.kda_recurrent_spec(layer, q, k, v, g, beta, np.array([0, T], np.int32), pool, table,
                           np.array([2], np.int32), o)
    f = ref.bf16_bits_to_f64
    for h in range(H):
        qh = np.stack([f(q[t, h]) / math.sqrt(np.sum(f(q[t, h]) ** 2) + 1e-6)
                       * float(np.float32(layer.scale)) for t in range(T)])
        kh = np.stack([f(k[t, h]) / math.sqrt(np.sum(f(k[t, h]) ** 2) + 1e-6) for t in range(T)])
        x = f(g[:, h]) + layer.g_bias.reshape(H, K)[h].astype(np.float64)
        A = math.exp(float(layer.a_log[h]))
        gg = -A * np.log1p(np.exp(x)) if lower_bound is None else lower_bound / (1 + np.exp(-A * x))
        bb = 1 / (1 + np.exp(-f(beta[:, h])))
        S0 = pool0[2, h].astype(np.float64).T
        states, outs = [], []
        for n in range(1, T + 1):
            P = [(np.eye(K) - bb[t] * np.outer(kh[t], kh[t])) @ np.diag(np.exp(gg[t])) for t in range(n)]
            M = np.eye(K)
            for t in range(n):
                M = P[t] @ M
            Sn = M @ S0
            for t in range(n):
                Lm = np.eye(K)
                for s in range(t + 1, n):
                    Lm = P[s] @ Lm
                Sn = Sn + Lm @ (bb[t] * np.outer(kh[t], f(v[t, h])))
            states.append(Sn)
            outs.append(Sn.T @ qh[n - 1])
        assert np.allclose(pool[3, h].T, states[0], rtol=1e-6, atol=1e-7)    # column 0: 1 token
        assert np.allclose(pool[2, h].T, states[1], rtol=1e-6, atol=1e-7)    # column 1: 2 tokens
        for t in range(T):
            assert np.array_equal(o[t, h], ref.f64_to_bf16_bits(outs[t]))
    for blk in (0, 1, 4, 5):   # column 2 is null; column 3 (block 5) has no fourth token
        assert np.array_equal(pool[blk], pool0[blk])


def test_spec_last_column_equals_the_plain_recurrence():
    """A full window with every column set: column T - 1 holds the state the
    plain recurrence stores, and the outputs are the plain recurrence's."""
    b = make_batch("tiny")
    layer = ref.Layer(b.a_log, b.g_bias, b.scale, b.lower_bound)
    t = b.tokens
    N, Tn = b.num_rows, 4
    pool0 = b.initial_pool()
    nslots = 1 + N + N * Tn
    pool_s = np.zeros((nslots,) + pool0.shape[1:], np.float32)
    pool_s[:b.num_slots] = pool0
    table = np.zeros((N, Tn), np.int32)
    for i in range(N):
        table[i] = b.num_slots + i * Tn + np.arange(Tn)
        table[i, 0] = b.state_indices[i]           # source in column 0 (one accepted)
    o_s = np.zeros((t.num_tokens, b.H, 128), np.uint16)
    ref.kda_recurrent_spec(layer, t.q, t.k, t.v, t.g, t.beta, b.cu_seqlens, pool_s, table,
                           np.ones(N, np.int32), o_s)
    pool_r = pool0.copy()
    o_r = np.zeros_like(o_s)
    ref.kda_recurrent(layer, t.q, t.k, t.v, t.g, t.beta, b.cu_seqlens, pool_r, b.state_indices, o_r)
    assert np.array_equal(o_s, o_r)
    for i in range(N):
        assert np.array_equal(pool_s[table[i, Tn - 1]], pool_r[b.state_indices[i]])


# ------------------------------------------------- align + deferred commit --

def _align_case():
    b = make_batch("tiny")
    layer = ref.Layer(b.a_log, b.g_bias, b.scale, b.lower_bound)
    t = b.tokens
    ntok = t.num_tokens
    pool = np.zeros((32, b.H, b.K, b.K), np.float32)
    pool[:b.num_slots] = b.initial_pool()
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K)
    o = np.zeros((ntok, b.H, b.K), np.uint16)
    ref.kda_verify(layer, t.q, t.k, t.v, t.g, t.beta, b.cu_seqlens, pool, b.state_indices, rec, o)
    nacc = np.array([3, 1, 4, 2], np.int32)
    # row 0 crosses a boundary, rows 1 and 3 stay in their source block, row 2
    # ends in another block
    bt = np.array([[20, 21], [2, 22], [23, 24], [4, 25]], np.int32)
    al = ref.Align(bt, np.array([2, 0, 4, 1], np.int32), 4)
    return b, layer, pool, rec, ntok, nacc, al


@pytest.mark.parametrize("eager", [[1, 1, 1, 1], [0, 0, 0, 0], [1, 0, 1, 0], [0, 1, 0, 1]])
@pytest.mark.parametrize("bad_slot", [False, True])
def test_align_deferred_commit_against_align_and_deferred(eager, bad_slot):
    """Eager rows commit exactly as the align commit does; the others leave
    the pool alone and leave their n' in pending (what the plain deferred
    commit writes, also for a row whose slot is outside the pool)."""
    b, layer, pool, rec, ntok, nacc, al = _align_case()
    if bad_slot:
        b.state_indices = b.state_indices.copy()
        b.state_indices[2] = 99
    eager = np.array(eager, np.uint8)
    full = pool.copy()
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, full, b.state_indices, rec, nacc, al)
    got = pool.copy()
    pend = np.full(b.num_rows, -9, np.int32)
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, got, b.state_indices, rec, nacc, al,
                         pending=pend, eager=eager)
    # pending as the plain deferred commit writes it
    p2 = np.full(b.num_rows, -9, np.int32)
    ref.kda_commit(layer, b.cu_seqlens, ntok, pool.copy(), b.state_indices, rec, nacc,
                   pending=p2, eager=eager)
    assert np.array_equal(pend, p2)
    plan = ref.commit_plan(b.cu_seqlens, ntok, nacc, b.state_indices, b.Q, al)
    touched = set()
    for i in range(b.num_rows):
        n, final, bnd, blen = (int(x) for x in plan[i])
        blocks = {final} | ({bnd} if 0 < blen < n and bnd > 0 else set())
        touched |= blocks
        for blk in blocks:
            want = full[blk] if eager[i] else pool[blk]
            assert np.array_equal(got[blk], want), f"row {i} block {blk}"
    for blk in range(pool.shape[0]):
        if blk not in touched:
            assert np.array_equal(got[blk], pool[blk])


def test_align_deferred_rows_fold_in_place():
    """A deferred row whose final block is its source and that crosses no
    boundary: the later fold (the flush) gives the align commit's state."""
    b, layer, pool, rec, ntok, nacc, al = _align_case()
    full = pool.copy()
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, full, b.state_indices, rec, nacc, al)
    got = pool.copy()
    pend = np.zeros(b.num_rows, np.int32)
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, got, b.state_indices, rec, nacc, al,
                         pending=pend, eager=np.zeros(b.num_rows, np.uint8))
    empty = np.zeros((0, b.H, b.K), np.uint16)
    ref.kda_verify_deferred(layer, empty, empty, empty, empty, np.zeros((0, b.H), np.uint16),
                            np.zeros(b.num_rows + 1, np.int32), got, b.state_indices, rec, pend,
                            ref.Records.empty(b.num_rows, b.H, b.Q, b.K), None, empty)
    for i in (1, 3):   # final block == source, no boundary
        s = int(b.state_indices[i])
        assert np.array_equal(got[s], full[s]), f"row {i}"
