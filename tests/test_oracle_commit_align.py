"""Pins of the oracle's commit plan, align-mode commit and conv-state
compaction, against values worked by hand from the pages (a golden file),
closed forms, and the already-pinned plain commit."""

import os

import numpy as np
import pytest

from oracle import kda_ref as ref
from workloads import make_batch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_plan():
    rows = []
    for line in open(os.path.join(GOLDEN, "commit_plan_align.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        left, right = line.split("|")
        rows.append(([int(x) for x in left.split()], [int(x) for x in right.split()]))
    return rows


def test_commit_plan_align_golden():
    rows = _golden_plan()
    N = len(rows)
    src = np.array([r[0][1] for r in rows], np.int32)
    cached = np.array([r[0][2] for r in rows], np.int32)
    nacc = np.array([r[0][3] for r in rows], np.int32)
    bt = np.array([[100 * i + c + 1 for c in range(4)] for i in range(N)], np.int32)
    cu = (np.arange(N + 1) * 4).astype(np.int32)
    plan = ref.commit_plan(cu, 4 * N, nacc, src, 4, ref.Align(bt, cached, 4))
    want = np.array([r[1] for r in rows], np.int64)
    assert np.array_equal(plan, want), np.argwhere(plan != want)


def test_commit_plan_without_align_is_in_place():
    rows = _golden_plan()
    N = len(rows)
    src = np.array([r[0][1] for r in rows], np.int32)
    nacc = np.array([r[0][3] for r in rows], np.int32)
    cu = (np.arange(N + 1) * 4).astype(np.int32)
    plan = ref.commit_plan(cu, 4 * N, nacc, src, 4)
    for i, (inp, out) in enumerate(rows):
        n = out[0]
        assert tuple(plan[i]) == ((n, src[i], 0, 0) if n > 0 else (0, 0, 0, 0))


def test_commit_plan_short_rows_clamp_to_their_span():
    # T_i = 1: n' <= 1 whatever was accepted; the final column follows n'.
    cu = np.array([0, 1, 2], np.int32)
    bt = np.array([[11, 12, 13], [21, 22, 23]], np.int32)
    plan = ref.commit_plan(cu, 2, np.array([4, 1], np.int32), np.array([5, 6], np.int32), 4,
                           ref.Align(bt, np.array([3, 4], np.int32), 2))
    # row 0: n' = 1, c = 3: final col 3 // 2 = 1, next 4 reached -> boundary col 1, length 1
    # row 1: n' = 1, c = 4: final col 4 // 2 = 2, next 6 not reached, length 2
    assert plan.tolist() == [[1, 12, 12, 1], [1, 23, 0, 2]]


# ---------------------------------------------------------- align commit --

def _tiny_with_records():
    b = make_batch("tiny")
    layer = ref.Layer(b.a_log, b.g_bias, b.scale, b.lower_bound)
    t = b.tokens
    toks = (t.q, t.k, t.v, t.g, t.beta)
    ntok = t.q.shape[0]
    pool = np.zeros((32, b.H, b.K, b.K), np.float32)
    pool[:b.num_slots] = b.initial_pool()
    rec = ref.Records.empty(b.num_rows, b.H, b.Q, b.K)
    o = np.zeros((ntok, b.H, b.K), np.uint16)
    ref.kda_verify(layer, *toks, b.cu_seqlens, pool, b.state_indices, rec, o)
    return b, layer, pool, rec, ntok


def _commit_prefix(layer, b, pool, rec, ntok, i, n):
    """The state of row i after its first n records, by the plain commit."""
    p = pool.copy()
    nacc = np.zeros(b.num_rows, np.int32)
    nacc[i] = n
    ref.kda_commit(layer, b.cu_seqlens, ntok, p, b.state_indices, rec, nacc)
    return p[b.state_indices[i]]


def test_commit_align_final_and_boundary_states():
    b, layer, pool, rec, ntok = _tiny_with_records()
    assert b.num_rows == 4 and b.Q == 4 and np.all(b.seq_lens() == 4)
    bt = np.array([[10 + 4 * i + c for c in range(4)] for i in range(4)], np.int32)
    cached = np.array([1, 2, 3, 0], np.int32)
    nacc = np.array([3, 2, 4, 1], np.int32)
    al = ref.Align(bt, cached, 2)
    # worked by hand (block size 2):
    #  row 0: c 1, n' 3 -> final col 1 (11), next 2 reached: boundary col 0 (10), length 1
    #  row 1: c 2, n' 2 -> final col 1 (15), next 4 reached: col 1 = final, length 2 = n'
    #  row 2: c 3, n' 4 -> final col 3 (21), next 4 reached: boundary col 1 (19), length 1
    #  row 3: c 0, n' 1 -> final col 0 (22), next 2 not reached
    plan = ref.commit_plan(b.cu_seqlens, ntok, nacc, b.state_indices, b.Q, al)
    assert plan.tolist() == [[3, 11, 10, 1], [2, 15, 15, 2], [4, 21, 19, 1], [1, 22, 0, 2]]
    work = pool.copy()
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, work, b.state_indices, rec, nacc, al)
    written = {11, 10, 15, 21, 19, 22}
    for i, (n, final, bnd, blen) in enumerate(plan.tolist()):
        assert np.array_equal(work[final], _commit_prefix(layer, b, pool, rec, ntok, i, n))
        if 0 < blen < n:
            assert np.array_equal(work[bnd], _commit_prefix(layer, b, pool, rec, ntok, i, blen))
    for s in range(32):
        if s not in written:
            assert np.array_equal(work[s], pool[s]), f"block {s} written"


def test_commit_align_in_place_equals_commit():
    # One block per request holding everything: final = source, no boundary.
    b, layer, pool, rec, ntok = _tiny_with_records()
    bt = np.zeros((4, 2), np.int32)
    bt[:, 0] = b.state_indices
    al = ref.Align(bt, np.zeros(4, np.int32), 64)
    nacc = np.array([4, 0, 2, 3], np.int32)
    a, p = pool.copy(), pool.copy()
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, a, b.state_indices, rec, nacc, al)
    ref.kda_commit(layer, b.cu_seqlens, ntok, p, b.state_indices, rec, nacc)
    assert np.array_equal(a, p)


def test_commit_align_null_final_block_skips_the_row():
    b, layer, pool, rec, ntok = _tiny_with_records()
    bt = np.array([[0, 0], [20, 21], [0, 22], [23, 0]], np.int32)
    al = ref.Align(bt, np.zeros(4, np.int32), 4)
    work = pool.copy()
    ref.kda_commit_align(layer, b.cu_seqlens, ntok, work, b.state_indices, rec,
                         np.array([2, 2, 2, 2], np.int32), al)
    changed = [s for s in range(32) if not np.array_equal(work[s], pool[s])]
    assert changed == [20, 23]


# ---------------------------------------------------------- conv compaction --

def _ramp(blocks=40, dim=3, width=6):
    b, d, c = np.meshgrid(np.arange(blocks), np.arange(dim), np.arange(width), indexing="ij")
    return (b * 100 + d * 10 + c).astype(np.float32)


def test_conv_compact_in_place_closed_form():
    conv = _ramp()
    conv0 = conv.copy()
    src = np.array([1, 2, 3, 4, 5, 0], np.int32)
    nacc = np.array([1, 2, 4, 0, 3, 2], np.int32)
    cu = (np.arange(7) * 4).astype(np.int32)
    ref.conv_compact(conv, cu, 24, nacc, src, Q=4, history=3)
    for i in range(6):
        s, n = int(src[i]), int(nacc[i])
        if s == 0:
            continue
        if n == 0:
            assert np.array_equal(conv[s], conv0[s])
            continue
        for d in range(3):
            assert conv[s, d, :3].tolist() == [s * 100 + d * 10 + n - 1 + j for j in range(3)]
            assert np.array_equal(conv[s, d, 3:], conv0[s, d, 3:])
    untouched = [x for x in range(40) if x not in (1, 2, 3, 5)]
    assert np.array_equal(conv[untouched], conv0[untouched])


def test_conv_compact_align_closed_form():
    conv = _ramp()
    conv0 = conv.copy()
    src = np.array([1, 2, 3], np.int32)
    nacc = np.array([3, 2, 4], np.int32)
    bt = np.array([[10, 11, 12, 13], [14, 15, 16, 17], [18, 19, 20, 21]], np.int32)
    al = ref.Align(bt, np.array([1, 2, 3], np.int32), 2)
    cu = np.array([0, 4, 8, 12], np.int32)
    ref.conv_compact(conv, cu, 12, nacc, src, Q=4, history=3, align=al)
    # rows as worked by hand in test_commit_align_final_and_boundary_states
    # (source, n', final, boundary, boundary length)
    for s, n, final, bnd, blen in ((1, 3, 11, 10, 1), (2, 2, 15, 15, 2), (3, 4, 21, 19, 1)):
        for d in range(3):
            assert conv[final, d, :3].tolist() == [s * 100 + d * 10 + n - 1 + j for j in range(3)]
            if bnd != final:
                assert conv[bnd, d, :3].tolist() == [s * 100 + d * 10 + blen - 1 + j for j in range(3)]
    assert np.array_equal(conv[1:4], conv0[1:4])          # sources are not destinations here
    assert np.array_equal(conv[22:], conv0[22:])


def test_conv_compact_copies_bits_exactly():
    rng = np.random.default_rng(3)
    conv = rng.integers(0, 1 << 16, size=(8, 5, 7), dtype=np.uint16)
    conv[2, 1, 3] = 0x7FC1                                  # a NaN payload
    conv0 = conv.copy()
    ref.conv_compact(conv, np.array([0, 4], np.int32), 4, np.array([4], np.int32),
                     np.array([2], np.int32), Q=4, history=4)
    assert np.array_equal(conv[2, :, :4], conv0[2, :, 3:7])
