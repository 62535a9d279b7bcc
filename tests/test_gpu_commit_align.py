"""GPU parity of the align-mode commit and of the conv-state compaction
against the oracle (commit_plan, kda_commit_align, conv_compact)."""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_deferred

from .helpers import DevTokens, check_state, dev_records, records_host, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _align_inputs(B, rng):
    """Block tables whose blocks (>= 100) are no row's source, cached counts
    that cross a block boundary on some rows and not on others, and a few
    null final blocks."""
    width, bs = 4, 2
    bt = np.array([[100 + width * i + c for c in range(width)] for i in range(B)], np.int32)
    cached = rng.integers(-1, 9, size=B).astype(np.int32)
    bt[3, :] = 0                      # row 3: null blocks everywhere
    return bt, cached, bs


@pytest.mark.parametrize("layers", [1, 3])
def test_commit_align_against_oracle(layers):
    B, H = 12, 4
    say(f"align commit vs oracle: B={B} H={H} layers={layers}")
    run = make_deferred(B=B, H=H, layers=layers, steps=1)
    rng = np.random.default_rng(11)
    bt, cached, bs = _align_inputs(B, rng)
    nblocks = 100 + 4 * B
    si, cu = to_dev(run.state_indices), to_dev(run.cu_seqlens)
    nacc_np = run.num_accepted(0)
    Ls, pools0, recs = [], [], []
    for l in range(layers):
        p = run.params[l]
        Ls.append(kda.Layer(a_log=to_dev(p.a_log), g_bias=to_dev(p.g_bias), scale=run.scale,
                            lower_bound=run.lower_bound))
        pool = np.zeros((nblocks, H, 128, 128), np.float32)
        pool[:run.num_slots] = run.initial_pool(l)
        pools0.append(pool)
        rec = dev_records(B, H, run.Q)
        o = torch.empty((B * run.T, H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_verify(Ls[l], *DevTokens(run.tokens(l, 0)).args(), cu, to_dev(pool), si, rec, o)
        recs.append(rec)
    pools = [to_dev(p) for p in pools0]
    al = kda.Align(to_dev(bt), to_dev(cached), bs)
    kda.kda_commit_layers(Ls, cu, pools, si, recs, to_dev(nacc_np), align=al)
    torch.cuda.synchronize()
    oal = ref.Align(bt, cached, bs)
    plan = ref.commit_plan(run.cu_seqlens, B * run.T, nacc_np, run.state_indices, run.Q, oal)
    say(f"  plan rows with a boundary store: {int(np.sum((plan[:, 3] < plan[:, 0]) & (plan[:, 2] > 0)))}")
    for l in range(layers):
        p = run.params[l]
        want = pools0[l].copy()
        ref.kda_commit_align(ref.Layer(p.a_log, p.g_bias, run.scale, run.lower_bound),
                             run.cu_seqlens, B * run.T, want, run.state_indices,
                             records_host(recs[l]), nacc_np, oal)
        got = pools[l].cpu().numpy()
        written = {int(b) for b in np.flatnonzero(np.any(want != pools0[l], axis=(1, 2, 3)))}
        for b in written:
            check_state(got[b], want[b], what=f"layer {l} block {b}")
        for b in range(nblocks):
            if b not in written:
                assert np.array_equal(got[b], pools0[l][b]), f"layer {l} block {b} written"


@pytest.mark.parametrize("B,H,layers", [(12, 4, 1), (12, 4, 3), (2049, 1, 1)])
def test_commit_align_deferred_against_oracle(B, H, layers):
    """The deferred commit in align mode: the eager rows commit into their
    align blocks now, the others only record their counts (row list for up
    to 2048 rows, the full grid beyond)."""
    say(f"align deferred commit vs oracle: B={B} H={H} layers={layers}")
    run = make_deferred(B=B, H=H, layers=layers, steps=1)
    rng = np.random.default_rng(12)
    width, bs = 4, 2
    nblocks = run.num_slots + width * B
    bt = (run.num_slots + np.arange(B * width, dtype=np.int32)).reshape(B, width)
    bt[3, :] = 0
    cached = rng.integers(-1, 9, size=B).astype(np.int32)
    eager = (rng.random(B) < 0.5).astype(np.uint8)
    si, cu, rr = to_dev(run.state_indices), to_dev(run.cu_seqlens), to_dev(run.record_rows)
    nacc_np = run.num_accepted(0)
    Ls, pools0, recs = [], [], []
    for l in range(layers):
        p = run.params[l]
        Ls.append(kda.Layer(a_log=to_dev(p.a_log), g_bias=to_dev(p.g_bias), scale=run.scale,
                            lower_bound=run.lower_bound))
        pool = np.zeros((nblocks, H, 128, 128), np.float32)
        pool[:run.num_slots] = run.initial_pool(l)
        pools0.append(pool)
        rec = dev_records(B, H, run.Q)
        o = torch.empty((B * run.T, H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_verify(Ls[l], *DevTokens(run.tokens(l, 0)).args(), cu, to_dev(pool), si, rec, o,
                       record_rows=rr)
        recs.append(rec)
    pools = [to_dev(p) for p in pools0]
    pending = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    al = kda.Align(to_dev(bt), to_dev(cached), bs)
    kda.kda_commit_layers(Ls, cu, pools, si, recs, to_dev(nacc_np), record_rows=rr,
                          pending=pending, eager=to_dev(eager), align=al)
    torch.cuda.synchronize()
    oal = ref.Align(bt, cached, bs)
    want_pending = np.full(B, -9, np.int32)
    for l in range(layers):
        p = run.params[l]
        want = pools0[l].copy()
        ref.kda_commit_align(ref.Layer(p.a_log, p.g_bias, run.scale, run.lower_bound),
                             run.cu_seqlens, B * run.T, want, run.state_indices,
                             records_host(recs[l]), nacc_np, oal, record_rows=run.record_rows,
                             pending=want_pending, eager=eager)
        got = pools[l].cpu().numpy()
        written = np.flatnonzero(np.any(want != pools0[l], axis=(1, 2, 3)))
        say(f"  layer {l}: {len(written)} blocks written by eager rows")
        for b in written:
            check_state(got[b], want[b], what=f"layer {l} block {b}")
        same = np.ones(nblocks, bool)
        same[written] = False
        assert np.array_equal(got[same], pools0[l][same]), f"layer {l}: a block no row writes changed"
    assert np.array_equal(pending.cpu().numpy(), want_pending), "pending counts"


def test_commit_align_bits_equal_prefix_commits():
    """The final block holds the bits of a plain commit of n' records, the
    boundary block those of a plain commit of the boundary length."""
    B, H = 10, 2
    run = make_deferred(B=B, H=H, layers=1, steps=1)
    rng = np.random.default_rng(4)
    bt, cached, bs = _align_inputs(B, rng)
    nblocks = 100 + 4 * B
    si, cu = to_dev(run.state_indices), to_dev(run.cu_seqlens)
    p = run.params[0]
    L = kda.Layer(a_log=to_dev(p.a_log), g_bias=to_dev(p.g_bias), scale=run.scale,
                  lower_bound=run.lower_bound)
    pool0 = np.zeros((nblocks, H, 128, 128), np.float32)
    pool0[:run.num_slots] = run.initial_pool(0)
    rec = dev_records(B, H, run.Q)
    o = torch.empty((B * run.T, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_verify(L, *DevTokens(run.tokens(0, 0)).args(), cu, to_dev(pool0), si, rec, o)
    nacc_np = np.full(B, run.Q, np.int32)
    work = to_dev(pool0)
    kda.kda_commit_layers([L], cu, [work], si, [rec], to_dev(nacc_np), align=kda.Align(to_dev(bt), to_dev(cached), bs))
    plan = ref.commit_plan(run.cu_seqlens, B * run.T, nacc_np, run.state_indices, run.Q,
                           ref.Align(bt, cached, bs))
    got = work.cpu().numpy()
    for i in range(B):
        n, final, bnd, blen = (int(x) for x in plan[i])
        if n == 0 or final == 0:
            continue
        for length, block in ((n, final), (blen, bnd)):
            # a boundary store happens only below n'; when the boundary block
            # is the final block (its column clamped to the table), the final
            # state, stored last, is what it holds
            if block == 0 or (length != n and (length > n or block == final)):
                continue
            plain = to_dev(pool0)
            acc = np.zeros(B, np.int32)
            acc[i] = length
            kda.kda_commit(L, cu, plain, si, rec, to_dev(acc))
            assert np.array_equal(got[block], plain.cpu().numpy()[run.state_indices[i]]), \
                f"row {i} block {block} after {length} records"


@pytest.mark.parametrize("aligned", [False, True])
def test_conv_compact_against_oracle(aligned):
    B, layers, dim, hist, Q = 40, 3, 300, 3, 4
    width = Q + hist - 1
    say(f"conv compaction vs oracle: B={B} layers={layers} dim={dim} align={aligned}")
    rng = np.random.default_rng(7)
    blocks = 100 + 4 * B if aligned else B + 1
    src = rng.permutation(np.arange(1, B + 1)).astype(np.int32)
    src[[5, 9]] = [0, -2]
    T = rng.integers(0, Q + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    nacc = rng.integers(-1, Q + 2, size=B).astype(np.int32)
    al_np, al_dev = None, None
    if aligned:
        bt, cached, bs = _align_inputs(B, rng)
        al_np = ref.Align(bt, cached, bs)
        al_dev = kda.Align(to_dev(bt), to_dev(cached), bs)
    states0, devs = [], []
    for l in range(layers):
        c = rng.integers(0, 1 << 16, size=(blocks, dim, width), dtype=np.uint16)
        states0.append(c)
        if l == 1:   # tokens-major storage: [blocks, width, dim] viewed as [blocks, dim, width]
            d = to_dev(np.ascontiguousarray(c.transpose(0, 2, 1)).view(np.int16)).transpose(1, 2)
        else:
            d = to_dev(c.view(np.int16))
        devs.append(d)
    kda.kda_conv_compact(devs, to_dev(cu), to_dev(src), to_dev(nacc), Q, hist, align=al_dev)
    torch.cuda.synchronize()
    for l in range(layers):
        want = states0[l].copy()
        ref.conv_compact(want, cu, int(cu[-1]), nacc, src, Q, hist, al_np)
        got = devs[l].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"layer {l}: {np.argwhere(got != want)[:5].tolist()}"


@pytest.mark.parametrize("dim,hist,Q", [(300, 3, 4), (2500, 3, 4), (2056, 4, 8), (301, 3, 4),
                                        (4096, 1, 4)])
def test_conv_compact_dense_layers(dim, hist, Q):
    """Every layer in the dense [blocks, channels, width] layout, in place:
    the span kernel when channels x width is a whole number of 16-byte
    units (one or several spans per row, a short last span), else the
    per-channel kernel; bitwise against the oracle either way."""
    B, layers = 24, 2
    width = Q + hist - 1
    say(f"conv compaction dense layers: dim={dim} hist={hist} Q={Q} width={width}")
    rng = np.random.default_rng(dim + hist)
    blocks = B + 3
    src = rng.permutation(np.arange(1, B + 1)).astype(np.int32)
    src[[2, 7]] = [0, -1]
    T = rng.integers(0, Q + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    nacc = rng.integers(-1, Q + 2, size=B).astype(np.int32)
    states0 = [rng.integers(0, 1 << 16, size=(blocks, dim, width), dtype=np.uint16)
               for _ in range(layers)]
    devs = [to_dev(c.view(np.int16)) for c in states0]
    kda.kda_conv_compact(devs, to_dev(cu), to_dev(src), to_dev(nacc), Q, hist)
    torch.cuda.synchronize()
    for l in range(layers):
        want = states0[l].copy()
        ref.conv_compact(want, cu, int(cu[-1]), nacc, src, Q, hist)
        got = devs[l].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"layer {l}: {np.argwhere(got != want)[:5].tolist()}"


def test_conv_compact_padded_blocks():
    """Dense rows inside blocks with padding between them (the block stride
    longer than channels x width) and a misaligned start: the span kernel
    for the first, the per-channel kernel for the second; the padding and
    everything outside the moved columns keep their bits."""
    B, dim, hist, Q = 12, 1024, 3, 4
    width = Q + hist - 1
    rng = np.random.default_rng(23)
    blocks = B + 2
    src = rng.permutation(np.arange(1, B + 1)).astype(np.int32)
    T = rng.integers(0, Q + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    nacc = rng.integers(-1, Q + 2, size=B).astype(np.int32)
    for pad, offset in ((8, 0), (8, 1)):
        say(f"conv compaction padded blocks: pad={pad} offset={offset}")
        stride = dim * width + pad
        flat0 = rng.integers(0, 1 << 16, size=blocks * stride + offset, dtype=np.uint16)
        flat = to_dev(flat0.view(np.int16))
        view = torch.as_strided(flat, (blocks, dim, width), (stride, width, 1), offset)
        kda.kda_conv_compact([view], to_dev(cu), to_dev(src), to_dev(nacc), Q, hist)
        torch.cuda.synchronize()
        want_flat = flat0.copy()
        want = np.lib.stride_tricks.as_strided(want_flat[offset:], (blocks, dim, width),
                                               (stride * 2, width * 2, 2))
        tmp = np.ascontiguousarray(want)
        ref.conv_compact(tmp, cu, int(cu[-1]), nacc, src, Q, hist)
        want[...] = tmp
        got = flat.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want_flat), f"pad={pad} offset={offset}: {np.argwhere(got != want_flat)[:5].tolist()}"
