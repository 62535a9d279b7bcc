"""GPU parity of the deferred commit: several layers, several steps, a pending
replay folded into the next verify, eager rows committed at once, and a
final flush; against the oracle's sequential (eager) replay and, bitwise,
against the GPU's own eager flow."""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_deferred

from .helpers import (DevTokens, bits_host, check_o, check_state, dev_records, oracle_records,
                      to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_layer(run, layer):
    p = run.params[layer]
    return kda.Layer(a_log=to_dev(p.a_log), g_bias=to_dev(p.g_bias), scale=run.scale,
                     lower_bound=run.lower_bound)


def gpu_flows(run, max_seqlen=None):
    """Run the deferred and the eager flow on the GPU; return per (layer, step)
    outputs and the final pools of both. max_seqlen: the eager verify's
    window bound (the short kernels), as the benchmark passes it."""
    B, H, Q = run.B, run.H, run.Q
    si = to_dev(run.state_indices)
    rr = to_dev(run.record_rows)
    cu = to_dev(run.cu_seqlens)
    layers = [dev_layer(run, l) for l in range(run.layers)]
    pools_d, pools_e = [], []
    for l in range(run.layers):
        p = to_dev(run.initial_pool(l))
        pools_d.append(p)
        pools_e.append(p.clone())
    recs_d = [[dev_records(B, H, Q), dev_records(B, H, Q)] for _ in range(run.layers)]
    recs_e = [dev_records(B, H, Q) for _ in range(run.layers)]
    pending = torch.zeros(B, dtype=torch.int32, device=DEV)
    outs_d, outs_e = {}, {}
    ntok = B * run.T
    for s in range(run.steps):
        nacc = to_dev(run.num_accepted(s))
        eager = to_dev(run.eager(s))
        toks = [DevTokens(run.tokens(l, s)) for l in range(run.layers)]
        for l in range(run.layers):
            od = torch.empty((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
            kda.kda_verify_deferred(layers[l], *toks[l].args(), cu, pools_d[l], si,
                                    recs_d[l][(s + 1) % 2], pending, recs_d[l][s % 2], od,
                                    record_rows=rr)
            oe = torch.empty_like(od)
            kda.kda_verify(layers[l], *toks[l].args(), cu, pools_e[l], si, recs_e[l], oe,
                           record_rows=rr, max_seqlen=max_seqlen)
            outs_d[l, s], outs_e[l, s] = od, oe
        for l in range(run.layers):
            kda.kda_commit(layers[l], cu, pools_d[l], si, recs_d[l][s % 2], nacc, record_rows=rr,
                           pending=pending, eager=eager)
            kda.kda_commit(layers[l], cu, pools_e[l], si, recs_e[l], nacc, record_rows=rr)
        torch.cuda.synchronize()
        # pending[r] = 0 for eager rows, n' otherwise
        n = np.minimum(np.maximum(run.num_accepted(s), 0), run.Q)
        want = np.zeros(B, np.int32)
        want[run.record_rows] = np.where(run.eager(s) != 0, 0, n)
        assert np.array_equal(pending.cpu().numpy(), want), f"pending after step {s}"
    last = (run.steps - 1) % 2
    for l in range(run.layers):
        kda.kda_flush(layers[l], pools_d[l], si, recs_d[l][last], pending, recs_d[l][1 - last],
                      record_rows=rr)
    torch.cuda.synchronize()
    return outs_d, outs_e, pools_d, pools_e


def oracle_flow(run, layer, rows):
    """Sequential replay of one layer for the given rows (others skipped)."""
    B, H, Q = run.B, run.H, run.Q
    p = run.params[layer]
    lay = ref.Layer(p.a_log, p.g_bias, run.scale, run.lower_bound)
    si = np.zeros(B, np.int32)
    si[rows] = run.state_indices[rows]
    pool = np.zeros((run.num_slots, H, 128, 128), np.float32)
    for r in rows:
        pool[si[r]] = run.slot_state(layer, int(si[r]))
    outs = []
    for s in range(run.steps):
        t = run.tokens(layer, s)
        o = np.zeros((B * run.T, H, 128), np.uint16)
        rec = oracle_records(B, H, Q)
        ref.kda_verify(lay, t.q, t.k, t.v, t.g, t.beta, run.cu_seqlens, pool, si, rec, o,
                       record_rows=run.record_rows)
        ref.kda_commit(lay, run.cu_seqlens, B * run.T, pool, si, rec, run.num_accepted(s),
                       record_rows=run.record_rows)
        outs.append(o)
    return outs, pool


def compare(run, outs_d, outs_e, pools_d, pools_e, sample):
    for key in outs_d:
        assert torch.equal(outs_d[key].view(torch.int16), outs_e[key].view(torch.int16)), \
            f"deferred o differs from eager o at (layer, step) {key}"
    for l in range(run.layers):
        assert torch.equal(pools_d[l].view(torch.int32), pools_e[l].view(torch.int32)), \
            f"deferred pool differs from eager pool, layer {l}"
    for layer, rows in sample:
        say(f"  oracle replay layer {layer} rows {rows}")
        outs, pool = oracle_flow(run, layer, rows)
        mask = np.zeros((run.B * run.T, 1, 1), bool)
        for r in rows:
            mask[r * run.T:(r + 1) * run.T] = True
        for s in range(run.steps):
            check_o(bits_host(outs_d[layer, s]), outs[s], mask=mask,
                    what=f"deferred o layer {layer} step {s}, {len(rows)} rows")
        pg = pools_d[layer].cpu().numpy()
        for r in rows:
            slot = int(run.state_indices[r])
            check_state(pg[slot], pool[slot], what=f"state layer {layer} row {r}")


def test_deferred_small_all_rows():
    run = make_deferred(B=24, H=4, layers=2, steps=4)
    say("case deferred B=24 H=4 layers=2 steps=4")
    res = gpu_flows(run)
    compare(run, *res, sample=[(0, list(range(24))), (1, list(range(24)))])


def test_deferred_full_size():
    run = make_deferred()
    say(f"case deferred B={run.B} H={run.H} layers={run.layers} steps={run.steps}")
    # the eager verify as the benchmark runs it: window bound T (short kernels)
    res = gpu_flows(run, max_seqlen=run.T)
    rng = np.random.default_rng(5)
    rows0 = sorted([0, run.B - 1, *rng.choice(np.arange(1, run.B - 1), 30, replace=False).tolist()])
    compare(run, *res, sample=[(0, rows0), (5, [1, 42, 300, 511]), (7, [0, 9, 255, 510])])


@pytest.mark.parametrize("B", [2048, 2049])
def test_deferred_row_list_capacity(B):
    """A deferring commit builds the list of rows that replay now; 2048 rows
    is the most the list holds (every 64-row chunk in use), 2049 takes the
    full grid. Both must match the eager flow bitwise and the oracle on the
    first and last rows."""
    run = make_deferred(B=B, H=1, layers=2, steps=3)
    say(f"case deferred row list B={B} H=1 layers=2 steps=3")
    res = gpu_flows(run)
    compare(run, *res, sample=[(1, [0, B - 1])])


@pytest.mark.parametrize("B,H", [(32, 16), (128, 32)])
def test_deferred_eight_token_windows(B, H):
    """Record window and windows of 8 tokens, with 512 and 4096 (row, head)
    pairs (64- and 128-row tiles). The deferred flow's folded states equal
    the eager flow's commits bit for bit (one replay code), and its outputs
    equal the eager flow's bit for bit too: both verify a chunk from the
    same state with the same matrix-core code, whatever the tile size
    (checked against the oracle's tolerance first, to report the size of any
    difference)."""
    from workloads import make_batch
    from .helpers import dev_layer
    batch = make_batch("deep", B=B, H=H)
    B, H, Q = batch.num_rows, batch.H, batch.Q
    assert Q == 8 and np.all(batch.seq_lens() == 8)
    say(f"case deferred 8-token windows B={B} H={H}")
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    cu, si = to_dev(batch.cu_seqlens), to_dev(batch.state_indices)
    nacc = to_dev(batch.num_accepted.astype(np.int32))
    pool0 = to_dev(batch.initial_pool())
    pool_e, pool_d = pool0.clone(), pool0.clone()
    ntok = batch.tokens.num_tokens
    rec_e = dev_records(B, H, Q)
    rec_d = [dev_records(B, H, Q), dev_records(B, H, Q)]
    pending = torch.zeros(B, dtype=torch.int32, device=DEV)
    outs = []
    for step in range(3):
        oe = torch.empty((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
        od = torch.empty_like(oe)
        kda.kda_verify(L, *toks.args(), cu, pool_e, si, rec_e, oe)
        kda.kda_verify_deferred(L, *toks.args(), cu, pool_d, si, rec_d[(step + 1) % 2], pending,
                                rec_d[step % 2], od)
        kda.kda_commit(L, cu, pool_e, si, rec_e, nacc)
        kda.kda_commit(L, cu, pool_d, si, rec_d[step % 2], nacc, pending=pending)
        outs.append((oe, od))
    kda.kda_flush(L, pool_d, si, rec_d[2 % 2], pending, rec_d[(2 + 1) % 2])
    torch.cuda.synchronize()
    for step, (oe, od) in enumerate(outs):
        check_o(bits_host(od), bits_host(oe), what=f"deferred o vs eager o, step {step}")
        assert torch.equal(od.view(torch.int16), oe.view(torch.int16)), \
            f"deferred o differs from eager o at step {step}"
    assert torch.equal(pool_e.view(torch.int32), pool_d.view(torch.int32)), "pools differ"
