"""GPU parity of the multi-layer calls: kda_commit_layers and kda_flush_layers
give, layer by layer, the same bits as kda_commit and kda_flush called once
per layer (eager and deferred mode, pending counts included), and the
committed states match the oracle's commit of the same records."""

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


def setup(run):
    """Per-layer params, pools (one copy per flow) and the records of one
    verify of each layer's step-0 tokens."""
    B, H, Q = run.B, run.H, run.Q
    si, rr, cu = to_dev(run.state_indices), to_dev(run.record_rows), to_dev(run.cu_seqlens)
    layers, pools, recs = [], [], []
    for l in range(run.layers):
        p = run.params[l]
        layers.append(kda.Layer(a_log=to_dev(p.a_log), g_bias=to_dev(p.g_bias), scale=run.scale,
                                lower_bound=run.lower_bound))
        pools.append(to_dev(run.initial_pool(l)))
        rec = dev_records(B, H, Q)
        o = torch.empty((B * run.T, H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_verify(layers[l], *DevTokens(run.tokens(l, 0)).args(), cu, pools[l], si, rec, o,
                       record_rows=rr)
        recs.append(rec)
    torch.cuda.synchronize()
    return layers, pools, recs, si, rr, cu


def bits(t):
    return t.view(torch.int32)


@pytest.mark.parametrize("B,H,layers", [(24, 4, 3), (16, 2, 16)])
def test_commit_layers_matches_per_layer(B, H, layers):
    say(f"commit_layers vs per-layer commit: B={B} H={H} layers={layers}")
    run = make_deferred(B=B, H=H, layers=layers, steps=1)
    Ls, pools, recs, si, rr, cu = setup(run)
    nacc = to_dev(run.num_accepted(0))
    eager = to_dev(run.eager(0))
    # eager mode
    one = [p.clone() for p in pools]
    many = [p.clone() for p in pools]
    for l in range(layers):
        kda.kda_commit(Ls[l], cu, one[l], si, recs[l], nacc, record_rows=rr)
    kda.kda_commit_layers(Ls, cu, many, si, recs, nacc, record_rows=rr)
    torch.cuda.synchronize()
    for l in range(layers):
        assert torch.equal(bits(one[l]), bits(many[l])), f"eager mode, layer {l}"
    # deferred mode: pending counts and the eager rows' commits
    one = [p.clone() for p in pools]
    many = [p.clone() for p in pools]
    pend1 = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    pend2 = pend1.clone()
    for l in range(layers):
        kda.kda_commit(Ls[l], cu, one[l], si, recs[l], nacc, record_rows=rr, pending=pend1,
                       eager=eager)
    kda.kda_commit_layers(Ls, cu, many, si, recs, nacc, record_rows=rr, pending=pend2, eager=eager)
    torch.cuda.synchronize()
    assert torch.equal(pend1, pend2), "pending counts"
    for l in range(layers):
        assert torch.equal(bits(one[l]), bits(many[l])), f"deferred mode, layer {l}"


def test_commit_layers_against_oracle():
    B, H, L = 12, 4, 3
    say(f"commit_layers vs oracle: B={B} H={H} layers={L}")
    run = make_deferred(B=B, H=H, layers=L, steps=1)
    Ls, pools, recs, si, rr, cu = setup(run)
    nacc_np = run.num_accepted(0)
    work = [p.clone() for p in pools]
    kda.kda_commit_layers(Ls, cu, work, si, recs, to_dev(nacc_np), record_rows=rr)
    torch.cuda.synchronize()
    for l in range(L):
        p = run.params[l]
        lay = ref.Layer(p.a_log, p.g_bias, run.scale, run.lower_bound)
        pool = pools[l].cpu().numpy().copy()
        ref.kda_commit(lay, run.cu_seqlens, B * run.T, pool, run.state_indices,
                       records_host(recs[l]), nacc_np, record_rows=run.record_rows)
        got = work[l].cpu().numpy()
        for s in run.state_indices:
            check_state(got[s], pool[s], what=f"layer {l} slot {s}")


def test_flush_layers_matches_per_layer():
    B, H, L = 20, 4, 4
    say(f"flush_layers vs per-layer flush: B={B} H={H} layers={L}")
    run = make_deferred(B=B, H=H, layers=L, steps=1)
    Ls, pools, recs, si, rr, cu = setup(run)
    pending = to_dev(np.random.default_rng(5).integers(-2, run.Q + 3, size=B).astype(np.int32))
    spare = [dev_records(B, H, run.Q) for _ in range(L)]
    one = [p.clone() for p in pools]
    many = [p.clone() for p in pools]
    for l in range(L):
        kda.kda_flush(Ls[l], one[l], si, recs[l], pending, spare[l], record_rows=rr)
    kda.kda_flush_layers(Ls, many, si, recs, pending, record_rows=rr)
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.equal(bits(one[l]), bits(many[l])), f"layer {l}"
    # the fold changed the slots of rows with a positive count, and only those
    pend = pending.cpu().numpy()
    for l in range(L):
        before, after = pools[l].cpu().numpy(), many[l].cpu().numpy()
        for i, s in enumerate(run.state_indices):
            changed = not np.array_equal(before[s], after[s])
            assert changed == (pend[run.record_rows[i]] > 0), f"layer {l} row {i}"


@pytest.mark.parametrize("name,layers", [("decode", 12), ("deep", 4), ("ragged", 4)])
def test_commit_layers_full_size(name, layers):
    """The benchmark's commit launch: every layer of a full-size workload in
    one kda_commit_layers call gives, layer by layer, the bits of kda_commit
    (itself bit-exact with kda_recurrent over the accepted prefix at these
    sizes). Each layer has its own checkpoints (seeded N(0, 0.02) on the
    device) and the records of its own verify."""
    from workloads import make_batch
    from .helpers import dev_layer
    batch = make_batch(name)
    B, H, Q = batch.num_rows, batch.H, batch.Q
    say(f"commit_layers full size: {name} B={B} H={H} layers={layers}")
    lay = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    cu, si, nacc = to_dev(batch.cu_seqlens), to_dev(batch.state_indices), to_dev(batch.num_accepted)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4242)
    o = torch.empty((batch.tokens.num_tokens, H, 128), dtype=torch.bfloat16, device=DEV)
    one, many, recs = [], [], []
    for _ in range(layers):
        p = torch.empty((batch.num_slots, H, 128, 128), dtype=torch.float32, device=DEV)
        p.normal_(0.0, 0.02, generator=gen)
        rec = dev_records(B, H, Q)
        kda.kda_verify(lay, *toks.args(), cu, p, si, rec, o)
        one.append(p)
        many.append(p.clone())
        recs.append(rec)
    for l in range(layers):
        kda.kda_commit(lay, cu, one[l], si, recs[l], nacc)
    kda.kda_commit_layers([lay] * layers, cu, many, si, recs, nacc)
    torch.cuda.synchronize()
    for l in range(layers):
        assert torch.equal(bits(one[l]), bits(many[l])), f"{name}: layer {l}"
    del one, many, recs
    torch.cuda.empty_cache()
