"""A verify + commit step captured in a HIP graph: every replay, with eager
work and synchronisations between the replays, gives the eager results bit
for bit. The library's calls enqueue one kernel each (no memset, no
allocation), so the captured graph holds the two kernels only."""

import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from workloads import make_batch

from .helpers import DevTokens, dev_layer, dev_records, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7E7E


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("name,B,H", [("tiny", None, None), ("ragged", 32, 8), ("deep", 16, 8)])
def test_graph_replay_matches_eager(name, B, H):
    say(f"graph replay vs eager: {name} B={B} H={H}")
    batch = make_batch(name, B=B, H=H)
    rows, H, Q = batch.num_rows, batch.H, batch.Q
    ntok = batch.tokens.num_tokens
    layer = dev_layer(batch)
    tok = DevTokens(batch.tokens)
    cu, si = to_dev(batch.cu_seqlens), to_dev(batch.state_indices)
    nacc = to_dev(batch.num_accepted)
    pool0 = to_dev(batch.initial_pool())

    def step(pool, rec, o, stream):
        kda.kda_verify(layer, *tok.args(), cu, pool, si, rec, o, stream=stream)
        kda.kda_commit(layer, cu, pool, si, rec, nacc, stream=stream)

    # eager reference
    pool_e = pool0.clone()
    rec_e = dev_records(rows, H, Q, fill=SENT)
    o_e = torch.full((ntok, H, 128), 0, dtype=torch.bfloat16, device=DEV)
    step(pool_e, rec_e, o_e, None)
    torch.cuda.synchronize()

    # capture one step on a side stream
    pool_g = pool0.clone()
    rec_g = dev_records(rows, H, Q, fill=SENT)
    o_g = torch.zeros((ntok, H, 128), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(pool_g, rec_g, o_g, side)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pool_g, rec_g, o_g, torch.cuda.current_stream())

    for rep in range(4):
        # reset the inputs the step overwrites, eagerly, then replay
        pool_g.copy_(pool0)
        for t in (rec_g.k, rec_g.v, rec_g.g, rec_g.beta):
            t.view(torch.int16).fill_(np.int16(np.uint16(SENT).view(np.int16)))
        o_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(o_g), bits(o_e)), f"o differs on replay {rep}"
        assert torch.equal(bits(pool_g), bits(pool_e)), f"pool differs on replay {rep}"
        for a, b, what in ((rec_g.k, rec_e.k, "k"), (rec_g.v, rec_e.v, "v"),
                           (rec_g.g, rec_e.g, "g"), (rec_g.beta, rec_e.beta, "beta")):
            assert torch.equal(bits(a), bits(b)), f"records {what} differ on replay {rep}"
        # unrelated eager work between replays
        _ = (pool0.sum() + pool_g.abs().max()).item()
    say("  4 replays bitwise equal to eager")


def test_graph_replay_of_the_serving_step():
    """The benchmark's step in one graph: every layer's window-bounded
    kda_verify (short kernels, predicted spans), then one kda_commit_layers;
    replays equal the eager step bit for bit."""
    batch = make_batch("decode", B=16, H=8)
    rows, H, Q = batch.num_rows, batch.H, batch.Q
    ntok = batch.tokens.num_tokens
    L = 3
    say(f"graph replay of the serving step: decode B={rows} H={H}, {L} layers")
    layer = dev_layer(batch)
    tok = DevTokens(batch.tokens)
    cu, si, nacc = to_dev(batch.cu_seqlens), to_dev(batch.state_indices), to_dev(batch.num_accepted)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    pools0 = []
    for _ in range(L):
        p = torch.empty((batch.num_slots, H, 128, 128), dtype=torch.float32, device=DEV)
        p.normal_(0.0, 0.02, generator=gen)
        pools0.append(p)

    def step(pools, recs, outs, stream):
        for l in range(L):
            kda.kda_verify(layer, *tok.args(), cu, pools[l], si, recs[l], outs[l], stream=stream,
                           max_seqlen=4)
        kda.kda_commit_layers([layer] * L, cu, pools, si, recs, nacc, stream=stream)

    def fresh():
        return ([p.clone() for p in pools0], [dev_records(rows, H, Q, fill=SENT) for _ in range(L)],
                [torch.zeros((ntok, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(L)])

    pe, re_, oe = fresh()
    step(pe, re_, oe, None)
    torch.cuda.synchronize()

    pg, rg, og = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(pg, rg, og, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(pg, rg, og, torch.cuda.current_stream())
    for rep in range(4):
        for l in range(L):
            pg[l].copy_(pools0[l])
            og[l].zero_()
            for t in (rg[l].k, rg[l].v, rg[l].g, rg[l].beta):
                t.view(torch.int16).fill_(np.int16(np.uint16(SENT).view(np.int16)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(bits(og[l]), bits(oe[l])), f"layer {l}: o differs on replay {rep}"
            assert torch.equal(bits(pg[l]), bits(pe[l])), f"layer {l}: pool differs on replay {rep}"
            assert torch.equal(bits(rg[l].v), bits(re_[l].v)), f"layer {l}: records differ on replay {rep}"
        _ = (pools0[0].sum() + pg[0].abs().max()).item()
    say("  4 replays bitwise equal to eager")
