"""GPU parity of kda_recurrent_spec, the stock speculative step (one state
stored per verified token): against the oracle, and column t bit for bit
against kda_recurrent over the same t + 1 tokens."""

import os
import sys

import numpy as np
import pytest
import torch

import linear_attention_speculative_kda_amd as kda
from oracle import kda_ref as ref
from workloads import make_batch
from workloads.configs import Tokens

from .helpers import (DevTokens, bits_host, check_o, check_state, dev_layer, oracle_layer,
                      to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENT = 0x7E7E
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def spec_table(batch, cols, seed=3):
    """Distinct blocks for every row's columns (slot 0 stays null), the
    source column from the accepted counts holding the row's checkpoint."""
    B = batch.num_rows
    nslots = 1 + B * cols
    rng = np.random.default_rng(seed)
    blocks = (rng.permutation(nslots - 1) + 1).astype(np.int32).reshape(B, cols)
    return blocks, nslots


def gather_prefix(batch, n):
    """The first min(n, T_i) tokens of every row, packed, and their cu_seqlens."""
    T = batch.seq_lens()
    m = np.minimum(T, n)
    idx = np.concatenate([np.arange(batch.cu_seqlens[i], batch.cu_seqlens[i] + m[i])
                          for i in range(batch.num_rows)]).astype(np.int64)
    cu = np.zeros(batch.num_rows + 1, np.int32)
    cu[1:] = np.cumsum(m)
    t = batch.tokens
    return Tokens(qkv=t.qkv[idx], g=t.g[idx], beta=t.beta[idx], H=t.H), cu


def run_spec(batch, pool_np, table, nacc):
    L = dev_layer(batch)
    toks = DevTokens(batch.tokens)
    pool = to_dev(pool_np)
    o = torch.full((batch.tokens.num_tokens, batch.H, 128), 0, dtype=torch.int16, device=DEV)
    o.fill_(np.int16(np.uint16(SENT).view(np.int16)))
    kda.kda_recurrent_spec(L, *toks.args(), to_dev(batch.cu_seqlens), pool, to_dev(table),
                           None if nacc is None else to_dev(nacc.astype(np.int32)),
                           o.view(torch.bfloat16))
    torch.cuda.synchronize()
    return pool.cpu().numpy(), bits_host(o)


def columns_bitexact(batch, pool_np, table, nacc):
    """Column t of every row holds the bits kda_recurrent stores after the
    row's first t + 1 tokens from its source block."""
    cols = table.shape[1]
    say(f"spec columns vs recurrent: {batch.name} B={batch.num_rows} H={batch.H} cols={cols}")
    got, _ = run_spec(batch, pool_np, table, nacc)
    T = batch.seq_lens()
    src_col = np.minimum(np.maximum(nacc if nacc is not None else np.ones(batch.num_rows), 1), cols) - 1
    src = table[np.arange(batch.num_rows), src_col.astype(np.int64)]
    L = dev_layer(batch)
    for t in range(cols):
        ptoks, pcu = gather_prefix(batch, t + 1)
        pool = to_dev(pool_np)
        o = torch.empty((max(ptoks.num_tokens, 1), batch.H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_recurrent(L, *DevTokens(ptoks).args(), to_dev(pcu), pool, to_dev(src.astype(np.int32)),
                          o[:ptoks.num_tokens])
        torch.cuda.synchronize()
        want = pool.cpu().numpy()
        for i in range(batch.num_rows):
            if T[i] > t and src[i] > 0:
                blk = int(table[i, t])
                assert np.array_equal(got[blk].view(np.int32), want[src[i]].view(np.int32)), \
                    f"row {i} column {t} (block {blk}) differs from the recurrence over {t + 1} tokens"


@pytest.mark.parametrize("name,B,H", [("tiny", None, None), ("ragged", 24, 4), ("decode", None, None)])
def test_spec_columns_bitexact_with_recurrent(name, B, H):
    batch = make_batch(name, B=B, H=H)
    cols = int(batch.seq_lens().max())
    table, nslots = spec_table(batch, cols)
    pool_np = np.zeros((nslots, batch.H, 128, 128), np.float32)
    rng = np.random.default_rng(7)
    nacc = rng.integers(1, cols + 1, size=batch.num_rows).astype(np.int32)
    src = table[np.arange(batch.num_rows), nacc - 1]
    pool_np[src] = (rng.standard_normal((batch.num_rows, batch.H, 128, 128), dtype=np.float32)
                    * np.float32(0.02))
    columns_bitexact(batch, pool_np, table, nacc)


def test_spec_against_oracle_golden_columns():
    """The column rules of the hand-worked table (null columns, clamped
    counts, a null source, windows longer and shorter than the row, blocks
    outside the pool) against the oracle; blocks no column names stay
    untouched."""
    rows = []
    for line in open(os.path.join(GOLDEN, "spec_columns.txt")):
        line = line.split("#")[0].strip()
        if line:
            l = [int(x) for x in line.split("|")[0].split()]
            rows.append(l)
    N, H, nslots = len(rows), 4, 40
    T = np.array([r[1] for r in rows])
    acc = np.array([r[2] for r in rows], np.int32)
    table = np.array([r[3:7] for r in rows], np.int32)
    base = make_batch("ragged", B=24, H=H)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(T)
    assert cu[-1] <= base.tokens.num_tokens
    say(f"spec golden columns: rows={N} tokens={cu[-1]}")
    t = base.tokens
    ntok = int(cu[-1])
    batch = base
    batch.tokens = Tokens(qkv=t.qkv[:ntok], g=t.g[:ntok], beta=t.beta[:ntok], H=H)
    batch.cu_seqlens = cu
    rng = np.random.default_rng(8)
    pool_np = (rng.standard_normal((nslots, H, 128, 128), dtype=np.float32) * np.float32(0.02))
    got, o_gpu = run_spec(batch, pool_np, table, acc)
    pool_ref = pool_np.copy()
    o_ref = np.full((ntok, H, 128), SENT, np.uint16)
    ref.kda_recurrent_spec(oracle_layer(batch), batch.tokens.q, batch.tokens.k, batch.tokens.v,
                           batch.tokens.g, batch.tokens.beta, cu, pool_ref, table, acc, o_ref)
    written = [b for b in range(nslots) if not np.array_equal(pool_ref[b], pool_np[b])]
    for b in range(nslots):
        if b in written:
            check_state(got[b], pool_ref[b], what=f"block {b}")
        else:
            assert np.array_equal(got[b], pool_np[b]), f"block {b} written"
    live = o_ref != SENT
    assert np.array_equal(o_gpu == SENT, ~live), "outputs written where the oracle writes none"
    check_o(o_gpu, o_ref, mask=live, what="spec golden o")


def test_spec_full_size_decode_against_oracle():
    """The decode workload's shape (B=64, H=32, T=4, four columns), as the
    benchmark runs it: sampled rows against the oracle, every column's
    state within the state tolerance."""
    batch = make_batch("decode")
    cols = 4
    table, nslots = spec_table(batch, cols)
    rng = np.random.default_rng(9)
    nacc = rng.integers(1, cols + 1, size=batch.num_rows).astype(np.int32)
    src = table[np.arange(batch.num_rows), nacc - 1]
    pool_np = np.zeros((nslots, batch.H, 128, 128), np.float32)
    pool_np[src] = (rng.standard_normal((batch.num_rows, batch.H, 128, 128), dtype=np.float32)
                    * np.float32(0.02))
    say("spec full size decode vs oracle")
    got, o_gpu = run_spec(batch, pool_np, table, nacc)
    sample = [0, 1, 17, 40, 62, 63]
    keep = np.zeros(batch.num_rows, bool)
    keep[sample] = True
    tab_ref = np.where(keep[:, None], table, 0).astype(np.int32)
    pool_ref = pool_np.copy()
    o_ref = np.full_like(o_gpu, SENT)
    t = batch.tokens
    ref.kda_recurrent_spec(oracle_layer(batch), t.q, t.k, t.v, t.g, t.beta, batch.cu_seqlens,
                           pool_ref, tab_ref, nacc, o_ref)
    mask = np.zeros((t.num_tokens, 1, 1), bool)
    for i in sample:
        mask[batch.cu_seqlens[i]:batch.cu_seqlens[i + 1]] = True
        for c in range(cols):
            check_state(got[table[i, c]], pool_ref[table[i, c]], what=f"row {i} column {c}")
    check_o(o_gpu, o_ref, mask=mask, what="spec decode o, 6 rows")
