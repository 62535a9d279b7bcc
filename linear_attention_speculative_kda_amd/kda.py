"""Python front end of libkda: the calls of include/kda.h (recurrent, the
stock speculative step, verify, commit, deferred verify and flush, the multi-layer commit and flush, the
conv-state compaction), taking torch tensors that live on the GPU.
Marshalling only; the computation is in HIP.

Tensor conventions (K = V = 128):
  q, k, v, g      [num_tokens, H, K] bf16 (or any 2-byte dtype holding bf16
                  bits), head stride K, element stride 1, any token stride that
                  is a multiple of 4 (q/k/v may be column blocks of one
                  projection output); g must be the same shape.
  beta            [num_tokens, H], element stride 1.
  o               [num_tokens, H, V] bf16, dense.
  cu_seqlens      int32 [num_rows + 1]; state_indices int32 [num_rows].
  pool            fp32 [num_slots, H, V, K], inner dims dense.
  Records         raw bf16 records with a scratch row at index 0.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import _lib

HEAD_DIM = 128


@dataclass
class Layer:
    a_log: torch.Tensor          # fp32 [H]
    g_bias: torch.Tensor         # fp32 [H * K]
    scale: float
    lower_bound: float | None = None   # None: unbounded softplus gate

    @property
    def num_heads(self) -> int:
        return int(self.a_log.numel())

    def c_struct(self) -> _lib.KdaLayer:
        _need(self.a_log, torch.float32, "a_log")
        _need(self.g_bias, torch.float32, "g_bias")
        if self.g_bias.numel() != self.num_heads * HEAD_DIM:
            raise ValueError("g_bias must hold H * 128 values")
        return _lib.KdaLayer(
            num_heads=self.num_heads, head_dim=HEAD_DIM, scale=float(self.scale),
            has_lower_bound=0 if self.lower_bound is None else 1,
            lower_bound=0.0 if self.lower_bound is None else float(self.lower_bound),
            a_log=self.a_log.data_ptr(), g_bias=self.g_bias.data_ptr())


@dataclass
class Records:
    """Raw records: k, g, v [rows+1, H, window, K] and beta [rows+1, H, window]
    (bf16); index 0 is the scratch row of record row -1."""
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor

    @property
    def rows(self) -> int:
        return self.k.shape[0] - 1

    @property
    def window(self) -> int:
        return self.k.shape[2]

    def c_struct(self) -> _lib.KdaRecords:
        for name in ("k", "v", "g", "beta"):
            t = getattr(self, name)
            if t.element_size() != 2 or not t.is_contiguous():
                raise ValueError(f"records.{name} must be a contiguous 2-byte tensor")
        return _lib.KdaRecords(k=self.k.data_ptr(), v=self.v.data_ptr(), g=self.g.data_ptr(),
                               beta=self.beta.data_ptr(), rows=self.rows, window=self.window)


def allocate_records(rows: int, num_heads: int, window: int, device,
                     dtype: torch.dtype = torch.bfloat16) -> Records:
    shape = (rows + 1, num_heads, window, HEAD_DIM)
    return Records(k=torch.empty(shape, dtype=dtype, device=device),
                   v=torch.empty(shape, dtype=dtype, device=device),
                   g=torch.empty(shape, dtype=dtype, device=device),
                   beta=torch.empty(shape[:3], dtype=dtype, device=device))


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _act(t: torch.Tensor, name: str, H: int) -> int:
    """Check a [tokens, H, K] activation view; return its token stride."""
    if t.element_size() != 2:
        raise TypeError(f"{name} must hold bf16 (2-byte) values")
    if t.dim() != 3 or t.shape[1] != H or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [tokens, {H}, {HEAD_DIM}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
        raise ValueError(f"{name} needs head stride {HEAD_DIM} and element stride 1")
    return t.stride(0)


def _tokens(q, k, v, g, beta, cu_seqlens, H: int, max_seqlen: int | None = None) -> _lib.KdaTokens:
    n = q.shape[0]
    for t, name in ((k, "k"), (v, "v"), (g, "g")):
        if t.shape[0] != n:
            raise ValueError(f"{name} has {t.shape[0]} tokens, q has {n}")
    if beta.element_size() != 2 or beta.dim() != 2 or beta.shape != (n, H) or (n > 0 and beta.stride(1) != 1):
        raise ValueError("beta must be [tokens, H] of bf16 with element stride 1")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    return _lib.KdaTokens(
        q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), g=g.data_ptr(), beta=beta.data_ptr(),
        stride_q=_act(q, "q", H), stride_k=_act(k, "k", H), stride_v=_act(v, "v", H),
        stride_g=_act(g, "g", H), stride_beta=beta.stride(0) if n > 0 else H,
        cu_seqlens=cu_seqlens.data_ptr(), num_rows=cu_seqlens.numel() - 1, num_tokens=n,
        max_seqlen=0 if max_seqlen is None else int(max_seqlen))


def _pool(pool: torch.Tensor, state_indices: torch.Tensor, H: int, rows: int | None = None) -> _lib.KdaPool:
    if pool.dtype != torch.float32 or pool.dim() != 4 or pool.shape[1:] != (H, HEAD_DIM, HEAD_DIM):
        raise ValueError(f"pool must be fp32 [slots, {H}, {HEAD_DIM}, {HEAD_DIM}]")
    if pool.stride()[1:] != (HEAD_DIM * HEAD_DIM, HEAD_DIM, 1):
        raise ValueError("pool inner dims must be dense")
    _need(state_indices, torch.int32, "state_indices")
    if rows is not None and state_indices.numel() < rows:
        raise ValueError(f"state_indices has {state_indices.numel()} entries, needs {rows}")
    return _lib.KdaPool(state=pool.data_ptr(), slot_stride=pool.stride(0),
                        num_slots=pool.shape[0], state_indices=state_indices.data_ptr())


def _opt_ptr(t: torch.Tensor | None, dtype, name: str, min_len: int = 0):
    if t is None:
        return None
    _need(t, dtype, name)
    if t.numel() < min_len:
        raise ValueError(f"{name} has {t.numel()} entries, needs {min_len}")
    return t.data_ptr()


def _on_gpu(ref: torch.Tensor, *tensors) -> None:
    """Every tensor handed to the kernels must live on the pool's GPU: a host
    pointer would be dereferenced by the device."""
    if not ref.is_cuda:
        raise ValueError("tensors must be on a GPU")
    for t in tensors:
        if t is None:
            continue
        if isinstance(t, Records):
            _on_gpu(ref, t.k, t.v, t.g, t.beta)
        elif isinstance(t, Layer):
            _on_gpu(ref, t.a_log, t.g_bias)
        elif t.device != ref.device:
            raise ValueError(f"tensor on {t.device}, expected {ref.device}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _out(o: torch.Tensor, n: int, H: int) -> int:
    if o.element_size() != 2 or not o.is_contiguous() or o.shape != (n, H, HEAD_DIM):
        raise ValueError(f"o must be a contiguous bf16 [{n}, {H}, {HEAD_DIM}] tensor")
    return o.data_ptr()


def check_rows(cu_seqlens, state_indices, num_slots: int, num_tokens: int | None = None,
               record_rows=None, rec_rows: int | None = None, max_seqlen: int | None = None) -> None:
    """Check on the host the row metadata the kernels only range-check
    (libkda's kda_check_rows): well-formed spans, windows within max_seqlen,
    slots below num_slots and distinct, record rows in range and distinct.
    The int32 tensors may live on any device (they are copied to the host,
    which synchronises with the GPU). Raises KdaError naming the first bad
    row."""
    lib = _lib.load()
    cu = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    si = state_indices.detach().to("cpu", torch.int32).contiguous()
    rows = cu.numel() - 1
    if si.numel() < rows:
        raise ValueError(f"state_indices has {si.numel()} entries, needs {rows}")
    rr = None if record_rows is None else record_rows.detach().to("cpu", torch.int32).contiguous()
    if rr is not None and rr.numel() < rows:
        raise ValueError(f"record_rows has {rr.numel()} entries, needs {rows}")
    ntok = int(cu[-1]) if num_tokens is None and rows > 0 else int(num_tokens or 0)
    bad, what = ctypes.c_int32(-1), ctypes.c_int32(0)
    st = lib.kda_check_rows(cu.data_ptr(), rows, ntok, si.data_ptr(), int(num_slots),
                            None if rr is None else rr.data_ptr(),
                            -1 if rec_rows is None else int(rec_rows),
                            0 if max_seqlen is None else int(max_seqlen),
                            ctypes.byref(bad), ctypes.byref(what))
    if st == _lib.KDA_ERR_METADATA:
        raise _lib.KdaError("kda_check_rows", st,
                            f"row {bad.value}: {_lib.ROW_ISSUES.get(what.value, what.value)}")
    _lib.check("kda_check_rows", st)


# KDA_DEBUG_VALIDATE=1: every call below first checks its row metadata on the
# host (a synchronising copy; for debugging only).
_DEBUG_VALIDATE = os.environ.get("KDA_DEBUG_VALIDATE", "0") == "1"


def _debug_rows(cu_seqlens, state_indices, pool, num_tokens=None, record_rows=None,
                rec: "Records | None" = None, max_seqlen=None) -> None:
    if _DEBUG_VALIDATE:
        check_rows(cu_seqlens, state_indices, pool.shape[0], num_tokens=num_tokens,
                   record_rows=record_rows, rec_rows=None if rec is None else rec.rows,
                   max_seqlen=max_seqlen)


def kda_recurrent(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices, o,
                  stream=None) -> None:
    """Plain recurrence: o for every token, final state stored in place."""
    _on_gpu(pool, layer, q, k, v, g, beta, cu_seqlens, state_indices, o)
    _debug_rows(cu_seqlens, state_indices, pool, q.shape[0])
    lib = _lib.load()
    H = layer.num_heads
    L, T, P = layer.c_struct(), _tokens(q, k, v, g, beta, cu_seqlens, H), _pool(pool, state_indices, H, cu_seqlens.numel() - 1)
    st = lib.kda_recurrent(ctypes.byref(L), ctypes.byref(T), ctypes.byref(P),
                           _out(o, q.shape[0], H), _stream(stream))
    _lib.check("kda_recurrent", st)


def kda_recurrent_spec(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_table,
                       num_accepted=None, o=None, stream=None) -> None:
    """The stock speculative step: each row runs its window from the block in
    column num_accepted - 1 of its row of ``state_table`` (int32 [rows,
    cols]; column 0 without counts) and stores the state after token t into
    the block of column t (0: none). o for every token."""
    _on_gpu(pool, layer, q, k, v, g, beta, cu_seqlens, state_table, num_accepted, o)
    lib = _lib.load()
    H = layer.num_heads
    rows = cu_seqlens.numel() - 1
    if state_table.dtype != torch.int32 or state_table.dim() != 2 or state_table.stride(1) != 1:
        raise ValueError("state_table must be an int32 [rows, cols] tensor with unit column stride")
    if state_table.shape[0] < rows:
        raise ValueError(f"state_table has {state_table.shape[0]} rows, needs {rows}")
    L, T = layer.c_struct(), _tokens(q, k, v, g, beta, cu_seqlens, H)
    P = _pool(pool, torch.zeros(1, dtype=torch.int32, device=pool.device), H)
    P.state_indices = None
    tab = _lib.KdaSpecTable(indices=state_table.data_ptr(), row_stride=state_table.stride(0),
                            cols=state_table.shape[1],
                            num_accepted=_opt_ptr(num_accepted, torch.int32, "num_accepted", rows))
    st = lib.kda_recurrent_spec(ctypes.byref(L), ctypes.byref(T), ctypes.byref(P), ctypes.byref(tab),
                                _out(o, q.shape[0], H), _stream(stream))
    _lib.check("kda_recurrent_spec", st)


def kda_verify(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices,
               rec: Records, o, record_rows=None, stream=None, max_seqlen: int | None = None) -> None:
    """Verify from the checkpoints: o and raw records; the pool is read only.
    ``max_seqlen``: an upper bound on every row's window that the caller
    guarantees (None: unknown); with 1..8 the short kernels run and rows
    longer than it are skipped."""
    _on_gpu(pool, layer, q, k, v, g, beta, cu_seqlens, state_indices, rec, o, record_rows)
    _debug_rows(cu_seqlens, state_indices, pool, q.shape[0], record_rows, rec, max_seqlen)
    lib = _lib.load()
    H = layer.num_heads
    L, T, P = layer.c_struct(), _tokens(q, k, v, g, beta, cu_seqlens, H, max_seqlen), _pool(pool, state_indices, H, cu_seqlens.numel() - 1)
    R = rec.c_struct()
    st = lib.kda_verify(ctypes.byref(L), ctypes.byref(T), ctypes.byref(P), ctypes.byref(R),
                        _opt_ptr(record_rows, torch.int32, "record_rows", cu_seqlens.numel() - 1),
                        _out(o, q.shape[0], H), _stream(stream))
    _lib.check("kda_verify", st)


def kda_commit(layer: Layer, cu_seqlens, pool, state_indices, rec: Records, num_accepted,
               record_rows=None, pending=None, eager=None, stream=None) -> None:
    """Commit the accepted prefix (or, with ``pending``, defer it)."""
    _on_gpu(pool, layer, cu_seqlens, state_indices, rec, num_accepted, record_rows, pending, eager)
    _debug_rows(cu_seqlens, state_indices, pool, None, record_rows, rec)
    lib = _lib.load()
    H = layer.num_heads
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    L, P, R = layer.c_struct(), _pool(pool, state_indices, H, cu_seqlens.numel() - 1), rec.c_struct()
    st = lib.kda_commit(ctypes.byref(L), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                        ctypes.byref(P), ctypes.byref(R),
                        _opt_ptr(record_rows, torch.int32, "record_rows", cu_seqlens.numel() - 1),
                        _opt_ptr(num_accepted, torch.int32, "num_accepted", cu_seqlens.numel() - 1),
                        _opt_ptr(pending, torch.int32, "pending", rec.rows),
                        _opt_ptr(eager, torch.uint8, "eager", cu_seqlens.numel() - 1), _stream(stream))
    _lib.check("kda_commit", st)


def kda_verify_deferred(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices,
                        rec_prev: Records, pending, rec_next: Records, o, record_rows=None,
                        stream=None) -> None:
    """Fold the pending replays into the checkpoints, then verify."""
    _on_gpu(pool, layer, q, k, v, g, beta, cu_seqlens, state_indices, rec_prev, pending,
            rec_next, o, record_rows)
    _debug_rows(cu_seqlens, state_indices, pool, q.shape[0], record_rows, rec_next)
    lib = _lib.load()
    H = layer.num_heads
    L, T, P = layer.c_struct(), _tokens(q, k, v, g, beta, cu_seqlens, H), _pool(pool, state_indices, H, cu_seqlens.numel() - 1)
    Rp, Rn = rec_prev.c_struct(), rec_next.c_struct()
    st = lib.kda_verify_deferred(ctypes.byref(L), ctypes.byref(T), ctypes.byref(P),
                                 ctypes.byref(Rp), _opt_ptr(pending, torch.int32, "pending", rec_prev.rows),
                                 ctypes.byref(Rn), _opt_ptr(record_rows, torch.int32, "record_rows", cu_seqlens.numel() - 1),
                                 _out(o, q.shape[0], H), _stream(stream))
    _lib.check("kda_verify_deferred", st)


def kda_flush(layer: Layer, pool, state_indices, rec_prev: Records, pending, rec_next: Records,
              record_rows=None, stream=None) -> None:
    """Fold every pending replay without verifying anything: kda_verify_deferred
    with an empty window on every row."""
    dev = pool.device
    n = state_indices.numel()
    H = layer.num_heads
    empty = torch.empty((0, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    kda_verify_deferred(layer, empty, empty, empty, empty,
                        torch.empty((0, H), dtype=torch.bfloat16, device=dev), cu, pool,
                        state_indices, rec_prev, pending, rec_next, empty, record_rows, stream)


MAX_LAYERS = 16   # layers per multi-layer launch


def _layer_arrays(layers, pools, state_indices, recs, rows: int):
    n = len(layers)
    if not (1 <= n <= MAX_LAYERS) or len(pools) != n or len(recs) != n:
        raise ValueError(f"1..{MAX_LAYERS} layers with one pool and one record set each")
    H = layers[0].num_heads
    Ls = (_lib.KdaLayer * n)(*[l.c_struct() for l in layers])
    Ps = (_lib.KdaPool * n)(*[_pool(p, state_indices, H, rows) for p in pools])
    Rs = (_lib.KdaRecords * n)(*[r.c_struct() for r in recs])
    return n, Ls, Ps, Rs


class Align:
    """Align mode of the commit: block ids per request row (int32 [rows,
    width], 0 = null block), the tokens each request had cached before the
    step (int32 [rows]) and the tokens per block."""

    def __init__(self, block_table: torch.Tensor, num_computed: torch.Tensor, block_size: int):
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be an int32 [rows, width] tensor with unit column stride")
        _need(num_computed, torch.int32, "num_computed")
        self.block_table, self.num_computed, self.block_size = block_table, num_computed, int(block_size)

    def c_struct(self, rows: int) -> _lib.KdaAlign:
        if self.block_table.shape[0] < rows or self.num_computed.numel() < rows:
            raise ValueError(f"align tables need at least {rows} rows")
        return _lib.KdaAlign(block_table=self.block_table.data_ptr(),
                             row_stride=self.block_table.stride(0),
                             width=self.block_table.shape[1],
                             num_computed=self.num_computed.data_ptr(),
                             block_size=self.block_size)


def kda_commit_layers(layers, cu_seqlens, pools, state_indices, recs, num_accepted,
                      record_rows=None, pending=None, eager=None, align: Align | None = None,
                      stream=None) -> None:
    """kda_commit for every layer in one launch. The layers share the row
    metadata and the state indices; each has its own pool and records. With
    ``align`` the final (and boundary) block of the block table is written
    instead of the source."""
    _on_gpu(pools[0], cu_seqlens, state_indices, num_accepted, record_rows, pending, eager,
            *layers, *pools, *recs, *(() if align is None else (align.block_table, align.num_computed)))
    _debug_rows(cu_seqlens, state_indices, pools[0], None, record_rows, recs[0])
    lib = _lib.load()
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    rows = cu_seqlens.numel() - 1
    n, Ls, Ps, Rs = _layer_arrays(layers, pools, state_indices, recs, rows)
    A = None if align is None else ctypes.byref(align.c_struct(rows))
    st = lib.kda_commit_layers(Ls, Ps, Rs, n, cu_seqlens.data_ptr(), rows,
                               _opt_ptr(record_rows, torch.int32, "record_rows", rows),
                               _opt_ptr(num_accepted, torch.int32, "num_accepted", rows),
                               _opt_ptr(pending, torch.int32, "pending", recs[0].rows),
                               _opt_ptr(eager, torch.uint8, "eager", rows), A, _stream(stream))
    _lib.check("kda_commit_layers", st)


def kda_conv_compact(conv_states, cu_seqlens, state_indices, num_accepted, window: int,
                     history: int, align: Align | None = None, stream=None) -> None:
    """The conv-state half of the commit for every layer in one launch.
    conv_states: 16-bit tensors [blocks, channels, width] (any strides), one
    per layer; the window after the accepted tokens moves to the front of
    the final block (and, in align mode, of the boundary block)."""
    _on_gpu(conv_states[0], cu_seqlens, state_indices, num_accepted, *conv_states,
            *(() if align is None else (align.block_table, align.num_computed)))
    lib = _lib.load()
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    rows = cu_seqlens.numel() - 1
    c0 = conv_states[0]
    for c in conv_states:
        if c.element_size() != 2 or c.dim() != 3 or c.shape[1:] != c0.shape[1:]:
            raise ValueError("conv states must be 16-bit [blocks, channels, width] tensors of one shape")
    arr = (_lib.KdaConvState * len(conv_states))(*[
        _lib.KdaConvState(state=c.data_ptr(), block_stride=c.stride(0), dim_stride=c.stride(1),
                          token_stride=c.stride(2), num_blocks=c.shape[0]) for c in conv_states])
    A = None if align is None else ctypes.byref(align.c_struct(rows))
    st = lib.kda_conv_compact(arr, len(conv_states), c0.shape[1], int(history), c0.shape[2],
                              cu_seqlens.data_ptr(), rows,
                              _opt_ptr(state_indices, torch.int32, "state_indices", rows),
                              _opt_ptr(num_accepted, torch.int32, "num_accepted", rows),
                              int(window), A, _stream(stream))
    _lib.check("kda_conv_compact", st)


def kda_flush_layers(layers, pools, state_indices, rec_prev, pending, record_rows=None,
                     stream=None) -> None:
    """Replay every pending commit of every layer in one launch (the flush)."""
    _on_gpu(pools[0], state_indices, pending, record_rows, *layers, *pools, *rec_prev)
    lib = _lib.load()
    rows = state_indices.numel()
    n, Ls, Ps, Rs = _layer_arrays(layers, pools, state_indices, rec_prev, rows)
    st = lib.kda_flush_layers(Ls, Ps, Rs, n, rows,
                              _opt_ptr(record_rows, torch.int32, "record_rows", rows),
                              _opt_ptr(pending, torch.int32, "pending", rec_prev[0].rows),
                              _stream(stream))
    _lib.check("kda_flush_layers", st)
