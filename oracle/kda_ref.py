"""CPU oracle for KDA speculative verify and accepted-token commit ("RecoverSSM").

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it, to check the HIP library and to time a plain CPU reference.

What it computes (sources are the four web pages on the method):

* The KDA recurrence (a gated delta rule with one decay per key channel), as
  the per-token loop of ``_verify_kernel`` on the page "recoverssm.py
  (GLM-5.3-Flash KDA speculative verify with one checkpoint state per
  request)". Per token, with the state S of shape [K, V]:
      q^ = scale * q / sqrt(sum(q*q) + 1e-6),   k^ = k / sqrt(sum(k*k) + 1e-6)
      g  = gate(g_raw + g_bias)                 (one value per key channel)
      beta = sigmoid(beta_raw)
      S  = diag(exp(g)) S
      u  = beta * (v - S^T k^)
      S  = S + k^ u^T
      o  = S^T q^
* The bounded gate lower_bound * sigmoid(exp(A_log) * x) of that same loop and
  of the kda.py page's FlashKDA-prefill docstring, and the unbounded softplus
  gate -exp(A_log) * softplus(x), which the kda.py page names (layer
  constructor) but does not print (this is a reading; see ``gate``).
* The RecoverSSM contract (recoverssm.py module docstring, ``_verify_kernel``,
  ``_prepare_commit_plan_kernel``): verify runs each row's window from its
  checkpoint, writes outputs and raw records and leaves the checkpoint alone;
  commit replays the first n' = min(max(n, 0), T_i, Q) records and writes the
  checkpoint in place.
* The commit plan and its align mode (recoverssm.py, ``_prepare_commit_plan_kernel``
  and ``_replay_indices_kernel``): with a block table per request, the state
  after the last committed token goes to the block holding that token and the
  state at a crossed block boundary to that boundary's block; and the
  conv-state compaction of the same commit (``_compact_conv_state_kernel``).
* The stock speculative path that RecoverSSM replaces (recoverssm.py module
  docstring; kda.py, ``_forward``, its spec branch into the fused recurrent
  kernel with a row of state indices per request; recoverssm.py,
  ``_replay_indices_kernel``, which states how that kernel uses the row): the
  recurrence from the state in column num_accepted - 1 of the row, storing
  the state after token t into the block of column t; see
  ``kda_recurrent_spec``.
* The deferred commit of the page "vllm.models.kimi_k3.nvidia.specialized_decode
  .recoverssm.context" (``KDADeferredCommitContext.commit`` / ``flush``,
  ``KDARecoverSSMDeferred``): commit turns n' into ``pending[record_row]``
  except for eager rows, committed at once; the next verify folds the pending
  replay into the checkpoint before it verifies.

Everything is float64. Inputs are taken as the GPU library takes them: bf16
bit patterns (uint16) are widened exactly; fp32 parameters and checkpoints are
widened exactly. Outputs are rounded once: o to bf16 round-to-nearest-even,
checkpoints to fp32 round-to-nearest-even (numpy's float64 -> float32 cast).

Layouts (the same as the library's boundary):
  q, k, g       uint16 [tokens, H, K]     v uint16 [tokens, H, V]
  beta          uint16 [tokens, H]        o uint16 [tokens, H, V]
  pool          float32 [slots, H, V, K]  (K fastest; S = stored^T)
  records       uint16 k,g [rows+1, H, Q, K], v [rows+1, H, Q, V],
                beta [rows+1, H, Q]; record row r lives at index r + 1 and
                index 0 is the scratch row of record row -1, which nothing reads.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Added to the squared norm, inside the square root (``_verify_kernel``).
L2_EPS = 1e-6


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits, 8 exponent bits)
    with round-to-nearest, ties to even, straight from float64 (no detour
    through fp32, which would round twice)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    ax = np.abs(x)
    tiny = 2.0 ** -126                      # smallest normal bf16
    sub = finite & (ax < tiny)
    nrm = finite & ~sub
    # Subnormal range: a fixed quantum of 2^-133.
    out[sub] = np.rint(x[sub] * 2.0 ** 133) * 2.0 ** -133
    # Normal range: x = m * 2^e with 0.5 <= |m| < 1; keep 8 bits of m.
    m, e = np.frexp(x[nrm])
    out[nrm] = np.ldexp(np.rint(m * 256.0), e - 8)
    out[~finite] = x[~finite]
    # Values at or above 2^128 after rounding overflow to infinity.
    big = finite & (np.abs(out) >= 2.0 ** 128)
    out[big] = np.copysign(np.inf, x[big])
    # The rounded values are exact in fp32; bf16 is the top 16 bits.
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(x)] = np.uint16(0x7FC0)
    return bits


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round to fp32, nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# Elementary functions of the per-token step
# --------------------------------------------------------------------------

def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)), split by sign so that no exp overflows."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + exp(x)), written as max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """x / sqrt(sum(x^2) + 1e-6) over the last axis (``_verify_kernel``)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def gate(x: np.ndarray, a_log: np.ndarray, lower_bound: float | None) -> np.ndarray:
    """Per-key-channel log-decay g from x = g_raw + g_bias.

    Bounded ("safe") gate, ``_verify_kernel`` and the kda.py FlashKDA-prefill
    docstring: g = lower_bound * sigmoid(exp(A_log) * x), so g lies in
    (lower_bound, 0).
    Unbounded gate (``lower_bound is None``), named "the default unbounded
    softplus gate" on the kda.py page (layer constructor) without a formula:
    read as g = -exp(A_log) * softplus(x) <= 0. Parity unpinned beyond its
    properties: no page prints this formula.

    ``a_log`` broadcasts against the leading axes of ``x`` (one per head).
    """
    a = np.exp(np.asarray(a_log, dtype=np.float64))
    if lower_bound is None:
        return -a * softplus(x)
    return float(lower_bound) * sigmoid(a * x)


def kda_step(S: np.ndarray, q_hat: np.ndarray | None, k_hat: np.ndarray,
             v: np.ndarray, g: np.ndarray, beta: np.ndarray):
    """One token of the recurrence, in the order of ``_verify_kernel``'s loop:
    decay the key channels, delta-rule update, then read the output from the
    updated state.

    S [..., K, V]; q_hat, k_hat, g [..., K]; v [..., V]; beta [...].
    Returns (S', o) with o [..., V], or (S', None) when q_hat is None.
    """
    S = np.exp(g)[..., :, None] * S
    u = beta[..., None] * (v - np.einsum("...kv,...k->...v", S, k_hat))
    S = S + k_hat[..., :, None] * u[..., None, :]
    o = None if q_hat is None else np.einsum("...kv,...k->...v", S, q_hat)
    return S, o


# --------------------------------------------------------------------------
# The library's four calls
# --------------------------------------------------------------------------

@dataclass
class Layer:
    """One layer's gate parameters. a_log float32 [H]; g_bias float32 [H*K]."""
    a_log: np.ndarray
    g_bias: np.ndarray
    scale: float
    lower_bound: float | None = None   # None: unbounded softplus gate


@dataclass
class Records:
    """Raw per-token inputs saved by verify for the commit (bf16 bits)."""
    k: np.ndarray      # [rows+1, H, Q, K]
    v: np.ndarray      # [rows+1, H, Q, V]
    g: np.ndarray      # [rows+1, H, Q, K]
    beta: np.ndarray   # [rows+1, H, Q]

    @property
    def rows(self) -> int:
        return self.k.shape[0] - 1

    @property
    def window(self) -> int:
        return self.k.shape[2]

    @staticmethod
    def empty(rows: int, H: int, Q: int, K: int, fill: int = 0) -> "Records":
        return Records(
            k=np.full((rows + 1, H, Q, K), fill, np.uint16),
            v=np.full((rows + 1, H, Q, K), fill, np.uint16),
            g=np.full((rows + 1, H, Q, K), fill, np.uint16),
            beta=np.full((rows + 1, H, Q), fill, np.uint16),
        )

    def copy(self) -> "Records":
        return Records(self.k.copy(), self.v.copy(), self.g.copy(), self.beta.copy())


def _head_params(layer: Layer, H: int, K: int):
    return (np.asarray(layer.g_bias, np.float32).astype(np.float64).reshape(H, K),
            np.asarray(layer.a_log, np.float32).astype(np.float64).reshape(H, 1))


def _prepare(layer: Layer, H: int, K: int, q_bits, k_bits, v_bits, g_bits, b_bits):
    """Widen one token's raw inputs (all heads) and form q^, k^, g, beta."""
    g_bias, a_log = _head_params(layer, H, K)
    k_hat = l2_normalize(bf16_bits_to_f64(k_bits))
    q_hat = None
    if q_bits is not None:
        q_hat = l2_normalize(bf16_bits_to_f64(q_bits)) * float(np.float32(layer.scale))
    g = gate(bf16_bits_to_f64(g_bits) + g_bias, a_log, layer.lower_bound)
    beta = sigmoid(bf16_bits_to_f64(b_bits))
    return q_hat, k_hat, bf16_bits_to_f64(v_bits), g, beta


def _row_span(cu_seqlens, i: int, num_tokens: int):
    """Token range of row i; a malformed span counts as an empty row."""
    bos, eos = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
    if bos < 0 or eos < bos or eos > num_tokens:
        return bos, 0
    return bos, eos - bos


def _slot_ok(slot: int, num_slots: int) -> bool:
    # Slot 0 is the null block and slots <= 0 mean "skip this row"
    # (``_verify_kernel`` returns before any store).
    return 0 < slot < num_slots


def _record_index(record_rows, i: int, rows: int) -> int:
    """Storage index of row i's records: record row r lives at r + 1 and
    record row -1 (or anything out of range) at the scratch index 0."""
    r = i if record_rows is None else int(record_rows[i])
    return r + 1 if 0 <= r < rows else 0


def _load_state(pool: np.ndarray, slot: int) -> np.ndarray:
    # The pool stores [H, V, K]; the math uses S [H, K, V].
    return pool[slot].astype(np.float64).transpose(0, 2, 1)


def _store_state(pool: np.ndarray, slot: int, S: np.ndarray) -> None:
    pool[slot] = f64_to_f32(S.transpose(0, 2, 1))


def _replay(layer: Layer, S: np.ndarray, rec: Records, ri: int, n: int,
            start: int = 0) -> np.ndarray:
    """Run records start .. n-1 of storage row ri through the recurrence
    (no output: the commit only needs the state)."""
    H, K = S.shape[0], S.shape[1]
    for t in range(start, n):
        _, k_hat, v, g, beta = _prepare(layer, H, K, None, rec.k[ri, :, t],
                                        rec.v[ri, :, t], rec.g[ri, :, t],
                                        rec.beta[ri, :, t])
        S, _ = kda_step(S, None, k_hat, v, g, beta)
    return S


def _run_tokens(layer: Layer, S: np.ndarray, q, k, v, g, beta, bos: int, T: int, o):
    H, K = S.shape[0], S.shape[1]
    for t in range(T):
        tok = bos + t
        q_hat, k_hat, vv, gg, bb = _prepare(layer, H, K, q[tok], k[tok], v[tok],
                                            g[tok], beta[tok])
        S, out = kda_step(S, q_hat, k_hat, vv, gg, bb)
        o[tok] = f64_to_bf16_bits(out)
    return S


def kda_recurrent(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices, o) -> None:
    """Plain full-state recurrence: every token of every valid row, from the
    row's slot; writes o and stores the final state in the slot in place."""
    N, ntok, H = len(state_indices), q.shape[0], q.shape[1]
    for i in range(N):
        bos, T = _row_span(cu_seqlens, i, ntok)
        slot = int(state_indices[i])
        if T == 0 or not _slot_ok(slot, pool.shape[0]):
            continue
        S = _run_tokens(layer, _load_state(pool, slot), q, k, v, g, beta, bos, T, o)
        _store_state(pool, slot, S)


def spec_source_column(num_accepted, i: int, cols: int) -> int:
    """Column of row i's state-index row that holds its initial state:
    num_accepted[i] - 1, the state after the last token accepted in the
    previous step (recoverssm.py, ``_replay_indices_kernel``: the stock
    kernel reads its initial state at column num_accepted - 1). Counts are
    clamped to 1..cols (a reading: the pages pass at least one accepted token,
    the bonus token, and never more than the row holds); no counts: column 0."""
    if num_accepted is None:
        return 0
    return min(max(int(num_accepted[i]), 1), int(cols)) - 1


def kda_recurrent_spec(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_table,
                       num_accepted, o) -> None:
    """The stock full-state speculative step (recoverssm.py module docstring:
    it keeps 1 + num_spec recurrent states per request and writes one full
    state per verified token; kda.py ``_forward``: the spec branch calls the
    fused recurrent kernel with a [rows, columns] table of state indices and
    the accepted counts; recoverssm.py ``_replay_indices_kernel``: that
    kernel reads its initial state at column num_accepted - 1 and stores the
    state after token t to the block of column t unless it is the null block).

    state_table int32 [rows, cols]. For each row i with T_i > 0 whose source
    block s = state_table[i, spec_source_column(...)] is in (0, num_slots):
    run the T_i tokens from pool[s], write o for each, and after token t
    (t < cols) store the state into pool[state_table[i, t]] when that block
    is in (0, num_slots). The initial state is read before anything is
    stored, so a column may name the source block itself. Rows whose blocks
    overlap another row's are outside the contract."""
    N, ntok, H = state_table.shape[0], q.shape[0], q.shape[1]
    cols = state_table.shape[1]
    K = q.shape[2]
    nslots = pool.shape[0]
    for i in range(N):
        bos, T = _row_span(cu_seqlens, i, ntok)
        src = int(state_table[i, spec_source_column(num_accepted, i, cols)])
        if T == 0 or not _slot_ok(src, nslots):
            continue
        S = _load_state(pool, src)
        for t in range(T):
            tok = bos + t
            q_hat, k_hat, vv, gg, bb = _prepare(layer, H, K, q[tok], k[tok], v[tok],
                                                g[tok], beta[tok])
            S, out = kda_step(S, q_hat, k_hat, vv, gg, bb)
            o[tok] = f64_to_bf16_bits(out)
            if t < cols:
                dst = int(state_table[i, t])
                if _slot_ok(dst, nslots):
                    _store_state(pool, dst, S)


def _write_records(rec: Records, ri: int, k, v, g, beta, bos: int, T: int) -> None:
    # Records are the raw bf16 inputs (``_verify_kernel``); the window holds Q
    # tokens, so tokens at or beyond Q are not recorded.
    n = min(T, rec.window)
    rec.k[ri, :, :n] = k[bos:bos + n].transpose(1, 0, 2)
    rec.v[ri, :, :n] = v[bos:bos + n].transpose(1, 0, 2)
    rec.g[ri, :, :n] = g[bos:bos + n].transpose(1, 0, 2)
    rec.beta[ri, :, :n] = beta[bos:bos + n].transpose(1, 0)


def kda_verify(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices,
               rec: Records, o, record_rows=None) -> None:
    """Verify each valid row's window from its checkpoint: write o and the raw
    records; the pool is not written."""
    N, ntok, H = len(state_indices), q.shape[0], q.shape[1]
    for i in range(N):
        bos, T = _row_span(cu_seqlens, i, ntok)
        slot = int(state_indices[i])
        if T == 0 or not _slot_ok(slot, pool.shape[0]):
            continue
        _run_tokens(layer, _load_state(pool, slot), q, k, v, g, beta, bos, T, o)
        _write_records(rec, _record_index(record_rows, i, rec.rows), k, v, g, beta, bos, T)


def commit_length(n: int, T: int, Q: int) -> int:
    """n' = min(max(n, 0), T_i, Q) (``_prepare_commit_plan_kernel``)."""
    return min(max(int(n), 0), int(T), int(Q))


def kda_commit(layer: Layer, cu_seqlens, num_tokens: int, pool, state_indices,
               rec: Records, num_accepted, record_rows=None, pending=None,
               eager=None) -> None:
    """Commit the accepted prefix.

    Without ``pending``: every valid row (slot > 0, n' > 0, a record row)
    replays its first n' records from the slot and writes the slot in place.
    With ``pending`` (the deferred mode): pending[r] = 0 for eager rows and n'
    otherwise (0 for rows that are not valid); eager rows are committed now,
    the rest wait for the next deferred verify. Rows without a record row
    (-1) are never committed.
    """
    N = len(state_indices)
    for i in range(N):
        _, T = _row_span(cu_seqlens, i, num_tokens)
        slot = int(state_indices[i])
        n = commit_length(num_accepted[i], T, rec.window)
        ri = _record_index(record_rows, i, rec.rows)
        valid = _slot_ok(slot, pool.shape[0]) and n > 0 and ri > 0
        now = True
        if pending is not None:
            now = eager is not None and bool(eager[i])
            if ri > 0:
                pending[ri - 1] = 0 if now else (n if valid else 0)
        if valid and now:
            _store_state(pool, slot, _replay(layer, _load_state(pool, slot), rec, ri, n))


@dataclass
class Align:
    """Align mode of the commit: one row of block ids per request row (block 0
    is the null block), the tokens each request had cached before the step,
    and the tokens per block."""
    block_table: np.ndarray    # int32 [rows, width]
    num_computed: np.ndarray   # int32 [rows]
    block_size: int


def commit_plan(cu_seqlens, num_tokens: int, num_accepted, state_indices, Q: int,
                align: Align | None = None) -> np.ndarray:
    """Per row (n', final block, boundary block, boundary length), as
    ``_prepare_commit_plan_kernel`` computes them (int64 [rows, 4]).

    n' = min(max(n, 0), T_i, Q). Without align the final block is the source
    (the row's state index) and there is no boundary. With align, c = tokens
    cached before the step (a negative count counts as 0, a reading):
      final column    = min(max(c + n' - 1, 0) // block_size, width - 1)
      next boundary   = (c // block_size + 1) * block_size
      boundary length = next boundary - c
      boundary block  = the block at column next boundary // block_size - 1
                        when c + n' reaches the next boundary (and that column
                        is inside the table, a reading), else the null block.
    Rows with a source <= 0 or n' = 0 get (0, 0, 0, 0)."""
    N = len(state_indices)
    plan = np.zeros((N, 4), np.int64)
    for i in range(N):
        _, T = _row_span(cu_seqlens, i, num_tokens)
        n = commit_length(num_accepted[i], T, Q)
        src = int(state_indices[i])
        final, bnd, blen = src, 0, 0
        if align is not None:
            bs = int(align.block_size)
            width = align.block_table.shape[1]
            c = max(int(align.num_computed[i]), 0)
            col = min(max(c + n - 1, 0) // bs, width - 1)
            final = int(align.block_table[i, col])
            nb = (c // bs + 1) * bs
            blen = nb - c
            bcol = nb // bs - 1
            if c + n >= nb and bcol < width:
                bnd = int(align.block_table[i, bcol])
        if src > 0 and n > 0:
            plan[i] = (n, final, bnd, blen)
    return plan


def kda_commit_align(layer: Layer, cu_seqlens, num_tokens: int, pool, state_indices,
                     rec: Records, num_accepted, align: Align, record_rows=None,
                     pending=None, eager=None) -> None:
    """The commit in align mode (``_replay_indices_kernel`` and the commit's
    replay): replay the first n' records from the source block; the state
    after the first boundary-length records goes to the boundary block when
    that length is below n' and the block is not null; the state after n'
    records goes to the final block. A row is skipped without a source, a
    final block (not null and inside the pool) or a record row. Blocks that
    are out of the pool are not written (a reading for memory safety).
    Destination blocks are assumed to be no other row's source.

    With ``pending`` (the deferred commit in align mode: recoverssm.context,
    ``KDADeferredCommitContext.commit`` takes the block table together with
    ``pending``, and ``KDARecoverSSMDeferred.eager`` marks the rows committed
    after sampling, in align mode those near a block boundary): the counts
    are written as in ``kda_commit`` (pending[r] = 0 for eager rows, else n'
    for rows with a source, n' > 0 and a record row, else 0) and only the
    eager rows commit now, in align mode as above. The other rows' replay
    waits for the next deferred verify, which folds it in place at the row's
    slot, so a caller defers only rows whose final block is their source and
    that cross no block boundary (a reading: the pages print neither
    ``_defer_commit_kernel`` nor the fold's plan)."""
    plan = commit_plan(cu_seqlens, num_tokens, num_accepted, state_indices, rec.window, align)
    nslots = pool.shape[0]
    for i in range(len(state_indices)):
        n, final, bnd, blen = (int(x) for x in plan[i])
        src = int(state_indices[i])
        ri = _record_index(record_rows, i, rec.rows)
        if pending is not None:
            now = eager is not None and bool(eager[i])
            if ri > 0:
                pending[ri - 1] = 0 if now else (n if (n > 0 and _slot_ok(src, nslots)) else 0)
            if not now:
                continue
        if n == 0 or ri == 0 or not _slot_ok(src, nslots) or not _slot_ok(final, nslots):
            continue
        S = _load_state(pool, src)
        if 0 < blen < n and _slot_ok(bnd, nslots):
            S = _replay(layer, S, rec, ri, blen)
            _store_state(pool, bnd, S)
            S = _replay(layer, S, rec, ri, n, start=blen)
        else:
            S = _replay(layer, S, rec, ri, n)
        _store_state(pool, final, S)


def conv_compact(conv: np.ndarray, cu_seqlens, num_tokens: int, num_accepted, state_indices,
                 Q: int, history: int, align: Align | None = None) -> None:
    """The conv-state compaction of the commit (``_compact_conv_state_kernel``).

    conv [blocks, channels, width], any element type, copied exactly. After a
    verify, the token axis of a row's source block holds the last history - 1
    inputs before the window, then the window's inputs; after n' accepted
    tokens the last ``history`` inputs are columns n' - 1 .. n' + history - 2.
    They move to columns 0 .. history - 1 of the final block (the source
    itself without align). In align mode the columns from boundary length - 1
    also go to the boundary block, when there is one. Rows without a source
    or final block inside the table, or with n' = 0, are left alone; all of a
    row's reads come before its writes."""
    plan = commit_plan(cu_seqlens, num_tokens, num_accepted, state_indices, Q, align)
    nb = conv.shape[0]
    for i in range(len(state_indices)):
        n, final, bnd, blen = (int(x) for x in plan[i])
        src = int(state_indices[i])
        if n == 0 or not 0 < src < nb or not 0 < final < nb:
            continue
        vals = conv[src, :, n - 1:n - 1 + history].copy()
        if align is not None and 0 < bnd < nb:
            bvals = conv[src, :, blen - 1:blen - 1 + history].copy()
            conv[bnd, :, :history] = bvals
        conv[final, :, :history] = vals


def kda_verify_deferred(layer: Layer, q, k, v, g, beta, cu_seqlens, pool, state_indices,
                        rec_prev: Records, pending, rec_next: Records, record_rows,
                        o) -> None:
    """Fold each valid row's pending replay, then verify its new window.

    p = min(max(pending[r], 0), Q) records of ``rec_prev`` are replayed from
    the slot and, if p > 0, the slot is written. The row's T_i new tokens are
    then verified from that stored state, writing o and ``rec_next``. With
    T_i = 0 only the fold runs (this is the flush). ``pending`` is read only.
    """
    N, ntok, H = len(state_indices), q.shape[0], q.shape[1]
    for i in range(N):
        bos, T = _row_span(cu_seqlens, i, ntok)
        slot = int(state_indices[i])
        if not _slot_ok(slot, pool.shape[0]):
            continue
        ri = _record_index(record_rows, i, rec_prev.rows)
        p = min(max(int(pending[ri - 1]), 0), rec_prev.window) if ri > 0 else 0
        if p > 0:
            _store_state(pool, slot, _replay(layer, _load_state(pool, slot), rec_prev, ri, p))
        if T == 0:
            continue
        _run_tokens(layer, _load_state(pool, slot), q, k, v, g, beta, bos, T, o)
        _write_records(rec_next, _record_index(record_rows, i, rec_next.rows),
                       k, v, g, beta, bos, T)
