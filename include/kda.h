/*
 * kda.h -- C ABI of libkda: KDA (Kimi Delta Attention) speculative verify and
 * accepted-token commit with one fp32 checkpoint state per request
 * ("RecoverSSM"), hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The method, per token and per head, with the state S of shape [K, V]
 * (pages: "recoverssm.py (GLM-5.3-Flash KDA speculative verify with one
 * checkpoint state per request)", _verify_kernel per-token loop):
 *     q^ = scale * q / sqrt(sum(q*q) + 1e-6)      k^ = k / sqrt(sum(k*k) + 1e-6)
 *     g  = lower_bound * sigmoid(exp(A_log) * (g_raw + g_bias))  (bounded gate)
 *        | -exp(A_log) * softplus(g_raw + g_bias)                 (unbounded gate)
 *     beta = sigmoid(beta_raw)
 *     S = diag(exp(g)) S;  u = beta * (v - S^T k^);  S = S + k^ u^T;  o = S^T q^
 * The unbounded gate is named but not printed on the kda.py page (layer
 * constructor); the formula above is this library's reading of it.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer inside the structs and every array argument is a DEVICE
 *   pointer unless marked "host". The structs themselves live in host memory
 *   and are read only during the call.
 * - bf16 values are passed as uint16_t bit patterns.
 * - Token arrays: q, k, v, g are [num_tokens, H, 128] with the head stride
 *   128 elements and a token stride given in elements (q/k/v may be column
 *   blocks of one projection output); beta is [num_tokens, H] with a token
 *   stride. o is dense [num_tokens, H, 128].
 * - A request row i owns tokens [cu_seqlens[i], cu_seqlens[i+1]) (T_i of
 *   them). A row with state_indices[i] <= 0 is skipped: nothing of it is read
 *   or written (slot 0 is the null block). A row whose span is malformed
 *   (negative start, end before start or beyond num_tokens) or whose slot is
 *   >= num_slots is also skipped: the kernels range-check every index they
 *   read from device memory, so bad metadata cannot make them access memory
 *   out of bounds. Distinct rows must use distinct slots.
 * - Checkpoint pool: fp32 [num_slots, H, V, K], K fastest (each (slot, head)
 *   is one dense 128 x 128 block of 64 KiB; the stored block is S^T). The
 *   slot stride is given in elements and must be a multiple of 4; the
 *   pointer must be 16-byte aligned.
 * - Records (raw bf16 inputs saved by verify for the commit; the record
 *   layout is re-chosen head-major so that one (row, head) is contiguous):
 *       k, g [rows+1, H, Q, 128], v [rows+1, H, Q, 128], beta [rows+1, H, Q]
 *   where Q = window (tokens per record row). Record row r is stored at
 *   index r + 1; index 0 is a scratch row: rows whose record row is -1 (or
 *   out of range) write their records there and nothing reads it (pages:
 *   "vllm.models.kimi_k3...recoverssm.context", allocate_records). Only the
 *   first Q tokens of a row are recorded.
 * - Calls are asynchronous on `stream`, enqueue at most one kernel, never
 *   allocate, never synchronise and never abort. The caller owns every
 *   buffer. The host checks below run before anything is enqueued; on any
 *   error nothing is enqueued. num_rows == 0 returns KDA_OK with no launch.
 * - Device metadata that the host cannot see (cu_seqlens, state_indices,
 *   record_rows, num_accepted, pending, eager) is only range-checked inside
 *   the kernels as described above.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,         /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,        /* inconsistent sizes (H <= 0, head_dim, window, strides, eager without pending) */
  KDA_ERR_CAPACITY = 3,     /* more rows than record rows (identity record mapping) */
  KDA_ERR_ALIGN = 4,        /* pointer or stride not aligned for the vector loads */
  KDA_ERR_ALIAS = 5,        /* an output range overlaps an input or another output */
  KDA_ERR_UNSUPPORTED = 6,  /* head_dim other than 128 */
  KDA_ERR_LAUNCH = 7,       /* the HIP launch reported an error */
  KDA_ERR_METADATA = 8      /* kda_check_rows: a row breaks a precondition (see kda_row_issue) */
} kda_status;

/* What kda_check_rows found wrong with a row. */
typedef enum kda_row_issue {
  KDA_ROW_OK = 0,
  KDA_ROW_SPAN = 1,          /* cu_seqlens[i] < 0, cu_seqlens[i+1] < cu_seqlens[i] or > num_tokens */
  KDA_ROW_WINDOW = 2,        /* T_i > max_seqlen (max_seqlen > 0) */
  KDA_ROW_SLOT_RANGE = 3,    /* state_indices[i] >= num_slots */
  KDA_ROW_SLOT_DUP = 4,      /* a slot used by an earlier row */
  KDA_ROW_RECORD_RANGE = 5,  /* record row < -1 or >= rec_rows */
  KDA_ROW_RECORD_DUP = 6     /* a record row used by an earlier row */
} kda_row_issue;

/* One layer's gate parameters (host struct). */
typedef struct kda_layer {
  int32_t num_heads;        /* H > 0 */
  int32_t head_dim;         /* K == V; must be 128 */
  float scale;              /* multiplies q^ (normally head_dim^-0.5) */
  int32_t has_lower_bound;  /* 1: bounded gate with lower_bound; 0: unbounded gate */
  float lower_bound;        /* e.g. -5; ignored when has_lower_bound == 0 */
  const float* a_log;       /* [H] fp32 */
  const float* g_bias;      /* [H * head_dim] fp32, 16-byte aligned */
} kda_layer;

/* A packed ragged batch of raw activations (host struct of device pointers). */
typedef struct kda_tokens {
  const uint16_t* q;        /* [num_tokens, H, K] bf16, token stride stride_q */
  const uint16_t* k;        /* [num_tokens, H, K] bf16, token stride stride_k */
  const uint16_t* v;        /* [num_tokens, H, V] bf16, token stride stride_v */
  const uint16_t* g;        /* [num_tokens, H, K] bf16 raw gate, token stride stride_g */
  const uint16_t* beta;     /* [num_tokens, H] bf16 raw beta, token stride stride_beta */
  int64_t stride_q, stride_k, stride_v, stride_g, stride_beta;   /* elements */
  const int32_t* cu_seqlens;  /* [num_rows + 1] int32 */
  int32_t num_rows;
  int32_t num_tokens;       /* rows of the token arrays (and of o) */
  /* An upper bound on every row's window T_i that the caller guarantees, or
   * 0 when unknown (pages: kda.py, _forward, where the speculative window's
   * maximum query length num_spec + 1 is known on the host and handed to the
   * short convolution). Used by kda_verify only: with 1 <= max_seqlen <= 8 it
   * runs kernels built for windows of at most that many tokens; larger
   * values run the general kernels. A row with a slot and T_i > max_seqlen
   * breaks the caller's guarantee and is not verified: every output of its
   * tokens is set to NaN (bf16 0x7FC0) and so is the beta record of each of
   * its recorded tokens (the first min(T_i, Q)); its other records are not
   * written. The error thus shows in the outputs, and a commit that replays
   * such a row (n' > 0) stores NaN, never a plausible checkpoint (pages:
   * recoverssm.py, _check_config fails where a commit would otherwise go
   * wrong silently). kda_check_rows reports such rows on the host
   * (KDA_ROW_WINDOW). Negative -> KDA_ERR_SHAPE (every call). */
  int32_t max_seqlen;
} kda_tokens;

/* The checkpoint pool of one layer (host struct of device pointers). */
typedef struct kda_pool {
  float* state;                  /* [num_slots, H, 128, 128] fp32, K fastest */
  int64_t slot_stride;           /* elements between slots, >= H*128*128, multiple of 4 */
  int32_t num_slots;
  const int32_t* state_indices;  /* [num_rows] int32 slot per row; <= 0: skip the row */
} kda_pool;

/* Raw bf16 records (host struct of device pointers); pointers are the
 * allocation bases, i.e. the scratch row at index 0. */
typedef struct kda_records {
  uint16_t* k;              /* [rows + 1, H, window, 128] */
  uint16_t* v;              /* [rows + 1, H, window, 128] */
  uint16_t* g;              /* [rows + 1, H, window, 128] */
  uint16_t* beta;           /* [rows + 1, H, window] */
  int32_t rows;             /* record rows (not counting the scratch row) */
  int32_t window;           /* Q: tokens per record row, 1..64 */
} kda_records;

/* Align mode of the commit (host struct of device pointers; pages:
 * recoverssm.py, _prepare_commit_plan_kernel with its align mode and
 * _replay_indices_kernel). Per request row i, with c = num_computed[i] (the
 * tokens cached before the step; negative counts as 0) and bs = block_size:
 *   final block    = block_table[i][min(max(c + n' - 1, 0) / bs, width - 1)]
 *   next boundary  = (c / bs + 1) * bs, boundary length = next - c
 *   boundary block = block_table[i][next / bs - 1] when c + n' >= next and that
 *                    column is below width, else none.
 * The state after n' records goes to the final block; the state after the
 * boundary length goes to the boundary block when that length is below n'.
 * Block 0 is the null block: a row whose final block is 0 (or outside the
 * pool) commits nothing. Destination blocks must not be another row's
 * source. */
typedef struct kda_align {
  const int32_t* block_table;   /* [num_rows, width] int32, row stride row_stride elements */
  int64_t row_stride;           /* >= width */
  int32_t width;                /* >= 1 */
  const int32_t* num_computed;  /* [num_rows] int32 */
  int32_t block_size;           /* tokens per block, >= 1 */
} kda_align;

/* The block ids of the stock speculative step (host struct of device
 * pointers): per request row, one block per window position. */
typedef struct kda_spec_table {
  const int32_t* indices;       /* [num_rows, cols] int32, row stride row_stride elements */
  int64_t row_stride;           /* >= cols */
  int32_t cols;                 /* >= 1: 1 + num_spec positions */
  const int32_t* num_accepted;  /* [num_rows] int32, or NULL (the source is column 0) */
} kda_spec_table;

/* One layer's conv state (host struct of a device pointer): 16-bit elements
 * [num_blocks, channels, width] with element strides. */
typedef struct kda_conv_state {
  uint16_t* state;
  int64_t block_stride, dim_stride, token_stride;   /* elements, >= 1 */
  int32_t num_blocks;
} kda_conv_state;

/*
 * kda_recurrent -- the plain full-state recurrence (pages: recoverssm.py,
 * _verify_kernel's per-token body, which is the stock fused recurrent KDA
 * kernel's; kda.py, the plain-decode call of the recurrent kernel).
 * For each valid row: load the row's checkpoint, run all T_i tokens (any
 * length), write o for each token, store the final state into the slot in
 * place. It is the equivalence reference of kda_commit: committing n tokens
 * gives the same bits as kda_recurrent over those n tokens.
 *   o: [num_tokens, H, 128] bf16 output; rows that are skipped are not written.
 * Errors: NULL -> KDA_ERR_NULL; head_dim != 128 -> KDA_ERR_UNSUPPORTED;
 * H <= 0, negative sizes or strides too small -> KDA_ERR_SHAPE; misaligned
 * (state 16 B, q/k/v/g 8 B with token strides multiple of 4) -> KDA_ERR_ALIGN;
 * o overlapping the pool or a token array, or a token array overlapping the
 * pool (which is written) -> KDA_ERR_ALIAS.
 */
kda_status kda_recurrent(const kda_layer* layer, const kda_tokens* tokens,
                         const kda_pool* pool, uint16_t* o, hipStream_t stream);

/*
 * kda_recurrent_spec -- the stock speculative step that RecoverSSM replaces,
 * one full state stored per verified token (pages: recoverssm.py, module
 * docstring: the stock path keeps 1 + num_spec states per request; kda.py,
 * _forward, its speculative branch into the fused recurrent kernel with a
 * row of state indices per request and the accepted counts; recoverssm.py,
 * _replay_indices_kernel: that kernel reads the initial state at column
 * num_accepted - 1 and stores the state after token t to column t unless
 * it is the null block). Kept as the baseline whose state traffic the
 * verify + commit removes.
 * For each row i with T_i > 0: the source column is
 * c = min(max(num_accepted[i], 1), cols) - 1 (0 when num_accepted is NULL)
 * and the source block table->indices[i][c]; a source outside
 * (0, num_slots) skips the row (nothing written). Otherwise run the T_i
 * tokens from the source with the per-token code of kda_recurrent, write o
 * for each token, and after token t < cols store the state into block
 * indices[i][t] when it lies in (0, num_slots). The source is read before
 * any store, so a column may name the source itself. The state in column t
 * has the bits kda_recurrent stores after the same t + 1 tokens.
 *   pool: pool->state_indices is not used (may be NULL).
 *   o: [num_tokens, H, 128] bf16.
 * Blocks named by one row must not be named by another row. Errors as
 * kda_recurrent, plus: table NULL -> KDA_ERR_NULL; cols < 1 or
 * row_stride < cols -> KDA_ERR_SHAPE; the block ids or the counts
 * overlapping the pool or o -> KDA_ERR_ALIAS.
 */
kda_status kda_recurrent_spec(const kda_layer* layer, const kda_tokens* tokens,
                              const kda_pool* pool, const kda_spec_table* table,
                              uint16_t* o, hipStream_t stream);

/*
 * kda_verify -- speculative verify from the checkpoint (pages: recoverssm.py,
 * module docstring and _verify_kernel / kda_recoverssm_verify). For each valid
 * row: run its T_i window tokens from the checkpoint, write o, and write the
 * raw k, v, g, beta of tokens 0..min(T_i, Q)-1 to record row r, where
 * r = record_rows[i] (record_rows == NULL: r = i, which needs
 * num_rows <= rec->rows, else KDA_ERR_CAPACITY). The pool is read only: no
 * state is written. With tokens->max_seqlen in 1..8 the rows within the
 * bound give the same bits as without it, and the rows longer than it get
 * NaN outputs and NaN beta records (see kda_tokens).
 * Errors as kda_recurrent, plus: records overlapping o, the pool or the
 * token arrays -> KDA_ERR_ALIAS; misaligned records -> KDA_ERR_ALIGN.
 */
kda_status kda_verify(const kda_layer* layer, const kda_tokens* tokens,
                      const kda_pool* pool, const kda_records* rec,
                      const int32_t* record_rows, uint16_t* o, hipStream_t stream);

/*
 * kda_commit -- commit the accepted prefix (pages: recoverssm.py,
 * _prepare_commit_plan_kernel and Glm5NextRecoverSSMCommitContext.commit;
 * deferred mode: recoverssm.context, KDADeferredCommitContext.commit).
 * For row i: T_i from cu_seqlens, n' = min(max(num_accepted[i], 0), T_i, Q),
 * r = record_rows ? record_rows[i] : i. The row is valid when its slot is in
 * (0, num_slots), n' > 0 and 0 <= r < rec->rows.
 *  - pending == NULL: every valid row replays records 0..n'-1 of record row r
 *    from its slot and stores the state into the slot in place.
 *  - pending != NULL (deferred): for 0 <= r < rec->rows,
 *    pending[r] = eager[i] ? 0 : (valid ? n' : 0); rows with eager[i] != 0
 *    are committed now as above; the others wait for kda_verify_deferred.
 *    eager == NULL: no row is eager.
 *   num_accepted: [num_rows] int32; pending: [rec->rows] int32, indexed by
 *   record row; eager: [num_rows] uint8 mask.
 * Errors: NULL pointers -> KDA_ERR_NULL; eager without pending ->
 * KDA_ERR_SHAPE; record_rows == NULL with num_rows > rec->rows ->
 * KDA_ERR_CAPACITY; the pool overlapping the records -> KDA_ERR_ALIAS.
 */
kda_status kda_commit(const kda_layer* layer, const int32_t* cu_seqlens, int32_t num_rows,
                      const kda_pool* pool, const kda_records* rec,
                      const int32_t* record_rows, const int32_t* num_accepted,
                      int32_t* pending, const uint8_t* eager, hipStream_t stream);

/*
 * kda_verify_deferred -- fold the pending commit, then verify, in one pass
 * (pages: recoverssm.context, module summary and KDARecoverSSMDeferred: the
 * next verify replays the pending commit in the same pass).
 * For each row with a slot in (0, num_slots): r = record_rows[i];
 * p = min(max(pending[r], 0), rec_prev->window) when 0 <= r < rec_prev->rows,
 * else 0. Replay records 0..p-1 of rec_prev row r from the slot; if p > 0
 * store the state into the slot. Then verify the row's T_i tokens from that
 * state exactly as kda_verify does, writing o and rec_next row r. With
 * every T_i == 0 this is the flush (fold only). pending is read only.
 * rec_prev and rec_next must be different buffers with the same rows, window.
 * Errors as kda_verify, plus: rec_prev overlapping rec_next -> KDA_ERR_ALIAS;
 * mismatched rows/window -> KDA_ERR_SHAPE.
 */
kda_status kda_verify_deferred(const kda_layer* layer, const kda_tokens* tokens,
                               const kda_pool* pool, const kda_records* rec_prev,
                               const int32_t* pending, const kda_records* rec_next,
                               const int32_t* record_rows, uint16_t* o, hipStream_t stream);

/*
 * kda_commit_layers -- kda_commit for several layers in one launch (pages:
 * recoverssm.py, Glm5NextRecoverSSMCommitContext construction, which keeps
 * per-layer base-address arrays, and its commit, whose kernels run over
 * every layer in one grid; recoverssm.context, the deferred context's state
 * commit over num_layers x num_heads). After acceptance every layer's commit
 * is independent of the others, so one grid of layers x rows x heads x tiles
 * replaces num_layers launches.
 *   layers, pools, recs: HOST arrays of num_layers structs, 1..16 layers.
 *   Every layer: the same num_heads and head_dim, records with the same rows
 *   and window, and pools sharing one state_indices array (the same pointer:
 *   a request's slot number is the same in every layer's pool).
 *   cu_seqlens, num_rows, record_rows, num_accepted, pending, eager: shared,
 *   with the meaning of kda_commit; each layer does exactly what kda_commit
 *   would do for it (same bits). pending (deferred mode) holds one count per
 *   record row for all layers and is written once, as the first layer's pool
 *   sees the row (a slot at or beyond that pool's num_slots counts as
 *   skipped there).
 *   align (host struct, may be NULL): the align mode above, which writes
 *   the final (and boundary) block instead of the source. With pending as
 *   well (the deferred commit in align mode; pages: recoverssm.context,
 *   KDADeferredCommitContext.commit takes the block table with pending, and
 *   KDARecoverSSMDeferred.eager marks the rows committed after sampling, in
 *   align mode those near a block boundary): the eager rows commit now in
 *   align mode; the other rows only get their count,
 *   pending[r] = (slot in (0, num_slots) and n' > 0) ? n' : 0, and the next
 *   kda_verify_deferred replays them in place at their slot, so a caller
 *   defers only rows whose final block is their slot and that cross no
 *   block boundary.
 * Errors as kda_commit, plus: num_layers outside 1..16, layers that differ
 * in num_heads or record shape, or pools with different state_indices ->
 * KDA_ERR_SHAPE; a layer's pool or records overlapping another layer's pool
 * or records -> KDA_ERR_ALIAS; align with a NULL table or count array ->
 * KDA_ERR_NULL, with width < 1, block_size < 1 or row_stride < width ->
 * KDA_ERR_SHAPE.
 */
kda_status kda_commit_layers(const kda_layer* layers, const kda_pool* pools,
                             const kda_records* recs, int32_t num_layers,
                             const int32_t* cu_seqlens, int32_t num_rows,
                             const int32_t* record_rows, const int32_t* num_accepted,
                             int32_t* pending, const uint8_t* eager, const kda_align* align,
                             hipStream_t stream);

/*
 * kda_flush_layers -- the flush of the deferred commit for several layers in
 * one launch (pages: recoverssm.context, KDADeferredCommitContext.flush,
 * which replays every pending commit without a verify). For each layer and
 * each row with a slot in (0, num_slots): r = record_rows[i] (NULL: r = i),
 * p = min(max(pending[r], 0), rec_prev->window) when 0 <= r < rows, else 0;
 * replay records 0..p-1 of that layer's rec_prev row r from the slot and,
 * if p > 0, store the state in place. This is kda_verify_deferred with every
 * window empty, bit for bit; no token array is read and pending is read only.
 *   layers, pools, rec_prev: HOST arrays of num_layers structs, 1..16 layers,
 *   with the constraints of kda_commit_layers.
 * Errors as kda_commit_layers; pending NULL -> KDA_ERR_NULL.
 */
kda_status kda_flush_layers(const kda_layer* layers, const kda_pool* pools,
                            const kda_records* rec_prev, int32_t num_layers, int32_t num_rows,
                            const int32_t* record_rows, const int32_t* pending,
                            hipStream_t stream);

/*
 * kda_conv_compact -- the conv-state half of the commit, for num_layers
 * layers in one launch (pages: recoverssm.py, _compact_conv_state_kernel).
 * After a verify, the token axis of a row's conv-state block holds the last
 * history - 1 inputs before the window, then the window's inputs. For each
 * layer and row i with 0 < state_indices[i] < num_blocks and
 * n' = min(max(num_accepted[i], 0), T_i, window) > 0: columns n' - 1 ..
 * n' + history - 2 of the source block move to columns 0 .. history - 1 of
 * the final block (the source itself when align is NULL; see kda_align);
 * in align mode the columns from boundary length - 1 also go to the
 * boundary block, when there is one. Every row reads before it writes;
 * values are copied as 16-bit patterns. Blocks outside 1..num_blocks-1 are
 * skipped.
 *   layers: HOST array of num_layers (1..64) conv states.
 *   conv_dim: channels (>= 1); history: 1..8; width: columns of the token
 *   axis, >= window + history - 1; window: 1..64.
 *   cu_seqlens [num_rows + 1], state_indices, num_accepted [num_rows] int32;
 *   num_rows <= 65535.
 * Errors: NULL pointers -> KDA_ERR_NULL; sizes out of range ->
 * KDA_ERR_SHAPE; a misaligned state -> KDA_ERR_ALIGN; two layers' states
 * overlapping -> KDA_ERR_ALIAS; align as for kda_commit_layers.
 */
kda_status kda_conv_compact(const kda_conv_state* layers, int32_t num_layers, int32_t conv_dim,
                            int32_t history, int32_t width, const int32_t* cu_seqlens,
                            int32_t num_rows, const int32_t* state_indices,
                            const int32_t* num_accepted, int32_t window,
                            const kda_align* align, hipStream_t stream);

/* Host: a static, human-readable name for a status code. */
const char* kda_status_string(kda_status status);

/*
 * kda_check_rows -- host-side check of the row metadata that the kernels
 * only range-check (an opt-in debugging aid: the calls above never read
 * device metadata on the host). Every pointer here is a HOST pointer.
 * Rows with state_indices[i] <= 0 are skipped rows and pass; for the others:
 * a well-formed span within num_tokens, T_i <= max_seqlen when max_seqlen > 0
 * (the window bound of kda_tokens), a slot below num_slots and not shared
 * with another row (distinct slots: one checkpoint state per request, pages:
 * recoverssm.py, module docstring), and a record row (record_rows[i], or i when record_rows is NULL)
 * that is -1 (the scratch row: nothing is recorded) or below rec_rows and
 * not shared with another row. rec_rows < 0 skips the record-row checks.
 * Returns KDA_OK, or KDA_ERR_METADATA with *bad_row = the first offending row
 * and *issue = what is wrong with it (both optional); KDA_ERR_NULL for
 * missing arrays, KDA_ERR_SHAPE for negative sizes. Reads only; allocates
 * host memory for the duplicate checks (num_slots and rec_rows flags).
 */
kda_status kda_check_rows(const int32_t* cu_seqlens, int32_t num_rows, int32_t num_tokens,
                          const int32_t* state_indices, int32_t num_slots,
                          const int32_t* record_rows, int32_t rec_rows, int32_t max_seqlen,
                          int32_t* bad_row, int32_t* issue);

/* Host: the library's build identification (static string). */
const char* kda_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
