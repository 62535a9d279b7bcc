// libkda: KDA speculative verify / accepted-token commit ("RecoverSSM") for
// AMD Instinct MI355X (gfx950, CDNA4, wave64).
//
// The method (pages: "recoverssm.py (GLM-5.3-Flash KDA speculative verify with
// one checkpoint state per request)", _verify_kernel per-token loop): per head
// a fp32 state S[K, V]; per token decay the key channels by exp(g), delta rule
// u = beta * (v - S^T k^), rank-1 update S += k^ u^T, output o = S^T q^.
//
// Kernel design (one kernel body serves the recurrent, verify, commit and
// deferred calls, single- or multi-layer):
//  * One workgroup of NW waves (4; 8 for the commit and for the deferred
//    verify of 4-token windows on 128-row tiles) per (request row, head,
//    V-tile of BV = 8*R*NW value rows). The fp32 K x BV state tile lives in
//    VGPRs: a group of 8 adjacent lanes owns one value row; each lane holds
//    16 key channels of it (4 chunks of 4 consecutive channels, chunk j at
//    j*32 + 4*(lane%8)), so one 128-bit load per chunk and the 8 lanes of a
//    group read 128 contiguous bytes. Each lane holds R rows, whatever NW.
//  * The per-token vectors shared by all rows (k^, q^, exp(g), beta and the
//    tile's slice of v) are computed once per workgroup, 8 tokens at a time,
//    by half-waves (one token each, 4 channels per lane) into LDS. The token
//    loads go out first and the state tile's right after, so the staging runs
//    while the tile is in flight; barriers wait for LDS operations only.
//  * Commit, recurrence and the deferred fold step the state token by token
//    (two reductions over K per token and row: 16-term in-lane FMA chains plus
//    a 3-step DPP butterfly across the 8 lanes of the group, which gives all 8
//    lanes the same bits). Every one of them runs the same per-token code with
//    the same lane layout, so a commit of n records gives the bits of the
//    plain recurrence over the same n tokens.
//  * A commit that defers (only the eager rows replay now) runs over a list of
//    the rows with work, built in every workgroup of a grid sized to the
//    resident capacity, instead of one workgroup per (row, head, tile).
//  * Verify computes its window in chunked form against the checkpoint: 2T
//    dot products per value row and a T x T triangular recurrence, no state
//    stepping and no state write (a window longer than one chunk advances
//    the state in registers from one chunk to the next).
//  * With the caller's bound on the windows (kda_tokens.max_seqlen), verify
//    runs short kernels without the long-window code (fewer registers, more
//    resident waves); the 4-token ones issue the window's token loads at the
//    predicted uniform span before the row metadata arrives.
//  * The state is streamed: the verify's tile loads and the commit's and
//    deferred fold's loads and stores are non-temporal, since every
//    checkpoint is touched once per kernel and step.
//  * Matrix cores (fp32 MFMA) for the verify's dot products on tiles of 16
//    or more rows per wave: each wave moves its rows through its own LDS
//    into the operand layout, so the tile still loads in whole lines. The
//    per-token replay (commit, recurrence, fold) is a handful of FMAs per
//    state element against a state read once and written at most once:
//    bound by HBM bandwidth, on the vector lanes.
//  * -ffp-contract=off: every FMA is an explicit fmaf, nothing is contracted
//    or reassociated by the compiler.
//  * Every index read from device memory (cu_seqlens, slots, record rows,
//    accepted and pending counts, block tables) is range-checked before use.
// The conv-state compaction of the commit is a separate small copy kernel
// (16-byte spans through LDS for the dense in-place layout).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "kda.h"

namespace {

constexpr int KD = 128;        // head dim (K == V)
constexpr int NTHREADS = 256;  // 4 waves: every kernel but the 8-wave deferred verify
constexpr int NWAVES = 4;
constexpr int CH = 8;          // tokens staged in LDS per chunk
constexpr int MAX_WINDOW = 64;

enum Mode : int { kRecurrent = 0, kVerify = 1, kCommit = 2, kDeferred = 3, kSpec = 4 };

// Align mode of the commit: a row of block ids per request row, the tokens
// each request had cached before the step, and the tokens per block.
struct AlignRef {
  const int* bt;           // nullptr: no align mode
  long long row_stride;    // elements between rows of bt
  int width;
  const int* num_computed;
  int block_size;
};

// A row's commit plan (recoverssm.py, _prepare_commit_plan_kernel): n', the
// final block (the source without align; in align mode the block holding the
// last committed token), and the boundary block (0: none) and length. A
// negative cached count counts as 0, and a boundary column beyond the block
// table gives no boundary block.
struct Plan {
  int n, final_block, boundary_block, boundary_len;
};

__device__ __forceinline__ Plan commit_plan_row(const AlignRef& al, int row, int n, int src) {
  Plan pl;
  pl.n = n;
  pl.final_block = src;
  pl.boundary_block = 0;
  pl.boundary_len = 0;
  if (al.bt) {
    const long long bs = al.block_size;
    long long cached = al.num_computed[row];
    cached = cached < 0 ? 0 : cached;
    long long last = cached + n - 1;
    last = last < 0 ? 0 : last;
    long long col = last / bs;
    col = col < al.width - 1 ? col : al.width - 1;
    const int* bt_row = al.bt + (long long)row * al.row_stride;
    pl.final_block = bt_row[col];
    const long long next = (cached / bs + 1) * bs;
    pl.boundary_len = (int)(next - cached);
    const long long bcol = next / bs - 1;
    if (cached + n >= next && bcol < al.width) pl.boundary_block = bt_row[bcol];
  }
  return pl;
}

struct Params {
  // layer
  const float* a_log;
  const float* g_bias;
  float scale;
  float lower_bound;
  int has_lb;
  int H;
  // tokens
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  long long sq, sk, sv, sg, sb;
  const int* cu;
  int num_rows;
  int num_tokens;
  int guess_len;           // short verify: predicted uniform window length, 0: none
  int max_seqlen;          // short verify: the caller's bound on every window
  // pool
  float* state;
  long long slot_stride;
  int num_slots;
  const int* slots;
  // records written by verify (rec / rec_next) or read by commit (rec)
  uint16_t* rk;
  uint16_t* rv;
  uint16_t* rg;
  uint16_t* rb;
  int rec_rows;
  int Q;
  // records read by the deferred fold (rec_prev)
  const uint16_t* pk;
  const uint16_t* pv;
  const uint16_t* pg;
  const uint16_t* pb;
  const int* record_rows;
  const int* num_accepted;
  int* pending;            // commit (deferred mode): written
  const unsigned char* eager;
  const int* pending_in;   // verify_deferred: read
  uint16_t* o;
  int tiles;               // V tiles per (row, head)
  int total_blocks;        // workgroups of the launch (all layers)
  int layer_blocks;        // workgroups per layer
  int flush;               // deferred fold only: every window is empty, no token is read
  int pending_skip;        // commit, deferred mode: this launch does not write pending
  AlignRef align;          // commit: block table (align.bt == nullptr: in place)
  // stock speculative step (kSpec): a row of block ids per request row
  const int* spec_idx;
  long long spec_stride;
  int spec_cols;
  const int* spec_acc;     // accepted counts (nullptr: the source is column 0)
};

// Per-layer pointers of a multi-layer launch (the rest of Params is shared:
// row metadata, state indices, head count, record window).
constexpr int kMaxLayers = 16;
struct LayerRef {
  const float* a_log;
  const float* g_bias;
  float scale;
  float lower_bound;
  int has_lb;
  int num_slots;
  long long slot_stride;
  float* state;
  uint16_t *rk, *rv, *rg, *rb;                // commit: the records replayed
  const uint16_t *pk, *pv, *pg, *pb;          // fold: the previous records
};
struct LayerTable {
  LayerRef l[kMaxLayers];
};

// ---------------------------------------------------------------- helpers --

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);                                  // nearest, ties to even
  return (uint16_t)(u >> 16);
}

// Hardware transcendentals (v_exp_f32 = 2^x, v_log_f32 = log2 x, v_rcp_f32,
// v_rsq_f32; about 1 ulp each). Every call of the library goes through the
// same functions, so all of them round alike.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

// log(1 + y) for y >= 0 with a relative error of a few ulp even for tiny y:
// log(u) * y / (u - 1) with u = 1 + y rounded (the correction cancels the
// rounding of u).
__device__ __forceinline__ float log1p_hw(float y) {
  const float u = 1.0f + y;
  const float l = __builtin_amdgcn_logf(u) * kLn2;
  return u == 1.0f ? y : l * (y * rcp_hw(u - 1.0f));
}

__device__ __forceinline__ float sigmoid_hw(float x) { return rcp_hw(1.0f + exp_hw(-x)); }

// Decay factor exp(g) of one key channel from x = g_raw + g_bias, A = exp(A_log).
//   bounded:   g = lb * sigmoid(A x)
//   unbounded: g = -A * softplus(x), softplus(x) = max(x, 0) + log1p(exp(-|x|))
__device__ __forceinline__ float decay_of(float x, float A, int has_lb, float lb) {
  if (has_lb) return exp_hw(lb * sigmoid_hw(A * x));
  const float sp = fmaxf(x, 0.0f) + log1p_hw(exp_hw(-fabsf(x)));
  return exp_hw(-(A * sp));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a group; every lane gets the same bits (each step
// adds the same two operands in both partner lanes).
__device__ __forceinline__ float reduce8(float x) {
  x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp<0x141>(x);  // row_half_mirror: lane i <-> 7-i
  return x;
}

// Sum over the 32 lanes of a half-wave; every lane gets the same bits. The
// two 16-lane rows of each half-wave are summed in their lanes (DPP), then
// added as scalars read from the rows' first lanes (no LDS round trip: a
// ds_swizzle across the rows waited behind the workgroup's other LDS
// traffic). Either half of the wave adds the same two row sums.
__device__ __forceinline__ float reduce32(float x) {
  x = reduce8(x);
  x = x + dpp<0x140>(x);  // row_mirror: lane i <-> 15-i (the other 8-group)
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
}

__device__ __forceinline__ void unpack4(uint2 raw, float out[4]) {
  out[0] = bf16_to_f32(raw.x & 0xFFFFu);
  out[1] = bf16_to_f32(raw.x >> 16);
  out[2] = bf16_to_f32(raw.y & 0xFFFFu);
  out[3] = bf16_to_f32(raw.y >> 16);
}

__device__ __forceinline__ float dot4(const float a[4], const float b[4]) {
  float s = a[0] * b[0];
  s = fmaf(a[1], b[1], s);
  s = fmaf(a[2], b[2], s);
  s = fmaf(a[3], b[3], s);
  return s;
}

// Workgroup barrier for data handed between waves through LDS.
// __syncthreads() is a workgroup release/acquire fence plus s_barrier, and
// the fence waits for every outstanding global load and store of the wave
// (vmcnt 0): a workgroup that has just issued its state-tile loads would
// wait for the whole tile at its first barrier, before the token staging
// that does not need it. LDS data only needs the wave's own LDS operations
// finished (lgkmcnt 0) before the barrier; no kernel here hands global
// memory between the waves of a workgroup.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A load of a workgroup-uniform value that this kernel never writes, through
// the constant address space so that it becomes a scalar load. A plain load
// may be emitted as a vector load when the kernel also stores to global
// memory, and its first use would then wait for every vector load issued
// before it.
template <class T>
__device__ __forceinline__ T scalar_load(const T* ptr) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(ptr));
}

// LDS staging area for one chunk of up to NT tokens.
template <int BV, int NT>
struct Stage {
  float kh[NT][KD];   // k^
  float qh[NT][KD];   // q^ (scale folded in)
  float dk[NT][KD];   // exp(g)
  float vt[NT][BV];   // the tile's slice of v
  float bt[NT];       // beta
};

// The chunk-form verify additionally keeps, for the window's tokens t and
// s <= t (Gamma_t = the decay product over tokens 1..t, P(s,t) the product
// over tokens s+1..t, both diagonal over key channels):
//   al(t) = Gamma_t k^_t,  ga(t) = Gamma_t q^_t,
//   M[t][s] = k^_s . P(s,t) k^_t  (s < t),   N[t][s] = k^_s . P(s,t) q^_t.
// The 2 NT decayed vectors are the rows of av, in the order the matrix-core
// dot products take them as the rows of their A operand: row
// 8 (t / 4) + t % 4 is al(t), the same plus 4 is ga(t); row 2 NT is zero
// (the A rows of tokens beyond the window read it). A row is padded to 132
// floats (528 bytes), so that 16 lanes reading one 16-byte column of 16
// rows hit 16 different bank groups.
constexpr int kAvStride = KD + 4;

__device__ __forceinline__ int al_row(int t) { return 8 * (t >> 2) + (t & 3); }
__device__ __forceinline__ int ga_row(int t) { return 8 * (t >> 2) + 4 + (t & 3); }

template <int BV, int NT>
struct StageChunk : Stage<BV, NT> {
  float av[2 * NT + 1][kAvStride];
  float M[NT][NT];
  float N[NT][NT];
  __device__ float* al(int t) { return av[al_row(t)]; }
  __device__ float* ga(int t) { return av[ga_row(t)]; }
  __device__ const float* al(int t) const { return av[al_row(t)]; }
  __device__ const float* ga(int t) const { return av[ga_row(t)]; }
};

// Per-workgroup constants.
struct Ctx {
  int bos, ri, head, tile, H;
  float A;            // exp(A_log[head])
  int tid, wave, p8, grp, hw, l32;
};

// Sum over K of x[k] * y[k] for one value row: 16 channels in this lane,
// then the 8 lanes of the row group.
__device__ __forceinline__ float row_dot(const float x[16], const float y[16]) {
  float acc[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float a = x[4 * jj] * y[4 * jj];
    a = fmaf(x[4 * jj + 1], y[4 * jj + 1], a);
    a = fmaf(x[4 * jj + 2], y[4 * jj + 2], a);
    a = fmaf(x[4 * jj + 3], y[4 * jj + 3], a);
    acc[jj] = a;
  }
  return reduce8((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// Read this lane's 16 key channels of an LDS vector.
__device__ __forceinline__ void lds_row16(const float* vec, int p8, float out[16]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float4 a = *reinterpret_cast<const float4*>(vec + jj * 32 + p8 * 4);
    out[4 * jj + 0] = a.x; out[4 * jj + 1] = a.y; out[4 * jj + 2] = a.z; out[4 * jj + 3] = a.w;
  }
}

template <int R, int BV>
__device__ __forceinline__ int row_in_tile(int rr, const Ctx& c) {
  constexpr int NW = BV / (8 * R);   // waves of the workgroup
  return (rr * NW + c.wave) * 8 + c.grp;
}

// A 16-byte load of state; NT: non-temporal (streamed: the line is not kept
// in the caches, nor allocated in the MALL). The verify reads each
// checkpoint once, and the commit reads each once before overwriting it
// whole, so their state loads stream and no longer evict lines that other
// kernels will read or write back. Only where a wave's 8-lane groups read
// whole 128-byte lines (load_tile): the matrix-core layout reads 64 bytes of
// a line per instruction, and streaming its loads fetched lines twice
// (deep-draft verify 144.7 -> 154 us). The commit and the deferred fold also
// stream the new state out (store_tile<..., true>): nothing reads it back
// before the next step, and a write that stays dirty in the MALL is written
// back later while other kernels stream their own state (12-layer decode
// step 77.4 -> 75.6 us per layer). With both, the deferred verify streams
// its state loads as well (decode deferred flow 64.7 -> 57.1 us per layer;
// with its stores cached, streaming its loads alone had not paid).
template <bool NT>
__device__ __forceinline__ float4 ld_state4(const float* src) {
  if constexpr (NT) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(src));
    return make_float4(x.x, x.y, x.z, x.w);
  } else {
    return *reinterpret_cast<const float4*>(src);
  }
}

template <int R, int BV, bool NT = false>
__device__ __forceinline__ void load_tile(float (&S)[R][16], const float* sbase, const Ctx& c) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const float* src = sbase + (c.tile * BV + row_in_tile<R, BV>(rr, c)) * KD + c.p8 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = ld_state4<NT>(src + j * 32);
      S[rr][4 * j + 0] = x.x; S[rr][4 * j + 1] = x.y; S[rr][4 * j + 2] = x.z; S[rr][4 * j + 3] = x.w;
    }
  }
}

template <int R, int BV, bool NT = false>
__device__ __forceinline__ void store_tile(const float (&S)[R][16], float* sbase, const Ctx& c) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    float* dst = sbase + (c.tile * BV + row_in_tile<R, BV>(rr, c)) * KD + c.p8 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (NT) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        f4v x;
        x.x = S[rr][4 * j + 0]; x.y = S[rr][4 * j + 1]; x.z = S[rr][4 * j + 2]; x.w = S[rr][4 * j + 3];
        __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(dst + j * 32));
      } else {
        float4 x;
        x.x = S[rr][4 * j + 0]; x.y = S[rr][4 * j + 1]; x.z = S[rr][4 * j + 2]; x.w = S[rr][4 * j + 3];
        *reinterpret_cast<float4*>(dst + j * 32) = x;
      }
    }
  }
}

// One staged token's raw inputs in registers (a half-wave per token, 4
// channels per lane).
template <int BV>
struct Raw {
  uint2 k, g, q;
  float4 gb;          // g_bias of the lane's 4 key channels
  uint16_t v[BV / 32];
  uint16_t b;
  bool active;
};

// Issue the loads of tokens c0 .. c0+m-1 of a segment. fold: records of
// storage row ri (no q); otherwise window tokens bos + j.
template <int MODE, int BV>
__device__ __forceinline__ void stage_load(Raw<BV>& x, const Params& p, const Ctx& c, bool fold,
                                           int c0, int m) {
  constexpr int VPL = BV / 32;
  // Branch-free: the half-waves without a token read the head's g_bias row
  // instead (512 bytes, more than any of the reads below spans) and drop
  // what they read. A branch around the loads would put a control-flow join
  // between them and the next loads, where the compiler's register copies
  // wait for them to arrive.
  x.active = c.hw < m;
  const int j = c0 + c.hw, l32 = c.l32;
  const uint16_t* safe = reinterpret_cast<const uint16_t*>(p.g_bias + c.head * KD);
  const uint16_t *k = safe, *g = safe, *v = safe, *b = safe, *q = safe;
  if (x.active) {
    if (fold) {
      const long long base = ((long long)c.ri * c.H + c.head) * p.Q + j;
      k = ((MODE == kDeferred) ? p.pk : p.rk) + base * KD;
      g = ((MODE == kDeferred) ? p.pg : p.rg) + base * KD;
      v = ((MODE == kDeferred) ? p.pv : p.rv) + base * KD;
      b = ((MODE == kDeferred) ? p.pb : p.rb) + base;
    } else {
      const long long tok = (long long)c.bos + j;
      k = p.k + tok * p.sk + c.head * KD;
      g = p.g + tok * p.sg + c.head * KD;
      v = p.v + tok * p.sv + c.head * KD;
      b = p.beta + tok * p.sb + c.head;
      q = p.q + tok * p.sq + c.head * KD;
    }
  }
  x.k = *reinterpret_cast<const uint2*>(k + 4 * l32);
  x.g = *reinterpret_cast<const uint2*>(g + 4 * l32);
  x.gb = *reinterpret_cast<const float4*>(p.g_bias + c.head * KD + 4 * l32);
  x.q = fold ? make_uint2(0, 0) : *reinterpret_cast<const uint2*>(q + 4 * l32);
#pragma unroll
  for (int e = 0; e < VPL; ++e) x.v[e] = v[c.tile * BV + l32 * VPL + e];
  // kept as loaded (every use is by lane 0 of the half-wave): a select here
  // would make the wave wait for all of these loads before issuing the next
  // ones (the row metadata, the state tile)
  x.b = *b;
}

// Write a staged window token's raw inputs to its record row (the first Q
// tokens of the row; the tile-0 workgroup writes k, g and beta, every tile
// its slice of v).
template <int BV>
__device__ __forceinline__ void store_records(const Raw<BV>& x, const Params& p, const Ctx& c, int c0) {
  constexpr int VPL = BV / 32;
  const int l32 = c.l32, j = c0 + c.hw;
  if (!x.active || j >= p.Q) return;
  const long long base = ((long long)c.ri * c.H + c.head) * p.Q + j;
  if (c.tile == 0) {
    *reinterpret_cast<uint2*>(p.rk + base * KD + 4 * l32) = x.k;
    *reinterpret_cast<uint2*>(p.rg + base * KD + 4 * l32) = x.g;
    if (l32 == 0) p.rb[base] = x.b;
  }
#pragma unroll
  for (int e = 0; e < VPL; ++e) p.rv[base * KD + c.tile * BV + l32 * VPL + e] = x.v[e];
}

// Turn the loaded raw inputs into the per-token vectors in LDS; for window
// tokens of the verify modes also write the raw inputs to the records
// unless `records` is false (the caller then calls store_records itself).
template <int MODE, int BV, int NT>
__device__ __forceinline__ void stage_compute(Stage<BV, NT>& st, const Raw<BV>& x, const Params& p,
                                              const Ctx& c, bool fold, int c0, bool records = true) {
  constexpr int VPL = BV / 32;
  if (!x.active) return;
  const int hw = c.hw, l32 = c.l32;
  float kx[4], gx[4];
  unpack4(x.k, kx);
  unpack4(x.g, gx);
  const float kinv = rsqrt_hw(reduce32(dot4(kx, kx)) + 1e-6f);
  float4 kh, dk;
  kh.x = kx[0] * kinv; kh.y = kx[1] * kinv; kh.z = kx[2] * kinv; kh.w = kx[3] * kinv;
  dk.x = decay_of(gx[0] + x.gb.x, c.A, p.has_lb, p.lower_bound);
  dk.y = decay_of(gx[1] + x.gb.y, c.A, p.has_lb, p.lower_bound);
  dk.z = decay_of(gx[2] + x.gb.z, c.A, p.has_lb, p.lower_bound);
  dk.w = decay_of(gx[3] + x.gb.w, c.A, p.has_lb, p.lower_bound);
  *reinterpret_cast<float4*>(&st.kh[hw][4 * l32]) = kh;
  *reinterpret_cast<float4*>(&st.dk[hw][4 * l32]) = dk;
  if (!fold) {
    float qx[4];
    unpack4(x.q, qx);
    const float qinv = rsqrt_hw(reduce32(dot4(qx, qx)) + 1e-6f);
    float4 qh;
    qh.x = (qx[0] * qinv) * p.scale; qh.y = (qx[1] * qinv) * p.scale;
    qh.z = (qx[2] * qinv) * p.scale; qh.w = (qx[3] * qinv) * p.scale;
    *reinterpret_cast<float4*>(&st.qh[hw][4 * l32]) = qh;
  }
#pragma unroll
  for (int e = 0; e < VPL; ++e) st.vt[hw][l32 * VPL + e] = bf16_to_f32(x.v[e]);
  if (l32 == 0) st.bt[hw] = sigmoid_hw(bf16_to_f32(x.b));
  if ((MODE == kVerify || MODE == kDeferred) && !fold && records) store_records<BV>(x, p, c, c0);
}

// The per-token recurrence over m staged tokens, state in registers. With
// `out`, token t's output goes to o[tok0 + t]. SPEC (the stock speculative
// step): after token t the state also goes to the block of column
// col0 + t of the row's block ids `spec_row`, unless that column is past
// the row or names the null block (or one outside the pool).
template <int R, int BV, int NT, bool SPEC = false>
__device__ __forceinline__ void seq_tokens(float (&S)[R][16], const Stage<BV, NT>& st, const Params& p,
                                           const Ctx& c, int m, bool out, long long tok0,
                                           const int* spec_row = nullptr, int col0 = 0) {
  for (int t = 0; t < m; ++t) {
    float kh[16], dk[16];
    lds_row16(st.kh[t], c.p8, kh);
    lds_row16(st.dk[t], c.p8, dk);
    const float beta = st.bt[t];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      // decay the key channels
#pragma unroll
      for (int e = 0; e < 16; ++e) S[rr][e] = S[rr][e] * dk[e];
      // delta rule against the decayed state, then the rank-1 update
      const float kv = row_dot(S[rr], kh);
      const float u = beta * (st.vt[t][row_in_tile<R, BV>(rr, c)] - kv);
#pragma unroll
      for (int e = 0; e < 16; ++e) S[rr][e] = fmaf(kh[e], u, S[rr][e]);
    }
    if (out) {
      float qh[16];
      lds_row16(st.qh[t], c.p8, qh);
      uint16_t* orow = p.o + ((tok0 + t) * c.H + c.head) * KD + c.tile * BV;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const float ov = row_dot(S[rr], qh);
        if (c.p8 == 0) orow[row_in_tile<R, BV>(rr, c)] = f32_to_bf16(ov);
      }
    }
    if constexpr (SPEC) {
      const int col = col0 + t;
      if (col < p.spec_cols) {
        const int dst = scalar_load(spec_row + col);
        if (dst > 0 && dst < p.num_slots)
          store_tile<R, BV, true>(S, p.state + (long long)dst * p.slot_stride +
                                         (long long)c.head * KD * KD, c);
      }
    }
  }
}

// Verify of a chunk of m <= TMAX staged tokens (the chunked form) from the
// state S0 in registers, without stepping the state token by token.
// Unrolling the recurrence from S0:
//   a_t = (Gamma_t S0)^T k^_t,  b_t = (Gamma_t S0)^T q^_t
//   u_t = beta_t (v_t - a_t - sum_{s<t} M[t][s] u_s)
//   o_t = b_t + sum_{s<=t} N[t][s] u_s
// which is the per-token loop's math (decay, delta rule, update, output)
// with 2m dot products per value row instead of 4m passes over it. Windows
// longer than one chunk run chunk after chunk (chunk_advance in between).
//
// coef_phase: the per-chunk vectors and coefficients, from the staged k^,
// q^, exp(g), by threads 0..255 (c.hw and c.l32 relative to them; the
// threads beyond them in an 8-wave workgroup take no part).
template <int BV, int TMAX, int NT>
__device__ __forceinline__ void coef_phase(StageChunk<BV, NT>& st, const Ctx& c, int T) {
  // Decayed vectors: threads 128..255, one key channel each (all of the
  // channel's staged values are read first, then a short product chain).
  if (c.tid >= KD && c.tid < 2 * KD) {
    const int ch = c.tid - KD;
    float kk[TMAX], qq[TMAX], dd[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        kk[t] = st.kh[t][ch];
        qq[t] = st.qh[t][ch];
        dd[t] = st.dk[t][ch];
      }
    }
    float gam = 1.0f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        gam = gam * dd[t];
        st.al(t)[ch] = gam * kk[t];
        st.ga(t)[ch] = gam * qq[t];
      }
    }
    st.av[2 * NT][ch] = 0.0f;
  }
  // Coefficients: the T(T+1)/2 pairs (s, t), s <= t, numbered t(t+1)/2 + s,
  // dealt to the 16 rows of 16 lanes (pair q to row q % 16; one pass for up
  // to 5 tokens, two for 6 or 7, three for 8); lane j of a
  // row covers the key channels 4j..4j+3 and 64+4j..64+4j+3, and the row
  // sums with 4 DPP steps. Every chunk size computes a pair with the same
  // operations, so the chunk size does not change the bits.
  {
    const int r16 = c.tid >> 4, j = c.tid & 15;
    const int npairs = T * (T + 1) / 2;
    constexpr int kSlots = (TMAX * (TMAX + 1) / 2 + 15) / 16;
#pragma unroll
    for (int slot = 0; slot < kSlots; ++slot) {
      const int q = r16 + 16 * slot;
      // (a pass with no live pair is skipped: the test is uniform)
      if (16 * slot < npairs && q < TMAX * (TMAX + 1) / 2) {
        const bool live = q < npairs;
        // pair number q -> (s, t): t is the largest with t(t+1)/2 <= q
        int t = 0;
#pragma unroll
        for (int u = 1; u < TMAX; ++u) t += (u * (u + 1) / 2 <= q) ? 1 : 0;
        const int sidx = live ? q - t * (t + 1) / 2 : 0;
        const int tidx = live ? t : 0;
        float4 wa = *reinterpret_cast<const float4*>(&st.kh[sidx][4 * j]);
        float4 wb = *reinterpret_cast<const float4*>(&st.kh[sidx][64 + 4 * j]);
#pragma unroll
        for (int r = 1; r < TMAX; ++r) {
          if (r > sidx && r <= tidx) {
            const float4 da = *reinterpret_cast<const float4*>(&st.dk[r][4 * j]);
            const float4 db = *reinterpret_cast<const float4*>(&st.dk[r][64 + 4 * j]);
            wa.x *= da.x; wa.y *= da.y; wa.z *= da.z; wa.w *= da.w;
            wb.x *= db.x; wb.y *= db.y; wb.z *= db.z; wb.w *= db.w;
          }
        }
        const float4 xa = *reinterpret_cast<const float4*>(&st.qh[tidx][4 * j]);
        const float4 xb = *reinterpret_cast<const float4*>(&st.qh[tidx][64 + 4 * j]);
        const float4 ya = *reinterpret_cast<const float4*>(&st.kh[tidx][4 * j]);
        const float4 yb = *reinterpret_cast<const float4*>(&st.kh[tidx][64 + 4 * j]);
        float nts = wa.x * xa.x;
        nts = fmaf(wa.y, xa.y, nts);
        nts = fmaf(wa.z, xa.z, nts);
        nts = fmaf(wa.w, xa.w, nts);
        nts = fmaf(wb.x, xb.x, nts);
        nts = fmaf(wb.y, xb.y, nts);
        nts = fmaf(wb.z, xb.z, nts);
        nts = fmaf(wb.w, xb.w, nts);
        float mts = wa.x * ya.x;
        mts = fmaf(wa.y, ya.y, mts);
        mts = fmaf(wa.z, ya.z, mts);
        mts = fmaf(wa.w, ya.w, mts);
        mts = fmaf(wb.x, yb.x, mts);
        mts = fmaf(wb.y, yb.y, mts);
        mts = fmaf(wb.z, yb.z, mts);
        mts = fmaf(wb.w, yb.w, mts);
        nts = reduce8(nts);
        mts = reduce8(mts);
        nts = nts + dpp<0x140>(nts);   // row_mirror: the other 8 lanes of the row
        mts = mts + dpp<0x140>(mts);
        if (live && j == 0) {
          st.N[tidx][sidx] = nts;
          st.M[tidx][sidx] = sidx < tidx ? mts : 0.0f;
        }
      }
    }
  }
}

// chunk_dots: the 2T dot products per value row against the chunk's start
// state (a_t with Gamma_t k^_t, b_t with Gamma_t q^_t).
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void chunk_dots(const float (&S)[R][16], const StageChunk<BV, NT>& st,
                                           const Ctx& c, int T, float (&a)[R][TMAX],
                                           float (&b)[R][TMAX]) {
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      float v16[16];
      lds_row16(st.al(t), c.p8, v16);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) a[rr][t] = row_dot(S[rr], v16);
      lds_row16(st.ga(t), c.p8, v16);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) b[rr][t] = row_dot(S[rr], v16);
    }
  }
}

// chunk_recur: the T x T triangular recurrence per value row and the
// outputs (lane p8 of the group stores token p8's output, to o[tok0 + p8]);
// u receives the chunk's u_t.
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void chunk_recur(const StageChunk<BV, NT>& st, const Params& p,
                                            const Ctx& c, int T, long long tok0,
                                            const float (&a)[R][TMAX], const float (&b)[R][TMAX],
                                            float (&u)[R][TMAX]) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int vloc = row_in_tile<R, BV>(rr, c);
    float mine = 0.0f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float x = st.vt[t][vloc] - a[rr][t];
#pragma unroll
        for (int s = 0; s < t; ++s) x = fmaf(-st.M[t][s], u[rr][s], x);
        u[rr][t] = st.bt[t] * x;
        float y = b[rr][t];
#pragma unroll
        for (int s = 0; s <= t; ++s) y = fmaf(st.N[t][s], u[rr][s], y);
        if (c.p8 == t) mine = y;
      }
    }
    if (c.p8 < T)
      p.o[((tok0 + c.p8) * c.H + c.head) * KD + c.tile * BV + vloc] = f32_to_bf16(mine);
  }
}

// chunk_advance: the state after the chunk's T tokens, for a window longer
// than one chunk: per token the decay and the rank-1 update with the u_t the
// chunk form found (the per-token step without its dot products).
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void chunk_advance(float (&S)[R][16], const StageChunk<BV, NT>& st,
                                              const Ctx& c, int T, const float (&u)[R][TMAX]) {
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      float kh[16], dk[16];
      lds_row16(st.kh[t], c.p8, kh);
      lds_row16(st.dk[t], c.p8, dk);
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[rr][e] = fmaf(kh[e], u[rr][t], S[rr][e] * dk[e]);
    }
  }
}

// One chunk of T <= TMAX window tokens; with `more`, S is advanced past them
// for the next chunk.
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void chunk_verify(float (&S)[R][16], StageChunk<BV, NT>& st,
                                             const Params& p, const Ctx& c, int T, long long tok0,
                                             bool more = false) {
  coef_phase<BV, TMAX, NT>(st, c, T);
  lds_barrier();
  float a[R][TMAX], b[R][TMAX], u[R][TMAX];
  chunk_dots<R, BV, TMAX, NT>(S, st, c, T, a, b);
  chunk_recur<R, BV, TMAX, NT>(st, p, c, T, tok0, a, b, u);
  if (more) chunk_advance<R, BV, TMAX, NT>(S, st, c, T, u);
}

// ------------------------------------------------- matrix-core chunk verify --
//
// The 2T dot products per value row (a_t with al(t), b_t with ga(t)) form a
// small matrix product D = A B: A the decayed vectors (rows of av) over the
// key channels, B the state tile (key channel x value row). fp32 MFMA
// (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums) computes it, so the
// vector lanes keep only the staging, the coefficients and the recurrence
// (with the dot products on the vector lanes, they were the verify's bound:
// taking them out took the decode-size verify from 34.5 to 25.1 us).
//
// The state stays in the streamed vector layout (whole 128-byte lines per
// load: a lane group of 8 holds one value row). The MFMA operand layout
// wants one value row per lane (lane l: row l % 16, key group l / 16), so
// each wave moves its rows through its own 2 KiB of LDS, 32 key channels at
// a time: block blk of a wave = its register sets 2 blk and 2 blk + 1 (16
// value rows, MFMA row i = 8 (set parity) + group); the chunk of 4 keys
// that lane p8 of a group holds goes to unit p8 ^ ((i / 2) % 8) of row i
// (16-byte units, 8 per row), which keeps both the writes and the reads
// free of bank conflicts. Lane (i, g) then reads the units of key chunks
// 2g and 2g + 1 of row i, and the A values of the same keys from av row i.
// For T <= 4 only A rows 0..7 exist (rows 8..15 read as zero).
//
// D register r of lane (i, g) holds A row 4 g + r against value row i:
// a_t (g even) or b_t (g odd) for t = 4 (g / 2) + r. The rows' a_t, b_t are
// regrouped through the same per-wave LDS and the recurrence runs one value
// row per lane.

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Per-wave LDS of the matrix-core path: the transpose buffer (16 rows x 32
// keys), then, once the products are done, the regrouped a_t, b_t of the
// wave's rows (20 floats per row: a_0..a_7, b_0..b_7, padding).
template <int R, int NW>
struct XBuf {
  static constexpr int kFloats = (16 * 32 > 16 * (R / 2) * 20) ? 16 * 32 : 16 * (R / 2) * 20;
  float w[NW][kFloats];
};

// The tile row of MFMA row i of block blk (register sets 2 blk, 2 blk + 1).
template <int R, int BV>
__device__ __forceinline__ int xrow(int blk, int i, const Ctx& c) {
  constexpr int NW = BV / (8 * R);
  return ((2 * blk + (i >> 3)) * NW + c.wave) * 8 + (i & 7);
}

template <int R, int BV, int NT>
__device__ __forceinline__ void xpose_dots(const float (&S)[R][16], const StageChunk<BV, NT>& st,
                                           float* xb, const Ctx& c, int T, floatx4 (&D)[R / 2]) {
  const int lane = c.tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int t = 4 * (i >> 3) + (i & 3);
  const bool live = i < 2 * NT && t < T;
  const float* arow = st.av[live ? i : 2 * NT] + 8 * g;
  const int grp = c.grp, p8 = c.p8;
  float* w0 = xb + grp * 32 + 4 * (p8 ^ ((grp >> 1) & 7));
  float* w1 = xb + (8 + grp) * 32 + 4 * (p8 ^ (((8 + grp) >> 1) & 7));
  const float* r0 = xb + i * 32 + 4 * ((2 * g) ^ ((i >> 1) & 7));
  const float* r1 = xb + i * 32 + 4 * ((2 * g + 1) ^ ((i >> 1) & 7));
#pragma unroll
  for (int blk = 0; blk < R / 2; ++blk) {
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // this lane's 4 keys 32 q + 4 p8 .. of its two rows of the block
      *reinterpret_cast<float4*>(w0) =
          make_float4(S[2 * blk][4 * q], S[2 * blk][4 * q + 1], S[2 * blk][4 * q + 2], S[2 * blk][4 * q + 3]);
      *reinterpret_cast<float4*>(w1) = make_float4(S[2 * blk + 1][4 * q], S[2 * blk + 1][4 * q + 1],
                                                   S[2 * blk + 1][4 * q + 2], S[2 * blk + 1][4 * q + 3]);
      // (a wave's LDS operations run in order: the reads see the writes)
      const float4 b0 = *reinterpret_cast<const float4*>(r0);
      const float4 b1 = *reinterpret_cast<const float4*>(r1);
      const float4 a0 = *reinterpret_cast<const float4*>(arow + 32 * q);
      const float4 a1 = *reinterpret_cast<const float4*>(arow + 32 * q + 4);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.x, b0.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.x, b1.x, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.y, b0.y, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.y, b1.y, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.z, b0.z, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.z, b1.z, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.w, b0.w, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.w, b1.w, acc1, 0, 0, 0);
    }
    D[blk] = acc0 + acc1;
  }
}

// The triangular recurrence and the outputs, one value row per lane, after
// the a_t, b_t of the wave's rows are regrouped through its LDS (lane
// 16 blk + i takes MFMA row i of block blk).
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void xpose_recur(const floatx4 (&D)[R / 2], const StageChunk<BV, NT>& st,
                                            float* xb, const Params& p, const Ctx& c, int T,
                                            long long tok0) {
  const int lane = c.tid & 63;
  const int g = lane >> 4;
  const int col = (g & 1) * 8 + 4 * (g >> 1);
  if (TMAX > 4 || g < 2) {
#pragma unroll
    for (int blk = 0; blk < R / 2; ++blk)
      *reinterpret_cast<float4*>(xb + (blk * 16 + (lane & 15)) * 20 + col) =
          make_float4(D[blk].x, D[blk].y, D[blk].z, D[blk].w);
  }
  if (lane >= 16 * (R / 2)) return;
  const int blk = lane >> 4, i = lane & 15;
  const int vloc = xrow<R, BV>(blk, i, c);
  const float* rowd = xb + lane * 20;
  float a[TMAX], b[TMAX], u[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    a[t] = rowd[t];
    b[t] = rowd[8 + t];
  }
  uint16_t* orow = p.o + (tok0 * c.H + c.head) * KD + c.tile * BV + vloc;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      float x = st.vt[t][vloc] - a[t];
#pragma unroll
      for (int s2 = 0; s2 < t; ++s2) x = fmaf(-st.M[t][s2], u[s2], x);
      u[t] = st.bt[t] * x;
      float y = b[t];
#pragma unroll
      for (int s2 = 0; s2 <= t; ++s2) y = fmaf(st.N[t][s2], u[s2], y);
      orow[(long long)t * c.H * KD] = f32_to_bf16(y);
    }
  }
}

// One chunk of T <= TMAX window tokens from the state in registers, the
// dot products on the matrix cores (tiles of 64 or 128 value rows).
template <int R, int BV, int TMAX, int NT>
__device__ __forceinline__ void chunk_verify_mfma(const float (&S)[R][16], StageChunk<BV, NT>& st,
                                                  XBuf<R, BV / (8 * R)>& xb, const Params& p, const Ctx& c, int T,
                                                  long long tok0) {
  static_assert(R >= 2, "the matrix-core path takes 16 value rows per wave");
  coef_phase<BV, TMAX, NT>(st, c, T);
  lds_barrier();
  floatx4 D[R / 2];
  xpose_dots<R, BV, NT>(S, st, xb.w[c.wave], c, T, D);
  xpose_recur<R, BV, TMAX, NT>(D, st, xb.w[c.wave], p, c, T, tok0);
}

// A chunk that fits the window: the matrix-core form where the tile allows
// it, else the vector form.
template <int R, int BV, int TMAX, int NT, class XB>
__device__ __forceinline__ void chunk_verify_one(float (&S)[R][16], StageChunk<BV, NT>& st, XB& xb,
                                                 const Params& p, const Ctx& c, int T, long long tok0) {
  if constexpr (R >= 2) {
    chunk_verify_mfma<R, BV, TMAX, NT>(S, st, xb, p, c, T, tok0);
  } else {
    chunk_verify<R, BV, TMAX, NT>(S, st, p, c, T, tok0);
  }
}

// A row longer than the caller's window bound reached a short verify kernel:
// a broken precondition that must not pass silently. Its outputs become NaN
// (this workgroup's value rows of every token of the row) and so do the
// beta records of its recorded tokens (the tile-0 workgroup), so that a
// commit replaying them cannot produce a plausible checkpoint (recoverssm.py
// page, _check_config: fail where a commit would otherwise go wrong
// silently). Nothing else of the row is written.
constexpr uint16_t kBf16NaN = 0x7FC0;

template <int BV>
__device__ __forceinline__ void poison_row(const Params& p, const Ctx& c, int T) {
  for (int i = c.tid; i < T * BV; i += (int)blockDim.x) {
    const int t = i / BV, vr = i - t * BV;
    p.o[((long long)(c.bos + t) * c.H + c.head) * KD + c.tile * BV + vr] = kBf16NaN;
  }
  if (c.tile == 0) {
    const int n = T < p.Q ? T : p.Q;
    for (int t = c.tid; t < n; t += (int)blockDim.x)
      p.rb[((long long)c.ri * c.H + c.head) * p.Q + t] = kBf16NaN;
  }
}

// ------------------------------------------------------------------ kernel --

// One workgroup's work: (row, head, tile) from its logical block index b.
// The commit's view of a request row: its span length T (a malformed span
// counts as empty), n' = the accepted count clamped to [0, min(T, Q)], and
// whether the row replays its records in this call (always, unless the call
// defers: then only the rows marked eager).
__device__ __forceinline__ int commit_span(const Params& p, int row) {
  const int bos = p.cu[row];
  const int T = p.cu[row + 1] - bos;
  return (bos < 0 || T < 0) ? 0 : T;
}
__device__ __forceinline__ int commit_count(const Params& p, int row, int T) {
  int n = p.num_accepted[row];
  n = n < 0 ? 0 : n;
  n = n < T ? n : T;
  return n < p.Q ? n : p.Q;
}
// The stock speculative step reads a row's initial state from column
// num_accepted - 1 of its block ids (counts clamped to 1..cols; no counts:
// column 0).
__device__ __forceinline__ int spec_source(const Params& p, int row) {
  int col = 0;
  if (p.spec_acc) {
    int n = p.spec_acc[row];
    n = n < 1 ? 1 : n;
    n = n > p.spec_cols ? p.spec_cols : n;
    col = n - 1;
  }
  return p.spec_idx[(long long)row * p.spec_stride + col];
}

__device__ __forceinline__ bool commit_now(const Params& p, int row) {
  return p.pending == nullptr || (p.eager != nullptr && p.eager[row] != 0);
}

// SHORT (verify only): a kernel for windows within the caller's bound
// p.max_seqlen <= TMAX; it has no code for longer windows, whose registers
// would set the allocation of the whole kernel, and it poisons the outputs
// and beta records of a row longer than the bound (poison_row). (The
// same cut in the deferred verify, 106 -> 96 VGPRs at 64-row tiles, ran 3%
// slower: the extra resident workgroups contend in its fold and store.)
template <int MODE, int R, int TMAX, bool SHORT = false, int NW = NWAVES>
__device__ __forceinline__ void kda_block(const Params& p, int b) {
  constexpr int BV = R * NW * 8;   // value rows per workgroup (NW waves)
  constexpr bool kChunk = (MODE == kVerify || MODE == kDeferred);
  // tokens staged at a time: the verify modes stage one chunk of a window
  // (TMAX) and replay records in chunks of the same size; the other modes
  // stage up to CH records or tokens
  constexpr int SNT = kChunk ? TMAX : CH;
  using StageT = typename std::conditional<kChunk, StageChunk<BV, SNT>, Stage<BV, SNT>>::type;
  __shared__ StageT st;
  // the matrix-core verify's per-wave LDS
  struct NoXBuf {};
  using XBufT = typename std::conditional<(kChunk && R >= 2), XBuf<R, NW>, NoXBuf>::type;
  __shared__ XBufT xbuf;

  Ctx c;
  c.tid = threadIdx.x;
  c.wave = c.tid >> 6;
  c.p8 = c.tid & 7;           // position inside the 8-lane row group
  c.grp = (c.tid & 63) >> 3;  // row group inside the wave
  c.hw = c.tid >> 5;          // half-wave: token slot when staging
  c.l32 = c.tid & 31;         // 4 channels per lane when staging

  c.tile = b % p.tiles;
  const int rh = b / p.tiles;
  c.head = rh % p.H;
  const int row = rh / p.H;
  c.H = p.H;

  // Short verify of uniform windows (the usual speculative batch: every row
  // has the same 1 + num_spec tokens, row i from token i * len): the window's
  // token loads go out at the predicted span before the row metadata
  // arrives. The prediction is checked against cu_seqlens before any use;
  // a row that does not match loads its tokens again.
  Raw<BV> raw;
  const int gl = (SHORT && TMAX == 4) ? p.guess_len : 0;
  if (gl > 0) {
    Ctx cs = c;
    cs.bos = row * gl;
    stage_load<MODE, BV>(raw, p, cs, false, 0, gl);
  }

  // ---- row prologue: span, slot, record row, counts -----------------------
  const bool flush = MODE == kDeferred && p.flush;
  const int bos = flush ? 0 : p.cu[row];
  const int eos = flush ? 0 : p.cu[row + 1];
  int T = eos - bos;
  if (bos < 0 || T < 0 || (MODE != kCommit && eos > p.num_tokens)) T = 0;
  c.bos = bos;
  const int slot = MODE == kSpec ? spec_source(p, row) : p.slots[row];
  const bool slot_ok = slot > 0 && slot < p.num_slots;
  const int r = p.record_rows ? p.record_rows[row] : row;
  c.ri = (r >= 0 && r < p.rec_rows) ? r + 1 : 0;   // storage index, 0 = scratch

  int nfold = 0;   // records replayed into the state (commit / deferred fold)
  int nmain = 0;   // window tokens run with outputs (recurrent / verify)
  float* fbase = nullptr;   // commit: where the final state goes (the source without align)
  float* bbase = nullptr;   // align mode: where the boundary state goes, after blen records
  int blen = 0;
  if (MODE == kCommit) {
    const int n = commit_count(p, row, T);
    bool final_ok = true;
    if (p.align.bt && slot_ok && n > 0) {
      const Plan pl = commit_plan_row(p.align, row, n, slot);
      final_ok = pl.final_block > 0 && pl.final_block < p.num_slots;
      const long long head_off = (long long)c.head * KD * KD;
      if (final_ok) fbase = p.state + (long long)pl.final_block * p.slot_stride + head_off;
      if (pl.boundary_len < n && pl.boundary_block > 0 && pl.boundary_block < p.num_slots) {
        bbase = p.state + (long long)pl.boundary_block * p.slot_stride + head_off;
        blen = pl.boundary_len;
      }
    }
    const bool valid = slot_ok && n > 0 && c.ri > 0 && final_ok;
    const bool now = commit_now(p, row);
    if (p.pending) {
      // a deferred replay runs in place at the row's slot (the next
      // deferred verify), so the align blocks do not enter the count
      if (!p.pending_skip && c.ri > 0 && c.head == 0 && c.tile == 0 && c.tid == 0)
        p.pending[c.ri - 1] = now ? 0 : ((slot_ok && n > 0) ? n : 0);
    }
    nfold = (valid && now) ? n : 0;
  } else if (MODE == kDeferred) {
    if (c.ri > 0) {
      int pn = p.pending_in[c.ri - 1];
      pn = pn < 0 ? 0 : pn;
      nfold = pn < p.Q ? pn : p.Q;
    }
    nmain = T;
  } else {
    nmain = T;
  }
  if (!slot_ok || (nfold == 0 && nmain == 0)) return;
  c.A = exp_hw(scalar_load(p.a_log + c.head));
  float* sbase = p.state + (long long)slot * p.slot_stride + (long long)c.head * KD * KD;
  if (fbase == nullptr) fbase = sbase;
  const bool chunk = kChunk && nmain <= (SHORT ? p.max_seqlen : TMAX);

  // Verify of a window that fits one chunk: straight-line code from the
  // loads to the outputs. A control-flow join between the state loads and
  // their first use lets the compiler copy the state registers there, which
  // waits for the whole tile before the token staging can start.
  // (kda_verify_deferred takes it too for rows with nothing to fold.)
  if constexpr (MODE == kVerify || MODE == kDeferred) {
    if (chunk && nfold == 0) {
      if (!(gl > 0 && bos == row * gl && nmain == gl)) stage_load<MODE, BV>(raw, p, c, false, 0, nmain);
      __builtin_amdgcn_sched_barrier(0);
      float S[R][16];
      load_tile<R, BV, true>(S, sbase, c);
      __builtin_amdgcn_sched_barrier(0);
      stage_compute<MODE, BV, SNT>(st, raw, p, c, false, 0, false);
      lds_barrier();
      chunk_verify_one<R, BV, TMAX, SNT>(S, st, xbuf, p, c, nmain, (long long)bos);
      // the records last: stores issued behind the state loads would make
      // later register reuse wait for those loads
      store_records<BV>(raw, p, c, 0);
      return;
    }
    if constexpr (SHORT) {   // a window longer than the caller's bound
      poison_row<BV>(p, c, nmain);
      return;
    }
  }

  // Deferred verify of a row with a pending replay (it fits one chunk: the
  // count is clamped to the record window): the window's token loads go out
  // with the records' and the tile's, so the verify's inputs are in
  // registers by the time the folded state has been stored, and no load
  // issued behind that store waits for its write.
  if constexpr (MODE == kDeferred) {
    if (chunk && nfold <= SNT) {
      Raw<BV> rf, rv;
      stage_load<MODE, BV>(rf, p, c, true, 0, nfold);
      stage_load<MODE, BV>(rv, p, c, false, 0, nmain);
      __builtin_amdgcn_sched_barrier(0);
      float S[R][16];
      load_tile<R, BV, true>(S, sbase, c);
      __builtin_amdgcn_sched_barrier(0);
      stage_compute<MODE, BV, SNT>(st, rf, p, c, true, 0);
      lds_barrier();
      seq_tokens<R, BV, SNT>(S, st, p, c, nfold, false, 0);
      store_tile<R, BV, true>(S, fbase, c);
      if (nmain > 0) {
        lds_barrier();   // the fold's staged tokens are consumed
        stage_compute<MODE, BV, SNT>(st, rv, p, c, false, 0, false);
        lds_barrier();
        chunk_verify_one<R, BV, TMAX, SNT>(S, st, xbuf, p, c, nmain, (long long)bos);
        store_records<BV>(rv, p, c, 0);
      }
      return;
    }
  }

  // The first chunk's token loads go out before the state tile's: loads
  // complete in issue order, so the staging math then waits for its own
  // inputs only while the 64 KiB tile is still in flight.
  const bool first_fold = nfold > 0;
  constexpr bool kStreamStore = MODE == kCommit || MODE == kDeferred;
  // align mode: the replay stops at blen for the boundary store
  const int seg0 = (bbase != nullptr) ? blen : nfold;
  // window tokens per pass: one chunk (TMAX) in the chunked modes
  constexpr int WCH = kChunk ? TMAX : CH;
  stage_load<MODE, BV>(raw, p, c, first_fold, 0, first_fold ? (seg0 < SNT ? seg0 : SNT)
                                                             : (nmain < WCH ? nmain : WCH));
  __builtin_amdgcn_sched_barrier(0);
  float S[R][16];
  load_tile<R, BV, MODE != kRecurrent>(S, sbase, c);
  __builtin_amdgcn_sched_barrier(0);

  // ---- fold: replay records into the state (commit, deferred fold) --------
  if (nfold > 0) {
    for (int c0 = 0; c0 < nfold;) {
      const int end = (bbase != nullptr && c0 < blen) ? blen : nfold;
      const int m = (end - c0) < SNT ? (end - c0) : SNT;
      if (c0 > 0) stage_load<MODE, BV>(raw, p, c, true, c0, m);
      lds_barrier();  // the previous chunk is consumed
      stage_compute<MODE, BV, SNT>(st, raw, p, c, true, c0);
      lds_barrier();
      seq_tokens<R, BV, SNT>(S, st, p, c, m, false, 0);
      c0 += m;
      if (bbase != nullptr && c0 == blen) store_tile<R, BV, kStreamStore>(S, bbase, c);
    }
    store_tile<R, BV, kStreamStore>(S, fbase, c);
    if (nmain > 0) stage_load<MODE, BV>(raw, p, c, false, 0, nmain < WCH ? nmain : WCH);
  }

  // ---- window: outputs (recurrent, verify, deferred verify) ---------------
  if (nmain > 0) {
    if constexpr (kChunk) {
      // chunks of TMAX tokens in chunked form, the state advanced in
      // registers between them (no per-token loop with outputs here: its
      // registers would set the whole kernel's allocation)
      for (int c0 = 0; c0 < nmain; c0 += TMAX) {
        const int m = (nmain - c0) < TMAX ? (nmain - c0) : TMAX;
        // the lane indices pass through an empty asm statement once per
        // chunk, so the compiler derives the chunk's LDS and global
        // addresses inside the loop instead of keeping them all live
        // across it
        Ctx cl = c;
        asm volatile("" : "+v"(cl.p8), "+v"(cl.grp), "+v"(cl.hw), "+v"(cl.l32), "+v"(cl.tid),
                     "+v"(cl.wave));
        if (c0 > 0) stage_load<MODE, BV>(raw, p, cl, false, c0, m);
        lds_barrier();
        stage_compute<MODE, BV, SNT>(st, raw, p, cl, false, c0);
        lds_barrier();
        chunk_verify<R, BV, TMAX, SNT>(S, st, p, cl, m, (long long)bos + c0, c0 + m < nmain);
      }
      return;
    }
    for (int c0 = 0; c0 < nmain; c0 += SNT) {
      const int m = (nmain - c0) < SNT ? (nmain - c0) : SNT;
      if (c0 > 0) stage_load<MODE, BV>(raw, p, c, false, c0, m);
      lds_barrier();
      stage_compute<MODE, BV, SNT>(st, raw, p, c, false, c0);
      lds_barrier();
      if constexpr (MODE == kSpec)
        seq_tokens<R, BV, SNT, true>(S, st, p, c, m, true, (long long)bos + c0,
                                    p.spec_idx + (long long)row * p.spec_stride, c0);
      else
        seq_tokens<R, BV, SNT>(S, st, p, c, m, true, (long long)bos + c0);
    }
    if (MODE == kRecurrent) store_tile<R, BV>(S, sbase, c);
  }
}

// XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
// consecutive logical blocks (the V-tiles and heads of one request, the
// layers of a multi-layer launch) are mapped to one XCD and share its L2.
__device__ __forceinline__ int logical_block(int nb) {
  const int b = blockIdx.x;
  return (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
}

// The 4-token short verify on 64-row tiles holds 84 + 8 registers by the
// compiler's choice (5 waves per SIMD); held to 6 waves it fits in 76
// without spills and runs 2% faster (decode workload; 7 or 8 waves need
// spills and run 11% and 38% slower).
template <int MODE, int R, int TMAX, bool SHORT, int NW>
constexpr int kda_waves() {
  return (MODE == kVerify && SHORT && TMAX == 4 && R == 2 && NW == 4) ? 6 : 1;
}

template <int MODE, int R, int TMAX, bool SHORT = false, int NW = NWAVES>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kda_waves<MODE, R, TMAX, SHORT, NW>())))
void kda_kernel(Params p) {
  kda_block<MODE, R, TMAX, SHORT, NW>(p, logical_block(p.total_blocks));
}

// The same work for several layers in one grid: logical block b belongs to
// layer b / layer_blocks, whose pool, records and gate parameters replace
// the shared ones.
__device__ __forceinline__ void apply_layer(Params& p, const LayerRef& L) {
  p.a_log = L.a_log;
  p.g_bias = L.g_bias;
  p.scale = L.scale;
  p.lower_bound = L.lower_bound;
  p.has_lb = L.has_lb;
  p.num_slots = L.num_slots;
  p.slot_stride = L.slot_stride;
  p.state = L.state;
  p.rk = L.rk; p.rv = L.rv; p.rg = L.rg; p.rb = L.rb;
  p.pk = L.pk; p.pv = L.pv; p.pg = L.pg; p.pb = L.pb;
}

template <int MODE, int R, int TMAX, int NW = NWAVES>
__global__ __launch_bounds__(NW * 64) void kda_kernel_layers(Params p, LayerTable t) {
  int b = logical_block(p.total_blocks);
  const int l = b / p.layer_blocks;
  b -= l * p.layer_blocks;
  apply_layer(p, t.l[l]);
  // pending is one array per request row, shared by the layers (they share
  // the state indices, so every layer would write the same counts): layer 0
  // writes it
  if (l != 0) p.pending_skip = 1;
  kda_block<MODE, R, TMAX, false, NW>(p, b);
}

// Commit over a list of rows. A deferring commit replays records for the
// eager rows only, and an eager one skips the rows with nothing accepted; a
// workgroup per (row, layer, head, tile) would then spend most of the launch
// starting workgroups that only read the row metadata and exit. Here a grid
// sized to the resident capacity first builds, in every workgroup alike,
// the list of rows that may replay (row order: one ballot per 64 rows, then
// prefix counts), and then takes every G-th (row, layer, head, tile) unit of
// that list; each unit is the ordinary commit workgroup body, which decides
// for itself (the list is a superset: the slot's upper bound and the align
// blocks are checked per layer there). Workgroup 0 writes the pending
// counts of all rows, as the first layer's workgroups do in the full grid.
constexpr int kListRows = 2048;

template <int R, int NW = NWAVES>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(R == 1 ? 5 : 1)))
void kda_commit_list(Params p, LayerTable t, int num_layers) {
  __shared__ unsigned long long mask[kListRows / 64];
  __shared__ unsigned short list[kListRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunks = (p.num_rows + 63) >> 6;
  const bool write_pending = p.pending != nullptr && blockIdx.x == 0;
  const int slots0 = t.l[0].num_slots;
  for (int k = wave; k < nchunks; k += NW) {
    const int row = k * 64 + lane;
    bool work = false;
    if (row < p.num_rows) {
      const int T = commit_span(p, row);
      const int n = commit_count(p, row, T);
      const int slot = p.slots[row];
      const int r = p.record_rows ? p.record_rows[row] : row;
      const int ri = (r >= 0 && r < p.rec_rows) ? r + 1 : 0;
      const bool now = commit_now(p, row);
      work = now && n > 0 && slot > 0 && ri > 0;
      if (write_pending && ri > 0) {
        const bool valid = slot > 0 && slot < slots0 && n > 0;   // as the first layer sees it
        p.pending[ri - 1] = now ? 0 : (valid ? n : 0);
      }
    }
    const unsigned long long m = __ballot(work);
    if (lane == 0) mask[k] = m;
  }
  lds_barrier();
  int count = 0;
  for (int k = 0; k < nchunks; ++k) {
    const unsigned long long m = mask[k];
    if ((k & (NW - 1)) == wave && ((m >> lane) & 1ull))
      list[count + __popcll(m & ((1ull << lane) - 1ull))] = (unsigned short)(k * 64 + lane);
    count += __popcll(m);
  }
  lds_barrier();
  const int per_layer = p.H * p.tiles;
  const int per_row = num_layers * per_layer;
  const long long units = (long long)count * per_row;
  const int G = gridDim.x;
  p.pending_skip = 1;
  for (long long u = logical_block(G); u < units; u += G) {
    const int e = (int)(u / per_row);
    int rem = (int)(u - (long long)e * per_row);
    const int l = rem / per_layer;
    rem -= l * per_layer;
    apply_layer(p, t.l[l]);
    kda_block<kCommit, R, CH, false, NW>(p, (int)list[e] * per_layer + rem);
  }
}

// ------------------------------------------------------- conv compaction --
//
// The other half of the commit (recoverssm.py, _compact_conv_state_kernel):
// after a verify, the token axis of a row's conv-state block holds the last
// history - 1 inputs before the window and then the window's inputs; after n'
// accepted tokens the last `history` inputs are columns n' - 1 ..
// n' + history - 2, and they move to columns 0 .. history - 1 of the final
// block (in align mode the columns from boundary_len - 1 also go to the
// boundary block). A workgroup covers 2048 channels of one (row, layer), 8
// per thread; a thread reads all of its values before it writes any. The
// element values are copied as 16-bit patterns.
constexpr int kMaxConvLayers = 64;
constexpr int kMaxHistory = 8;
constexpr int kConvThreads = 256;

struct ConvRef {
  uint16_t* state;
  long long block_stride, dim_stride, token_stride;
  int num_blocks;
};
struct ConvParams {
  const int* cu;
  const int* slots;
  const int* num_accepted;
  int num_rows, conv_dim, history, window;
  int width;          // token columns per channel
  int chans;          // in-place kernel: channels per workgroup (a multiple of 8)
  AlignRef align;
};
struct ConvTable {
  ConvRef l[kMaxConvLayers];
};

constexpr int kConvPerThread = 8;   // channels per thread: loads in flight, fewer workgroups

template <int HIST>
__global__ __launch_bounds__(kConvThreads) void conv_compact_kernel(ConvParams p, ConvTable t) {
  const int row = blockIdx.y;
  const ConvRef& L = t.l[blockIdx.z];
  const int src = p.slots[row];
  if (src <= 0 || src >= L.num_blocks) return;
  const int bos = p.cu[row], eos = p.cu[row + 1];
  int T = eos - bos;
  if (bos < 0 || T < 0) T = 0;
  int n = p.num_accepted[row];
  n = n < 0 ? 0 : n;
  n = n < T ? n : T;
  n = n < p.window ? n : p.window;
  if (n == 0) return;
  const Plan pl = commit_plan_row(p.align, row, n, src);
  if (pl.final_block <= 0 || pl.final_block >= L.num_blocks) return;
  const bool boundary = p.align.bt != nullptr && pl.boundary_block > 0 &&
                        pl.boundary_block < L.num_blocks;
  const uint16_t* in = L.state + (long long)src * L.block_stride;
  uint16_t* fout = L.state + (long long)pl.final_block * L.block_stride;
  uint16_t* bout = L.state + (long long)pl.boundary_block * L.block_stride;
  const long long f0 = (long long)(n - 1) * L.token_stride;
  const long long b0 = (long long)(pl.boundary_len - 1) * L.token_stride;
  const int d0 = blockIdx.x * kConvThreads * kConvPerThread + threadIdx.x;
  uint16_t fv[kConvPerThread][HIST], bv[kConvPerThread][HIST];
#pragma unroll
  for (int u = 0; u < kConvPerThread; ++u) {
    const int d = d0 + u * kConvThreads;
    if (d < p.conv_dim) {
      const uint16_t* x = in + (long long)d * L.dim_stride;
#pragma unroll
      for (int j = 0; j < HIST; ++j) {
        fv[u][j] = x[f0 + (long long)j * L.token_stride];
        if (boundary) bv[u][j] = x[b0 + (long long)j * L.token_stride];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kConvPerThread; ++u) {
    const int d = d0 + u * kConvThreads;
    if (d < p.conv_dim) {
      const long long off = (long long)d * L.dim_stride;
#pragma unroll
      for (int j = 0; j < HIST; ++j)
        if (boundary) bout[off + (long long)j * L.token_stride] = bv[u][j];
#pragma unroll
      for (int j = 0; j < HIST; ++j) fout[off + (long long)j * L.token_stride] = fv[u][j];
    }
  }
}

// The in-place compaction (no block table) of a dense [blocks, channels,
// width] layout: the channel rows of a span are one contiguous run of
// bytes, and every 128-byte line of it is read and written anyway (a row
// is a few columns). A workgroup moves `chans` channels of one (row, layer):
// 16-byte loads of the whole span into LDS, the kept columns moved to the
// front of each row there (one thread per channel, all of its reads before
// its writes), 16-byte stores of the span back. The columns from HIST on
// are written back as they were read.
constexpr int kConvSpanBytes = 32768;

template <int HIST>
__global__ __launch_bounds__(kConvThreads) void conv_compact_span_kernel(ConvParams p, ConvTable t) {
  __shared__ uint4 buf[kConvSpanBytes / 16];
  const int row = blockIdx.y;
  const ConvRef& L = t.l[blockIdx.z];
  const int src = p.slots[row];
  if (src <= 0 || src >= L.num_blocks) return;
  const int bos = p.cu[row], eos = p.cu[row + 1];
  int T = eos - bos;
  if (bos < 0 || T < 0) T = 0;
  int n = p.num_accepted[row];
  n = n < 0 ? 0 : n;
  n = n < T ? n : T;
  n = n < p.window ? n : p.window;
  if (n == 0) return;
  const int w = p.width;
  const int c0 = blockIdx.x * p.chans;
  const int nch = (p.conv_dim - c0) < p.chans ? (p.conv_dim - c0) : p.chans;
  uint4* span = reinterpret_cast<uint4*>(L.state + (long long)src * L.block_stride + (long long)c0 * w);
  const int nvec = nch * w / 8;   // the host keeps spans whole 16-byte units
  for (int i = threadIdx.x; i < nvec; i += kConvThreads) buf[i] = span[i];
  __syncthreads();
  uint16_t* b16 = reinterpret_cast<uint16_t*>(buf);
  for (int ch = threadIdx.x; ch < nch; ch += kConvThreads) {
    uint16_t v[HIST];
#pragma unroll
    for (int j = 0; j < HIST; ++j) v[j] = b16[ch * w + n - 1 + j];
#pragma unroll
    for (int j = 0; j < HIST; ++j) b16[ch * w + j] = v[j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nvec; i += kConvThreads) span[i] = buf[i];
}

// ------------------------------------------------------------------- host --

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, long long bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Bytes spanned by a strided [rows, inner] array of `elem`-byte elements.
long long span_bytes(long long rows, long long stride, long long inner, long long elem) {
  if (rows <= 0) return 0;
  return ((rows - 1) * stride + inner) * elem;
}

kda_status check_layer(const kda_layer* L) {
  if (!L || !L->a_log || !L->g_bias) return KDA_ERR_NULL;
  if (L->head_dim != KD) return KDA_ERR_UNSUPPORTED;
  if (L->num_heads <= 0) return KDA_ERR_SHAPE;
  if (!aligned(L->g_bias, 16) || !aligned(L->a_log, 4)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// Per-row arrays (state_indices, num_accepted, ...) may be NULL when there
// are no rows.
kda_status check_pool(const kda_pool* P, int H, int num_rows) {
  if (!P || !P->state || (num_rows > 0 && !P->state_indices)) return KDA_ERR_NULL;
  if (P->num_slots <= 0 || P->slot_stride < (long long)H * KD * KD) return KDA_ERR_SHAPE;
  if (!aligned(P->state, 16) || (P->slot_stride % 4) != 0) return KDA_ERR_ALIGN;
  return KDA_OK;
}

kda_status check_tokens(const kda_tokens* t, int H) {
  if (!t || !t->cu_seqlens) return KDA_ERR_NULL;
  if (t->num_rows < 0 || t->num_tokens < 0 || t->max_seqlen < 0) return KDA_ERR_SHAPE;
  // With no tokens every row is empty and no token array is read.
  if (t->num_rows == 0 || t->num_tokens == 0) return KDA_OK;
  if (!t->q || !t->k || !t->v || !t->g || !t->beta) return KDA_ERR_NULL;
  const long long hk = (long long)H * KD;
  if (t->stride_q < hk || t->stride_k < hk || t->stride_v < hk || t->stride_g < hk ||
      t->stride_beta < H)
    return KDA_ERR_SHAPE;
  if (!aligned(t->q, 8) || !aligned(t->k, 8) || !aligned(t->v, 8) || !aligned(t->g, 8) ||
      !aligned(t->beta, 2))
    return KDA_ERR_ALIGN;
  if ((t->stride_q | t->stride_k | t->stride_v | t->stride_g) % 4 != 0) return KDA_ERR_ALIGN;
  return KDA_OK;
}

kda_status check_records(const kda_records* r) {
  if (!r || !r->k || !r->v || !r->g || !r->beta) return KDA_ERR_NULL;
  if (r->rows < 0 || r->window < 1 || r->window > MAX_WINDOW) return KDA_ERR_SHAPE;
  if (!aligned(r->k, 8) || !aligned(r->v, 8) || !aligned(r->g, 8) || !aligned(r->beta, 2))
    return KDA_ERR_ALIGN;
  return KDA_OK;
}

struct Ranges {
  Range a[8];
  int n = 0;
  void add(Range r) { a[n++] = r; }
};

void token_ranges(const kda_tokens* t, int H, Ranges& out) {
  const long long n = t->num_tokens, hk = (long long)H * KD;
  out.add(range_of(t->q, span_bytes(n, t->stride_q, hk, 2)));
  out.add(range_of(t->k, span_bytes(n, t->stride_k, hk, 2)));
  out.add(range_of(t->v, span_bytes(n, t->stride_v, hk, 2)));
  out.add(range_of(t->g, span_bytes(n, t->stride_g, hk, 2)));
  out.add(range_of(t->beta, span_bytes(n, t->stride_beta, H, 2)));
}

void record_ranges(const kda_records* r, int H, Ranges& out) {
  const long long per = (long long)(r->rows + 1) * H * r->window;
  out.add(range_of(r->k, per * KD * 2));
  out.add(range_of(r->v, per * KD * 2));
  out.add(range_of(r->g, per * KD * 2));
  out.add(range_of(r->beta, per * 2));
}

Range pool_range(const kda_pool* P, int H) {
  return range_of(P->state, ((long long)(P->num_slots - 1) * P->slot_stride + (long long)H * KD * KD) * 4);
}

bool any_overlap(Range x, const Ranges& set) {
  for (int i = 0; i < set.n; ++i)
    if (overlap(x, set.a[i])) return true;
  return false;
}

// Record buffers must not overlap each other.
bool records_self_overlap(const Ranges& rr) {
  for (int i = 0; i < rr.n; ++i)
    for (int j = i + 1; j < rr.n; ++j)
      if (overlap(rr.a[i], rr.a[j])) return true;
  return false;
}

Params base_params(const kda_layer* L) {
  Params p{};
  p.a_log = L->a_log;
  p.g_bias = L->g_bias;
  p.scale = L->scale;
  p.lower_bound = L->lower_bound;
  p.has_lb = L->has_lower_bound ? 1 : 0;
  p.H = L->num_heads;
  return p;
}

void set_tokens(Params& p, const kda_tokens* t) {
  p.q = t->q; p.k = t->k; p.v = t->v; p.g = t->g; p.beta = t->beta;
  p.sq = t->stride_q; p.sk = t->stride_k; p.sv = t->stride_v; p.sg = t->stride_g;
  p.sb = t->stride_beta;
  p.cu = t->cu_seqlens;
  p.num_rows = t->num_rows;
  p.num_tokens = t->num_tokens;
}

void set_pool(Params& p, const kda_pool* P) {
  p.state = P->state;
  p.slot_stride = P->slot_stride;
  p.num_slots = P->num_slots;
  p.slots = P->state_indices;
}

void set_records(Params& p, const kda_records* r) {
  p.rk = r->k; p.rv = r->v; p.rg = r->g; p.rb = r->beta;
  p.rec_rows = r->rows;
  p.Q = r->window;
}

// Rows of the state tile per workgroup: 32 * R (measured on MI355X at
// H = 32, K = V = 128). The commit and the plain recurrence keep the
// workgroups short and numerous (32 rows: four tiles per head). The verify
// calls repeat the per-head token staging and coefficients in every tile,
// so larger tiles pay off once there are enough (row, head) pairs to fill
// the chip: 128 rows from 4096 pairs, 64 from 512, else 32. The per-row
// arithmetic does not depend on the tile size. KDA_TILE_ROWS in
// {32, 64, 128} forces a size (read once).
int tile_rows_for(int mode, long long pairs) {
  static int forced = -2;
  if (forced == -2) {
    forced = -1;
    const char* env = getenv("KDA_TILE_ROWS");
    if (env) {
      const int v = atoi(env);
      if (v == 32 || v == 64 || v == 128) forced = v;
    }
  }
  if (forced > 0) return forced;
  if (mode == kCommit || mode == kRecurrent || mode == kSpec) return 32;
  if ((mode == kVerify && pairs >= 4096) || (mode == kDeferred && pairs >= 512)) return 128;
  return pairs >= 512 ? 64 : 32;
}

template <int MODE, int R, int TMAX, bool SHORT = false, int NW = NWAVES>
kda_status launch_r(Params& p, hipStream_t stream) {
  p.tiles = KD / (R * NW * 8);
  const long long blocks = (long long)p.num_rows * p.H * p.tiles;
  if (blocks > 0x7FFFFFFFLL) return KDA_ERR_SHAPE;
  p.total_blocks = (int)blocks;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_kernel<MODE, R, TMAX, SHORT, NW>),
                                       dim3((unsigned)blocks), dim3(NW * 64), args, 0, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// The verify modes keep 2 * R * TMAX dot products in registers: windows of
// up to 4 tokens get a kernel with TMAX = 4 (fewer registers, more waves);
// longer windows TMAX = 8 (CH). Rows longer than TMAX still run, chunk after
// chunk, except in the short kernels.
template <int MODE, int TMAX, bool SHORT = false>
kda_status launch_t(Params& p, hipStream_t stream) {
  switch (tile_rows_for(MODE, (long long)p.num_rows * p.H)) {
    // (the single-layer commit as the multi-layer one: 8 waves, 54.9 ->
    // 54.4 us; the recurrence kernels keep 4, the stock step ran 1.6%
    // slower with 8)
    case 32: return launch_r<MODE, 1, TMAX, SHORT, (MODE == kCommit ? 8 : NWAVES)>(p, stream);
    case 64: return launch_r<MODE, 2, TMAX, SHORT>(p, stream);
    default:
      // the deferred verify of 4-token windows on 128-row tiles runs as 8
      // waves of 16 rows (decode workload: 58.2 -> 55.7 us against 64-row
      // tiles of 4 waves; B = 512: 324.9 -> 322.9 us); with 8-token windows
      // it keeps 64-row tiles (128 rows in 8 waves: 1% slower on the
      // deep-draft and ragged workloads); the verify takes 4 waves of 32
      if constexpr (MODE == kDeferred && TMAX == 4) return launch_r<MODE, 2, TMAX, SHORT, 8>(p, stream);
      else if constexpr (MODE == kDeferred) return launch_r<MODE, 2, TMAX, SHORT>(p, stream);
      else return launch_r<MODE, 4, TMAX, SHORT>(p, stream);
  }
}

template <int MODE, int R, int TMAX, int NW = NWAVES>
kda_status launch_layers_r(Params& p, LayerTable& t, int num_layers, hipStream_t stream) {
  p.tiles = KD / (R * NW * 8);
  const long long per = (long long)p.num_rows * p.H * p.tiles;
  const long long blocks = per * num_layers;
  if (blocks > 0x7FFFFFFFLL) return KDA_ERR_SHAPE;
  p.layer_blocks = (int)per;
  p.total_blocks = (int)blocks;
  void* args[] = {&p, &t};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_kernel_layers<MODE, R, TMAX, NW>),
                                       dim3((unsigned)blocks), dim3(NW * 64), args, 0, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// Multi-layer launches: commit (per-token replay, any window) and the
// deferred fold with empty windows (the flush).
template <int MODE>
kda_status launch_layers(Params& p, LayerTable& t, int num_layers, hipStream_t stream) {
  constexpr int TMAX = MODE == kDeferred ? 4 : CH;   // the fold does not use the chunk path
  switch (tile_rows_for(MODE, (long long)p.num_rows * p.H)) {
    // the commit's smallest tiles as 8 waves of 8 rows (64 rows per
    // workgroup, one record staging for all of them): the decode
    // workload's 12-layer commit 540.9 -> 520.2 us against 32-row tiles of
    // 4 waves (2 waves: 531.1, 16 waves: 520.6)
    case 32: return launch_layers_r<MODE, 1, TMAX, (MODE == kCommit ? 8 : NWAVES)>(p, t, num_layers, stream);
    case 64: return launch_layers_r<MODE, 2, TMAX>(p, t, num_layers, stream);
    // (the flush keeps 64-row tiles where the deferred verify takes 128)
    default: return launch_layers_r<MODE, MODE == kDeferred ? 2 : 4, TMAX>(p, t, num_layers, stream);
  }
}

// The row-list commit: the default when the call defers (most rows then
// have nothing to replay now), else the full grid. KDA_COMMIT_LIST=0 / 1
// forces the full grid / the list (read once). Calls with more rows than
// the list holds take the full grid.
bool commit_by_list(const Params& p) {
  static int forced = -2;
  if (forced == -2) {
    forced = -1;
    const char* env = getenv("KDA_COMMIT_LIST");
    if (env && (env[0] == '0' || env[0] == '1') && env[1] == 0) forced = env[0] - '0';
  }
  if (p.num_rows > kListRows) return false;
  return forced >= 0 ? forced == 1 : p.pending != nullptr;
}

// Workgroups of kda_commit_list<R, NW> resident at once on the current device
// (compute units x workgroups per unit), queried once per device.
template <int R, int NW>
int list_capacity() {
  constexpr int kDevices = 64;
  static int cap[kDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kDevices && cap[dev] > 0) return cap[dev];
  int occ = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &occ, reinterpret_cast<const void*>(&kda_commit_list<R, NW>), NW * 64, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int c = occ * cus;
  if (dev < kDevices) cap[dev] = c;
  return c;
}

template <int R, int NW = NWAVES>
kda_status launch_list_r(Params& p, LayerTable& t, int num_layers, hipStream_t stream) {
  p.tiles = KD / (R * NW * 8);
  const long long full = (long long)p.num_rows * p.H * p.tiles * num_layers;
  long long grid = list_capacity<R, NW>();
  if (grid < 1) return KDA_ERR_LAUNCH;
  if (grid > full) grid = full;
  p.total_blocks = (int)grid;
  void* args[] = {&p, &t, &num_layers};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_commit_list<R, NW>),
                                       dim3((unsigned)grid), dim3(NW * 64), args, 0, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status launch_list(Params& p, LayerTable& t, int num_layers, hipStream_t stream) {
  switch (tile_rows_for(kCommit, (long long)p.num_rows * p.H)) {
    // 8 waves of 8 rows, as the full-grid commit (B = 512 deferred
    // workload: deferred flow 398.0 -> 392.4 us per layer-step)
    case 32: return launch_list_r<1, 8>(p, t, num_layers, stream);
    case 64: return launch_list_r<2>(p, t, num_layers, stream);
    default: return launch_list_r<4>(p, t, num_layers, stream);
  }
}

// The one-entry layer table of a single-layer call.
LayerTable single_layer(const Params& p) {
  LayerTable t{};
  LayerRef& r = t.l[0];
  r.a_log = p.a_log;
  r.g_bias = p.g_bias;
  r.scale = p.scale;
  r.lower_bound = p.lower_bound;
  r.has_lb = p.has_lb;
  r.num_slots = p.num_slots;
  r.slot_stride = p.slot_stride;
  r.state = p.state;
  r.rk = p.rk; r.rv = p.rv; r.rg = p.rg; r.rb = p.rb;
  r.pk = p.pk; r.pv = p.pv; r.pg = p.pg; r.pb = p.pb;
  return t;
}

template <int MODE>
kda_status launch(Params& p, hipStream_t stream) {
  if ((MODE == kVerify || MODE == kDeferred) && p.Q <= 4) return launch_t<MODE, 4>(p, stream);
  return launch_t<MODE, CH>(p, stream);
}

// kda_verify with the caller's bound on every window (1..CH tokens): the
// short kernels, TMAX = 4 for bounds up to 4. When the token count is a
// whole multiple of the row count within the bound, the rows are predicted
// to be uniform windows of that length (checked per row in the kernel).
kda_status launch_verify_short(Params& p, int max_seqlen, hipStream_t stream) {
  const int g = p.num_tokens % p.num_rows == 0 ? p.num_tokens / p.num_rows : 0;
  p.guess_len = (g >= 1 && g <= max_seqlen) ? g : 0;
  p.max_seqlen = max_seqlen;
  if (max_seqlen <= 4) return launch_t<kVerify, 4, true>(p, stream);
  return launch_t<kVerify, CH, true>(p, stream);
}

}  // namespace

// --------------------------------------------------------------- C ABI ----

static kda_status check_align(const kda_align* a, int num_rows) {
  if (!a) return KDA_OK;
  if (num_rows > 0 && (!a->block_table || !a->num_computed)) return KDA_ERR_NULL;
  if (a->width < 1 || a->block_size < 1 || a->row_stride < a->width) return KDA_ERR_SHAPE;
  return KDA_OK;
}

AlignRef align_ref(const kda_align* a) {
  AlignRef r{};
  if (a) {
    r.bt = a->block_table;
    r.row_stride = a->row_stride;
    r.width = a->width;
    r.num_computed = a->num_computed;
    r.block_size = a->block_size;
  }
  return r;
}

// Elements spanned by one layer's conv state: the last element's offset + 1.
static long long conv_span(const kda_conv_state* c, int conv_dim, int width) {
  return (long long)(c->num_blocks - 1) * c->block_stride + (long long)(conv_dim - 1) * c->dim_stride +
         (long long)(width - 1) * c->token_stride + 1;
}

// Checks shared by the multi-layer calls: every layer valid, the same head
// count, the same record shape, one state-index array, and no two layers'
// pools or records overlapping each other or (with `pending`) the counts.
static kda_status check_layers(const kda_layer* layers, const kda_pool* pools, const kda_records* recs,
                        int num_layers, int num_rows, const int32_t* pending) {
  if (!layers || !pools || !recs) return KDA_ERR_NULL;
  if (num_layers < 1 || num_layers > kMaxLayers || num_rows < 0) return KDA_ERR_SHAPE;
  kda_status s;
  const int H = layers[0].num_heads;
  for (int l = 0; l < num_layers; ++l) {
    if ((s = check_layer(&layers[l])) != KDA_OK) return s;
    if (layers[l].num_heads != H) return KDA_ERR_SHAPE;
    if ((s = check_pool(&pools[l], H, num_rows)) != KDA_OK) return s;
    if ((s = check_records(&recs[l])) != KDA_OK) return s;
    if (recs[l].rows != recs[0].rows || recs[l].window != recs[0].window) return KDA_ERR_SHAPE;
    if (pools[l].state_indices != pools[0].state_indices) return KDA_ERR_SHAPE;
  }
  for (int l = 0; l < num_layers; ++l) {
    const Range pl = pool_range(&pools[l], H);
    Ranges rl;
    record_ranges(&recs[l], H, rl);
    if (records_self_overlap(rl)) return KDA_ERR_ALIAS;
    for (int m = 0; m < num_layers; ++m) {
      Ranges rm;
      record_ranges(&recs[m], H, rm);
      if (any_overlap(pl, rm)) return KDA_ERR_ALIAS;
      if (m > l && overlap(pl, pool_range(&pools[m], H))) return KDA_ERR_ALIAS;
      if (m > l)
        for (int i = 0; i < rl.n; ++i)
          if (any_overlap(rl.a[i], rm)) return KDA_ERR_ALIAS;
    }
    if (pending) {
      const Range pr = range_of(pending, (long long)recs[0].rows * 4);
      if (overlap(pr, pl) || any_overlap(pr, rl)) return KDA_ERR_ALIAS;
    }
  }
  return KDA_OK;
}

void fill_layer_table(LayerTable& t, const kda_layer* layers, const kda_pool* pools,
                      const kda_records* recs, int num_layers, bool fold) {
  for (int l = 0; l < num_layers; ++l) {
    LayerRef& r = t.l[l];
    r.a_log = layers[l].a_log;
    r.g_bias = layers[l].g_bias;
    r.scale = layers[l].scale;
    r.lower_bound = layers[l].lower_bound;
    r.has_lb = layers[l].has_lower_bound ? 1 : 0;
    r.num_slots = pools[l].num_slots;
    r.slot_stride = pools[l].slot_stride;
    r.state = pools[l].state;
    r.rk = recs[l].k; r.rv = recs[l].v; r.rg = recs[l].g; r.rb = recs[l].beta;
    if (fold) {
      r.pk = recs[l].k; r.pv = recs[l].v; r.pg = recs[l].g; r.pb = recs[l].beta;
    } else {
      r.pk = r.pv = r.pg = r.pb = nullptr;
    }
  }
}

extern "C" {

kda_status kda_recurrent(const kda_layer* layer, const kda_tokens* tokens, const kda_pool* pool,
                         uint16_t* o, hipStream_t stream) {
  kda_status s = check_layer(layer);
  if (s != KDA_OK) return s;
  const int H = layer->num_heads;
  if ((s = check_tokens(tokens, H)) != KDA_OK) return s;
  if ((s = check_pool(pool, H, tokens->num_rows)) != KDA_OK) return s;
  if (tokens->num_rows == 0) return KDA_OK;
  if (!o && tokens->num_tokens > 0) return KDA_ERR_NULL;
  if (!aligned(o, 2)) return KDA_ERR_ALIGN;
  Ranges in;
  token_ranges(tokens, H, in);
  const Range prange = pool_range(pool, H);
  if (any_overlap(prange, in)) return KDA_ERR_ALIAS;   // the pool is written
  in.add(prange);
  const Range orange = range_of(o, (long long)tokens->num_tokens * H * KD * 2);
  if (any_overlap(orange, in)) return KDA_ERR_ALIAS;
  Params p = base_params(layer);
  set_tokens(p, tokens);
  set_pool(p, pool);
  p.o = o;
  p.Q = 1;
  return launch<kRecurrent>(p, stream);
}

kda_status kda_recurrent_spec(const kda_layer* layer, const kda_tokens* tokens, const kda_pool* pool,
                              const kda_spec_table* table, uint16_t* o, hipStream_t stream) {
  kda_status s = check_layer(layer);
  if (s != KDA_OK) return s;
  const int H = layer->num_heads;
  if ((s = check_tokens(tokens, H)) != KDA_OK) return s;
  if (!table) return KDA_ERR_NULL;
  if ((s = check_pool(pool, H, 0)) != KDA_OK) return s;   // state_indices: not used
  if (table->cols < 1 || table->row_stride < table->cols) return KDA_ERR_SHAPE;
  if (tokens->num_rows == 0) return KDA_OK;
  if (!table->indices) return KDA_ERR_NULL;
  if (!o && tokens->num_tokens > 0) return KDA_ERR_NULL;
  if (!aligned(o, 2)) return KDA_ERR_ALIGN;
  Ranges in;
  token_ranges(tokens, H, in);
  const Range prange = pool_range(pool, H);
  if (any_overlap(prange, in)) return KDA_ERR_ALIAS;   // the pool is written
  in.add(prange);
  const Range orange = range_of(o, (long long)tokens->num_tokens * H * KD * 2);
  if (any_overlap(orange, in)) return KDA_ERR_ALIAS;
  // the block ids and counts are read while the pool and o are written
  const Range trange = range_of(table->indices,
                                ((long long)(tokens->num_rows - 1) * table->row_stride + table->cols) * 4);
  const Range arange = range_of(table->num_accepted, table->num_accepted ? (long long)tokens->num_rows * 4 : 0);
  if (overlap(trange, prange) || overlap(trange, orange) || overlap(arange, prange) ||
      overlap(arange, orange))
    return KDA_ERR_ALIAS;
  Params p = base_params(layer);
  set_tokens(p, tokens);
  set_pool(p, pool);
  p.slots = nullptr;
  p.o = o;
  p.Q = 1;
  p.spec_idx = table->indices;
  p.spec_stride = table->row_stride;
  p.spec_cols = table->cols;
  p.spec_acc = table->num_accepted;
  return launch<kSpec>(p, stream);
}

kda_status kda_verify(const kda_layer* layer, const kda_tokens* tokens, const kda_pool* pool,
                      const kda_records* rec, const int32_t* record_rows, uint16_t* o,
                      hipStream_t stream) {
  kda_status s = check_layer(layer);
  if (s != KDA_OK) return s;
  const int H = layer->num_heads;
  if ((s = check_tokens(tokens, H)) != KDA_OK) return s;
  if ((s = check_pool(pool, H, tokens->num_rows)) != KDA_OK) return s;
  if ((s = check_records(rec)) != KDA_OK) return s;
  if (tokens->num_rows == 0) return KDA_OK;
  if (!o && tokens->num_tokens > 0) return KDA_ERR_NULL;
  if (!aligned(o, 2)) return KDA_ERR_ALIGN;
  if (!record_rows && tokens->num_rows > rec->rows) return KDA_ERR_CAPACITY;
  Ranges in;
  token_ranges(tokens, H, in);
  in.add(pool_range(pool, H));
  Ranges rr;
  record_ranges(rec, H, rr);
  const Range orange = range_of(o, (long long)tokens->num_tokens * H * KD * 2);
  if (any_overlap(orange, in) || any_overlap(orange, rr) || records_self_overlap(rr)) return KDA_ERR_ALIAS;
  for (int i = 0; i < rr.n; ++i)
    if (any_overlap(rr.a[i], in)) return KDA_ERR_ALIAS;
  Params p = base_params(layer);
  set_tokens(p, tokens);
  set_pool(p, pool);
  set_records(p, rec);
  p.record_rows = record_rows;
  p.o = o;
  if (tokens->max_seqlen >= 1 && tokens->max_seqlen <= CH)
    return launch_verify_short(p, tokens->max_seqlen, stream);
  return launch<kVerify>(p, stream);
}

kda_status kda_commit(const kda_layer* layer, const int32_t* cu_seqlens, int32_t num_rows,
                      const kda_pool* pool, const kda_records* rec, const int32_t* record_rows,
                      const int32_t* num_accepted, int32_t* pending, const uint8_t* eager,
                      hipStream_t stream) {
  kda_status s = check_layer(layer);
  if (s != KDA_OK) return s;
  const int H = layer->num_heads;
  if (num_rows < 0) return KDA_ERR_SHAPE;
  if (!cu_seqlens || (num_rows > 0 && !num_accepted)) return KDA_ERR_NULL;
  if ((s = check_pool(pool, H, num_rows)) != KDA_OK) return s;
  if ((s = check_records(rec)) != KDA_OK) return s;
  if (eager && !pending) return KDA_ERR_SHAPE;
  if (num_rows == 0) return KDA_OK;
  if (!record_rows && num_rows > rec->rows) return KDA_ERR_CAPACITY;
  Ranges rr;
  record_ranges(rec, H, rr);
  if (any_overlap(pool_range(pool, H), rr) || records_self_overlap(rr)) return KDA_ERR_ALIAS;
  if (pending) {
    const Range pr = range_of(pending, (long long)rec->rows * 4);
    if (overlap(pr, pool_range(pool, H)) || any_overlap(pr, rr)) return KDA_ERR_ALIAS;
  }
  Params p = base_params(layer);
  p.cu = cu_seqlens;
  p.num_rows = num_rows;
  p.num_tokens = 0x7FFFFFFF;
  set_pool(p, pool);
  set_records(p, rec);
  p.record_rows = record_rows;
  p.num_accepted = num_accepted;
  p.pending = pending;
  p.eager = eager;
  if (commit_by_list(p)) {
    LayerTable t = single_layer(p);
    return launch_list(p, t, 1, stream);
  }
  return launch<kCommit>(p, stream);
}

kda_status kda_verify_deferred(const kda_layer* layer, const kda_tokens* tokens,
                               const kda_pool* pool, const kda_records* rec_prev,
                               const int32_t* pending, const kda_records* rec_next,
                               const int32_t* record_rows, uint16_t* o, hipStream_t stream) {
  kda_status s = check_layer(layer);
  if (s != KDA_OK) return s;
  const int H = layer->num_heads;
  if ((s = check_tokens(tokens, H)) != KDA_OK) return s;
  if ((s = check_pool(pool, H, tokens->num_rows)) != KDA_OK) return s;
  if ((s = check_records(rec_prev)) != KDA_OK) return s;
  if ((s = check_records(rec_next)) != KDA_OK) return s;
  if (!pending) return KDA_ERR_NULL;
  if (rec_prev->rows != rec_next->rows || rec_prev->window != rec_next->window) return KDA_ERR_SHAPE;
  if (tokens->num_rows == 0) return KDA_OK;
  if (!o && tokens->num_tokens > 0) return KDA_ERR_NULL;
  if (!aligned(o, 2)) return KDA_ERR_ALIGN;
  if (!record_rows && tokens->num_rows > rec_next->rows) return KDA_ERR_CAPACITY;
  Ranges in;
  token_ranges(tokens, H, in);
  Range prange = pool_range(pool, H);
  Ranges rp, rn;
  record_ranges(rec_prev, H, rp);
  record_ranges(rec_next, H, rn);
  const Range orange = range_of(o, (long long)tokens->num_tokens * H * KD * 2);
  if (records_self_overlap(rp) || records_self_overlap(rn)) return KDA_ERR_ALIAS;
  for (int i = 0; i < rn.n; ++i)
    if (any_overlap(rn.a[i], rp) || any_overlap(rn.a[i], in) || overlap(rn.a[i], prange) ||
        overlap(rn.a[i], orange))
      return KDA_ERR_ALIAS;
  for (int i = 0; i < rp.n; ++i)
    if (overlap(rp.a[i], prange) || overlap(rp.a[i], orange)) return KDA_ERR_ALIAS;
  if (any_overlap(orange, in) || overlap(orange, prange)) return KDA_ERR_ALIAS;
  const Range pend = range_of(pending, (long long)rec_prev->rows * 4);
  if (overlap(pend, prange) || any_overlap(pend, rn) || overlap(pend, orange)) return KDA_ERR_ALIAS;
  Params p = base_params(layer);
  set_tokens(p, tokens);
  set_pool(p, pool);
  set_records(p, rec_next);
  p.pk = rec_prev->k; p.pv = rec_prev->v; p.pg = rec_prev->g; p.pb = rec_prev->beta;
  p.record_rows = record_rows;
  p.pending_in = pending;
  p.o = o;
  return launch<kDeferred>(p, stream);
}

kda_status kda_commit_layers(const kda_layer* layers, const kda_pool* pools,
                             const kda_records* recs, int32_t num_layers, const int32_t* cu_seqlens,
                             int32_t num_rows, const int32_t* record_rows,
                             const int32_t* num_accepted, int32_t* pending, const uint8_t* eager,
                             const kda_align* align, hipStream_t stream) {
  kda_status s = check_layers(layers, pools, recs, num_layers, num_rows, pending);
  if (s != KDA_OK) return s;
  if (!cu_seqlens || (num_rows > 0 && !num_accepted)) return KDA_ERR_NULL;
  if (eager && !pending) return KDA_ERR_SHAPE;
  if ((s = check_align(align, num_rows)) != KDA_OK) return s;
  if (num_rows == 0) return KDA_OK;
  if (!record_rows && num_rows > recs[0].rows) return KDA_ERR_CAPACITY;
  Params p = base_params(&layers[0]);
  p.cu = cu_seqlens;
  p.num_rows = num_rows;
  p.num_tokens = 0x7FFFFFFF;
  set_pool(p, &pools[0]);
  set_records(p, &recs[0]);
  p.record_rows = record_rows;
  p.num_accepted = num_accepted;
  p.pending = pending;
  p.eager = eager;
  p.align = align_ref(align);
  LayerTable t{};
  fill_layer_table(t, layers, pools, recs, num_layers, false);
  if (commit_by_list(p)) return launch_list(p, t, num_layers, stream);
  return launch_layers<kCommit>(p, t, num_layers, stream);
}

kda_status kda_flush_layers(const kda_layer* layers, const kda_pool* pools,
                            const kda_records* rec_prev, int32_t num_layers, int32_t num_rows,
                            const int32_t* record_rows, const int32_t* pending, hipStream_t stream) {
  kda_status s = check_layers(layers, pools, rec_prev, num_layers, num_rows, pending);
  if (s != KDA_OK) return s;
  if (!pending) return KDA_ERR_NULL;
  if (num_rows == 0) return KDA_OK;
  if (!record_rows && num_rows > rec_prev[0].rows) return KDA_ERR_CAPACITY;
  Params p = base_params(&layers[0]);
  p.num_rows = num_rows;
  p.num_tokens = 0;
  p.flush = 1;
  set_pool(p, &pools[0]);
  set_records(p, &rec_prev[0]);
  p.pk = rec_prev[0].k; p.pv = rec_prev[0].v; p.pg = rec_prev[0].g; p.pb = rec_prev[0].beta;
  p.record_rows = record_rows;
  p.pending_in = pending;
  LayerTable t{};
  fill_layer_table(t, layers, pools, rec_prev, num_layers, true);
  return launch_layers<kDeferred>(p, t, num_layers, stream);
}

kda_status kda_conv_compact(const kda_conv_state* layers, int32_t num_layers, int32_t conv_dim,
                            int32_t history, int32_t width, const int32_t* cu_seqlens,
                            int32_t num_rows, const int32_t* state_indices,
                            const int32_t* num_accepted, int32_t window, const kda_align* align,
                            hipStream_t stream) {
  if (!layers) return KDA_ERR_NULL;
  if (num_layers < 1 || num_layers > kMaxConvLayers || num_rows < 0 || conv_dim < 1 ||
      history < 1 || history > kMaxHistory || window < 1 || window > MAX_WINDOW ||
      width < window + history - 1)
    return KDA_ERR_SHAPE;
  for (int l = 0; l < num_layers; ++l) {
    const kda_conv_state& c = layers[l];
    if (!c.state) return KDA_ERR_NULL;
    if (c.num_blocks < 1 || c.block_stride < 1 || c.dim_stride < 1 || c.token_stride < 1)
      return KDA_ERR_SHAPE;
    if (!aligned(c.state, 2)) return KDA_ERR_ALIGN;
  }
  for (int l = 0; l < num_layers; ++l)
    for (int m = l + 1; m < num_layers; ++m)
      if (overlap(range_of(layers[l].state, conv_span(&layers[l], conv_dim, width) * 2),
                  range_of(layers[m].state, conv_span(&layers[m], conv_dim, width) * 2)))
        return KDA_ERR_ALIAS;
  if (num_rows > 0 && (!cu_seqlens || !state_indices || !num_accepted)) return KDA_ERR_NULL;
  kda_status s;
  if ((s = check_align(align, num_rows)) != KDA_OK) return s;
  if (num_rows == 0) return KDA_OK;
  if (num_rows > 65535) return KDA_ERR_SHAPE;   // rows are the grid's second dimension
  ConvParams p{};
  p.cu = cu_seqlens;
  p.slots = state_indices;
  p.num_accepted = num_accepted;
  p.num_rows = num_rows;
  p.conv_dim = conv_dim;
  p.history = history;
  p.window = window;
  p.width = width;
  p.align = align_ref(align);
  ConvTable t{};
  for (int l = 0; l < num_layers; ++l) {
    t.l[l].state = layers[l].state;
    t.l[l].block_stride = layers[l].block_stride;
    t.l[l].dim_stride = layers[l].dim_stride;
    t.l[l].token_stride = layers[l].token_stride;
    t.l[l].num_blocks = layers[l].num_blocks;
  }
  void* args[] = {&p, &t};
  // in place on dense rows, whole 16-byte units: the span kernel
  bool span = align == nullptr && (long long)conv_dim * width % 8 == 0;
  for (int l = 0; l < num_layers && span; ++l) {
    const kda_conv_state& c = layers[l];
    span = c.token_stride == 1 && c.dim_stride == width && c.block_stride % 8 == 0 &&
           c.block_stride >= (long long)conv_dim * width && aligned(c.state, 16);
  }
  if (span) {
    int chans = (kConvSpanBytes / 2 / width) & ~7;
    chans = chans < 1024 ? chans : 1024;
    if (chans >= 8) {
      p.chans = chans;
      const void* f = nullptr;
      switch (history) {
        case 1: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<1>); break;
        case 2: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<2>); break;
        case 3: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<3>); break;
        case 4: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<4>); break;
        case 5: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<5>); break;
        case 6: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<6>); break;
        case 7: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<7>); break;
        default: f = reinterpret_cast<const void*>(&conv_compact_span_kernel<8>); break;
      }
      const dim3 grid((unsigned)((conv_dim + chans - 1) / chans), (unsigned)num_rows,
                      (unsigned)num_layers);
      const hipError_t e = hipLaunchKernel(f, grid, dim3(kConvThreads), args, 0, stream);
      return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
    }
  }
  const void* fn = nullptr;
  switch (history) {
    case 1: fn = reinterpret_cast<const void*>(&conv_compact_kernel<1>); break;
    case 2: fn = reinterpret_cast<const void*>(&conv_compact_kernel<2>); break;
    case 3: fn = reinterpret_cast<const void*>(&conv_compact_kernel<3>); break;
    case 4: fn = reinterpret_cast<const void*>(&conv_compact_kernel<4>); break;
    case 5: fn = reinterpret_cast<const void*>(&conv_compact_kernel<5>); break;
    case 6: fn = reinterpret_cast<const void*>(&conv_compact_kernel<6>); break;
    case 7: fn = reinterpret_cast<const void*>(&conv_compact_kernel<7>); break;
    default: fn = reinterpret_cast<const void*>(&conv_compact_kernel<8>); break;
  }
  const int per_block = kConvThreads * kConvPerThread;
  const dim3 grid((unsigned)((conv_dim + per_block - 1) / per_block), (unsigned)num_rows,
                  (unsigned)num_layers);
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(kConvThreads), args, 0, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char* kda_status_string(kda_status status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: inconsistent sizes";
    case KDA_ERR_CAPACITY: return "KDA_ERR_CAPACITY: more rows than record rows";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointer or stride misaligned";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input or another output";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head_dim must be 128";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: kernel launch failed";
    case KDA_ERR_METADATA: return "KDA_ERR_METADATA: a row breaks a precondition";
  }
  return "unknown kda_status";
}

const char* kda_build_info(void) {
  return "libkda gfx950 (HIP, wave64, fp32 state, bf16 activations, head_dim 128)";
}

}  // extern "C"
