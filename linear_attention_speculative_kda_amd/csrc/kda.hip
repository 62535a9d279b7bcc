// libkda: KDA speculative verify / accepted-token commit ("RecoverSSM") for
// AMD Instinct MI355X (gfx950, CDNA4, wave64).
//
// The method (pages: "recoverssm.py (GLM-5.3-Flash KDA speculative verify with
// one checkpoint state per request)", _verify_kernel per-token loop): per head
// a fp32 state S[K, V]; per token decay the key channels by exp(g), delta rule
// u = beta * (v - S^T k^), rank-1 update S += k^ u^T, output o = S^T q^.
//
// Kernel design (one kernel template serves the four calls):
//  * One workgroup of 256 threads (4 waves) per (request row, head, V-tile of
//    BV = 32*R value rows). The fp32 K x BV state tile lives in VGPRs for the
//    whole token loop: a group of 8 adjacent lanes owns one value row; each
//    lane holds 16 key channels of it (4 chunks of 4 consecutive channels,
//    chunk j at j*32 + 4*(lane%8)), so one 128-bit load per chunk and the 8
//    lanes of a group read 128 contiguous bytes. Each lane holds R rows.
//  * The per-token vectors shared by all rows (k^, q^, exp(g), beta and the
//    tile's slice of v) are computed once per workgroup, 8 tokens at a time,
//    by half-waves (one token each, 4 channels per lane) into LDS. The state
//    tile's loads are issued before this staging so that they are in flight
//    meanwhile.
//  * The two reductions over K per token and row (S^T k^ and S^T q^) are
//    16-term in-lane FMA chains plus a 3-step DPP butterfly across the 8
//    lanes of the group (quad_perm 1032, quad_perm 2301, row_half_mirror).
//    A butterfly adds the same two operands in every lane, so all 8 lanes
//    get the same bits.
//  * No MFMA: per token the work is two matrix-vector products and a rank-1
//    update of a 64 KiB state that is read once and written at most once, so
//    the path is bound by HBM bandwidth, not by a dense contraction.
//  * Every call runs the same per-token code with the same lane layout, so a
//    commit of n records gives the bits of the plain recurrence over the same
//    n tokens. The build uses -ffp-contract=off: every FMA is an explicit
//    fmaf, nothing is contracted or reassociated by the compiler.
//  * Every index read from device memory (cu_seqlens, slots, record rows,
//    accepted counts, pending counts) is range-checked before use.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kda.h"

namespace {

constexpr int KD = 128;        // head dim (K == V)
constexpr int NTHREADS = 256;  // 4 waves
constexpr int NWAVES = 4;
constexpr int CH = 8;          // tokens staged in LDS per chunk
constexpr int MAX_WINDOW = 64;

enum Mode : int { kRecurrent = 0, kVerify = 1, kCommit = 2, kDeferred = 3 };

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
  int total_blocks;
};

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);                                  // nearest, ties to even
  return (uint16_t)(u >> 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a group; every lane gets the same bits.
__device__ __forceinline__ float reduce8(float x) {
  x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp<0x141>(x);  // row_half_mirror
  return x;
}

template <int XOR>
__device__ __forceinline__ float swz(float x) {
  // ds_swizzle bit mode: lane j of each 32-lane half reads lane j ^ XOR.
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (XOR << 10) | 0x1F));
}

// Sum over the 32 lanes of a half-wave; every lane gets the same bits.
__device__ __forceinline__ float reduce32(float x) {
  x = x + swz<1>(x);
  x = x + swz<2>(x);
  x = x + swz<4>(x);
  x = x + swz<8>(x);
  x = x + swz<16>(x);
  return x;
}

__device__ __forceinline__ void unpack4(uint2 raw, float out[4]) {
  out[0] = bf16_to_f32(raw.x & 0xFFFFu);
  out[1] = bf16_to_f32(raw.x >> 16);
  out[2] = bf16_to_f32(raw.y & 0xFFFFu);
  out[3] = bf16_to_f32(raw.y >> 16);
}

__device__ __forceinline__ float sum_sq4(const float x[4]) {
  float s = x[0] * x[0];
  s = fmaf(x[1], x[1], s);
  s = fmaf(x[2], x[2], s);
  s = fmaf(x[3], x[3], s);
  return s;
}

// Gate of one key channel from x = g_raw + g_bias (A = exp(A_log)).
__device__ __forceinline__ float gate_of(float x, float A, int has_lb, float lb) {
  if (has_lb) {
    // bounded: lb * sigmoid(A * x), written lb / (1 + exp(-(A * x)))
    return lb / (1.0f + expf(-(A * x)));
  }
  // unbounded: -A * softplus(x), softplus(x) = max(x, 0) + log1p(exp(-|x|))
  const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
  return -(A * sp);
}

// LDS staging area for one chunk of tokens.
template <int BV>
struct Stage {
  float kh[CH][KD];   // k^
  float qh[CH][KD];   // q^ (scale folded in)
  float dk[CH][KD];   // exp(g)
  float vt[CH][BV];   // the tile's slice of v
  float bt[CH];       // beta
};

// Where one token's raw inputs come from.
struct Src {
  const uint16_t* k;
  const uint16_t* g;
  const uint16_t* v;
  const uint16_t* b;
  const uint16_t* q;  // nullptr: no output for this token
};

// ------------------------------------------------------------------ kernel --

template <int MODE, int R>
__global__ __launch_bounds__(NTHREADS) void kda_kernel(Params p) {
  constexpr int BV = R * NWAVES * 8;   // value rows per workgroup
  constexpr int VPL = BV / 32;         // v values per lane when staging
  __shared__ Stage<BV> st;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p8 = lane & 7;    // position inside the 8-lane row group
  const int grp = lane >> 3;  // row group inside the wave

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
  // consecutive logical blocks (the V-tiles and heads of one request) are
  // mapped to one XCD and share its L2.
  int b = blockIdx.x;
  const int nb = p.total_blocks;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int tile = b % p.tiles;
  const int rh = b / p.tiles;
  const int head = rh % p.H;
  const int row = rh / p.H;
  const int H = p.H;

  // ---- row prologue: span, slot, record row, counts -----------------------
  const int bos = p.cu[row];
  const int eos = p.cu[row + 1];
  int T = eos - bos;
  if (bos < 0 || T < 0 || (MODE != kCommit && eos > p.num_tokens)) T = 0;
  const int slot = p.slots[row];
  const bool slot_ok = slot > 0 && slot < p.num_slots;
  const int r = p.record_rows ? p.record_rows[row] : row;
  const int ri = (r >= 0 && r < p.rec_rows) ? r + 1 : 0;   // storage index, 0 = scratch

  int nfold = 0;   // records replayed into the state (commit / deferred fold)
  int nmain = 0;   // window tokens run with outputs (recurrent / verify)
  if (MODE == kCommit) {
    int n = p.num_accepted[row];
    n = n < 0 ? 0 : n;
    n = n < T ? n : T;
    n = n < p.Q ? n : p.Q;
    const bool valid = slot_ok && n > 0 && ri > 0;
    bool now = true;
    if (p.pending) {
      now = p.eager != nullptr && p.eager[row] != 0;
      if (ri > 0 && head == 0 && tile == 0 && tid == 0) p.pending[ri - 1] = now ? 0 : (valid ? n : 0);
    }
    nfold = (valid && now) ? n : 0;
  } else if (MODE == kDeferred) {
    if (ri > 0) {
      int pn = p.pending_in[ri - 1];
      pn = pn < 0 ? 0 : pn;
      nfold = pn < p.Q ? pn : p.Q;
    }
    nmain = T;
  } else {
    nmain = T;
  }
  if (!slot_ok || (nfold == 0 && nmain == 0)) return;

  // ---- state tile: issue the loads ----------------------------------------
  float* sbase = p.state + (long long)slot * p.slot_stride + (long long)head * KD * KD;
  float S[R][16];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int vrow = tile * BV + (rr * NWAVES + wave) * 8 + grp;
    const float* src = sbase + vrow * KD + p8 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(src + j * 32);
      S[rr][4 * j + 0] = x.x;
      S[rr][4 * j + 1] = x.y;
      S[rr][4 * j + 2] = x.z;
      S[rr][4 * j + 3] = x.w;
    }
  }

  const float A = expf(p.a_log[head]);
  const int hw = tid >> 5;      // half-wave: token slot when staging
  const int l32 = tid & 31;     // 4 channels per lane when staging
  const float* gb = p.g_bias + head * KD + 4 * l32;

  // Two segments: the fold (records, no output) then the main window.
  for (int seg = 0; seg < 2; ++seg) {
    const bool fold = seg == 0;
    const int n = fold ? nfold : nmain;
    if (n == 0) continue;
    for (int c0 = 0; c0 < n; c0 += CH) {
      const int m = (n - c0) < CH ? (n - c0) : CH;
      __syncthreads();  // the previous chunk is consumed
      // ---- stage: one token per half-wave --------------------------------
      if (hw < m) {
        const int j = c0 + hw;
        Src s;
        if (fold) {
          const uint16_t* rk = (MODE == kDeferred) ? p.pk : p.rk;
          const uint16_t* rg = (MODE == kDeferred) ? p.pg : p.rg;
          const uint16_t* rv = (MODE == kDeferred) ? p.pv : p.rv;
          const uint16_t* rb = (MODE == kDeferred) ? p.pb : p.rb;
          const long long base = ((long long)ri * H + head) * p.Q + j;
          s.k = rk + base * KD;
          s.g = rg + base * KD;
          s.v = rv + base * KD;
          s.b = rb + base;
          s.q = nullptr;
        } else {
          const long long tok = (long long)bos + j;
          s.k = p.k + tok * p.sk + head * KD;
          s.g = p.g + tok * p.sg + head * KD;
          s.v = p.v + tok * p.sv + head * KD;
          s.b = p.beta + tok * p.sb + head;
          s.q = p.q + tok * p.sq + head * KD;
        }
        const uint2 kraw = *reinterpret_cast<const uint2*>(s.k + 4 * l32);
        const uint2 graw = *reinterpret_cast<const uint2*>(s.g + 4 * l32);
        float kx[4], gx[4];
        unpack4(kraw, kx);
        unpack4(graw, gx);
        const float kn = sqrtf(reduce32(sum_sq4(kx)) + 1e-6f);
        float4 kh, dk;
        kh.x = kx[0] / kn; kh.y = kx[1] / kn; kh.z = kx[2] / kn; kh.w = kx[3] / kn;
        dk.x = expf(gate_of(gx[0] + gb[0], A, p.has_lb, p.lower_bound));
        dk.y = expf(gate_of(gx[1] + gb[1], A, p.has_lb, p.lower_bound));
        dk.z = expf(gate_of(gx[2] + gb[2], A, p.has_lb, p.lower_bound));
        dk.w = expf(gate_of(gx[3] + gb[3], A, p.has_lb, p.lower_bound));
        *reinterpret_cast<float4*>(&st.kh[hw][4 * l32]) = kh;
        *reinterpret_cast<float4*>(&st.dk[hw][4 * l32]) = dk;
        if (!fold) {
          const uint2 qraw = *reinterpret_cast<const uint2*>(s.q + 4 * l32);
          float qx[4];
          unpack4(qraw, qx);
          const float qn = sqrtf(reduce32(sum_sq4(qx)) + 1e-6f);
          float4 qh;
          qh.x = (qx[0] / qn) * p.scale; qh.y = (qx[1] / qn) * p.scale;
          qh.z = (qx[2] / qn) * p.scale; qh.w = (qx[3] / qn) * p.scale;
          *reinterpret_cast<float4*>(&st.qh[hw][4 * l32]) = qh;
        }
        uint16_t vraw[VPL];
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
          vraw[e] = s.v[tile * BV + l32 * VPL + e];
          st.vt[hw][l32 * VPL + e] = bf16_to_f32(vraw[e]);
        }
        uint16_t braw = 0;
        if (l32 == 0) {
          braw = *s.b;
          st.bt[hw] = 1.0f / (1.0f + expf(-bf16_to_f32(braw)));
        }
        // Records of the window (verify): raw inputs, first Q tokens only.
        if ((MODE == kVerify || MODE == kDeferred) && !fold && j < p.Q) {
          const long long base = ((long long)ri * H + head) * p.Q + j;
          if (tile == 0) {
            *reinterpret_cast<uint2*>(p.rk + base * KD + 4 * l32) = kraw;
            *reinterpret_cast<uint2*>(p.rg + base * KD + 4 * l32) = graw;
            if (l32 == 0) p.rb[base] = braw;
          }
#pragma unroll
          for (int e = 0; e < VPL; ++e) p.rv[base * KD + tile * BV + l32 * VPL + e] = vraw[e];
        }
      }
      __syncthreads();

      // ---- token loop over the chunk -------------------------------------
      for (int t = 0; t < m; ++t) {
        float kh[16], dk[16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float4 a = *reinterpret_cast<const float4*>(&st.kh[t][jj * 32 + p8 * 4]);
          const float4 d = *reinterpret_cast<const float4*>(&st.dk[t][jj * 32 + p8 * 4]);
          kh[4 * jj + 0] = a.x; kh[4 * jj + 1] = a.y; kh[4 * jj + 2] = a.z; kh[4 * jj + 3] = a.w;
          dk[4 * jj + 0] = d.x; dk[4 * jj + 1] = d.y; dk[4 * jj + 2] = d.z; dk[4 * jj + 3] = d.w;
        }
        const float beta = st.bt[t];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const int vloc = (rr * NWAVES + wave) * 8 + grp;
          // decay the key channels
#pragma unroll
          for (int e = 0; e < 16; ++e) S[rr][e] = S[rr][e] * dk[e];
          // S^T k^ for this value row
          float acc[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float a = S[rr][4 * jj] * kh[4 * jj];
            a = fmaf(S[rr][4 * jj + 1], kh[4 * jj + 1], a);
            a = fmaf(S[rr][4 * jj + 2], kh[4 * jj + 2], a);
            a = fmaf(S[rr][4 * jj + 3], kh[4 * jj + 3], a);
            acc[jj] = a;
          }
          const float kv = reduce8((acc[0] + acc[1]) + (acc[2] + acc[3]));
          const float u = beta * (st.vt[t][vloc] - kv);
          // rank-1 update
#pragma unroll
          for (int e = 0; e < 16; ++e) S[rr][e] = fmaf(kh[e], u, S[rr][e]);
        }
        if (!fold) {
          float qh[16];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float4 a = *reinterpret_cast<const float4*>(&st.qh[t][jj * 32 + p8 * 4]);
            qh[4 * jj + 0] = a.x; qh[4 * jj + 1] = a.y; qh[4 * jj + 2] = a.z; qh[4 * jj + 3] = a.w;
          }
          const long long tok = (long long)bos + c0 + t;
          uint16_t* orow = p.o + (tok * H + head) * KD + tile * BV;
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            float acc[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float a = S[rr][4 * jj] * qh[4 * jj];
              a = fmaf(S[rr][4 * jj + 1], qh[4 * jj + 1], a);
              a = fmaf(S[rr][4 * jj + 2], qh[4 * jj + 2], a);
              a = fmaf(S[rr][4 * jj + 3], qh[4 * jj + 3], a);
              acc[jj] = a;
            }
            const float ov = reduce8((acc[0] + acc[1]) + (acc[2] + acc[3]));
            if (p8 == 0) orow[(rr * NWAVES + wave) * 8 + grp] = f32_to_bf16(ov);
          }
        }
      }
    }
    // The folded (deferred) or committed state goes back to the slot.
    const bool store = (fold && MODE == kDeferred) || (MODE == kCommit) || (!fold && MODE == kRecurrent);
    if (store) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int vrow = tile * BV + (rr * NWAVES + wave) * 8 + grp;
        float* dst = sbase + vrow * KD + p8 * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float4 x;
          x.x = S[rr][4 * j + 0]; x.y = S[rr][4 * j + 1]; x.z = S[rr][4 * j + 2]; x.w = S[rr][4 * j + 3];
          *reinterpret_cast<float4*>(dst + j * 32) = x;
        }
      }
    }
  }
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
  if (t->num_rows < 0 || t->num_tokens < 0) return KDA_ERR_SHAPE;
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

// Rows of the state tile per workgroup: 32 * R. One workgroup per (row, head)
// (128 rows) when there are enough (row, head) pairs to fill the chip;
// smaller batches split V into 2 or 4 tiles for more workgroups. The per-row
// arithmetic does not depend on the tile size. KDA_TILE_ROWS in {32, 64, 128}
// forces a size (read once).
int tile_rows_for(long long pairs) {
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
  if (pairs >= 2048) return 128;
  if (pairs >= 1024) return 64;
  return 32;
}

template <int MODE, int R>
kda_status launch_r(Params& p, hipStream_t stream) {
  p.tiles = KD / (32 * R);
  const long long blocks = (long long)p.num_rows * p.H * p.tiles;
  if (blocks > 0x7FFFFFFFLL) return KDA_ERR_SHAPE;
  p.total_blocks = (int)blocks;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&kda_kernel<MODE, R>),
                                       dim3((unsigned)blocks), dim3(NTHREADS), args, 0, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int MODE>
kda_status launch(Params& p, hipStream_t stream) {
  switch (tile_rows_for((long long)p.num_rows * p.H)) {
    case 32: return launch_r<MODE, 1>(p, stream);
    case 64: return launch_r<MODE, 2>(p, stream);
    default: return launch_r<MODE, 4>(p, stream);
  }
}

}  // namespace

// --------------------------------------------------------------- C ABI ----

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
  in.add(pool_range(pool, H));
  const Range orange = range_of(o, (long long)tokens->num_tokens * H * KD * 2);
  if (any_overlap(orange, in)) return KDA_ERR_ALIAS;
  Params p = base_params(layer);
  set_tokens(p, tokens);
  set_pool(p, pool);
  p.o = o;
  p.Q = 1;
  return launch<kRecurrent>(p, stream);
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
  }
  return "unknown kda_status";
}

const char* kda_build_info(void) {
  return "libkda gfx950 (HIP, wave64, fp32 state, bf16 activations, head_dim 128)";
}

}  // extern "C"
