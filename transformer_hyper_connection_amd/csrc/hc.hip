// libhc -- Hyper-Connections residual glue for AMD Instinct MI355X (gfx950).
//
// Sources (model-atlas pages, by title and part):
//   "Source layer, pairs pooled": Block code panel (hc_mixes, hc_pre, hc_post, forward)
//   "Reading weights":            reading-weight equation; split/Sinkhorn kernel panel
//   "Write the streams":          stream-update equation
//   "Final RMSNorm":              RMSNorm equation and class
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (no fused multiply-add
// is formed implicitly: the stream arithmetic of hc_post / hc_pre is the page's
// sequence of separately rounded fp32 products and sums, bit for bit).
//
// Kernels
//   tile_kernel<POST, RM, NORM>  everything that derives mixes (hc_mixes, block
//       entry, sublayer boundary): 64-token tiles x feature slices, about one
//       workgroup per compute unit; the 24-wide projection on the matrix cores
//       with the weight tiles shared through LDS; the slices of a tile meet once
//       in a workspace, then each writes its part of the read row.
//   row_kernel<POST, PRE, NORM, TPW>  streams only (hc_post, hc_pre, the stack
//       exit): whole token rows per wave, 1 KB per load or store.
//   split_kernel    hc_split_sinkhorn, one token per lane.
//   pack_kernel     fp32 projection weight -> bf16 hi/mid/lo terms in tile order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "hc.h"

namespace {

constexpr int kHC = 4;
constexpr int kMix = (2 + kHC) * kHC;  // 24 mix numbers
constexpr int kSplitRows = 3 * kMix;   // 72 = hi | mid | lo rows of the packed weight
constexpr int kNT = 5;                 // 16-column matrix tiles covering 72 (+8 zero) rows
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kFPL = 8;                // features per lane per matrix-core step
constexpr int kStepF = 4 * kFPL;       // features per matrix-core step (4 lane groups)
constexpr int kMaxD = 32768;
constexpr int kMaxNormD = 10240;

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_elem(u32 w, int h) { return h ? bf_hi(w) : bf_lo(w); }

// Two fp32 -> packed bf16 pair (element a in the low half), nearest-even.
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float round_bf16(float a) { return bf_lo(pack_bf16(a, 0.f)); }

__device__ __forceinline__ float dot2_bf16(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32 w0, u32 w1, u32 w2, u32 w3) {
  u32x4 v = {w0, w1, w2, w3};
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------- split / Sinkhorn
// One token: "Reading weights" split/Sinkhorn kernel panel and reading-weight
// equation.  fp32; the row/column divisions use the hardware reciprocal.
__device__ __forceinline__ float sigmoidf_(float u) { return __builtin_amdgcn_rcpf(1.0f + expf(-u)); }

__device__ void split_sinkhorn_one(const float* mx, float s0, float s1, float s2, const float* bs,
                                   int iters, float eps, float* pre_o, float* post_o, float* comb_o) {
  float pre[kHC], post[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    pre[j] = sigmoidf_(mx[j] * s0 + bs[j]) + eps;
    post[j] = 2.0f * sigmoidf_(mx[kHC + j] * s1 + bs[kHC + j]);
  }
  float A[kHC][kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    float mx_row = -INFINITY;
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      A[j][k] = mx[2 * kHC + j * kHC + k] * s2 + bs[2 * kHC + j * kHC + k];
      mx_row = fmaxf(mx_row, A[j][k]);
    }
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      A[j][k] = expf(A[j][k] - mx_row);
      rs = rs + A[j][k];
    }
    const float inv = __builtin_amdgcn_rcpf(rs);
#pragma unroll
    for (int k = 0; k < kHC; ++k) A[j][k] = A[j][k] * inv + eps;
  }
  auto col_norm = [&]() {
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      float cs = A[0][k];
#pragma unroll
      for (int j = 1; j < kHC; ++j) cs = cs + A[j][k];
      const float inv = __builtin_amdgcn_rcpf(cs + eps);
#pragma unroll
      for (int j = 0; j < kHC; ++j) A[j][k] = A[j][k] * inv;
    }
  };
  col_norm();
  for (int it = 1; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
      float rs = A[j][0];
#pragma unroll
      for (int k = 1; k < kHC; ++k) rs = rs + A[j][k];
      const float inv = __builtin_amdgcn_rcpf(rs + eps);
#pragma unroll
      for (int k = 0; k < kHC; ++k) A[j][k] = A[j][k] * inv;
    }
    col_norm();
  }
  *reinterpret_cast<f32x4*>(pre_o) = f32x4{pre[0], pre[1], pre[2], pre[3]};
  *reinterpret_cast<f32x4*>(post_o) = f32x4{post[0], post[1], post[2], post[3]};
#pragma unroll
  for (int j = 0; j < kHC; ++j)
    reinterpret_cast<f32x4*>(comb_o)[j] = f32x4{A[j][0], A[j][1], A[j][2], A[j][3]};
}

__global__ void __launch_bounds__(256) split_kernel(const float* __restrict__ mixes,
                                                    const float* __restrict__ scale,
                                                    const float* __restrict__ base, int64_t n, int iters,
                                                    float eps, float* __restrict__ pre,
                                                    float* __restrict__ post, float* __restrict__ comb) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  float mx[kMix], bs[kMix];
#pragma unroll
  for (int q = 0; q < kMix; q += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(mixes + t * kMix + q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(base + q);
    mx[q] = v[0]; mx[q + 1] = v[1]; mx[q + 2] = v[2]; mx[q + 3] = v[3];
    bs[q] = b[0]; bs[q + 1] = b[1]; bs[q + 2] = b[2]; bs[q + 3] = b[3];
  }
  split_sinkhorn_one(mx, scale[0], scale[1], scale[2], bs, iters, eps, pre + t * kHC, post + t * kHC,
                     comb + t * kHC * kHC);
}

// ------------------------------------------------------------------ weight pack
// Packed layout, in 16-byte lane records:
//   [step = f/32][stream k][tile nt][lane 0..63] -> 8 bf16
// record (step, k, nt, lane) holds split row qs = 16*nt + lane%16 at features
// k*d + 32*step + 8*(lane/16) + 0..7.  Split row qs < 24 is the hi term of
// projection row qs, 24..47 the mid term of row qs-24, 48..71 the lo term of
// row qs-48, 72..79 zero.  One 1 KB (step, k, nt) block is the B operand of one
// 16x16x32 matrix-core instruction.
__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ fn, int d,
                                                   u32x4* __restrict__ out, int records) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= records) return;
  const int lane = idx & 63;
  const int nt = (idx >> 6) % kNT;
  const int k = (idx / (64 * kNT)) % kHC;
  const int step = idx / (64 * kNT * kHC);
  const int qs = nt * 16 + (lane & 15);
  const int part = qs / kMix;  // 0 hi, 1 mid, 2 lo, 3 zero
  const int q = qs % kMix;
  const int f0 = step * kStepF + (lane >> 4) * kFPL;
  u32 w[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float r = 0.f;
      if (part < 3) {
        const float x = fn[(size_t)q * (kHC * d) + (size_t)k * d + f0 + 2 * e2 + h];
        const float hi = round_bf16(x);
        const float r1 = x - hi;  // exact
        const float mid = round_bf16(r1);
        const float r2 = r1 - mid;  // exact
        r = part == 0 ? hi : (part == 1 ? mid : round_bf16(r2));
      }
      v[h] = r;
    }
    w[e2] = pack_bf16(v[0], v[1]);
  }
  out[idx] = u32x4{w[0], w[1], w[2], w[3]};
}

// ================================================================ row kernel
// Streams without the projection: hc_post, hc_pre and the stack exit.  One workgroup = 8 waves x
// TPW tokens; a wave owns whole token rows, a lane 8 consecutive features of
// a 512-feature chunk, so every load and store moves 1 KB of one row.  The
// per-token coefficients are wave-uniform (scalar registers).  With NORM the
// read row stays in registers until its mean square is known.
struct RowArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const float* pre_in;
  const float* gamma;
  hc_bf16* x_out;
  hc_bf16* y_out;
  int64_t n;
  int d;
  float rms_eps;
};

constexpr int kRowChunk = 512;                   // features per wave instruction
constexpr int kRowMaxChunks = 10;                // per token held in registers (NORM)

template <bool POST>
__device__ __forceinline__ void row_load(u32x4 (&r)[kHC + 1], const u32x4* xrow, const u32x4* drow, int d,
                                         int f) {
#pragma unroll
  for (int j = 0; j < kHC; ++j) r[j] = ld_stream(xrow + (j * d + f) / 8);
  r[kHC] = POST ? ld_stream(drow + f / 8) : u32x4{0u, 0u, 0u, 0u};
}

// X'_k = post_k * delta + ((C_0k X_0 + C_1k X_1) + C_2k X_2) + C_3k X_3, one lane's 8 features
__device__ __forceinline__ void post_8(const u32x4 (&r)[kHC + 1], const float* cpost, const float* ccomb,
                                       u32 (&xp)[kHC][4]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float X[kHC][2], D[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < kHC; ++j) X[j][h] = bf_elem(r[j][e2], h);
      D[h] = bf_elem(r[kHC][e2], h);
    }
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float pa = cpost[k] * D[h];
        float sm = ccomb[0 * kHC + k] * X[0][h];
#pragma unroll
        for (int j = 1; j < kHC; ++j) sm = sm + ccomb[j * kHC + k] * X[j][h];
        v[h] = pa + sm;
      }
      xp[k][e2] = pack_bf16(v[0], v[1]);
    }
  }
}

// y = ((p_0 X'_0 + p_1 X'_1) + p_2 X'_2) + p_3 X'_3, one lane's 8 features
__device__ __forceinline__ void pre_8(const u32 (&xp)[kHC][4], const float* cpre, u32 (&yp)[4]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float s = cpre[0] * bf_elem(xp[0][e2], h);
#pragma unroll
      for (int k = 1; k < kHC; ++k) s = s + cpre[k] * bf_elem(xp[k][e2], h);
      v[h] = s;
    }
    yp[e2] = pack_bf16(v[0], v[1]);
  }
}

template <bool POST, bool PRE, bool NORM, int TPW>
__global__ void __launch_bounds__(kThreads) row_kernel(const RowArgs a) {
  static_assert(!NORM || PRE, "RMSNorm needs the read row");
  constexpr int MAXC = kRowMaxChunks * 2 / TPW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d = a.d;
  const int nch = (d + kRowChunk - 1) / kRowChunk;

  int64_t tok[TPW];
  bool tvalid[TPW];
  float cpost[TPW][kHC], ccomb[TPW][kHC * kHC], cpre[TPW][kHC];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = (int64_t)blockIdx.x * (kWaves * TPW) + wave * TPW + i;
    tvalid[i] = t < a.n;
    tok[i] = tvalid[i] ? t : 0;
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
      cpost[i][j] = POST ? a.post_in[tok[i] * kHC + j] : 0.f;
      cpre[i][j] = PRE ? a.pre_in[tok[i] * kHC + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kHC * kHC; ++j) ccomb[i][j] = POST ? a.comb_in[tok[i] * kHC * kHC + j] : 0.f;
  }

  u32 ykeep[NORM ? TPW : 1][NORM ? MAXC : 1][4];
  float ssy[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) ssy[i] = 0.f;

  auto chunk = [&](int c) {
    const int f0 = c * kRowChunk + lane * 8;
    const bool act = f0 < d;
    const int f = act ? f0 : 0;  // idle lanes of a partial chunk read feature 0 and never store
    u32x4 r[TPW][kHC + 1];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      row_load<POST>(r[i], reinterpret_cast<const u32x4*>(a.x + tok[i] * kHC * d),
                     reinterpret_cast<const u32x4*>(POST ? a.delta + tok[i] * d : a.x), d, f);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const bool st = act && tvalid[i];
      u32 xp[kHC][4];
      if constexpr (POST) {
        post_8(r[i], cpost[i], ccomb[i], xp);
        u32x4* xo = reinterpret_cast<u32x4*>(a.x_out + tok[i] * kHC * d);
        if (st) {
#pragma unroll
          for (int k = 0; k < kHC; ++k) st_stream(xo + (k * d + f) / 8, u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
        }
      } else {
#pragma unroll
        for (int k = 0; k < kHC; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) xp[k][e] = r[i][k][e];
      }
      if constexpr (PRE) {
        u32 yp[4];
        pre_8(xp, cpre[i], yp);
        if constexpr (NORM) {
          if (act) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ssy[i] = dot2_bf16(yp[e], yp[e], ssy[i]);
          }
#pragma unroll
          for (int cc = 0; cc < MAXC; ++cc)
            if (cc == c) {
#pragma unroll
              for (int e = 0; e < 4; ++e) ykeep[i][cc][e] = yp[e];
            }
        } else if (st) {
          st_stream(reinterpret_cast<u32x4*>(a.y_out + tok[i] * d) + f / 8, u32x4{yp[0], yp[1], yp[2], yp[3]});
        }
      }
    }
  };

  if constexpr (NORM) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (c < nch) chunk(c);
    // z = gamma * (y * r), r = 1/sqrt(mean y^2 + eps), per token row
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      float s = ssy[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      const float ry = 1.0f / sqrtf(s / (float)d + a.rms_eps);
      u32x4* yo = reinterpret_cast<u32x4*>(a.y_out + tok[i] * d);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int f = c * kRowChunk + lane * 8;
        if (c < nch && f < d && tvalid[i]) {
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + f);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + f + 4);
          const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
          u32 zp[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            zp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(ykeep[i][c][e2]) * ry), gm[2 * e2 + 1] * (bf_hi(ykeep[i][c][e2]) * ry));
          st_stream(yo + f / 8, u32x4{zp[0], zp[1], zp[2], zp[3]});
        }
      }
    }
  } else {
    for (int c = 0; c < nch; ++c) chunk(c);
  }
}

// ====================================================== boundary: two kernels
// Everything that derives mixes (hc_mixes, block entry, sublayer boundary)
// runs as two ordinary launches; the boundary between them is the only
// device-wide synchronisation.
//
// stream_kernel: tokens form tiles of 64 (4 row blocks of 16); the features
// of each stream are cut into S slices of F = d/S (a multiple of 64), S chosen
// so that tiles*S is about one workgroup per compute unit.  One workgroup
// handles one (tile, slice) pair.  Per 64-feature chunk, with waves 2r and
// 2r+1 sharing row block r:
//   stream phase: each wave owns 8 tokens, one per group of 8 lanes, with 8
//     features per lane (128 B per token and instruction).  X' = hc_post(...)
//     is stored and written into the row block's LDS tile in the matrix-core A
//     layout.  With a given pre the read row y is formed and stored as well.
//     The per-token sums the finish needs accumulate in registers: sum x'^2,
//     and for the RMSNorm either sum y^2 (given pre) or the 4x4 Gram matrix of
//     the X' streams (fresh pre: sum y^2 = p^T G p once p is known).
//   barrier; the next chunk's weight tiles (staged through registers) go into
//     the other half of a double-buffered LDS area.
//   matrix phase: each wave of the pair takes one of the chunk's two 32-
//     feature steps: 4 streams x 5 tiles of 16x16x32 bf16 MFMA, A and B from LDS.
// At the end each workgroup writes one record per token of its slice to the
// workspace: 24 projection dots, sum x'^2, the norm sums.
//
// finish_kernel: one workgroup per (tile, read slice).  It sums the tile's
// records over the S slices in slice order (so every workgroup derives
// bit-identical coefficients), derives the mixes, pre/post and the Sinkhorn
// comb with 4 lanes per token (one comb row each; the owner of a token writes
// them), and then writes its part of the read row: from the X' of the stream
// kernel read back with the derived pre (fresh pre), or by rescaling the y it
// stored (given pre with the RMSNorm).
constexpr int kTT = 64;                  // tokens per tile
constexpr int kCF = 64;                  // features per chunk
constexpr int kGram = kHC * (kHC + 1) / 2;   // 10 distinct Gram entries
constexpr int kRec = 36;                 // record: 24 dots, sum x'^2, then sum y^2 or the Gram entries; 9 x 16 B
constexpr int kMaxSlices = 32;           // S is the smallest divisor of d/64 reaching min(256/tiles, this)
constexpr int kFinThreads = 512;

enum ReadMode { kNoRead = 0, kGivenPre = 1, kFreshPre = 2 };

template <int RM, bool NORM>
constexpr int rec_used() { return kMix + 1 + (NORM ? (RM == kFreshPre ? kGram : 1) : 0); }

struct StreamArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const float* pre_in;
  const u32x4* fn;
  hc_bf16* x_out;
  hc_bf16* y_out;
  float* rec;         // [tiles][S][kTT][kRec]
  int64_t n;
  int d, S, F, tiles;
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Slot of A-operand lane L of step st in the LDS A tile.  The 8 lanes that
// write one token's 64 features hold L = 16*g + c (g = 0..3) for both steps:
// unswizzled, their 16-byte slots are 256 B apart, all in one bank group.
// XOR-ing the low 3 bits with (g, st) spreads them over 8 bank groups; per
// (step, stream) block it is a permutation that keeps each aligned group of
// 8 lanes together, so the operand reads stay conflict-free too.
__device__ __forceinline__ int a_swz(int L, int st) { return L ^ (((L >> 4) & 3) | (st << 2)); }

// a store that the finish kernel reads back soon (kept cacheable)
__device__ __forceinline__ void st_keep(u32x4* p, u32x4 v) { *p = v; }

template <bool POST, int RM, bool NORM>
__global__ void __launch_bounds__(kThreads, 1) stream_kernel(const StreamArgs a) {
  static_assert(!NORM || RM != kNoRead, "RMSNorm needs the read row");
  __shared__ u32x4 w_lds[2][2][kHC][kNT][64];          // weight tiles, double buffered (80 KB)
  __shared__ u32x4 a_lds[4][2][kHC][64];               // X' in A layout per row block (32 KB)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave >> 1, hw = wave & 1;   // row block, half (stream phase) / step (matrix phase)
  const int d = a.d, S = a.S, F = a.F;
  const int nch = F / kCF;
  // XCD-aware: consecutive blocks land on different XCDs.  Renumbered so that
  // each XCD holds a contiguous run, then taken slice-major: the workgroups of
  // an XCD share few slices, and so few weight columns in their L2.
  const int lin = (gridDim.x & 7) ? blockIdx.x : (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int slice = lin / a.tiles;
  const int tile = lin % a.tiles;
  const int fs = slice * F;                     // first feature of the slice (per stream)

  const int hl = lane >> 3;                     // token within the wave's 8
  const int fl = (lane & 7) * 8;                // first feature within the chunk
  const int m = rb * 16 + hw * 8 + hl;          // token within the tile
  const int a_st = fl >> 5, a_g = (fl >> 3) & 3;
  const int a_lane = a_g * 16 + hw * 8 + hl;    // A-layout lane of this lane's 8 features
  constexpr int kUsed = rec_used<RM, NORM>();
  constexpr int kQuads = (kUsed + 3) / 4;

  const int64_t t0 = (int64_t)tile * kTT;
  const bool tv = t0 + m < a.n;
  const unsigned lt = tv ? (unsigned)m : 0u;   // tokens past n read the tile's first and never store
  const hc_bf16* xb = a.x + t0 * kHC * d;
  const hc_bf16* db = POST ? a.delta + t0 * d : a.x;
  hc_bf16* xob = POST ? a.x_out + t0 * kHC * d : nullptr;
  hc_bf16* yb = RM == kGivenPre ? a.y_out + t0 * d : nullptr;

  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    cpost[j] = POST ? a.post_in[(t0 + lt) * kHC + j] : 0.f;
    cpre[j] = RM == kGivenPre ? a.pre_in[(t0 + lt) * kHC + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = POST ? a.comb_in[(t0 + lt) * kHC * kHC + j] : 0.f;

  u32x4 cur[kHC + 1];
  u32x4 wst[kNT];  // this wave's share (5 of 40 blocks) of the next chunk's weight tiles
  f32x4 acc[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ssx = 0.f, ssy = 0.f;
  float gram[kGram];
#pragma unroll
  for (int g = 0; g < kGram; ++g) gram[g] = 0.f;

  auto load_wst = [&](int c) {
    const int gstep = (fs + c * kCF) / 32;
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;          // (st, k, nt) = blk / 20, (blk / 5) % 4, blk % 5
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      wst[i] = a.fn[((size_t)((gstep + st) * kHC + k) * kNT + nt) * 64 + lane];
    }
  };
  auto store_wst = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      w_lds[buf][st][k][nt][lane] = wst[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[kHC + 1]) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int j = 0; j < kHC; ++j) dst[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * kHC * d + j * d + f)));
    dst[kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(db + (lt * d + f))) : u32x4{0u, 0u, 0u, 0u};
  };
  auto stream_phase = [&](int c) {
    const unsigned f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    if constexpr (POST) {
      post_8(cur, cpost, ccomb, xp);
      if (tv) {
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
          u32x4* p = reinterpret_cast<u32x4*>(xob + (lt * kHC * d + k * d + f));
          const u32x4 v = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
          if constexpr (RM == kFreshPre) st_keep(p, v); else st_stream(p, v);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kHC; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[k][e] = cur[k][e];
    }
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ssx = dot2_bf16(xp[k][e], xp[k][e], ssx);
      a_lds[rb][a_st][k][a_swz(a_lane, a_st)] = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
    }
    if constexpr (RM == kGivenPre) {
      u32 yp[4];
      pre_8(xp, cpre, yp);
      if constexpr (NORM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ssy = dot2_bf16(yp[e], yp[e], ssy);
      }
      if (tv) {
        u32x4* p = reinterpret_cast<u32x4*>(yb + (lt * d + f));
        const u32x4 v = u32x4{yp[0], yp[1], yp[2], yp[3]};
        if constexpr (NORM) st_keep(p, v); else st_stream(p, v);
      }
    }
    if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int g = 0;
#pragma unroll
        for (int j = 0; j < kHC; ++j)
#pragma unroll
          for (int l = j; l < kHC; ++l, ++g) gram[g] = dot2_bf16(xp[j][e], xp[l][e], gram[g]);
      }
    }
  };
  auto matrix_phase = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, a_lds[rb][hw][k][a_swz(lane, hw)]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            A, __builtin_bit_cast(bf16x8, w_lds[buf][hw][k][nt][lane]), acc[nt], 0, 0, 0);
    }
  };
  // one chunk: its streams are in registers; the next chunk's weights are
  // requested before any compute of this one, its streams before (given pre)
  // or after (fresh pre) the stream phase -- the faster order of each, measured
  auto chunk = [&](int c, bool more) {
    constexpr bool kEarly = RM != kFreshPre;
    u32x4 nxt[kHC + 1];
    if (more) {
      load_wst(c + 1);
      if (kEarly) load_stream(c + 1, nxt);
    }
    stream_phase(c);
    if (more && !kEarly) load_stream(c + 1, nxt);
    lds_barrier();                 // A tiles and chunk c's weights in place; previous matrix phase done
    if (more) store_wst((c + 1) & 1);
    matrix_phase(c & 1);
    lds_barrier();                 // matrix phase done before the A tiles are rewritten
    if (more) {
#pragma unroll
      for (int j = 0; j <= kHC; ++j) cur[j] = nxt[j];
    }
  };

  load_wst(0);
  load_stream(0, cur);
  store_wst(0);
  lds_barrier();
  for (int c = 0; c + 1 < nch; ++c) chunk(c, true);
  chunk(nch - 1, false);

  // ---- per-token records of this slice
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    ssx += __shfl_xor(ssx, o);
    if constexpr (RM == kGivenPre && NORM) ssy += __shfl_xor(ssy, o);
    if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
      for (int g = 0; g < kGram; ++g) gram[g] += __shfl_xor(gram[g], o);
    }
  }
  float* red = reinterpret_cast<float*>(&w_lds[0][0][0][0][0]);   // [4 rb][2 steps][16][80] | extra
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      red[((rb * 2 + hw) * 16 + 4 * (lane >> 4) + rr) * 80 + nt * 16 + (lane & 15)] = acc[nt][rr];
  float* extra = red + 4 * 2 * 16 * 80;                            // [kRec - kMix][kTT]
  if ((lane & 7) == 0) {
    extra[m] = ssx;
    if constexpr (RM == kGivenPre && NORM) extra[kTT + m] = ssy;
    if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
      for (int g = 0; g < kGram; ++g) extra[(1 + g) * kTT + m] = gram[g];
    }
  }
  lds_barrier();
  float* rec = a.rec + ((size_t)tile * S + slice) * kTT * kRec;
  for (int idx = threadIdx.x; idx < kTT * kQuads; idx += kThreads) {
    const int tm = idx / kQuads, q0 = (idx % kQuads) * 4;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + i;
      if (q < kMix) {
        const float* r0 = red + ((tm >> 4) * 2 * 16 + (tm & 15)) * 80;   // step 0
        const float* r1 = r0 + 16 * 80;                                 // step 1
        v[i] = ((r0[q] + r0[kMix + q]) + r0[2 * kMix + q]) + ((r1[q] + r1[kMix + q]) + r1[2 * kMix + q]);
      } else {
        v[i] = q < kUsed ? extra[(q - kMix) * kTT + tm] : 0.f;
      }
    }
    *reinterpret_cast<f32x4*>(rec + tm * kRec + q0) = f32x4{v[0], v[1], v[2], v[3]};
  }
}

struct FinishArgs {
  const float* rec;         // [tiles][S][kTT][kRec] from stream_kernel
  const hc_bf16* src;       // fresh pre: X' (or x at a block entry) [n, hc, d]; given pre: y [n, d]
  hc_bf16* y_out;
  const float* gamma;
  const float* hc_base;
  const float* hc_scale;
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  int64_t n;
  int d, S, S2, F2, tiles, iters;
  float hc_eps, norm_eps, rms_eps;
};

// Sum over the 4 lanes of a token's quad, by lane permutation within the
// quad (no LDS round trip).  Butterfly order: every lane of the quad obtains
// the same bits, (v0 + v1) + (v2 + v3) up to commutation.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_sum(float v) {
  const float u = v + quad_perm<0xB1>(v);      // lanes [1,0,3,2]
  return u + quad_perm<0x4E>(u);               // lanes [2,3,0,1]
}

template <int RM, bool NORM>
__global__ void __launch_bounds__(kFinThreads) finish_kernel(const FinishArgs a) {
  __shared__ float tot[kTT][kRec];          // the tile's records summed over the slices
  __shared__ float s_pre[kTT][kHC];         // derived pre (fresh read)
  __shared__ float s_r[kTT];                // RMSNorm factor of the read row
  __shared__ float g_lds[NORM ? kMaxNormD : 1];   // gamma of the read slice (F2 <= d <= kMaxNormD)
  constexpr int kUsed = rec_used<RM, NORM>();
  constexpr int kQuads = (kUsed + 3) / 4;
  const int tile = blockIdx.x / a.S2, sl2 = blockIdx.x % a.S2;
  const int64_t t0 = (int64_t)tile * kTT;
  const int valid = (int)min<int64_t>(kTT, a.n - t0);
  const int d = a.d, S = a.S;

  if constexpr (NORM) {
    for (int i = threadIdx.x; i < a.F2; i += kFinThreads) g_lds[i] = a.gamma[sl2 * a.F2 + i];
  }
  // ---- sum the tile's records over the slices, in slice order
  const float* rt = a.rec + (size_t)tile * S * kTT * kRec;
  for (int cell = threadIdx.x; cell < valid * kQuads; cell += kFinThreads) {
    const int tm = cell / kQuads, q0 = (cell % kQuads) * 4;
    const float* p = rt + tm * kRec + q0;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    int sl = 0;
    for (; sl + 8 <= S; sl += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(p + (size_t)(sl + u) * kTT * kRec);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; sl < S; ++sl) s += *reinterpret_cast<const f32x4*>(p + (size_t)sl * kTT * kRec);
    *reinterpret_cast<f32x4*>(&tot[tm][q0]) = s;
  }
  __syncthreads();

  // ---- derive: 4 lanes per token, lane j holds comb row j
  if (threadIdx.x < kTT * kHC) {
    const int tm = threadIdx.x >> 2, j = threadIdx.x & 3;
    const int64_t t = t0 + tm;
    const bool own = tm < valid && tm % a.S2 == sl2;
    const float* rec = tot[tm];
    const float rx = 1.0f / sqrtf(rec[kMix] / (float)(kHC * d) + a.norm_eps);
    if (own && a.mixes_out) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(rec + 4 * j);
      *reinterpret_cast<f32x4*>(a.mixes_out + t * kMix + 4 * j) = f32x4{v[0] * rx, v[1] * rx, v[2] * rx, v[3] * rx};
      if (j < 2) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(rec + 16 + 4 * j);
        *reinterpret_cast<f32x4*>(a.mixes_out + t * kMix + 16 + 4 * j) =
            f32x4{w[0] * rx, w[1] * rx, w[2] * rx, w[3] * rx};
      }
    }
    if (a.pre_out) {
      const float s0 = a.hc_scale[0], s1 = a.hc_scale[1], s2 = a.hc_scale[2];
      const float pre = sigmoidf_((rec[j] * rx) * s0 + a.hc_base[j]) + a.hc_eps;
      const float post = 2.0f * sigmoidf_((rec[kHC + j] * rx) * s1 + a.hc_base[kHC + j]);
      float A[kHC];
      float mxr = -INFINITY;
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        const int q = 2 * kHC + j * kHC + k;
        A[k] = (rec[q] * rx) * s2 + a.hc_base[q];
        mxr = fmaxf(mxr, A[k]);
      }
      float rsum = 0.f;
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        A[k] = expf(A[k] - mxr);
        rsum = rsum + A[k];
      }
      const float rinv = __builtin_amdgcn_rcpf(rsum);
#pragma unroll
      for (int k = 0; k < kHC; ++k) A[k] = A[k] * rinv + a.hc_eps;
      auto col_norm = [&]() {
#pragma unroll
        for (int k = 0; k < kHC; ++k) A[k] = A[k] * __builtin_amdgcn_rcpf(quad_sum(A[k]) + a.hc_eps);
      };
      col_norm();
      for (int it = 1; it < a.iters; ++it) {
        const float inv = __builtin_amdgcn_rcpf(((A[0] + A[1]) + A[2]) + A[3] + a.hc_eps);
#pragma unroll
        for (int k = 0; k < kHC; ++k) A[k] = A[k] * inv;
        col_norm();
      }
      if (own) {
        a.pre_out[t * kHC + j] = pre;
        a.post_out[t * kHC + j] = post;
        *reinterpret_cast<f32x4*>(a.comb_out + t * kHC * kHC + j * kHC) = f32x4{A[0], A[1], A[2], A[3]};
      }
      if constexpr (RM == kFreshPre) {
        s_pre[tm][j] = pre;
        if constexpr (NORM) {
          // sum_i y_i^2 = p^T G p over the whole row, G summed over the slices
          double p[kHC];
#pragma unroll
          for (int l = 0; l < kHC; ++l) p[l] = (double)__shfl(pre, (threadIdx.x & ~3) + l);
          double yy = 0.0;
          int g = 0;
#pragma unroll
          for (int l = 0; l < kHC; ++l)
#pragma unroll
            for (int l2 = l; l2 < kHC; ++l2, ++g)
              yy += (l == l2 ? 1.0 : 2.0) * p[l] * p[l2] * (double)rec[kMix + 1 + g];
          if (j == 0) s_r[tm] = 1.0f / sqrtf((float)(yy / (double)d) + a.rms_eps);
        }
      }
    }
    if constexpr (RM == kGivenPre && NORM) {
      if (j == 0) s_r[tm] = 1.0f / sqrtf(rec[kMix + 1] / (float)d + a.rms_eps);
    }
  }

  // ---- this workgroup's slice of the read row
  if constexpr (RM == kFreshPre || (RM == kGivenPre && NORM)) {
    __syncthreads();                 // s_pre, s_r in place
    const int m = threadIdx.x >> 3;              // token of the tile
    const int fl = (threadIdx.x & 7) * 8;        // first feature within the chunk
    const bool tv = m < valid;
    const unsigned lt = tv ? (unsigned)m : 0u;
    const int fs = sl2 * a.F2;
    const int nch = a.F2 / kCF;
    float p[kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) p[j] = RM == kFreshPre ? s_pre[lt][j] : 0.f;
    const float r = NORM ? s_r[lt] : 1.f;
    constexpr int NL = RM == kFreshPre ? kHC : 1;
    const int rstride = RM == kFreshPre ? kHC * d : d;
    const hc_bf16* src = a.src + (t0 + lt) * rstride;
    hc_bf16* yrow = a.y_out + (t0 + lt) * d;
    // chunks in batches of U, all loads of a batch in flight at once, last
    // written first (the most recent stores are the likeliest still cached)
    constexpr int U = RM == kFreshPre ? 5 : 8;
    for (int cb = nch; cb > 0; cb -= U) {
      u32x4 ld[U][NL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb - 1 - u;
        if (c >= 0) {
          const unsigned f = fs + c * kCF + fl;
#pragma unroll
          for (int k = 0; k < NL; ++k) ld[u][k] = ld_stream(reinterpret_cast<const u32x4*>(src + (k * d + f)));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb - 1 - u;
        if (c >= 0) {
          const unsigned f = fs + c * kCF + fl;
          u32 yp[4];
          if constexpr (RM == kFreshPre) {
            u32 xp[kHC][4];
#pragma unroll
            for (int k = 0; k < kHC; ++k)
#pragma unroll
              for (int e = 0; e < 4; ++e) xp[k][e] = ld[u][k][e];
            pre_8(xp, p, yp);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) yp[e] = ld[u][0][e];
          }
          if constexpr (NORM) {
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(g_lds + (f - fs));
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(g_lds + (f - fs) + 4);
            const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              yp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(yp[e2]) * r), gm[2 * e2 + 1] * (bf_hi(yp[e2]) * r));
          }
          if (tv) st_stream(reinterpret_cast<u32x4*>(yrow + f), u32x4{yp[0], yp[1], yp[2], yp[3]});
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side
thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_hd(int hc, int d) {
  if (hc != kHC) return fail(HC_ENOTSUP, "hc=%d: only hc=4 is supported", hc);
  if (d <= 0 || d % kCF != 0 || d > kMaxD)
    return fail(HC_ENOTSUP, "d=%d: d must be a positive multiple of %d, at most %d", d, kCF, kMaxD);
  return HC_OK;
}

#define HC_REQ(ptr)                                                                    \
  do {                                                                                 \
    if (!(ptr)) return fail(HC_EINVAL, "%s must not be NULL", #ptr);                   \
    if (!aligned16(ptr)) return fail(HC_EINVAL, "%s is not 16-byte aligned", #ptr);    \
  } while (0)
#define HC_OPT(ptr)                                                                    \
  do {                                                                                 \
    if ((ptr) && !aligned16(ptr)) return fail(HC_EINVAL, "%s is not 16-byte aligned", #ptr); \
  } while (0)

int check_n(int64_t n) {
  if (n < 0) return fail(HC_EINVAL, "n=%lld is negative", (long long)n);
  if (n > ((int64_t)1 << 31)) return fail(HC_EINVAL, "n=%lld is too large", (long long)n);
  return HC_OK;
}

int check_device() {
  int count = 0;
  const hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0)
    return fail(HC_ENODEV, "no HIP device: %s", e == hipSuccess ? "count is 0" : hipGetErrorName(e));
  return HC_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HC_EHIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return HC_OK;
}

// ---- boundary geometry and workspace
// Stream slices: the smallest divisor S of d/64 with tiles*S >= 256 (one
// workgroup for each of the 256 compute units of an MI355X), capped at
// kMaxSlices for short inputs.  Fixed by (n, d) alone so that the workspace
// size is too.  Read slices of the finish: likewise with tiles*S2 >= 512.
int divisor_at_least(int units, int64_t need) {
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && s >= need) return s;
  return units;
}
int stream_slices(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return divisor_at_least(d / kCF, std::min<int64_t>((256 + tiles - 1) / tiles, kMaxSlices));
}
int read_slices(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return divisor_at_least(d / kCF, std::min<int64_t>((512 + tiles - 1) / tiles, kMaxSlices));
}
size_t workspace_bytes(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return (size_t)tiles * stream_slices(n, d) * kTT * kRec * 4;
}

template <bool POST, int RM, bool NORM>
hipError_t launch_stream_t(const StreamArgs& a, unsigned grid, hipStream_t st) {
  StreamArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_kernel<POST, RM, NORM>), dim3(grid), dim3(kThreads),
                         args, 0, st);
}
template <int RM, bool NORM>
hipError_t launch_finish_t(const FinishArgs& a, unsigned grid, hipStream_t st) {
  FinishArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&finish_kernel<RM, NORM>), dim3(grid), dim3(kFinThreads),
                         args, 0, st);
}

// s: streams, pre_in, x_out/y_out set; f: split parameters and outputs, gamma set.
// phases: bit 0 the stream kernel, bit 1 the finish kernel.
int launch_boundary(bool post, int rm, bool norm, StreamArgs s, FinishArgs f, void* ws, size_t ws_bytes,
                    hipStream_t st, const char* what, int phases = 3) {
  const size_t need = workspace_bytes(s.n, s.d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  const int64_t tiles = (s.n + kTT - 1) / kTT;
  if (tiles * kMaxSlices > INT32_MAX) return fail(HC_ENOTSUP, "%s: n=%lld is too large", what, (long long)s.n);
  s.S = stream_slices(s.n, s.d);
  s.F = s.d / s.S;
  s.tiles = (int)tiles;
  s.rec = static_cast<float*>(ws);
  const unsigned grid1 = (unsigned)(tiles * s.S);
  hipError_t e = hipSuccess;
  if (phases & 1) switch ((post ? 8 : 0) | (rm << 1) | (norm ? 1 : 0)) {
    case 0x0: e = launch_stream_t<false, kNoRead, false>(s, grid1, st); break;
    case 0x2: e = launch_stream_t<false, kGivenPre, false>(s, grid1, st); break;
    case 0x3: e = launch_stream_t<false, kGivenPre, true>(s, grid1, st); break;
    case 0x4: e = launch_stream_t<false, kFreshPre, false>(s, grid1, st); break;
    case 0x5: e = launch_stream_t<false, kFreshPre, true>(s, grid1, st); break;
    case 0xA: e = launch_stream_t<true, kGivenPre, false>(s, grid1, st); break;
    case 0xB: e = launch_stream_t<true, kGivenPre, true>(s, grid1, st); break;
    case 0xC: e = launch_stream_t<true, kFreshPre, false>(s, grid1, st); break;
    case 0xD: e = launch_stream_t<true, kFreshPre, true>(s, grid1, st); break;
    default: return fail(HC_EINVAL, "%s: unsupported stage combination", what);
  }
  int rc = launched(e, what);
  if (rc || !(phases & 2)) return rc;
  const bool read = rm == kFreshPre || (rm == kGivenPre && norm);
  f.rec = s.rec;
  f.n = s.n; f.d = s.d; f.S = s.S; f.tiles = s.tiles;
  f.S2 = read ? read_slices(s.n, s.d) : 1;
  f.F2 = s.d / f.S2;
  f.y_out = s.y_out;
  f.src = rm == kFreshPre ? (post ? s.x_out : s.x) : s.y_out;
  const unsigned grid2 = (unsigned)(tiles * f.S2);
  if (rm == kFreshPre) e = norm ? launch_finish_t<kFreshPre, true>(f, grid2, st) : launch_finish_t<kFreshPre, false>(f, grid2, st);
  else if (rm == kGivenPre && norm) e = launch_finish_t<kGivenPre, true>(f, grid2, st);
  else e = launch_finish_t<kNoRead, false>(f, grid2, st);
  return launched(e, what);
}

template <bool POST, bool PRE, bool NORM, int TPW>
hipError_t launch_row_t(const RowArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.n + kWaves * TPW - 1) / (kWaves * TPW));
  RowArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&row_kernel<POST, PRE, NORM, TPW>), dim3(grid),
                         dim3(kThreads), args, 0, st);
}

int launch_row(bool post, bool pre, bool norm, const RowArgs& a, hipStream_t st, const char* what) {
  const bool wide = norm && a.d > kRowChunk * kRowMaxChunks;
  if (norm && a.d > kRowChunk * kRowMaxChunks * 2)
    return fail(HC_ENOTSUP, "%s: RMSNorm of the read row supports d <= %d", what, kRowChunk * kRowMaxChunks * 2);
  const int key = (post ? 4 : 0) | (pre ? 2 : 0) | (norm ? 1 : 0);
  hipError_t e;
  switch (key) {
    case 0b100: e = launch_row_t<true, false, false, 2>(a, st); break;
    case 0b010: e = launch_row_t<false, true, false, 2>(a, st); break;
    case 0b110: e = launch_row_t<true, true, false, 2>(a, st); break;
    case 0b011: e = wide ? launch_row_t<false, true, true, 1>(a, st) : launch_row_t<false, true, true, 2>(a, st); break;
    case 0b111: e = wide ? launch_row_t<true, true, true, 1>(a, st) : launch_row_t<true, true, true, 2>(a, st); break;
    default: return fail(HC_EINVAL, "%s: unsupported stage combination", what);
  }
  return launched(e, what);
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

int hc_version(void) { return 200; /* 0.2.0 */ }

const char* hc_strerror(int status) {
  switch (status) {
    case HC_OK: return "success";
    case HC_EINVAL: return "invalid argument";
    case HC_ENOTSUP: return "unsupported shape";
    case HC_EHIP: return "HIP error";
    case HC_ENODEV: return "no HIP device";
    default: return "unknown status";
  }
}

const char* hc_last_error(void) { return g_err; }

size_t hc_fn_packed_bytes(int hc, int d) {
  if (hc != kHC || d <= 0 || d % kCF != 0 || d > kMaxD) return 0;
  return (size_t)(d / kStepF) * kHC * kNT * 64 * 16;
}

int hc_fn_pack(const float* hc_fn, int hc, int d, void* fn_packed, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  HC_REQ(hc_fn);
  HC_REQ(fn_packed);
  if ((rc = check_device())) return rc;
  const int records = (d / kStepF) * kHC * kNT * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((records + 255) / 256), dim3(256), 0, (hipStream_t)stream, hc_fn, d,
                     reinterpret_cast<u32x4*>(fn_packed), records);
  return launched(hipGetLastError(), "pack_kernel");
}

size_t hc_workspace_bytes(int64_t n, int hc, int d) {
  if (hc != kHC || d <= 0 || d % kCF != 0 || d > kMaxD || n < 0) return 0;
  if (n == 0) return 0;
  return workspace_bytes(n, d);
}

int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base, int64_t n, int hc,
                      int iters, float hc_eps, float* pre, float* post, float* comb, void* stream) {
  g_err[0] = 0;
  int rc;
  if (hc != kHC) return fail(HC_ENOTSUP, "hc=%d: only hc=4 is supported", hc);
  if ((rc = check_n(n))) return rc;
  if (iters < 1) return fail(HC_EINVAL, "iters=%d: at least one Sinkhorn round is needed", iters);
  HC_REQ(mixes); HC_REQ(hc_scale); HC_REQ(hc_base); HC_REQ(pre); HC_REQ(post); HC_REQ(comb);
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  hipLaunchKernelGGL(split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     mixes, hc_scale, hc_base, n, iters, hc_eps, pre, post, comb);
  return launched(hipGetLastError(), "split_kernel");
}

int hc_mixes(const hc_bf16* x, const void* fn_packed, int64_t n, int hc, int d, float norm_eps, float* mixes,
             const float* hc_scale, const float* hc_base, int iters, float hc_eps, float* pre, float* post,
             float* comb, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(x); HC_REQ(fn_packed); HC_OPT(mixes);
  const bool split = pre || post || comb;
  if (split) {
    HC_REQ(pre); HC_REQ(post); HC_REQ(comb); HC_REQ(hc_scale); HC_REQ(hc_base);
    if (iters < 1) return fail(HC_EINVAL, "iters=%d: at least one Sinkhorn round is needed", iters);
  } else if (!mixes) {
    return fail(HC_EINVAL, "nothing to compute: mixes and pre/post/comb are all NULL");
  }
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  StreamArgs s{};
  s.n = n; s.d = d; s.x = x; s.fn = reinterpret_cast<const u32x4*>(fn_packed);
  FinishArgs f{};
  f.mixes_out = mixes; f.norm_eps = norm_eps; f.hc_scale = hc_scale; f.hc_base = hc_base; f.iters = iters;
  f.hc_eps = hc_eps;
  if (split) { f.pre_out = pre; f.post_out = post; f.comb_out = comb; }
  return launch_boundary(false, kNoRead, false, s, f, workspace, workspace_bytes, (hipStream_t)stream, "hc_mixes");
}

int hc_pre(const hc_bf16* x, const float* pre_mix, int64_t n, int hc, int d, hc_bf16* y, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(x); HC_REQ(pre_mix); HC_REQ(y);
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  RowArgs a{};
  a.n = n; a.d = d; a.x = x; a.pre_in = pre_mix; a.y_out = y;
  return launch_row(false, true, false, a, (hipStream_t)stream, "hc_pre");
}

int hc_post(const hc_bf16* delta, const hc_bf16* x, const float* post, const float* comb, int64_t n, int hc,
            int d, hc_bf16* x_out, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(delta); HC_REQ(x); HC_REQ(post); HC_REQ(comb); HC_REQ(x_out);
  if (x_out == x) return fail(HC_EINVAL, "x_out must not alias x");
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  RowArgs a{};
  a.n = n; a.d = d; a.delta = delta; a.x = x; a.post_in = post; a.comb_in = comb; a.x_out = x_out;
  return launch_row(true, false, false, a, (hipStream_t)stream, "hc_post");
}

size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d) { return hc_workspace_bytes(n, hc, d); }

static int boundary_phases(const hc_boundary_args* p, void* stream, int phases) {
  g_err[0] = 0;
  if (!p) return fail(HC_EINVAL, "args must not be NULL");
  if (p->struct_size < sizeof(hc_boundary_args))
    return fail(HC_EINVAL, "struct_size=%u, expected %zu", p->struct_size, sizeof(hc_boundary_args));
  int rc = check_hd(p->hc, p->d);
  if (rc) return rc;
  if ((rc = check_n(p->n))) return rc;
  const bool post = p->delta != nullptr;
  const bool mix = p->fn_packed != nullptr;
  const bool fresh = p->pre_in == nullptr;
  const bool norm = p->gamma != nullptr;
  HC_REQ(p->x); HC_REQ(p->y_out); HC_OPT(p->delta); HC_OPT(p->pre_in); HC_OPT(p->gamma);
  if (post) { HC_REQ(p->post_in); HC_REQ(p->comb_in); HC_REQ(p->x_out);
    if (p->x_out == p->x) return fail(HC_EINVAL, "x_out must not alias x"); }
  if (mix) {
    HC_REQ(p->fn_packed); HC_REQ(p->hc_base); HC_REQ(p->hc_scale);
    HC_REQ(p->pre_out); HC_REQ(p->post_out); HC_REQ(p->comb_out); HC_OPT(p->mixes_out);
    if (p->iters < 1) return fail(HC_EINVAL, "iters=%d: at least one Sinkhorn round is needed", p->iters);
  }
  if (fresh && !mix) return fail(HC_EINVAL, "pre_in is NULL but no mixes are derived (fn_packed is NULL)");
  if (norm && p->d > kRowChunk * kRowMaxChunks * 2)
    return fail(HC_ENOTSUP, "RMSNorm of the read row supports d <= %d", kRowChunk * kRowMaxChunks * 2);
  if (p->n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  const hipStream_t st = (hipStream_t)stream;

  if (!mix) {  // stack exit: write, read (+ norm); no projection; one kernel, the first phase
    if (!(phases & 1)) return HC_OK;
    RowArgs r{};
    r.n = p->n; r.d = p->d; r.x = p->x; r.delta = p->delta; r.post_in = p->post_in; r.comb_in = p->comb_in;
    r.pre_in = p->pre_in; r.gamma = p->gamma; r.x_out = p->x_out; r.y_out = p->y_out; r.rms_eps = p->rms_eps;
    return launch_row(post, true, norm, r, st, "hc_boundary (exit)");
  }
  StreamArgs s{};
  s.n = p->n; s.d = p->d; s.x = p->x; s.delta = p->delta; s.post_in = p->post_in; s.comb_in = p->comb_in;
  s.pre_in = p->pre_in; s.fn = reinterpret_cast<const u32x4*>(p->fn_packed); s.x_out = p->x_out;
  s.y_out = p->y_out;
  FinishArgs f{};
  f.gamma = p->gamma; f.hc_base = p->hc_base; f.hc_scale = p->hc_scale; f.mixes_out = p->mixes_out;
  f.pre_out = p->pre_out; f.post_out = p->post_out; f.comb_out = p->comb_out; f.iters = p->iters;
  f.hc_eps = p->hc_eps; f.norm_eps = p->norm_eps; f.rms_eps = p->rms_eps;
  return launch_boundary(post, fresh ? kFreshPre : kGivenPre, norm, s, f, p->workspace, p->workspace_bytes, st,
                         "hc_boundary", phases);
}

int hc_boundary(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 3); }
int hc_boundary_begin(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 1); }
int hc_boundary_end(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 2); }

}  // extern "C"
