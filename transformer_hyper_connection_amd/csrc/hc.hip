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
//   split_kernel_tiles<POST, PRE, NORM>  everything that derives mixes (hc_mixes,
//       block entry, sublayer boundary): 64-token tiles x feature slices, the
//       24-wide projection on the matrix cores with the weight tiles shared
//       through LDS, per-slice partials met in a workspace (see below).
//   row_kernel<POST, PRE, NORM, TPW>     streams only (hc_post, hc_pre, stack
//       exit, the read of a boundary that uses the pre it derives): whole token
//       rows per wave, 1 KB per load or store.
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
constexpr int kTM = 16;                // tokens per workgroup tile
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
// Streams without the projection: hc_post, hc_pre, the stack exit and the
// read of a boundary that uses the pre it derives.  One workgroup = 8 waves x
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

// ============================================================== split kernel
// Everything that derives mixes.  The tokens form tiles of 64 (4 row blocks of
// 16); the features of each stream are cut into S slices of F = d/S (a
// multiple of 64); one workgroup handles one (tile, slice) pair and loops over
// the tiles of its slice (grid <= number of CUs, all resident).  Waves 2r and
// 2r+1 share row block r: in the stream phase each owns 8 of its tokens (one
// per lane group of 8 lanes, 8 features per lane, 128 B per token and
// instruction); in the matrix phase each takes one of the chunk's two 32-
// feature steps.  Per 64-feature chunk:
//   stream phase: X' (and y) for the wave's 8 tokens; X' is stored and also
//     written into the row block's LDS tile in the matrix-core A layout;
//   barrier;  the weight tiles of the next chunk (staged through registers)
//     go into the other half of a double-buffered LDS area;
//   matrix phase: 4 streams x 5 tiles of 16x16x32 bf16 MFMA, A and B from LDS.
// After the slice: per-token partials (24 dots, sum x'^2, sum y^2) go to the
// workspace; the S workgroups of a tile meet at a counter; the owner of each
// token reduces its partials in slice order, derives the mixes and runs the
// split/Sinkhorn; every workgroup reads the row sums of squares it needs and
// rescales its slice of the read row, parked in LDS (NORM).
constexpr int kTT = 64;                  // tokens per tile
constexpr int kCF = 64;                  // features per chunk
constexpr int kMaxSliceY = 320;          // features per slice when the read row is parked in LDS
constexpr int kPartials = kMix + 2;      // per token per slice: 24 dots, sum x'^2, sum y^2
constexpr int kRec = 28;                 // partial record, padded to 7 x 16 B
constexpr size_t kWeightStageBytes = 2 * 2 * 4 * 5 * 64 * 16;   // LDS weight staging, reused by the finish
constexpr unsigned kSpinLimit = 1u << 23;

struct SplitArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const float* pre_in;
  const u32x4* fn;
  const float* hc_base;
  const float* hc_scale;
  const float* gamma;
  hc_bf16* x_out;
  hc_bf16* y_out;
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  unsigned* ws_err;   // sticky error word
  unsigned* ws_cnt;   // [tiles] arrivals
  unsigned* ws_done;  // [tiles] departures
  float* ws_part;     // [tiles][S][kTT][kRec]
  int64_t n;
  int d, S, F, tiles, iters;
  float hc_eps, norm_eps, rms_eps;
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroups of a tile meet through the workspace using device-coherent
// accesses only (buffer loads/stores with the system-coherence cache policy,
// relaxed device-scope atomics for the counters), so no cache-wide write-back
// or invalidation -- which a device-scope fence issues on this multi-L2
// part -- is needed.  A writer waits for its stores to complete before its
// workgroup raises the arrival counter; a reader issues its loads only after
// the counter has been seen complete.  The buffer descriptor also bounds
// every access to the workspace.
constexpr int kCoherent = 16;            // cache-policy bit: coherent at device scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(float* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void wait_vm_stores() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every vector memory operation of this wave completed
}

template <bool POST, bool PRE, bool NORM>
__global__ void __launch_bounds__(kThreads, 1) split_kernel_tiles(const SplitArgs a) {
  static_assert(!NORM || PRE, "RMSNorm needs the read row");
  __shared__ u32x4 w_lds[2][2][kHC][kNT][64];          // weight tiles, double buffered (80 KB)
  static_assert(sizeof(w_lds) == kWeightStageBytes, "LDS staging size");
  __shared__ u32x4 a_lds[4][2][kHC][64];               // X' in A layout per row block (32 KB)
  __shared__ u32x4 y_lds[NORM ? kTT : 1][kMaxSliceY / 8];  // read row of the slice (40 KB)
  __shared__ float s_ry[kTT];
  __shared__ float g_lds[NORM ? kMaxSliceY : 1];        // gamma of the slice

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave >> 1, hw = wave & 1;   // row block, half (stream phase) / step (matrix phase)
  const int d = a.d, S = a.S, F = a.F;
  const int nch = F / kCF;
  const int groups = gridDim.x / S;
  // XCD-aware: consecutive blocks land on different XCDs; the S blocks of a
  // tile group are taken 8 apart so that they share one XCD (and its L2)
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int lin = (gridDim.x & 7) ? blockIdx.x : xcd * (gridDim.x >> 3) + jx;
  const int slice = lin % S;
  const int group = lin / S;
  const int fs = slice * F;                     // first feature of the slice (per stream)

  const int hl = lane >> 3;                     // token within the wave's 8
  const int fl = (lane & 7) * 8;                // first feature within the chunk
  const int m = rb * 16 + hw * 8 + hl;          // token within the tile
  const int a_st = fl >> 5, a_g = (fl >> 3) & 3;
  const int a_lane = a_g * 16 + hw * 8 + hl;    // A-layout lane of this lane's 8 features
  if constexpr (NORM) {
    for (int i = threadIdx.x; i < F; i += kThreads) g_lds[i] = a.gamma[fs + i];
  }
  const unsigned tile_bytes = (unsigned)S * kTT * kRec * 4;   // one tile's partials

  for (int tile = group; tile < a.tiles; tile += groups) {
    const int64_t t0 = (int64_t)tile * kTT;
    const bool tv = t0 + m < a.n;
    const unsigned lt = tv ? (unsigned)m : 0u;   // tokens past n read the tile's first and never store
    const hc_bf16* xb = a.x + t0 * kHC * d;
    const hc_bf16* db = POST ? a.delta + t0 * d : a.x;
    hc_bf16* xob = POST ? a.x_out + t0 * kHC * d : nullptr;
    hc_bf16* yb = PRE ? a.y_out + t0 * d : nullptr;

    float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
      cpost[j] = POST ? a.post_in[(t0 + lt) * kHC + j] : 0.f;
      cpre[j] = PRE ? a.pre_in[(t0 + lt) * kHC + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = POST ? a.comb_in[(t0 + lt) * kHC * kHC + j] : 0.f;

    u32x4 cur[kHC + 1];
    u32x4 wst[kNT];  // this wave's share (5 of 40 blocks) of the next chunk's weight tiles
    f32x4 acc[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ssx = 0.f, ssy = 0.f;

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
    auto load_stream = [&](int c) {
      const unsigned f = fs + c * kCF + fl;
#pragma unroll
      for (int j = 0; j < kHC; ++j) cur[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * kHC * d + j * d + f)));
      cur[kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(db + (lt * d + f))) : u32x4{0u, 0u, 0u, 0u};
    };
    auto stream_phase = [&](int c) {
      const unsigned f = fs + c * kCF + fl;
      u32 xp[kHC][4];
      if constexpr (POST) {
        post_8(cur, cpost, ccomb, xp);
        if (tv) {
#pragma unroll
          for (int k = 0; k < kHC; ++k)
            st_stream(reinterpret_cast<u32x4*>(xob + (lt * kHC * d + k * d + f)),
                      u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
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
        a_lds[rb][a_st][k][a_lane] = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
      }
      if constexpr (PRE) {
        u32 yp[4];
        pre_8(xp, cpre, yp);
        if constexpr (NORM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ssy = dot2_bf16(yp[e], yp[e], ssy);
          y_lds[m][(c * kCF + fl) / 8] = u32x4{yp[0], yp[1], yp[2], yp[3]};
        } else if (tv) {
          st_stream(reinterpret_cast<u32x4*>(yb + (lt * d + f)), u32x4{yp[0], yp[1], yp[2], yp[3]});
        }
      }
    };
    auto matrix_phase = [&](int buf) {
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, a_lds[rb][hw][k][lane]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(bf16x8, w_lds[buf][hw][k][nt][lane]), acc[nt], 0, 0, 0);
      }
    };
    // one chunk: its streams are in registers; the next chunk's weights (then
    // streams) are requested before any compute of this one
    auto chunk = [&](int c, bool more) {
      if (more) load_wst(c + 1);
      stream_phase(c);
      if (more) load_stream(c + 1);
      lds_barrier();                 // A tiles and chunk c's weights in place; previous matrix phase done
      if (more) store_wst((c + 1) & 1);
      matrix_phase(c & 1);
      lds_barrier();                 // matrix phase done before the A tiles are rewritten
    };

    load_wst(0);
    load_stream(0);
    store_wst(0);
    lds_barrier();
    for (int c = 0; c + 1 < nch; ++c) chunk(c, true);
    chunk(nch - 1, false);

    // ---- per-token partials of this slice
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      ssx += __shfl_xor(ssx, o);
      ssy += __shfl_xor(ssy, o);
    }
    float* red = reinterpret_cast<float*>(&w_lds[0][0][0][0][0]);   // [4 rb][2 steps][16][80] | sums
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        red[((rb * 2 + hw) * 16 + 4 * (lane >> 4) + rr) * 80 + nt * 16 + (lane & 15)] = acc[nt][rr];
    float* sums = red + 4 * 2 * 16 * 80;                             // [2][kTT]
    if ((lane & 7) == 0) {
      sums[m] = ssx;
      sums[kTT + m] = ssy;
    }
    lds_barrier();
    float* tpw = a.ws_part + (size_t)tile * S * kTT * kRec;
    const __amdgpu_buffer_rsrc_t rs = ws_rsrc(tpw, tile_bytes);
    for (int idx = threadIdx.x; idx < kTT * (kRec / 4); idx += kThreads) {
      const int tm = idx / (kRec / 4), q0 = (idx % (kRec / 4)) * 4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + i;
        if (q < kMix) {
          const float* r0 = red + ((tm >> 4) * 2 * 16 + (tm & 15)) * 80;   // step 0
          const float* r1 = r0 + 16 * 80;                                 // step 1
          v[i] = ((r0[q] + r0[kMix + q]) + r0[2 * kMix + q]) + ((r1[q] + r1[kMix + q]) + r1[2 * kMix + q]);
        } else {
          v[i] = q < kPartials ? sums[(q - kMix) * kTT + tm] : 0.f;
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(f32x4{v[0], v[1], v[2], v[3]}, rs,
                                             ((slice * kTT + tm) * kRec + q0) * 4, 0, kCoherent);
    }
    wait_vm_stores();
    lds_barrier();
    // ---- meet the other slices of this tile
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(a.ws_cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned it = 0;
      while (__hip_atomic_load(a.ws_cnt + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)S) {
        __builtin_amdgcn_s_sleep(2);
        if (++it == kSpinLimit) {
          __hip_atomic_fetch_or(a.ws_err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    lds_barrier();
    // gather what this workgroup needs, all loads in flight at once:
    // the owned tokens' records from every slice, and every token's sum of y^2
    const int own = (kTT + S - 1) / S;            // tokens owned by this slice
    float* g_own = red;                           // [own][S][kRec]
    float* g_yy = red + own * S * kRec;           // [kTT][S]
    for (int i = threadIdx.x; i < own * S; i += kThreads) {
      const int o = i / S, sl = i % S;
      const int tm = min(slice * own + o, kTT - 1);
#pragma unroll
      for (int g4 = 0; g4 < kRec / 4; ++g4) {
        const f32x4 v = (f32x4)__builtin_amdgcn_raw_buffer_load_b128(rs, ((sl * kTT + tm) * kRec + g4 * 4) * 4, 0, kCoherent);
        *reinterpret_cast<f32x4*>(g_own + i * kRec + g4 * 4) = v;
      }
    }
    if constexpr (NORM) {
      for (int i = threadIdx.x; i < kTT * S; i += kThreads) {
        const int tm = i / S, sl = i % S;
        g_yy[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((sl * kTT + tm) * kRec + kMix + 1) * 4, 0, kCoherent));
      }
    }
    lds_barrier();
    if constexpr (NORM) {
      if (threadIdx.x < kTT) {
        float sy = 0.f;
        for (int sl = 0; sl < S; ++sl) sy += g_yy[threadIdx.x * S + sl];
        s_ry[threadIdx.x] = 1.0f / sqrtf(sy / (float)d + a.rms_eps);
      }
    }
    // owned tokens: mixes and the split/Sinkhorn, one token per lane of wave 0
    if (wave == 0 && lane < own) {
      const int tm = slice * own + lane;
      const int64_t t = t0 + tm;
      if (tm < kTT && t < a.n) {
        float dot[kMix];
#pragma unroll
        for (int q = 0; q < kMix; ++q) dot[q] = 0.f;
        float sx = 0.f;
        for (int sl = 0; sl < S; ++sl) {
          const float* pp = g_own + (lane * S + sl) * kRec;
#pragma unroll
          for (int q = 0; q < kMix; ++q) dot[q] += pp[q];
          sx += pp[kMix];
        }
        const float rx = 1.0f / sqrtf(sx / (float)(kHC * d) + a.norm_eps);
        float mx[kMix];
#pragma unroll
        for (int q = 0; q < kMix; ++q) mx[q] = dot[q] * rx;
        if (a.mixes_out) {
#pragma unroll
          for (int q = 0; q < kMix; q += 4)
            *reinterpret_cast<f32x4*>(a.mixes_out + t * kMix + q) = f32x4{mx[q], mx[q + 1], mx[q + 2], mx[q + 3]};
        }
        if (a.pre_out) {
          float bs[kMix];
#pragma unroll
          for (int q = 0; q < kMix; ++q) bs[q] = a.hc_base[q];
          split_sinkhorn_one(mx, a.hc_scale[0], a.hc_scale[1], a.hc_scale[2], bs, a.iters, a.hc_eps,
                             a.pre_out + t * kHC, a.post_out + t * kHC, a.comb_out + t * kHC * kHC);
        }
      }
    }
    if constexpr (NORM) lds_barrier();   // s_ry visible
    // ---- rescale the parked read row: z = gamma * (y * r)  (NORM)
    if constexpr (NORM) {
      if (tv) {
        const float ry = s_ry[m];
        for (int c = 0; c < nch; ++c) {
          const unsigned f = fs + c * kCF + fl;
          const u32x4 yv = y_lds[m][(c * kCF + fl) / 8];
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(g_lds + c * kCF + fl);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(g_lds + c * kCF + fl + 4);
          const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
          u32 zp[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            zp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(yv[e2]) * ry), gm[2 * e2 + 1] * (bf_hi(yv[e2]) * ry));
          st_stream(reinterpret_cast<u32x4*>(yb + (lt * d + f)), u32x4{zp[0], zp[1], zp[2], zp[3]});
        }
      }
    }
    lds_barrier();                   // all reads of the tile's partials, s_ry and y_lds done
    if (threadIdx.x == 0) {
      const unsigned prev = __hip_atomic_fetch_add(a.ws_done + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (unsigned)S - 1) {   // last one out leaves the counters zeroed for the next call
        __hip_atomic_store(a.ws_cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.ws_done + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

int check_device(int* ncu) {
  int count = 0, dev = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0)
    return fail(HC_ENODEV, "no HIP device: %s", e == hipSuccess ? "count is 0" : hipGetErrorName(e));
  if (ncu) {
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return fail(HC_EHIP, "device query failed: %s", hipGetErrorName(e));
  }
  return HC_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HC_EHIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return HC_OK;
}

// ---- split kernel geometry and workspace
// Slices per stream: the smallest divisor S of d/64 with F = d/S <= 320 (the
// read row of a slice fits the registers) and tiles*S >= 256 (enough
// workgroups for the 256 compute units of an MI355X).  Fixed by (n, d) alone
// so that the workspace size is too.
int split_slices(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  const int units = d / kCF;
  const int64_t need = std::max<int64_t>((d + kMaxSliceY - 1) / kMaxSliceY, (256 + tiles - 1) / tiles);
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && s >= need) return s;
  return units;
}

struct WsLayout {
  size_t err, cnt, done, part, total;
};

WsLayout ws_layout(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  const int S = split_slices(n, d);
  WsLayout w;
  w.err = 0;
  w.cnt = 256;
  w.done = w.cnt + ((size_t)tiles * 4 + 255) / 256 * 256;
  w.part = w.done + ((size_t)tiles * 4 + 255) / 256 * 256;
  w.total = w.part + (size_t)tiles * S * kTT * kRec * 4;
  return w;
}

template <bool POST, bool PRE, bool NORM>
hipError_t launch_split_t(const SplitArgs& a, int grid, hipStream_t st) {
  SplitArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&split_kernel_tiles<POST, PRE, NORM>),
                                    dim3(grid), dim3(kThreads), args, 0, st);
}

int launch_split(bool post, bool pre, bool norm, SplitArgs a, void* ws, size_t ws_bytes, int ncu,
                 hipStream_t st, const char* what) {
  const WsLayout L = ws_layout(a.n, a.d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, L.total);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < L.total) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, L.total);
  a.S = split_slices(a.n, a.d);
  a.F = a.d / a.S;
  a.tiles = (int)((a.n + kTT - 1) / kTT);
  char* base = static_cast<char*>(ws);
  a.ws_err = reinterpret_cast<unsigned*>(base + L.err);
  a.ws_cnt = reinterpret_cast<unsigned*>(base + L.cnt);
  a.ws_done = reinterpret_cast<unsigned*>(base + L.done);
  a.ws_part = reinterpret_cast<float*>(base + L.part);
  {  // the finish gathers the owned tokens' records (and, with RMSNorm, every token's
     // sum of y^2) into the weight staging area of LDS
    const int own = (kTT + a.S - 1) / a.S;
    const size_t gather = ((size_t)own * a.S * kRec + (norm ? (size_t)kTT * a.S : 0)) * 4;
    if (gather > kWeightStageBytes)
      return fail(HC_ENOTSUP, "%s: d=%d needs %zu bytes of LDS for the slice exchange (limit %zu)", what, a.d,
                  gather, kWeightStageBytes);
  }
  const int64_t total = (int64_t)a.tiles * a.S;
  int64_t cap = (int64_t)(ncu / a.S) * a.S;
  if (cap < a.S) return fail(HC_ENOTSUP, "%s: %d slices need as many resident workgroups, device has %d", what, a.S, ncu);
  const int grid = (int)std::min<int64_t>(total, cap);
  const int key = (post ? 4 : 0) | (pre ? 2 : 0) | (norm ? 1 : 0);
  hipError_t e;
  switch (key) {
    case 0b000: e = launch_split_t<false, false, false>(a, grid, st); break;
    case 0b100: e = launch_split_t<true, false, false>(a, grid, st); break;
    case 0b010: e = launch_split_t<false, true, false>(a, grid, st); break;
    case 0b011: e = launch_split_t<false, true, true>(a, grid, st); break;
    case 0b110: e = launch_split_t<true, true, false>(a, grid, st); break;
    case 0b111: e = launch_split_t<true, true, true>(a, grid, st); break;
    default: return fail(HC_EINVAL, "%s: unsupported stage combination", what);
  }
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
  if ((rc = check_device(nullptr))) return rc;
  const int records = (d / kStepF) * kHC * kNT * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((records + 255) / 256), dim3(256), 0, (hipStream_t)stream, hc_fn, d,
                     reinterpret_cast<u32x4*>(fn_packed), records);
  return launched(hipGetLastError(), "pack_kernel");
}

size_t hc_workspace_bytes(int64_t n, int hc, int d) {
  if (hc != kHC || d <= 0 || d % kCF != 0 || d > kMaxD || n < 0) return 0;
  if (n == 0) return 0;
  return ws_layout(n, d).total;
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
  if ((rc = check_device(nullptr))) return rc;
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
  int ncu = 0;
  if ((rc = check_device(&ncu))) return rc;
  SplitArgs a{};
  a.n = n; a.d = d; a.x = x; a.fn = reinterpret_cast<const u32x4*>(fn_packed); a.mixes_out = mixes;
  a.norm_eps = norm_eps; a.hc_scale = hc_scale; a.hc_base = hc_base; a.iters = iters; a.hc_eps = hc_eps;
  if (split) { a.pre_out = pre; a.post_out = post; a.comb_out = comb; }
  return launch_split(false, false, false, a, workspace, workspace_bytes, ncu, (hipStream_t)stream, "hc_mixes");
}

int hc_pre(const hc_bf16* x, const float* pre_mix, int64_t n, int hc, int d, hc_bf16* y, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(x); HC_REQ(pre_mix); HC_REQ(y);
  if (n == 0) return HC_OK;
  if ((rc = check_device(nullptr))) return rc;
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
  if ((rc = check_device(nullptr))) return rc;
  RowArgs a{};
  a.n = n; a.d = d; a.delta = delta; a.x = x; a.post_in = post; a.comb_in = comb; a.x_out = x_out;
  return launch_row(true, false, false, a, (hipStream_t)stream, "hc_post");
}

size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d) { return hc_workspace_bytes(n, hc, d); }

int hc_boundary(const hc_boundary_args* p, void* stream) {
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
  int ncu = 0;
  if ((rc = check_device(&ncu))) return rc;
  const hipStream_t st = (hipStream_t)stream;

  if (!mix) {  // stack exit: write, read (+ norm); no projection
    RowArgs r{};
    r.n = p->n; r.d = p->d; r.x = p->x; r.delta = p->delta; r.post_in = p->post_in; r.comb_in = p->comb_in;
    r.pre_in = p->pre_in; r.gamma = p->gamma; r.x_out = p->x_out; r.y_out = p->y_out; r.rms_eps = p->rms_eps;
    return launch_row(post, true, norm, r, st, "hc_boundary (exit)");
  }
  SplitArgs a{};
  a.n = p->n; a.d = p->d; a.x = p->x; a.delta = p->delta; a.post_in = p->post_in; a.comb_in = p->comb_in;
  a.pre_in = p->pre_in; a.fn = reinterpret_cast<const u32x4*>(p->fn_packed); a.hc_base = p->hc_base;
  a.hc_scale = p->hc_scale; a.gamma = p->gamma; a.x_out = p->x_out; a.y_out = p->y_out;
  a.mixes_out = p->mixes_out; a.pre_out = p->pre_out; a.post_out = p->post_out; a.comb_out = p->comb_out;
  a.iters = p->iters; a.hc_eps = p->hc_eps; a.norm_eps = p->norm_eps; a.rms_eps = p->rms_eps;
  if (!fresh) return launch_split(post, true, norm, a, p->workspace, p->workspace_bytes, ncu, st, "hc_boundary");
  // Read with the pre derived in this call: derive (and write), then read.
  SplitArgs a1 = a;
  a1.pre_in = nullptr; a1.y_out = nullptr; a1.gamma = nullptr;
  if ((rc = launch_split(post, false, false, a1, p->workspace, p->workspace_bytes, ncu, st, "hc_boundary (derive)")))
    return rc;
  RowArgs r{};
  r.n = p->n; r.d = p->d; r.x = post ? p->x_out : p->x; r.pre_in = p->pre_out; r.gamma = p->gamma;
  r.y_out = p->y_out; r.rms_eps = p->rms_eps;
  return launch_row(false, true, norm, r, st, "hc_boundary (read)");
}

}  // extern "C"
