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
//   tile_kernel<POST, MIX, PRE, NORM>  one workgroup = 16 tokens x all features.
//       8 waves; each wave walks feature steps of 64 (16 per lane) over the 4
//       streams.  POST: X' = hc_post(...) and store; MIX: sum of squares and the
//       24-wide projection on the matrix cores; PRE: y = hc_pre(X', pre_in);
//       NORM: y kept in registers until the row's mean square is known, then
//       RMS-normalised.  Epilogue: cross-wave reduction in LDS, then the
//       split/Sinkhorn of each token in registers.
//   split_kernel    hc_split_sinkhorn, one token per lane.
//   pack_kernel     fp32 projection weight -> bf16 hi/mid/lo terms in tile order.
#include <hip/hip_runtime.h>

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
constexpr int kFPL = 16;               // features per lane per step
constexpr int kStepF = 4 * kFPL;       // features per step (4 lane groups)
constexpr int kMaxD = 5120;
constexpr int kMaxSPW = kMaxD / (kStepF * kWaves);  // steps per wave at the largest d

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
// Packed layout, in 32-byte lane records:
//   [step = f/64][stream k][tile nt][lane 0..63] -> 16 bf16
// record (step, k, nt, lane) holds split row qs = 16*nt + lane%16 at features
// k*d + 64*step + 16*(lane/16) + 0..15.  Split row qs < 24 is the hi term of
// projection row qs, 24..47 the mid term of row qs-24, 48..71 the lo term of
// row qs-48, 72..79 zero.  One record is one lane's B operand for two
// 16x16x32 matrix-core steps.
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
  u32 w[8];
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) {
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
  out[2 * (size_t)idx] = u32x4{w[0], w[1], w[2], w[3]};
  out[2 * (size_t)idx + 1] = u32x4{w[4], w[5], w[6], w[7]};
}

// ------------------------------------------------------------------- tile kernel
struct TileArgs {
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
  int64_t n;
  int d;
  int iters;
  float hc_eps, norm_eps, rms_eps;
};

template <bool POST, bool MIX, bool PRE, bool NORM>
__global__ void __launch_bounds__(kThreads, 1) tile_kernel(const TileArgs a) {
  static_assert(!NORM || PRE, "RMSNorm needs the read row");
  __shared__ float s_mix[kWaves][kTM][kNT * 16];
  __shared__ float s_ssx[kWaves][kTM];
  __shared__ float s_ssy[kWaves][kTM];
  __shared__ float s_rx[kTM];
  __shared__ float s_ry[kTM];
  __shared__ float s_mixes[kTM][kMix];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;  // token within the tile
  const int g = lane >> 4;  // lane group: features [16g, 16g+16) of each step
  const int64_t t = (int64_t)blockIdx.x * kTM + m;
  const bool valid = t < a.n;
  const int d = a.d;
  const int nsteps = d / kStepF;

  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) cpost[j] = cpre[j] = 0.f;
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = 0.f;
  if (valid) {
    if constexpr (POST) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(a.post_in + t * kHC);
#pragma unroll
      for (int j = 0; j < kHC; ++j) cpost[j] = p[j];
#pragma unroll
      for (int j = 0; j < kHC; ++j) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(a.comb_in + t * kHC * kHC + j * kHC);
#pragma unroll
        for (int k = 0; k < kHC; ++k) ccomb[j * kHC + k] = c[k];
      }
    }
    if constexpr (PRE) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(a.pre_in + t * kHC);
#pragma unroll
      for (int j = 0; j < kHC; ++j) cpre[j] = p[j];
    }
  }

  const int64_t tc = valid ? t : 0;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + tc * kHC * d);
  const u32x4* drow = reinterpret_cast<const u32x4*>(POST ? a.delta + tc * d : a.x);
  u32x4* xorow = reinterpret_cast<u32x4*>(POST ? a.x_out + tc * kHC * d : nullptr);
  u32x4* yrow = reinterpret_cast<u32x4*>(PRE ? a.y_out + tc * d : nullptr);

  f32x4 acc[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ssx = 0.f, ssy = 0.f;
  u32 ykeep[NORM ? kMaxSPW : 1][8];

#pragma unroll
  for (int s = 0; s < kMaxSPW; ++s) {
    const int step = wave + s * kWaves;
    if (step >= nsteps) break;
    const int f = step * kStepF + g * kFPL;  // first feature of this lane
    u32x4 xr[kHC][2], dr[2];
    if (valid) {
#pragma unroll
      for (int j = 0; j < kHC; ++j) {
        xr[j][0] = ld_stream(xrow + (j * d + f) / 8);
        xr[j][1] = ld_stream(xrow + (j * d + f) / 8 + 1);
      }
      if constexpr (POST) {
        dr[0] = ld_stream(drow + f / 8);
        dr[1] = ld_stream(drow + f / 8 + 1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHC; ++j) xr[j][0] = xr[j][1] = u32x4{0u, 0u, 0u, 0u};
      dr[0] = dr[1] = u32x4{0u, 0u, 0u, 0u};
    }

    float yacc[kFPL];
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      u32 xp[8];
      if constexpr (POST) {
        // X'_k = post_k * delta + ((C_0k X_0 + C_1k X_1) + C_2k X_2) + C_3k X_3
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          float v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float dv = bf_elem(dr[e2 >> 2][e2 & 3], h);
            const float pa = cpost[k] * dv;
            float sm = ccomb[0 * kHC + k] * bf_elem(xr[0][e2 >> 2][e2 & 3], h);
#pragma unroll
            for (int j = 1; j < kHC; ++j) sm = sm + ccomb[j * kHC + k] * bf_elem(xr[j][e2 >> 2][e2 & 3], h);
            v[h] = pa + sm;
          }
          xp[e2] = pack_bf16(v[0], v[1]);
        }
        if (valid) {
          st_stream(xorow + (k * d + f) / 8, u32x4{xp[0], xp[1], xp[2], xp[3]});
          st_stream(xorow + (k * d + f) / 8 + 1, u32x4{xp[4], xp[5], xp[6], xp[7]});
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xp[e] = xr[k][0][e];
          xp[4 + e] = xr[k][1][e];
        }
      }
      if constexpr (MIX) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) ssx = dot2_bf16(xp[e2], xp[e2], ssx);
        const bf16x8 A0 = as_bf16x8(xp[0], xp[1], xp[2], xp[3]);
        const bf16x8 A1 = as_bf16x8(xp[4], xp[5], xp[6], xp[7]);
        const u32x4* wp = a.fn + ((size_t)(step * kHC + k) * kNT) * 128 + lane * 2;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const u32x4 b0 = wp[nt * 128];
          const u32x4 b1 = wp[nt * 128 + 1];
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8, b0), acc[nt], 0,
                                                            0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8, b1), acc[nt], 0,
                                                            0, 0);
        }
      }
      if constexpr (PRE) {
        // y = ((p_0 X'_0 + p_1 X'_1) + p_2 X'_2) + p_3 X'_3
#pragma unroll
        for (int e = 0; e < kFPL; ++e) {
          const float pv = cpre[k] * bf_elem(xp[e >> 1], e & 1);
          yacc[e] = (k == 0) ? pv : yacc[e] + pv;
        }
      }
    }
    if constexpr (PRE) {
      u32 yp[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) yp[e2] = pack_bf16(yacc[2 * e2], yacc[2 * e2 + 1]);
      if constexpr (NORM) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          ssy = dot2_bf16(yp[e2], yp[e2], ssy);
          ykeep[s][e2] = yp[e2];
        }
      } else if (valid) {
        st_stream(yrow + f / 8, u32x4{yp[0], yp[1], yp[2], yp[3]});
        st_stream(yrow + f / 8 + 1, u32x4{yp[4], yp[5], yp[6], yp[7]});
      }
    }
  }

  if constexpr (!(MIX || NORM)) return;

  // ---- cross-lane and cross-wave reductions
  if constexpr (MIX) {
    ssx += __shfl_xor(ssx, 16);
    ssx += __shfl_xor(ssx, 32);
    if (g == 0) s_ssx[wave][m] = ssx;
    // C layout of the 16x16 tile: lane holds rows 4g..4g+3 (tokens), column m
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_mix[wave][4 * g + r][nt * 16 + m] = acc[nt][r];
  }
  if constexpr (NORM) {
    ssy += __shfl_xor(ssy, 16);
    ssy += __shfl_xor(ssy, 32);
    if (g == 0) s_ssy[wave][m] = ssy;
  }
  __syncthreads();
  if (threadIdx.x < kTM) {
    const int tok = threadIdx.x;
    if constexpr (MIX) {
      float sx = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sx += s_ssx[w][tok];
      s_rx[tok] = 1.0f / sqrtf(sx / (float)(kHC * d) + a.norm_eps);
    }
    if constexpr (NORM) {
      float sy = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sy += s_ssy[w][tok];
      s_ry[tok] = 1.0f / sqrtf(sy / (float)d + a.rms_eps);
    }
  }
  if constexpr (MIX) {
    for (int idx = threadIdx.x; idx < kTM * kSplitRows; idx += kThreads) {
      const int tok = idx / kSplitRows, qs = idx % kSplitRows;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += s_mix[w][tok][qs];
      s_mix[0][tok][qs] = v;
    }
  }
  __syncthreads();
  if constexpr (MIX) {
    for (int idx = threadIdx.x; idx < kTM * kMix; idx += kThreads) {
      const int tok = idx / kMix, q = idx % kMix;
      const float dotv = (s_mix[0][tok][q] + s_mix[0][tok][kMix + q]) + s_mix[0][tok][2 * kMix + q];
      const float mv = dotv * s_rx[tok];
      s_mixes[tok][q] = mv;
      const int64_t tt = (int64_t)blockIdx.x * kTM + tok;
      if (a.mixes_out && tt < a.n) a.mixes_out[tt * kMix + q] = mv;
    }
    __syncthreads();
    if (a.pre_out && wave == 0 && lane < kTM) {
      const int64_t tt = (int64_t)blockIdx.x * kTM + lane;
      if (tt < a.n) {
        split_sinkhorn_one(s_mixes[lane], a.hc_scale[0], a.hc_scale[1], a.hc_scale[2], a.hc_base, a.iters,
                           a.hc_eps, a.pre_out + tt * kHC, a.post_out + tt * kHC,
                           a.comb_out + tt * kHC * kHC);
      }
    }
  }
  if constexpr (NORM) {
    const float ry = s_ry[m];
#pragma unroll
    for (int s = 0; s < kMaxSPW; ++s) {
      const int step = wave + s * kWaves;
      if (step >= nsteps) break;
      const int f = step * kStepF + g * kFPL;
      const f32x4* gp = reinterpret_cast<const f32x4*>(a.gamma + f);
      float gm[kFPL];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = gp[q4];
        gm[4 * q4] = v[0]; gm[4 * q4 + 1] = v[1]; gm[4 * q4 + 2] = v[2]; gm[4 * q4 + 3] = v[3];
      }
      u32 zp[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const float z0 = gm[2 * e2] * (bf_lo(ykeep[s][e2]) * ry);
        const float z1 = gm[2 * e2 + 1] * (bf_hi(ykeep[s][e2]) * ry);
        zp[e2] = pack_bf16(z0, z1);
      }
      if (valid) {
        st_stream(yrow + f / 8, u32x4{zp[0], zp[1], zp[2], zp[3]});
        st_stream(yrow + f / 8 + 1, u32x4{zp[4], zp[5], zp[6], zp[7]});
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
  if (d <= 0 || d % kStepF != 0 || d > kMaxD)
    return fail(HC_ENOTSUP, "d=%d: d must be a positive multiple of %d, at most %d", d, kStepF, kMaxD);
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
  if (n > ((int64_t)1 << 34)) return fail(HC_EINVAL, "n=%lld is too large", (long long)n);
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

template <bool POST, bool MIX, bool PRE, bool NORM>
hipError_t launch_tile_t(const TileArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.n + kTM - 1) / kTM);
  TileArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tile_kernel<POST, MIX, PRE, NORM>), dim3(grid),
                         dim3(kThreads), args, 0, st);
}

hipError_t launch_tile(bool post, bool mix, bool pre, bool norm, const TileArgs& a, hipStream_t st) {
  const int key = (post ? 8 : 0) | (mix ? 4 : 0) | (pre ? 2 : 0) | (norm ? 1 : 0);
  switch (key) {
    case 0b1000: return launch_tile_t<true, false, false, false>(a, st);
    case 0b0100: return launch_tile_t<false, true, false, false>(a, st);
    case 0b1100: return launch_tile_t<true, true, false, false>(a, st);
    case 0b0010: return launch_tile_t<false, false, true, false>(a, st);
    case 0b0011: return launch_tile_t<false, false, true, true>(a, st);
    case 0b1010: return launch_tile_t<true, false, true, false>(a, st);
    case 0b1011: return launch_tile_t<true, false, true, true>(a, st);
    case 0b0110: return launch_tile_t<false, true, true, false>(a, st);
    case 0b0111: return launch_tile_t<false, true, true, true>(a, st);
    case 0b1110: return launch_tile_t<true, true, true, false>(a, st);
    case 0b1111: return launch_tile_t<true, true, true, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

TileArgs base_args(int64_t n, int d) {
  TileArgs a{};
  a.n = n;
  a.d = d;
  a.iters = 1;
  return a;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

int hc_version(void) { return 100; /* 0.1.0 */ }

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
  if (hc != kHC || d <= 0 || d % kStepF != 0 || d > kMaxD) return 0;
  return (size_t)(d / kStepF) * kHC * kNT * 64 * 32;
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
             float* comb, void* stream) {
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
  TileArgs a = base_args(n, d);
  a.x = x; a.fn = reinterpret_cast<const u32x4*>(fn_packed); a.mixes_out = mixes;
  a.norm_eps = norm_eps; a.hc_scale = hc_scale; a.hc_base = hc_base; a.iters = iters; a.hc_eps = hc_eps;
  if (split) { a.pre_out = pre; a.post_out = post; a.comb_out = comb; }
  return launched(launch_tile(false, true, false, false, a, (hipStream_t)stream), "hc_mixes");
}

int hc_pre(const hc_bf16* x, const float* pre_mix, int64_t n, int hc, int d, hc_bf16* y, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(x); HC_REQ(pre_mix); HC_REQ(y);
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  TileArgs a = base_args(n, d);
  a.x = x; a.pre_in = pre_mix; a.y_out = y;
  return launched(launch_tile(false, false, true, false, a, (hipStream_t)stream), "hc_pre");
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
  TileArgs a = base_args(n, d);
  a.delta = delta; a.x = x; a.post_in = post; a.comb_in = comb; a.x_out = x_out;
  return launched(launch_tile(true, false, false, false, a, (hipStream_t)stream), "hc_post");
}

size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d) {
  (void)n; (void)hc; (void)d;
  return 0;
}

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
  if (p->n == 0) return HC_OK;
  if ((rc = check_device())) return rc;

  TileArgs a = base_args(p->n, p->d);
  a.x = p->x; a.delta = p->delta; a.post_in = p->post_in; a.comb_in = p->comb_in; a.pre_in = p->pre_in;
  a.fn = reinterpret_cast<const u32x4*>(p->fn_packed); a.hc_base = p->hc_base; a.hc_scale = p->hc_scale;
  a.gamma = p->gamma; a.x_out = p->x_out; a.y_out = p->y_out; a.mixes_out = p->mixes_out;
  a.pre_out = p->pre_out; a.post_out = p->post_out; a.comb_out = p->comb_out;
  a.iters = p->iters; a.hc_eps = p->hc_eps; a.norm_eps = p->norm_eps; a.rms_eps = p->rms_eps;
  const hipStream_t st = (hipStream_t)stream;
  if (!fresh) return launched(launch_tile(post, mix, true, norm, a, st), "hc_boundary");
  // Read with the pre derived in this call: derive first, then read.
  TileArgs a1 = a;
  a1.pre_in = nullptr; a1.y_out = nullptr; a1.gamma = nullptr;
  if ((rc = launched(launch_tile(post, true, false, false, a1, st), "hc_boundary (derive)"))) return rc;
  TileArgs a2 = base_args(p->n, p->d);
  a2.x = post ? p->x_out : p->x; a2.pre_in = p->pre_out; a2.gamma = p->gamma; a2.y_out = p->y_out;
  a2.rms_eps = p->rms_eps;
  return launched(launch_tile(false, false, true, norm, a2, st), "hc_boundary (read)");
}

}  // extern "C"
