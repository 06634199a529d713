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
// Kernels (hc = 4, the pages' setting)
//   stream_kernel<POST, RM, NORM, MEAN> + finish_kernel<RM, NORM>  everything
//       that derives mixes (hc_mixes, block entry, sublayer boundary) at any n:
//       64-token tiles x feature slices, about one workgroup per compute unit;
//       the 24-wide projection on the matrix cores with the weight tiles shared
//       through LDS; the per-slice sums meet in the workspace, and the finish
//       derives the coefficients and writes the read row.
//   decode_kernel<POST, READ>  the same for n <= 128 in one launch: the last
//       slice of a token tile to arrive sums the tile's records.
//   fused_kernel<POST, RM, NORM>  the single-launch schedule (opt-in).
//   row_kernel<POST, PRE, NORM, TPW, HC>  streams only (hc_post, hc_pre, the
//       stack exit): whole token rows per wave, 1 KB per load or store.
//   split_kernel<HC>  hc_split_sinkhorn, one token per lane.
//   pack_kernel     fp32 projection weight -> bf16 hi/mid/lo terms in tile order.
// hc = 2 and 8: row_kernel and split_kernel instantiated for that hc, and
//   mixes_generic_kernel<GM>, the projection in fp32 multiply-adds.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstddef>
#include <cstdio>

#include "hc.h"

namespace {

constexpr int kHC = 4;
constexpr int kMix = (2 + kHC) * kHC;  // 24 mix numbers
constexpr int kNT = 5;                 // packed 16-column weight tiles per 32-feature step and stream
constexpr int kAcc = 2;                // accumulator tiles: rows 0..15, and rows 16..23 (two halves)
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
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
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


// ------------------------------------------------------------- split / Sinkhorn
// "Reading weights" split/Sinkhorn kernel panel and reading-weight equation.
// fp32; the row/column divisions use the hardware reciprocal.
__device__ __forceinline__ float sigmoidf_(float u) { return __builtin_amdgcn_rcpf(1.0f + expf(-u)); }

// Lane-group sums by DPP, within the group (no LDS round trip).  Butterfly
// order: every lane of a group gets the same bits; for a quad (v0 + v1) +
// (v2 + v3) up to commutation.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_sum(float v) {
  const float u = v + quad_perm<0xB1>(v);      // lanes [1,0,3,2]
  return u + quad_perm<0x4E>(u);               // lanes [2,3,0,1]
}
// Sum over the 8 lanes of an aligned group: the two quad sums, each lane
// adding the other quad's (half-row mirror), the same bits in all 8 lanes.
__device__ __forceinline__ float oct_sum(float v) {
  const float u = quad_sum(v);
  return u + quad_perm<0x141>(u);
}
template <int HC>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (HC == 2) return v + quad_perm<0xB1>(v);
  else if constexpr (HC == 4) return quad_sum(v);
  else return oct_sum(v);
}

// The split and the Sinkhorn of "Reading weights" for one token, hc lanes per
// token: lane j holds mixes pre_j (mp), post_j (mq) and comb row j (mc), and
// writes pre_j, post_j and comb row j.  The column sums run across the lanes
// of the token.  Every lane of the group calls it (lanes of a token past n
// with valid false: they compute and store nothing).
template <int HC>
__device__ __forceinline__ void split_lanes(float mp, float mq, const float (&mc)[HC], const float* scale,
                                            const float* base, int iters, float eps, int j, bool valid,
                                            float* pre_o, float* post_o, float* comb_o) {
  const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
  const float pre = sigmoidf_(mp * s0 + base[j]) + eps;
  const float post = 2.0f * sigmoidf_(mq * s1 + base[HC + j]);
  float A[HC], mxr = -INFINITY;
#pragma unroll
  for (int k = 0; k < HC; ++k) {
    A[k] = mc[k] * s2 + base[2 * HC + j * HC + k];
    mxr = fmaxf(mxr, A[k]);
  }
  float rs = 0.f;
#pragma unroll
  for (int k = 0; k < HC; ++k) {
    A[k] = expf(A[k] - mxr);
    rs = rs + A[k];
  }
  const float rinv = __builtin_amdgcn_rcpf(rs);
#pragma unroll
  for (int k = 0; k < HC; ++k) A[k] = A[k] * rinv + eps;
  auto col_norm = [&]() {
#pragma unroll
    for (int k = 0; k < HC; ++k) A[k] = A[k] * __builtin_amdgcn_rcpf(group_sum<HC>(A[k]) + eps);
  };
  col_norm();
  for (int it = 1; it < iters; ++it) {
    float r2 = A[0];
#pragma unroll
    for (int k = 1; k < HC; ++k) r2 = r2 + A[k];
    const float inv = __builtin_amdgcn_rcpf(r2 + eps);
#pragma unroll
    for (int k = 0; k < HC; ++k) A[k] = A[k] * inv;
    col_norm();
  }
  if (valid) {
    pre_o[j] = pre;
    post_o[j] = post;
#pragma unroll
    for (int k = 0; k < HC; ++k) comb_o[j * HC + k] = A[k];
  }
}

// hc_split_sinkhorn: hc lanes per token.
template <int HC>
__global__ void __launch_bounds__(256) split_kernel(const float* __restrict__ mixes,
                                                    const float* __restrict__ scale,
                                                    const float* __restrict__ base, int64_t n, int iters,
                                                    float eps, float* __restrict__ pre,
                                                    float* __restrict__ post, float* __restrict__ comb) {
  constexpr int MIX = (2 + HC) * HC;
  const int j = threadIdx.x % HC;
  const int64_t tq = (int64_t)blockIdx.x * (256 / HC) + threadIdx.x / HC;
  const bool valid = tq < n;
  const int64_t t = valid ? tq : 0;   // lanes past n compute on token 0 (they take part in the sums)
  const float* m = mixes + t * MIX;
  float mc[HC];
#pragma unroll
  for (int k = 0; k < HC; ++k) mc[k] = m[2 * HC + j * HC + k];
  split_lanes<HC>(m[j], m[HC + j], mc, scale, base, iters, eps, j, valid, pre + t * HC, post + t * HC,
                  comb + t * HC * HC);
}

// ------------------------------------------------------------------ weight pack
// Each fp32 weight w is split into three bf16 terms, w = hi + mid + lo, each
// the nearest-even rounding of what is left (exact but for subnormal tails).
// Packed layout, in 16-byte lane records:
//   [step = f/32][stream k][tile nt][lane 0..63] -> 8 bf16
// record (step, k, nt, lane) holds, for column n = lane%16, the terms of one
// projection row at features k*d + 32*step + 8*(lane/16) + 0..7:
//   nt 0/1/2: hi/mid/lo of row n                      (accumulator tile 0)
//   nt 3:     hi of row 16+n (n < 8), mid of row 8+n  (accumulator tile 1)
//   nt 4:     lo of row 16+n (n < 8), zero            (accumulator tile 1)
// so that the three terms of a row meet in one accumulator column (tile 0),
// or in columns n and n+8 of tile 1 (summed once per token at the end).  One
// 1 KB (step, k, nt) block is the B operand of one 16x16x32 matrix-core
// instruction for a 64-lane wave.
__device__ __forceinline__ float split_term(float x, int part) {
  const float hi = round_bf16(x);
  if (part == 0) return hi;
  const float r1 = x - hi;  // exact
  const float mid = round_bf16(r1);
  if (part == 1) return mid;
  return round_bf16(r1 - mid);  // r1 - mid exact
}

__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ fn, int d,
                                                   u32x4* __restrict__ out, int records) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= records) return;
  const int lane = idx & 63;
  const int nt = (idx >> 6) % kNT;
  const int k = (idx / (64 * kNT)) % kHC;
  const int step = idx / (64 * kNT * kHC);
  const int n = lane & 15;
  int q, part;                       // projection row and split term; q < 0: zero
  if (nt < 3) { q = n; part = nt; }
  else if (nt == 3) { q = n < 8 ? 16 + n : 8 + n; part = n < 8 ? 0 : 1; }
  else { q = n < 8 ? 16 + n : -1; part = 2; }
  const int f0 = step * kStepF + (lane >> 4) * kFPL;
  u32 w[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[h] = q < 0 ? 0.f : split_term(fn[(size_t)q * (kHC * d) + (size_t)k * d + f0 + 2 * e2 + h], part);
    w[e2] = pack_bf16(v[0], v[1]);
  }
  out[idx] = u32x4{w[0], w[1], w[2], w[3]};
}

// ------------------------------------------- projection for hc other than 4
// The arithmetic of the hc = 4 kernels (bf16 streams times the three bf16
// terms of each fp32 weight on the matrix cores, fp32 accumulation) in a
// plainer schedule: the projection reads the written streams back instead of
// taking them from the write.  Packed layout for hc other than 4, 16-byte lane
// records [step = c/32][tile ct][lane 0..63] -> 8 bf16 (c the flattened
// feature j*d + i): column n = lane%16 of tile ct is packed column q = 16*ct
// + n, term q / MIXP (hi, mid, lo) of projection row q % MIXP (zero for rows
// >= MIX), at features 32*step + 8*(lane/16) + 0..7.  The three terms of a
// row sit in tiles rt, rt + RT, rt + 2 RT at the same column and so meet in
// the same accumulator register.
template <int HC>
struct GShape {
  static constexpr int MIX = (2 + HC) * HC;
  static constexpr int RT = (MIX + 15) / 16;        // 16-row tiles per term
  static constexpr int MIXP = RT * 16;
  static constexpr int NCT = 3 * RT;                // packed tiles per 32-feature step
  static constexpr int RECW = (MIX + 1 + 3) & ~3;   // record: MIX dots, sum x^2 (16 B multiple)
};

template <int HC>
__global__ void __launch_bounds__(256) gpack_kernel(const float* __restrict__ fn, int K,
                                                    u32x4* __restrict__ out, int records) {
  using G = GShape<HC>;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= records) return;
  const int lane = idx & 63, ct = (idx >> 6) % G::NCT, step = (idx >> 6) / G::NCT;
  const int q = 16 * ct + (lane & 15), term = q / G::MIXP, row = q % G::MIXP;
  const float* src = fn + (size_t)row * K + 32 * step + 8 * (lane >> 4);
  u32 w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = row < G::MIX ? split_term(src[2 * e], term) : 0.f;
    const float b = row < G::MIX ? split_term(src[2 * e + 1], term) : 0.f;
    w[e] = pack_bf16(a, b);
  }
  out[idx] = u32x4{w[0], w[1], w[2], w[3]};
}

constexpr int kGWaves = 4;                 // waves per workgroup
constexpr int kGThreads = kGWaves * 64;
constexpr int kGTok = kGWaves * 32;        // tokens per workgroup: 2 row tiles of 16 per wave
constexpr int kGChunk = 64;    // features per pipeline chunk (two 32-feature steps)

struct GMixArgs {
  const hc_bf16* x;
  const u32x4* fn;     // packed as above
  float* rec;          // [S][n][RECW] per-slice dots and sums of squares
  int64_t n;
  int xtok, xstr;      // elements per token / per stream of x (stride 0: expanded)
  int d, S, Fs;        // slices of the flattened feature range, Fs = hc*d/S features each
};

// One workgroup: 32 tokens per wave x one feature slice.  Per 64-feature chunk
// the weight tiles are staged through registers into a double-buffered LDS
// area shared by the waves; each wave streams the A tiles of its 32 tokens
// straight from memory, two chunks ahead.
template <int HC>
__global__ void __launch_bounds__(kGThreads, 2) gmix_kernel(const GMixArgs a) {
  using G = GShape<HC>;
  constexpr int NCT = G::NCT, RT = G::RT;
  constexpr int BREC = 2 * NCT * 64;            // 16-byte weight records per chunk
  constexpr int BPT = (BREC + kGThreads - 1) / kGThreads;
  __shared__ u32x4 w_lds[2][2 * NCT * 64];      // [buffer][step][tile][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // consecutive workgroups go to different XCDs: slice-major so the workgroups
  // reading one slice of the weights share an XCD (and its L2) where S allows
  const int slice = blockIdx.x % a.S, group = blockIdx.x / a.S;
  const int64_t tw = (int64_t)group * kGTok + wave * 32;
  const hc_bf16* xr[2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t t = tw + 16 * ti + (lane & 15);
    xr[ti] = a.x + (t < a.n ? t : 0) * a.xtok;    // rows past n read token 0 and are never stored
  }
  const int kg = 8 * (lane >> 4);
  const int c0 = slice * a.Fs;
  const int nch = a.Fs / kGChunk;

  auto load_a = [&](int ch, u32x4 (&A)[2][2]) {
    const int c = c0 + ch * kGChunk;              // a chunk never crosses a stream (d % 64 == 0)
    const int j = c / a.d, i = c - j * a.d + kg;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int st = 0; st < 2; ++st) A[ti][st] = ld_stream(reinterpret_cast<const u32x4*>(xr[ti] + j * a.xstr + i + 32 * st));
  };
  auto load_b = [&](int ch, u32x4 (&Bs)[BPT]) {
    const u32x4* src = a.fn + (size_t)((c0 + ch * kGChunk) / 32) * NCT * 64;
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
      const int idx = threadIdx.x + kGThreads * r;
      if (idx < BREC) Bs[r] = src[idx];
    }
  };
  auto store_b = [&](int buf, const u32x4 (&Bs)[BPT]) {
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
      const int idx = threadIdx.x + kGThreads * r;
      if (idx < BREC) w_lds[buf][idx] = Bs[r];
    }
  };

  f32x4 acc[2][NCT];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ti][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[2] = {0.f, 0.f};
  // The stream tiles run two chunks ahead in three register sets used in
  // rotation by a loop unrolled three times (a copy between sets would wait for
  // the loads in flight).  A chunk's weight loads are issued before its stream
  // loads, so that waiting for the former (the load counter is in order) does
  // not wait for the latter.
  u32x4 A0[2][2], A1[2][2], A2[2][2], Bs[BPT];
  auto step = [&](int ch, const u32x4 (&Ac)[2][2], u32x4 (&An)[2][2]) {
    const bool more = ch + 1 < nch;
    if (more) load_b(ch + 1, Bs);
    if (ch + 2 < nch) load_a(ch + 2, An);
    const u32x4* wb = w_lds[ch & 1];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, wb[(st * NCT + ct) * 64 + lane]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          acc[ti][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Ac[ti][st]), b,
                                                                acc[ti][ct], 0, 0, 0);
      }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss[ti] = dot2_bf16(Ac[ti][st][e], Ac[ti][st][e], ss[ti]);
    if (more) store_b((ch + 1) & 1, Bs);
    __syncthreads();                              // next weights in place; this chunk's reads done
  };
  load_b(0, Bs);
  load_a(0, A0);
  if (nch > 1) load_a(1, A1);
  store_b(0, Bs);
  __syncthreads();
  for (int ch = 0; ch < nch; ch += 3) {
    step(ch, A0, A2);
    if (ch + 1 < nch) step(ch + 1, A1, A0);
    if (ch + 2 < nch) step(ch + 2, A2, A1);
  }

  // sums of squares: the four lanes holding one token row (lane, +16, +32, +48)
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    ss[ti] += __shfl_xor(ss[ti], 16);
    ss[ti] += __shfl_xor(ss[ti], 32);
  }
  float* rs = a.rec + (size_t)slice * a.n * G::RECW;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = 16 * rt + (lane & 15);
      if (row < G::MIX) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = tw + 16 * ti + 4 * (lane >> 4) + r;   // accumulator row = token
          if (t < a.n) rs[t * G::RECW + row] = (acc[ti][rt][r] + acc[ti][rt + RT][r]) + acc[ti][rt + 2 * RT][r];
        }
      }
    }
    const int64_t t = tw + 16 * ti + lane;
    if (lane < 16 && t < a.n) rs[t * G::RECW + G::MIX] = ss[ti];
  }
}

struct GFinArgs {
  const float* rec;
  const float* hc_scale;
  const float* hc_base;
  float* mixes_out;    // or NULL
  float* pre_out;      // pre/post/comb, or all NULL
  float* post_out;
  float* comb_out;
  int64_t n;
  int S, K, iters;
  float norm_eps, hc_eps;
};

// hc lanes per token, lane j owning stream j: the slices' records summed in
// slice order, the RMS scale applied ("Source layer, pairs pooled":
// Block.hc_mixes), then the split and the Sinkhorn rounds of "Reading
// weights" with lane j holding comb row j (column sums across the hc lanes).

template <int HC>
__global__ void __launch_bounds__(256) gfinish_kernel(const GFinArgs a) {
  using G = GShape<HC>;
  const int j = threadIdx.x % HC;
  const int64_t tq = (int64_t)blockIdx.x * (256 / HC) + threadIdx.x / HC;
  const bool valid = tq < a.n;
  const int64_t t = valid ? tq : 0;   // lanes past n compute on token 0 (they take part in the shuffles)
  const float* r = a.rec + t * G::RECW;
  const size_t sstride = (size_t)a.n * G::RECW;
  float lp = r[j], lq = r[HC + j], ss = r[G::MIX], lc[HC];
#pragma unroll
  for (int k = 0; k < HC; ++k) lc[k] = r[2 * HC + j * HC + k];
#pragma unroll 4
  for (int s = 1; s < a.S; ++s) {
    r += sstride;
    lp = lp + r[j]; lq = lq + r[HC + j]; ss = ss + r[G::MIX];
#pragma unroll
    for (int k = 0; k < HC; ++k) lc[k] = lc[k] + r[2 * HC + j * HC + k];
  }
  const float rx = 1.0f / sqrtf(ss / (float)a.K + a.norm_eps);
  lp = lp * rx;
  lq = lq * rx;
#pragma unroll
  for (int k = 0; k < HC; ++k) lc[k] = lc[k] * rx;
  if (a.mixes_out && valid) {
    float* m = a.mixes_out + t * G::MIX;
    m[j] = lp;
    m[HC + j] = lq;
#pragma unroll
    for (int k = 0; k < HC; ++k) m[2 * HC + j * HC + k] = lc[k];
  }
  if (!a.pre_out) return;
  split_lanes<HC>(lp, lq, lc, a.hc_scale, a.hc_base, a.iters, a.hc_eps, j, valid, a.pre_out + t * HC,
                  a.post_out + t * HC, a.comb_out + t * HC * HC);
}

// The matrix-core step for one (A tile, 32-feature step, stream): the five
// weight tiles into the two accumulator tiles.
__device__ __forceinline__ void mfma_step(const bf16x8 A, const bf16x8 (&B)[kNT], f32x4 (&acc)[kAcc]) {
  acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[0], acc[0], 0, 0, 0);
  acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[1], acc[0], 0, 0, 0);
  acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[2], acc[0], 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[3], acc[1], 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[4], acc[1], 0, 0, 0);
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
  hc_bf16* x_mean;    // mean over the streams of X' (MTP tap), or NULL
  int64_t n;
  int xtok, xstr;     // elements per token / per stream of x (hc*d, d; or d, 0 when expanded)
  int d;
  float rms_eps;
};

constexpr int kRowChunk = 512;                   // features per wave instruction
constexpr int kRowMaxChunks = 10;                // per token held in registers (NORM)

template <bool POST, int HC = kHC>
__device__ __forceinline__ void row_load(u32x4 (&r)[HC + 1], const u32x4* xrow, const u32x4* drow, int xstr,
                                         int f) {
#pragma unroll
  for (int j = 0; j < HC; ++j) r[j] = ld_stream(xrow + (j * xstr + f) / 8);
  r[HC] = POST ? ld_stream(drow + f / 8) : u32x4{0u, 0u, 0u, 0u};
}

// X'_k = post_k * delta + ((C_0k X_0 + C_1k X_1) + C_2k X_2) + C_3k X_3, one lane's 8 features
template <int HC = kHC>
__device__ __forceinline__ void post_8(const u32x4 (&r)[HC + 1], const float* cpost, const float* ccomb,
                                       u32 (&xp)[HC][4]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float X[HC][2], D[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < HC; ++j) X[j][h] = bf_elem(r[j][e2], h);
      D[h] = bf_elem(r[HC][e2], h);
    }
#pragma unroll
    for (int k = 0; k < HC; ++k) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float pa = cpost[k] * D[h];
        float sm = ccomb[0 * HC + k] * X[0][h];
#pragma unroll
        for (int j = 1; j < HC; ++j) sm = sm + ccomb[j * HC + k] * X[j][h];
        v[h] = pa + sm;
      }
      xp[k][e2] = pack_bf16(v[0], v[1]);
    }
  }
}

// The MTP tap ("Final RMSNorm", the model driver: the mean over the streams of
// a block's input): (((X'_0 + X'_1) + X'_2) + X'_3) / 4 in fp32, one lane's 8
// features (the sum of four bf16 values is exact in fp32 but for extreme
// exponent spreads, and the quarter is exact).
template <int HC = kHC>
__device__ __forceinline__ u32x4 mean_8(const u32 (&xp)[HC][4]) {
  u32 m[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float sm = bf_elem(xp[0][e2], h);
#pragma unroll
      for (int k = 1; k < HC; ++k) sm = sm + bf_elem(xp[k][e2], h);
      v[h] = sm * (1.0f / HC);
    }
    m[e2] = pack_bf16(v[0], v[1]);
  }
  return u32x4{m[0], m[1], m[2], m[3]};
}

// y = ((p_0 X'_0 + p_1 X'_1) + p_2 X'_2) + p_3 X'_3, one lane's 8 features
template <int HC = kHC>
__device__ __forceinline__ void pre_8(const u32 (&xp)[HC][4], const float* cpre, u32 (&yp)[4]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float s = cpre[0] * bf_elem(xp[0][e2], h);
#pragma unroll
      for (int k = 1; k < HC; ++k) s = s + cpre[k] * bf_elem(xp[k][e2], h);
      v[h] = s;
    }
    yp[e2] = pack_bf16(v[0], v[1]);
  }
}

template <bool POST, bool PRE, bool NORM, int TPW, int HC = kHC>
__global__ void __launch_bounds__(kThreads) row_kernel(const RowArgs a) {
  static_assert(!NORM || PRE, "RMSNorm needs the read row");
  constexpr int MAXC = kRowMaxChunks * 2 / TPW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d = a.d;
  const int nch = (d + kRowChunk - 1) / kRowChunk;

  int64_t tok[TPW];
  bool tvalid[TPW];
  float cpost[TPW][HC], ccomb[TPW][HC * HC], cpre[TPW][HC];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = (int64_t)blockIdx.x * (kWaves * TPW) + wave * TPW + i;
    tvalid[i] = t < a.n;
    tok[i] = tvalid[i] ? t : 0;
#pragma unroll
    for (int j = 0; j < HC; ++j) {
      cpost[i][j] = POST ? a.post_in[tok[i] * HC + j] : 0.f;
      cpre[i][j] = PRE ? a.pre_in[tok[i] * HC + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < HC * HC; ++j) ccomb[i][j] = POST ? a.comb_in[tok[i] * HC * HC + j] : 0.f;
  }

  u32 ykeep[NORM ? TPW : 1][NORM ? MAXC : 1][4];
  float ssy[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) ssy[i] = 0.f;

  auto chunk = [&](int c) {
    const int f0 = c * kRowChunk + lane * 8;
    const bool act = f0 < d;
    const int f = act ? f0 : 0;  // idle lanes of a partial chunk read feature 0 and never store
    u32x4 r[TPW][HC + 1];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      row_load<POST, HC>(r[i], reinterpret_cast<const u32x4*>(a.x + tok[i] * a.xtok),
                     reinterpret_cast<const u32x4*>(POST ? a.delta + tok[i] * d : a.x), a.xstr, f);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const bool st = act && tvalid[i];
      u32 xp[HC][4];
      if constexpr (POST) {
        post_8<HC>(r[i], cpost[i], ccomb[i], xp);
        u32x4* xo = reinterpret_cast<u32x4*>(a.x_out + tok[i] * HC * d);
        if (st) {
#pragma unroll
          for (int k = 0; k < HC; ++k) st_stream(xo + (k * d + f) / 8, u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
        }
      } else {
#pragma unroll
        for (int k = 0; k < HC; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) xp[k][e] = r[i][k][e];
      }
      if (a.x_mean && st) st_stream(reinterpret_cast<u32x4*>(a.x_mean + tok[i] * d) + f / 8, mean_8<HC>(xp));
      if constexpr (PRE) {
        u32 yp[4];
        pre_8<HC>(xp, cpre[i], yp);
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
    // without the RMSNorm a row need not stay in one workgroup: the chunks of
    // a row are spread over gridDim.y workgroups (few tokens)
    for (int c = blockIdx.y; c < nch; c += gridDim.y) chunk(c);
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
  hc_bf16* x_mean;    // mean over the streams of X' (MTP tap), or NULL
  float* rec;         // [tiles][S][kTT][kRec]
  int64_t n;
  int xtok, xstr;     // elements per token / per stream of x (hc*d, d; or d, 0 when expanded)
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

template <int N> struct IC { static constexpr int v = N; };

// MEAN: the stream mean (x_mean) is written; a template parameter so that the
// calls without it carry none of its registers
template <bool POST, int RM, bool NORM, bool MEAN>
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
  const unsigned lt = tv ? (unsigned)m : 0u;   // tokens past n read the tile's first token
  const hc_bf16* xb = a.x + t0 * a.xtok;
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
  f32x4 acc[kAcc];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ssx = 0.f, ssy = 0.f;
  float gram[kGram];
#pragma unroll
  for (int g = 0; g < kGram; ++g) gram[g] = 0.f;

  auto load_wst = [&](int c, u32x4 (&dst)[kNT]) {
    const int gstep = (fs + c * kCF) / 32;
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;          // (st, k, nt) = blk / 20, (blk / 5) % 4, blk % 5
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      dst[i] = a.fn[((size_t)((gstep + st) * kHC + k) * kNT + nt) * 64 + lane];
    }
  };
  auto store_wst = [&](int buf, const u32x4 (&src)[kNT]) {
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      w_lds[buf][st][k][nt][lane] = src[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[kHC + 1]) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int j = 0; j < kHC; ++j) dst[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * (unsigned)a.xtok + j * (unsigned)a.xstr + f)));
    dst[kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(db + (lt * d + f))) : u32x4{0u, 0u, 0u, 0u};
  };
  auto stream_phase = [&](int c, const u32x4 (&src)[kHC + 1]) {
    const unsigned f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    if constexpr (POST) {
      post_8(src, cpost, ccomb, xp);
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
        for (int e = 0; e < 4; ++e) xp[k][e] = src[k][e];
    }
    // unconditional: a lane past n works on the tile's first token (lt = 0) and
    // stores the same bits as that token's lane; with no branch the wait counts
    // of the two-chunk loop need not assume a skipped store
    if constexpr (MEAN) st_stream(reinterpret_cast<u32x4*>(a.x_mean + (t0 + lt) * d + f), mean_8(xp));
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
      bf16x8 B[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) B[nt] = __builtin_bit_cast(bf16x8, w_lds[buf][hw][k][nt][lane]);
      mfma_step(A, B, acc);
    }
  };
  // one chunk: its streams are in registers; the next chunk's weights are
  // requested before any compute of this one, its streams before (given pre)
  // or after (fresh pre) the stream phase -- the faster order of each, measured
  auto chunk = [&](int c, bool more) {
    constexpr bool kEarly = RM != kFreshPre;
    u32x4 nxt[kHC + 1];
    if (more) {
      load_wst(c + 1, wst);
      if (kEarly) load_stream(c + 1, nxt);
    }
    stream_phase(c, cur);
    if (more && !kEarly) load_stream(c + 1, nxt);
    lds_barrier();                 // A tiles and chunk c's weights in place; previous matrix phase done
    if (more) store_wst((c + 1) & 1, wst);
    matrix_phase(c & 1);
    lds_barrier();                 // matrix phase done before the A tiles are rewritten
    if (more) {
#pragma unroll
      for (int j = 0; j <= kHC; ++j) cur[j] = nxt[j];
    }
  };
  // Two chunks in flight (the kernels that store no X'): while chunk c is
  // consumed, c+1 is arriving, and c+2 is requested as soon as c's stream
  // registers are free.  Each chunk's weights are requested before its streams,
  // so the wait for the weights (one chunk later) never waits for younger
  // stream loads.  Register sets alternate with the chunk's parity (loop
  // unrolled by two: no copies of loaded registers).  Measured at n = 4096:
  // hc_mixes' kernel 41.5 -> 38.4 us; with hc_post (X' stored) the same loop
  // is slower, 70.5 -> 71.9 us, so those keep one chunk in flight.
  auto deep_step = [&](int c, auto ISSUE, auto STORE, u32x4 (&s)[kHC + 1], u32x4 (&wfree)[kNT],
                       const u32x4 (&wnext)[kNT]) {
    __builtin_amdgcn_sched_barrier(0);             // nothing of chunk c moves into chunk c-1
    stream_phase(c, s);
    if constexpr (decltype(ISSUE)::v) {
      __builtin_amdgcn_sched_barrier(0);           // keep the issue order: weights, then streams
      load_wst(c + 2, wfree);
      __builtin_amdgcn_sched_barrier(0);
      load_stream(c + 2, s);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    if constexpr (decltype(STORE)::v) store_wst((c + 1) & 1, wnext);
    matrix_phase(c & 1);
    lds_barrier();
  };

  if constexpr (!POST) {
    u32x4 sB[kHC + 1], wB[kNT];
    const int c1 = nch > 1 ? 1 : 0;                // a single chunk loads chunk 0 twice (unused)
    load_wst(0, wst);
    __builtin_amdgcn_sched_barrier(0);
    load_stream(0, cur);
    __builtin_amdgcn_sched_barrier(0);
    load_wst(c1, wB);
    __builtin_amdgcn_sched_barrier(0);
    load_stream(c1, sB);
    __builtin_amdgcn_sched_barrier(0);
    store_wst(0, wst);
    lds_barrier();
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      deep_step(c, IC<1>{}, IC<1>{}, cur, wst, wB);
      deep_step(c + 1, IC<1>{}, IC<1>{}, sB, wB, wst);
    }
    const int left = nch - c;                       // 1..3: chunk c in cur, c+1 in sB
    if (left == 3) {
      deep_step(c, IC<1>{}, IC<1>{}, cur, wst, wB);
      deep_step(c + 1, IC<0>{}, IC<1>{}, sB, wB, wst);
      deep_step(c + 2, IC<0>{}, IC<0>{}, cur, wst, wB);
    } else if (left == 2) {
      deep_step(c, IC<0>{}, IC<1>{}, cur, wst, wB);
      deep_step(c + 1, IC<0>{}, IC<0>{}, sB, wB, wst);
    } else {
      deep_step(c, IC<0>{}, IC<0>{}, cur, wst, wB);
    }
  } else {
    load_wst(0, wst);
    load_stream(0, cur);
    store_wst(0, wst);
    lds_barrier();
    for (int c = 0; c + 1 < nch; ++c) chunk(c, true);
    chunk(nch - 1, false);
  }

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
  float* red = reinterpret_cast<float*>(&w_lds[0][0][0][0][0]);   // [4 rb][2 steps][16][32] | extra
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      red[((rb * 2 + hw) * 16 + 4 * (lane >> 4) + rr) * 32 + t * 16 + (lane & 15)] = acc[t][rr];
  float* extra = red + 4 * 2 * 16 * 32;                            // [kRec - kMix][kTT]
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
        const float* r0 = red + ((tm >> 4) * 2 * 16 + (tm & 15)) * 32;   // step 0
        const float* r1 = r0 + 16 * 32;                                 // step 1
        v[i] = q < 16 ? r0[q] + r1[q] : (r0[q] + r0[q + 8]) + (r1[q] + r1[q + 8]);
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
  int stok, sstr;           // fresh pre: elements per token / per stream of src
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

template <int RM, bool NORM>
__global__ void __launch_bounds__(kFinThreads) finish_kernel(const FinishArgs a) {
  __shared__ float tot[kTT][kRec];          // the tile's records summed over the slices
  __shared__ float s_pre[kTT][kHC];         // derived pre (fresh read)
  __shared__ float s_r[kTT];                // RMSNorm factor of the read row
  __shared__ float g_lds[NORM ? kMaxNormD : 1];   // gamma of the read slice (F2 <= d <= kMaxNormD)
  constexpr int kUsed = rec_used<RM, NORM>();
  constexpr int kQuads = (kUsed + 3) / 4;
  // XCD-aware: consecutive blocks land on different XCDs.  Renumbered so that
  // each XCD holds a contiguous run, the S2 workgroups of a tile share an XCD
  // and its L2, and the tile's records cross the fabric once instead of S2 times.
  const int lin = (gridDim.x & 7) ? blockIdx.x : (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int tile = lin / a.S2, sl2 = lin % a.S2;
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

  // ---- derive: 4 lanes per token, lane j of token dtm holds stream j.  The
  // read needs only pre and the RMSNorm factor of every token; the Sinkhorn
  // comb is needed only for the tokens this workgroup owns (writes) and runs
  // later, while the first reads of X' are in flight.
  const bool dthr = threadIdx.x < kTT * kHC;
  const int dtm = (threadIdx.x >> 2) & (kTT - 1), dj = threadIdx.x & 3;
  const bool own = dthr && dtm < valid && dtm % a.S2 == sl2;
  float d_pre = 0.f, d_post = 0.f, d_rx = 0.f;
  if (dthr) {
    const int tm = dtm, j = dj;
    const int64_t t = t0 + tm;
    const float* rec = tot[tm];
    const float rx = 1.0f / sqrtf(rec[kMix] / (float)(kHC * d) + a.norm_eps);
    d_rx = rx;
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
      const float pre = sigmoidf_((rec[j] * rx) * a.hc_scale[0] + a.hc_base[j]) + a.hc_eps;
      d_pre = pre;
      d_post = 2.0f * sigmoidf_((rec[kHC + j] * rx) * a.hc_scale[1] + a.hc_base[kHC + j]);
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
  // the owned tokens' comb (whole quads take part: ownership is per token)
  auto sinkhorn_owned = [&]() {
    if (!(own && a.pre_out)) return;
    const int tm = dtm, j = dj;
    const int64_t t = t0 + tm;
    const float* rec = tot[tm];
    const float s2 = a.hc_scale[2];
    float A[kHC];
    float mxr = -INFINITY;
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
      const int q = 2 * kHC + j * kHC + k;
      A[k] = (rec[q] * d_rx) * s2 + a.hc_base[q];
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
    a.pre_out[t * kHC + j] = d_pre;
    a.post_out[t * kHC + j] = d_post;
    *reinterpret_cast<f32x4*>(a.comb_out + t * kHC * kHC + j * kHC) = f32x4{A[0], A[1], A[2], A[3]};
  };
  if constexpr (!(RM == kFreshPre || (RM == kGivenPre && NORM))) sinkhorn_owned();

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
    const int rstride = RM == kFreshPre ? a.stok : d;
    const int sstr = RM == kFreshPre ? a.sstr : 0;
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
          for (int k = 0; k < NL; ++k) ld[u][k] = ld_stream(reinterpret_cast<const u32x4*>(src + (k * sstr + f)));
        }
      }
      if (cb == nch) sinkhorn_owned();   // while the first batch is in flight
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

// ======================================================= single-launch boundary
// fused_kernel<POST, RM, NORM>: the sublayer boundary in one launch, X' written
// once and read from the chip ("Source layer, pairs pooled": Block.forward).
//
// Work items are (tile of kFT = 16 tokens, slice of kFF = 512 features of each
// stream); the S = d/512 slices of a tile run on different workgroups.  The grid
// is persistent, one workgroup per compute unit, every workgroup resident, and a
// multiple of S; it walks the items in rounds, item r*G + w in round r, so the
// slices of a tile share a round.
//
// Segment k of a workgroup (one barrier between segments):
//   stream waves (8): the read row of item k-2 from its kept X' tile (its
//     coefficients were derived in segment k-1) -> z; then X' of item k =
//     hc_post(...) from the loads issued in segment k-1.  The loads of item k+1
//     go out before any store of item k (one vector-memory counter orders them);
//     X' is stored, put in the LDS A tile of item k (kept for its read row) and
//     its Gram entries summed.
//   matrix waves (4), at the same time: the 24 projection dots of item k-1 on
//     the matrix cores (weight tiles streamed from L2 into registers); publish
//     item k-1's per-token record (dots + Gram) for the other slices of its tile;
//     the outputs (mixes, pre/post, Sinkhorn comb) of the tokens this slice owns
//     in item k-2 (all 34 words of all S slices, written a segment earlier); the
//     read coefficients of item k-1: the 14 words the read needs (4 pre dots +
//     Gram), summed over the S slices in slice order by every slice workgroup of
//     the tile (the same bits everywhere) -> pre and the RMSNorm factor.
// Records travel through the workspace as 64-bit words (value, call tag): a word
// is valid when its tag is this call's, so no ordering between words is needed
// and no writer waits.  A reader polls until valid, a bounded number of times;
// a timeout sets an error flag instead of hanging.
constexpr int kFT = 16;                      // tokens per tile
constexpr int kFF = 512;                     // features per slice and stream
constexpr int kFSW = 8;                      // stream waves
constexpr int kFMW = 4;                      // matrix waves
constexpr int kFThreads = (kFSW + kFMW) * 64;
constexpr int kFKS = kFF / kStepF;           // 32-feature steps per slice (16)
constexpr int kFKB = kFKS * kHC;             // matrix-core K blocks per item (64)
constexpr int kFKBW = kFKB / kFMW;           // per matrix wave (16)
constexpr int kFPre = 4;                     // weight blocks in flight per matrix wave
constexpr int kFRec = 34;                    // record words per token and slice
constexpr int kFCoef = 5;                    // read coefficients per token: pre[4], RMSNorm factor
constexpr int kFMinD = 2 * kFF;              // S >= 2: at most 8 owned tokens per slice
constexpr int kFPollBatch = 10;              // slices polled per batch
constexpr int kCtrlBytes = 8192;             // control block at the head of the workspace
constexpr int kEpochCopies = 64;             // epoch word copies, 64 bytes apart
constexpr int kDoneWord = 1024, kErrWord = 1040;
constexpr unsigned kPollLimit = 1u << 14;    // polls of one word (about 1 us each) before a wait gives up
constexpr int64_t kFusedMaxN = (int64_t)1 << 26;   // item indices stay in int
typedef unsigned long long u64;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

enum : unsigned { kErrPollTimeout = 1u };

struct FusedArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const float* pre_in;
  const u32x4* fn;
  const float* gamma;
  const float* hc_base;
  const float* hc_scale;
  hc_bf16* x_out;
  hc_bf16* y_out;
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  u32* ctrl;          // workspace head (kCtrlBytes)
  u64* rec;           // [tiles][S][kFT][kFRec] tagged words
  int64_t n;
  int d, S, tiles, items, rounds, iters;
  float hc_eps, norm_eps, rms_eps;
};

// record word order per read mode: fresh [pre dots 0..3 | Gram 10 | dots 4..23];
// given pre with RMSNorm [sum y^2 | sum x'^2 | dots]; otherwise [sum x'^2 | dots]
template <int RM, bool NORM> constexpr int f_fast() { return RM == kFreshPre ? kHC + kGram : (RM == kGivenPre && NORM ? 1 : 0); }
template <int RM, bool NORM> __device__ __forceinline__ int f_dot(int q) {
  if constexpr (RM == kFreshPre) return q < kHC ? q : q + kGram;
  else return q + (NORM && RM == kGivenPre ? 2 : 1);
}
template <int RM, bool NORM> constexpr int f_ssx() { return RM == kGivenPre && NORM ? 1 : 0; }   // (not fresh)

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, u32 bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2); }
__device__ __forceinline__ void buf_st(rsrc_t r, u32 off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2); }

__device__ __forceinline__ u64 tag_word(float v, u32 tag) { return ((u64)tag << 32) | __float_as_uint(v); }
__device__ __forceinline__ void put_word(u64* p, u64 w) { __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 get_word(const u64* p) { return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// The word's value once its tag is this call's, polled again as needed.  After
// a wait of this lane has timed out (dead), no further waiting: the call then
// finishes quickly with the error flag set rather than polling on.
__device__ __forceinline__ float settle(const u64* p, u64 w, u32 tag, u32* err, bool& dead) {
  unsigned polls = 0;
  while ((u32)(w >> 32) != tag && !dead) {
    if (++polls > kPollLimit) { atomicOr(err, kErrPollTimeout); dead = true; break; }
    __builtin_amdgcn_s_sleep(8);
    w = get_word(p);
  }
  return __uint_as_float((u32)w);
}

// A-tile slot of matrix-core lane L at step parity st: the low 4 bits are
// XOR-ed with (2*(L/16) | st), a permutation within each 16-slot group, so that
// the 8 lanes writing one token's 64 features hit 8 different bank groups.
__device__ __forceinline__ int f_swz(int L, int st) { return (L & 48) | ((L & 15) ^ (((L >> 4) << 1) | st)); }

// One token's mixes / pre / post / comb from its summed record (in LDS, record
// word order), 4 lanes (one quad) per token, lane j holding comb row j
// ("Reading weights" kernel panel and reading-weight equation).  All four lanes
// of the quad call it.
template <int RM, bool NORM>
__device__ __forceinline__ void derive_outputs(const float* fs, float rx, int j, const FusedArgs& a, int64_t t) {
  if (a.mixes_out) {
#pragma unroll
    for (int i = 0; i < kMix / kHC; ++i) a.mixes_out[t * kMix + i * kHC + j] = fs[f_dot<RM, NORM>(i * kHC + j)] * rx;
  }
  const float s0 = a.hc_scale[0], s1 = a.hc_scale[1], s2 = a.hc_scale[2];
  const float pre = sigmoidf_((fs[f_dot<RM, NORM>(j)] * rx) * s0 + a.hc_base[j]) + a.hc_eps;
  const float post = 2.0f * sigmoidf_((fs[f_dot<RM, NORM>(kHC + j)] * rx) * s1 + a.hc_base[kHC + j]);
  float A[kHC];
  float mxr = -INFINITY;
#pragma unroll
  for (int k = 0; k < kHC; ++k) {
    const int q = 2 * kHC + j * kHC + k;
    A[k] = (fs[f_dot<RM, NORM>(q)] * rx) * s2 + a.hc_base[q];
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
  a.pre_out[t * kHC + j] = pre;
  a.post_out[t * kHC + j] = post;
  *reinterpret_cast<f32x4*>(a.comb_out + t * kHC * kHC + j * kHC) = f32x4{A[0], A[1], A[2], A[3]};
}

template <bool POST, int RM, bool NORM>
__global__ void __launch_bounds__(kFThreads, 1) fused_kernel(const FusedArgs a) {
  constexpr bool kFresh = RM == kFreshPre;
  constexpr bool kKeepY = RM == kGivenPre && NORM;       // y kept (registers) for the RMSNorm
  constexpr bool kFinish = kFresh || kKeepY;             // a read row is written after the exchange
  constexpr int kFast = f_fast<RM, NORM>();
  // LDS
  __shared__ u32x4 A_lds[2][kHC][kFKS][64];              // X' in matrix-core A layout, items k and k-1 (128 KB)
  __shared__ float red[kFMW][kFT][kMix];                 // per-matrix-wave partial dots
  __shared__ float gred[2][4][kFT][kGram + 2];           // per-chunk-pair Gram / sum x'^2 / sum y^2, by item parity
  __shared__ float cin[2][kFT][kHC + kHC * kHC + kHC];   // post_in, comb_in, pre_in of the streamed item
  __shared__ float gam[2][NORM ? kFF : 1];               // RMSNorm gain of the item being read
  __shared__ float coef[2][kFT][kFCoef];                 // read coefficients (pre, RMSNorm factor)
  __shared__ float fsum[kFMW][kFT / kFMW][kFRec];        // matrix-wave scratch: summed record words
  __shared__ u32 mcount;                                 // matrix-wave barrier counter

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = gridDim.x, w = blockIdx.x, S = a.S, d = a.d;
  u32* err = a.ctrl + kErrWord;
  const u32 epoch = __hip_atomic_load(a.ctrl + 16 * (w % kEpochCopies), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u32 tag = epoch + 1u == 0u ? 1u : epoch + 1u;
  if (threadIdx.x == 0) mcount = 0;

  // Position of this workgroup in a round: consecutive workgroups land on
  // different XCDs (round-robin), so they are renumbered XCD by XCD; items are
  // taken slice-major, position g -> (tile r*TPR + g%TPR, slice g/TPR), TPR = G/S
  // tiles per round.  A workgroup keeps its slice in every round, and the
  // workgroups of one XCD share one or two slices: their weight tiles stay in
  // that XCD's L2.  (Any bijection is correct; this one is for locality.)
  const int xcd = w & 7, xq = G >> 3, xr = G & 7;
  const int g_pos = xcd * xq + min(xcd, xr) + (w >> 3);
  const int TPR = G / S;
  struct Item { int tile, slice, valid; };
  auto item_of = [&](int r) {
    Item it;
    const int tile = r * TPR + g_pos % TPR;
    const bool ok = r >= 0 && r < a.rounds && tile < a.tiles;
    it.tile = ok ? tile : 0;
    it.slice = g_pos / TPR;
    it.valid = ok ? (int)min<int64_t>(kFT, a.n - (int64_t)tile * kFT) : 0;
    return it;
  };
  const u32 xrow = (u32)(kHC * d * 2), drow = (u32)(d * 2);
  const int K = a.rounds + 2;                            // segments: stream k, matrix k-1, read k-2

  if (wave < kFSW) {
    // ======================================================== stream waves
    // segment k: the read row of item k-2, then X' of item k
    const int tg = wave & 1, cp = wave >> 1;
    const int tl = lane >> 3, p = lane & 7;
    const int m = 8 * tg + tl;                             // token of the tile
    struct Res { rsrc_t x, dl, xo, yo; u32 fbyte; };
    auto res_of = [&](const Item& it) {
      Res q;
      const int64_t t0 = (int64_t)it.tile * kFT;
      q.x = make_rsrc(a.x + t0 * kHC * d, it.valid * xrow);
      q.dl = make_rsrc(POST ? a.delta + t0 * d : a.x, POST ? it.valid * drow : 0);
      q.xo = make_rsrc(POST ? a.x_out + t0 * kHC * d : a.x, POST ? it.valid * xrow : 0);
      q.yo = make_rsrc(a.y_out + t0 * d, it.valid * drow);
      q.fbyte = (u32)(it.slice * kFF + 2 * cp * 64 + 8 * p) * 2;
      return q;
    };
    u32x4 L[2][kHC + 1];
    auto issue = [&](const Res& q) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const u32 o = (u32)m * xrow + q.fbyte + cc * 128;
#pragma unroll
        for (int j = 0; j < kHC; ++j) L[cc][j] = buf_ld(q.x, o + j * drow);
        L[cc][kHC] = POST ? buf_ld(q.dl, (u32)m * drow + q.fbyte + cc * 128) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    u32 yk1[2][4], yk2[2][4];                            // given pre + RMSNorm: y of items k-1, k-2
    Res rc = res_of(item_of(0));
    issue(rc);
    __syncthreads();                                     // P: cin of item 0 in place
    for (int k = 0; k < K; ++k) {
      // ---- the read row of item k-2 (its coefficients arrived with the last barrier)
      if constexpr (kFinish) {
        const Res rp = res_of(item_of(k - 2));
        const int pb = k & 1;                            // (k-2) & 1
        const float* cf = coef[pb][m];
        float pr[kHC];
#pragma unroll
        for (int j = 0; j < kHC; ++j) pr[j] = cf[j];
        const float rn = NORM ? cf[kHC] : 1.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          u32 yv[4];
          if constexpr (kFresh) {
            const int ks = 2 * (2 * cp + cc) + (p >> 2);
            const int slot = f_swz(16 * (p & 3) + m, ks & 1);
            u32 xv[kHC][4];
#pragma unroll
            for (int kk = 0; kk < kHC; ++kk) {
              const u32x4 v = A_lds[pb][kk][ks][slot];
#pragma unroll
              for (int e = 0; e < 4; ++e) xv[kk][e] = v[e];
            }
            pre_8(xv, pr, yv);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[e] = yk2[cc][e];
          }
          if constexpr (NORM) {
            const float* gm = gam[pb] + (2 * cp + cc) * 64 + 8 * p;
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gm);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gm + 4);
            const float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              yv[e2] = pack_bf16(gg[2 * e2] * (bf_lo(yv[e2]) * rn), gg[2 * e2 + 1] * (bf_hi(yv[e2]) * rn));
          }
          buf_st(rp.yo, (u32)m * drow + rp.fbyte + cc * 128, u32x4{yv[0], yv[1], yv[2], yv[3]});
        }
      }
      // ---- X' of item k
      const Res rn_ = res_of(item_of(k + 1));
      const int sl = k & 1;
      const float* ci = cin[k & 1][m];
      float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
      for (int j = 0; j < kHC; ++j) { cpost[j] = ci[j]; cpre[j] = ci[kHC + kHC * kHC + j]; }
#pragma unroll
      for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = ci[kHC + j];
      u32 xp[2][kHC][4];
      u32 yp[2][4];
      float g[kGram + 2];
#pragma unroll
      for (int i = 0; i < kGram + 2; ++i) g[i] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if constexpr (POST) {
          post_8(L[cc], cpost, ccomb, xp[cc]);
        } else {
#pragma unroll
          for (int kk = 0; kk < kHC; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) xp[cc][kk][e] = L[cc][kk][e];
        }
        if constexpr (kFresh) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int gi = 0;
#pragma unroll
            for (int j = 0; j < kHC; ++j)
#pragma unroll
              for (int l = j; l < kHC; ++l, ++gi) g[gi] = dot2_bf16(xp[cc][j][e], xp[cc][l][e], g[gi]);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < kHC; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) g[kGram] = dot2_bf16(xp[cc][kk][e], xp[cc][kk][e], g[kGram]);
          pre_8(xp[cc], cpre, yp[cc]);
          if constexpr (NORM) {
#pragma unroll
            for (int e = 0; e < 4; ++e) g[kGram + 1] = dot2_bf16(yp[cc][e], yp[cc][e], g[kGram + 1]);
          }
        }
      }
      // the loads of item k+1 go out before any store of item k (one vector-memory counter orders them)
      issue(rn_);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const u32 o = (u32)m * xrow + rc.fbyte + cc * 128;
        if constexpr (POST) {
#pragma unroll
          for (int kk = 0; kk < kHC; ++kk)
            buf_st(rc.xo, o + kk * drow, u32x4{xp[cc][kk][0], xp[cc][kk][1], xp[cc][kk][2], xp[cc][kk][3]});
        }
        if constexpr (RM == kGivenPre && !NORM)
          buf_st(rc.yo, (u32)m * drow + rc.fbyte + cc * 128, u32x4{yp[cc][0], yp[cc][1], yp[cc][2], yp[cc][3]});
      }
      __builtin_amdgcn_sched_barrier(0);
      // X' into the A tile of item k: chunk c = 2cp+cc, step ks = 2c + p/4, A lane 16*(p%4) + m
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ks = 2 * (2 * cp + cc) + (p >> 2);
        const int slot = f_swz(16 * (p & 3) + m, ks & 1);
#pragma unroll
        for (int kk = 0; kk < kHC; ++kk)
          A_lds[sl][kk][ks][slot] = u32x4{xp[cc][kk][0], xp[cc][kk][1], xp[cc][kk][2], xp[cc][kk][3]};
      }
      // per-token sums over the 8 lanes of the token, then one lane writes this chunk pair's share
#pragma unroll
      for (int i = 0; i < kGram + 2; ++i) {
        g[i] += __shfl_xor(g[i], 1);
        g[i] += __shfl_xor(g[i], 2);
        g[i] += __shfl_xor(g[i], 4);
      }
      if (p == 0) {
#pragma unroll
        for (int i = 0; i < kGram + 2; ++i) gred[k & 1][cp][m][i] = g[i];
      }
      if constexpr (kKeepY) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 4; ++e) { yk2[cc][e] = yk1[cc][e]; yk1[cc][e] = yp[cc][e]; }
      }
      rc = rn_;
      __syncthreads();                                   // X(k)
    }
  } else {
    // ======================================================== matrix waves
    // segment k: the dots of item k-1 and its record; the outputs of the tokens
    // this slice owns in item k-2; the read coefficients of item k-1
    const int mw = wave - kFSW;
    const int lt = threadIdx.x - kFSW * 64;              // 0..255
    u32 mgen = 0;
    // the four matrix waves meet (LDS counter; bounded)
    auto mbar = [&]() {
      ++mgen;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_fetch_add(&mcount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      unsigned spins = 0;
      while (__hip_atomic_load(&mcount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kFMW * mgen) {
        if (++spins > kPollLimit * 64) { if (lane == 0) atomicOr(err, kErrPollTimeout); break; }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    // weight tiles of this workgroup's slice (the slice is the same in every
    // round): record (K block kb, tile nt, lane) at ((kb*kNT + nt)*64 + lane)*16 B
    constexpr u32 kSliceWt = (u32)kFKB * kNT * 64 * 16;
    const rsrc_t wres = make_rsrc(a.fn + (size_t)item_of(0).slice * (kSliceWt / 16), kSliceWt);
    const u32 wlane = (u32)lane * 16 + (u32)mw * kFKBW * kNT * 64 * 16;
    auto wt = [&](int j, int nt) {                     // weight tile nt of K block j of this wave
      return __builtin_amdgcn_raw_buffer_load_b128(wres, wlane, (j * kNT + nt) * 64 * 16, 0);
    };
    constexpr int kCin = kFT * (kHC + kHC * kHC + kHC);  // 384 floats
    auto cin_val = [&](const Item& it, int i) {
      const int tm = i / (kHC + kHC * kHC + kHC), q = i % (kHC + kHC * kHC + kHC);
      const int64_t t = (int64_t)it.tile * kFT + tm;
      if (tm >= it.valid) return 0.f;
      if (q < kHC) return POST ? a.post_in[t * kHC + q] : 0.f;
      if (q < kHC + kHC * kHC) return POST ? a.comb_in[t * kHC * kHC + (q - kHC)] : 0.f;
      return RM == kGivenPre ? a.pre_in[t * kHC + (q - kHC - kHC * kHC)] : 0.f;
    };
    {                                                    // prologue: cin of item 0
      const Item i0 = item_of(0);
      for (int i = lt; i < kCin; i += kFMW * 64) cin[0][i / (kCin / kFT)][i % (kCin / kFT)] = cin_val(i0, i);
    }
    u32x4 B[kFPre][kNT];
#pragma unroll
    for (int j = 0; j < kFPre; ++j)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) B[j][nt] = wt(j, nt);
    bool dead = false;
    __syncthreads();                                     // P
    for (int k = 0; k < K; ++k) {
      const Item im = item_of(k - 1), io = item_of(k - 2), in1 = item_of(k + 1);
      // ---- the dots of item k-1 (A tile k-1, weights prefetched)
      {
        const int sl = (k - 1) & 1;
        f32x4 acc[kAcc];
#pragma unroll
        for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kFKBW; ++j) {
          const int kb = mw * kFKBW + j;
          const int ks = kb >> 2, kk = kb & 3;
          const bf16x8 Av = __builtin_bit_cast(bf16x8, A_lds[sl][kk][ks][f_swz(lane, ks & 1)]);
          bf16x8 Bv[kNT];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) Bv[nt] = __builtin_bit_cast(bf16x8, B[j % kFPre][nt]);
          if (j + kFPre < kFKBW) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) B[j % kFPre][nt] = wt(j + kFPre, nt);
          }
          mfma_step(Av, Bv, acc);
        }
        // tile 1: columns c and c+8 hold the (hi+lo) and mid terms of row 16+c
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o = __shfl_xor(acc[1][i], 8);
          const int tm = 4 * (lane >> 4) + i, col = lane & 15;
          red[mw][tm][col] = acc[0][i];
          if (col < 8) red[mw][tm][16 + col] = acc[1][i] + o;
        }
      }
      // Requests with the weight loads of this segment behind them (one vector-memory
      // counter: a wait for a weight block waits for everything issued before it):
      // the staged inputs (stream coefficients of item k+1, RMSNorm gain of item k-1).
      const u64* ro = a.rec + (size_t)io.tile * S * kFT * kFRec;
      const int oi0 = mw;                                // first owned token index of this wave
      u64 ow[kFPollBatch];                               // words of this wave's first owned token, item k-2
      {
        const int otm = io.slice + oi0 * S;
        const bool act = io.valid > 0 && otm < io.valid && lane < kFRec;
#pragma unroll
        for (int b = 0; b < kFPollBatch; ++b)
          ow[b] = (act && b < S) ? get_word(ro + ((size_t)b * kFT + otm) * kFRec + lane) : 0ull;
      }
      float cv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) cv[u] = (lt + u * kFMW * 64 < kCin) ? cin_val(in1, lt + u * kFMW * 64) : 0.f;
      f32x4 gv = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NORM) gv = *reinterpret_cast<const f32x4*>(a.gamma + im.slice * kFF + 4 * (lt & (kFF / 4 - 1)));
      mbar();
      // ---- publish item k-1's record
      if (im.valid > 0) {
        u64* rb = a.rec + ((size_t)im.tile * S + im.slice) * kFT * kFRec;
        const float(*gr)[kFT][kGram + 2] = gred[(k - 1) & 1];
        const int tm = lt >> 4;
#pragma unroll
        for (int q = lt & 15; q < kFRec; q += 16) {
          if (tm >= im.valid) break;
          int qd = -1, gi = -1;
          if constexpr (kFresh) {
            if (q < kHC) qd = q;
            else if (q < kHC + kGram) gi = q - kHC;
            else qd = q - kGram;
          } else {
            const int base = kKeepY ? 2 : 1;
            if (q >= base + kMix) gi = -2;
            else if (q >= base) qd = q - base;
            else gi = (kKeepY && q == 0) ? kGram + 1 : kGram;
          }
          float v = 0.f;
          if (qd >= 0) v = ((red[0][tm][qd] + red[1][tm][qd]) + red[2][tm][qd]) + red[3][tm][qd];
          else if (gi >= 0) v = ((gr[0][tm][gi] + gr[1][tm][gi]) + gr[2][tm][gi]) + gr[3][tm][gi];
          put_word(rb + tm * kFRec + q, tag_word(v, tag));
        }
      }
      // ---- read coefficients of item k-1 (words written just now by the other
      //      slices): requested here, summed after the owned tokens of item k-2
      const u64* rm = a.rec + (size_t)im.tile * S * kFT * kFRec;
      const int fi = lane >> 4, fq = lane & 15, ftm = 4 * mw + fi;
      const bool fast_act = kFast > 0 && im.valid > 0 && fq < kFast && ftm < im.valid;
      u64 fw[kFPollBatch];
#pragma unroll
      for (int b = 0; b < kFPollBatch; ++b)
        fw[b] = (fast_act && b < S) ? get_word(rm + ((size_t)b * kFT + ftm) * kFRec + fq) : 0ull;
      // owned tokens: mixes, pre/post, Sinkhorn comb (first owned token from the words above)
      for (int oi = oi0; io.valid > 0 && io.slice + oi * S < io.valid; oi += kFMW) {
        const int tm = io.slice + oi * S;
        const bool act = lane < kFRec;
        float s = 0.f;
        for (int s0b = 0; s0b < S; s0b += kFPollBatch) {
          u64 wv[kFPollBatch];
#pragma unroll
          for (int b = 0; b < kFPollBatch; ++b)
            wv[b] = (oi == oi0 && s0b == 0) ? ow[b]
                    : ((act && s0b + b < S) ? get_word(ro + ((size_t)(s0b + b) * kFT + tm) * kFRec + lane) : 0ull);
#pragma unroll
          for (int b = 0; b < kFPollBatch; ++b)
            if (act && s0b + b < S) s += settle(ro + ((size_t)(s0b + b) * kFT + tm) * kFRec + lane, wv[b], tag, err, dead);
        }
        float* fs = fsum[mw][0];
        __builtin_amdgcn_wave_barrier();
        if (act) fs[lane] = s;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float ssx;
        if constexpr (kFresh) ssx = (fs[kHC + 0] + fs[kHC + 4]) + (fs[kHC + 7] + fs[kHC + 9]);
        else ssx = fs[f_ssx<RM, NORM>()];
        const float rx = 1.0f / sqrtf(ssx / (float)(kHC * d) + a.norm_eps);
        if (lane < kHC) derive_outputs<RM, NORM>(fs, rx, lane, a, (int64_t)io.tile * kFT + tm);
        __builtin_amdgcn_wave_barrier();
      }
      // read coefficients of item k-1: this wave takes tokens 4*mw .. 4*mw+3
      if constexpr (kFast > 0) {
        if (im.valid > 0) {
          float s = 0.f;
          for (int s0b = 0; s0b < S; s0b += kFPollBatch) {
            u64 wv[kFPollBatch];
#pragma unroll
            for (int b = 0; b < kFPollBatch; ++b)
              wv[b] = s0b == 0 ? fw[b]
                               : ((fast_act && s0b + b < S) ? get_word(rm + ((size_t)(s0b + b) * kFT + ftm) * kFRec + fq) : 0ull);
#pragma unroll
            for (int b = 0; b < kFPollBatch; ++b)
              if (fast_act && s0b + b < S) s += settle(rm + ((size_t)(s0b + b) * kFT + ftm) * kFRec + fq, wv[b], tag, err, dead);
          }
          __builtin_amdgcn_wave_barrier();
          if (fast_act) fsum[mw][fi][fq] = s;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (lane < 4 * kHC) {                          // quad per token: lane j of the quad = pre j
            const int i2 = lane >> 2, j = lane & 3, t2 = 4 * mw + i2;
            const float* fs = fsum[mw][i2];
            float pre = 0.f, rnv = 1.f;
            if constexpr (kFresh) {
              const float ssx = (fs[kHC + 0] + fs[kHC + 4]) + (fs[kHC + 7] + fs[kHC + 9]);
              const float rx = 1.0f / sqrtf(ssx / (float)(kHC * d) + a.norm_eps);
              pre = sigmoidf_((fs[j] * rx) * a.hc_scale[0] + a.hc_base[j]) + a.hc_eps;
              if constexpr (NORM) {
                double pd[kHC];
#pragma unroll
                for (int l = 0; l < kHC; ++l) pd[l] = (double)__shfl(pre, (lane & ~3) + l);
                double yy = 0.0;
                int gi = 0;
#pragma unroll
                for (int l = 0; l < kHC; ++l)
#pragma unroll
                  for (int l2 = l; l2 < kHC; ++l2, ++gi) yy += (l == l2 ? 1.0 : 2.0) * pd[l] * pd[l2] * (double)fs[kHC + gi];
                rnv = 1.0f / sqrtf((float)(yy / (double)d) + a.rms_eps);
              }
            } else {
              rnv = 1.0f / sqrtf(fs[0] / (float)d + a.rms_eps);
            }
            coef[(k - 1) & 1][t2][j] = pre;
            if (j == 0) coef[(k - 1) & 1][t2][kHC] = rnv;
          }
        }
      }
      // ---- staged inputs into LDS; the next item's first weight blocks
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = lt + u * kFMW * 64;
        if (i < kCin) cin[(k + 1) & 1][i / (kCin / kFT)][i % (kCin / kFT)] = cv[u];
      }
      if constexpr (NORM) {
        if (lt < kFF / 4) *reinterpret_cast<f32x4*>(&gam[(k - 1) & 1][4 * lt]) = gv;
      }
#pragma unroll
      for (int j = 0; j < kFPre; ++j)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) B[j][nt] = wt(j, nt);
      __syncthreads();                                   // X(k)
    }
  }
  // ---- the last workgroup out advances the call tag for the next call
  if (threadIdx.x == 0) {
    const u32 done = __hip_atomic_fetch_add(a.ctrl + kDoneWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (u32)G - 1u) {
      for (int i = 0; i < kEpochCopies; ++i)
        __hip_atomic_store(a.ctrl + 16 * i, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctrl + kDoneWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ======================================================= slice-resident boundary
// sweep_kernel<NORM>: the boundary with the freshly derived pre -- hc_post,
// hc_mixes on X', split and Sinkhorn, hc_pre with that pre (+ RMSNorm) -- in
// one launch that reads X and delta once and never reads X' back ("Source
// layer, pairs pooled": Block.forward; "Reading weights": the split kernel
// panel; "Final RMSNorm").  Built for the pages' width, d = 5120, at hc = 4.
//
// The width is cut into 32 slices of 160 features of each stream.  Token tiles
// (16 tokens) are dealt to the eight XCDs round robin (tile T to XCD T % 8);
// on an XCD every tile passes through all 32 workgroups, workgroup p taking
// slice p.  So a workgroup keeps one slice for the whole call and holds that
// slice's packed projection weights (the B operands of the matrix cores) in
// LDS, loaded once.  The grid is one workgroup per compute unit, all resident.
//
// Eight waves, two per SIMD: five stream waves (one lane per token and 8
// features of the slice), the projection wave, and exchange waves A and B.
// The stream waves never wait on global memory; the others never stream.
// Interval k, one workgroup barrier per interval (tile indices local to the
// XCD):
//   stream waves: the read row (y, or z with the RMSNorm) of tile k-7 from its
//     X' kept in registers (eight sets) and its coefficients in LDS; X' of
//     tile k+1 from the loads of two intervals ago, stored and put in the LDS
//     A tile; the loads of tile k+3.
//   projection wave: the 24 dots of tile k on the matrix cores, published as
//     words 0..23 of each token's record.
//   wave A: sum x'^2 and the 10 Gram entries of tile k from the A tile,
//     record words 24..35; the read coefficients of tile k-6 (requested an
//     interval earlier) into LDS; post_in and comb_in of tile k+2.
//   wave B (owner of one token of every other tile): sums the records of its
//     token of tile k-3 over the 32 slices (requested an interval earlier),
//     derives and publishes the read coefficients (pre, and the RMSNorm factor
//     from p^T G p) with mixes, pre and post; or requests the records of tile
//     k-2 and runs the Sinkhorn comb of its token of tile k-4.
// Exchange words are 64-bit (value, tag) stored and loaded with device scope;
// tags are the call epoch plus the tile index, so no ring slot needs clearing
// and no store waits.  Every request is issued at the start of an interval
// (ahead of the stream waves' burst in the compute unit's memory pipeline) and
// used an interval later.  Waits are bounded: a timeout sets the error mask and
// the call finishes with wrong values instead of hanging.  The last workgroup
// to finish advances the epoch.
constexpr int kWT = 16;                      // tokens per tile
constexpr int kWX = 8;                       // XCDs: tile T goes to XCD T % 8
constexpr int kWS = 32;                      // slices = workgroups per XCD
constexpr int kWD = 5120;                    // the width the schedule is built for
constexpr int kWF = kWD / kWS;               // 160 features per slice and stream
constexpr int kWG8 = kWF / 8;                // 20 lanes per token
constexpr int kWSt = kWF / kStepF;           // 5 matrix-core K steps per stream
constexpr int kWSW = kWT * kWG8 / 64;        // 5 stream waves
constexpr int kWThreads = (kWSW + 3) * 64;   // + exchange waves A, B and the projection wave
constexpr int kWGrid = kWX * kWS;            // 256 workgroups
constexpr int kWLag = 7;                     // read row of tile k - 7 in interval k
constexpr int kWXS = kWLag + 1;              // X' register sets, tile % 8
constexpr int kWRR = 16;                     // ring slots (records, read coefficients)
constexpr int kWRec = 36;                    // record words used: 24 dots, sum x'^2, 10 Gram, pad
constexpr int kWRecS = 48;                   // record stride (384 B, three 128-byte lines): dots in
                                             // words 0..23, sum x'^2 / Gram / pad in words 32..43
constexpr int kWSq = 32;                     // first sum-of-squares word
constexpr int kWCin = kHC + kHC * kHC;       // post_in, comb_in per token
constexpr int kWCoefW = 8;                   // read-coefficient words per token (5 used)
constexpr int kWEpochWord = 1152;            // control block: 8 epoch copies, 64 bytes apart
constexpr int kWDoneWord = 1280;
constexpr int kWaitLds = 0xC07F;             // s_waitcnt lgkmcnt(0) only (vmcnt 63, expcnt 7 untouched)
constexpr size_t kWRecBytes = sizeof(unsigned long long) * kWX * kWRR * kWS * kWT * kWRecS;
constexpr size_t kWCoefBytes = sizeof(unsigned long long) * kWX * kWRR * kWT * kWCoefW;
static_assert(kWSW * 64 == kWT * kWG8, "stream lanes cover the tile");
static_assert(kWF % kStepF == 0, "slice is whole matrix-core steps");

struct SweepArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const u32x4* fn;
  const float* gamma;
  const float* hc_base;
  const float* hc_scale;
  hc_bf16* x_out;
  hc_bf16* y_out;
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  u32* ctrl;          // workspace head (kCtrlBytes)
  u64* rec;           // [kWX][kWRR][kWS][kWT][kWRecS] tagged words
  u64* coef;          // [kWX][kWRR][kWT][kWCoefW]
  int64_t n;
  int ntiles, maxcnt, iters;
  float hc_eps, norm_eps, rms_eps;
};


// Sum over the 4 lanes c, c+4, c+8, c+12 of a row of 16 (one column of a 4x4
// block held one element per lane, lane 4j + c).  Rotating a row by 8 pairs
// lane l with l^8; the pair sums are then rotated by 4, which lands in the
// other pair whichever way the rotation runs: each lane adds the same two
// pair sums, so all four lanes get the same bits.
template <int CTRL>
__device__ __forceinline__ float row_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float col4_sum(float v) {
  const float u = v + row_dpp<0x128>(v);          // row_ror:8
  return u + row_dpp<0x124>(u);                   // row_ror:4
}
__device__ __forceinline__ float quad_max(float v) {
  const float u = fmaxf(v, quad_perm<0xB1>(v));
  return fmaxf(u, quad_perm<0x4E>(u));
}

template <bool NORM>
__global__ void __launch_bounds__(kWThreads, 1) sweep_kernel(const SweepArgs a) {
  __shared__ u32x4 w_lds[kWSt][kHC][kNT][64];      // the slice's weight tiles (100 KB)
  __shared__ u32x4 a_lds[2][kWSt][kHC][64];        // X' in A layout, by tile parity (40 KB)
  __shared__ float cin[2][kWT][kWCin];             // post_in, comb_in, by tile parity
  __shared__ float bcl[2][kWT][kHC + 1];           // pre and RMSNorm factor, by tile parity
  __shared__ float gsc[kWS][kWRec];                // owner: one token's records of all slices
  __shared__ float tot[2][kWRec];                  // owner: summed, by tile parity

  constexpr int d = kWD;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x % kWX, p = blockIdx.x / kWX;
  const int cnt = a.ntiles > x ? (a.ntiles - x + kWX - 1) / kWX : 0;   // tiles of this XCD
  const int K = cnt > 0 ? cnt + kWLag : 0;                            // the last interval's k
  // intervals k = -1 .. J-2: K + 1 of them, padded to a multiple of 8 (the
  // stream waves' loop is unrolled eight times with no early exit)
  const int J = (K + 1 + kWXS - 1) / kWXS * kWXS;
  u32* err = a.ctrl + kErrWord;
  const u32 epoch = __hip_atomic_load(a.ctrl + kWEpochWord + 16 * x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto tag_of = [&](int i) __attribute__((always_inline)) { return epoch + 1u + (u32)i; };
  auto tok0 = [&](int i) __attribute__((always_inline)) { return (int64_t)(x + kWX * i) * kWT; };   // first token of local tile i
  const int fs = p * kWF;                          // first feature of the slice (per stream)

  // ---- the slice's weight tiles into LDS (once)
  for (int idx = threadIdx.x; idx < kWSt * kHC * kNT * 64; idx += kWThreads) {
    const int l = idx & 63, nt = (idx >> 6) % kNT, k = (idx / (64 * kNT)) % kHC, s = idx / (64 * kNT * kHC);
    const int gstep = fs / kStepF + s;
    w_lds[s][k][nt][l] = a.fn[((size_t)(gstep * kHC + k) * kNT + nt) * 64 + l];
  }

  if (wave < kWSW) {
    // ======================================================== stream waves
    // Every memory access goes through a buffer resource sized to the tile's
    // valid tokens (0 for a tile past the end): tokens past n read zeros and
    // store nothing, with no branch, so every interval issues the same memory
    // instructions and the loads of the next two tiles stay in flight.
    const int u = wave * 64 + lane;
    const int tau = u / kWG8, g = u % kWG8;
    const int f = fs + 8 * g;                      // this lane's first feature (per stream)
    const int a_s = g >> 2, a_lane = (g & 3) * 16 + tau;
    const u32 xoff = (u32)((tau * kHC * d + f) * 2), doff = (u32)((tau * d + f) * 2);
    float gm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gm[e] = NORM ? a.gamma[f + e] : 1.f;
    u32x4 LS[2][kHC + 1];                          // loads in flight, by tile parity
    u32 XS[kWXS][kHC][4] = {};                     // X' kept for the read row, tile % 8
    auto valid_of = [&](int i) __attribute__((always_inline)) -> u32 {
      if (i < 0 || i >= cnt) return 0u;
      const int64_t left = a.n - tok0(i);
      return (u32)(left < kWT ? left : kWT);
    };
    auto issue = [&](int i, u32x4 (&L)[kHC + 1]) __attribute__((always_inline)) {
      const u32 v = valid_of(i);
      const int64_t t0 = v ? tok0(i) : 0;
      const rsrc_t rx = make_rsrc(a.x + t0 * kHC * d, v * (u32)(kHC * d * 2));
      const rsrc_t rd = make_rsrc(a.delta + t0 * d, v * (u32)(d * 2));
#pragma unroll
      for (int j = 0; j < kHC; ++j) L[j] = buf_ld(rx, xoff + (u32)(j * d * 2));
      L[kHC] = buf_ld(rd, doff);
    };
    // X' of tile i: stored, and into the A tile
    auto stream = [&](int i, const u32x4 (&L)[kHC + 1], u32 (&xp)[kHC][4]) __attribute__((always_inline)) {
      const u32 v = valid_of(i);
      const rsrc_t ro = make_rsrc(a.x_out + (v ? tok0(i) : 0) * kHC * d, v * (u32)(kHC * d * 2));
      const float* c = cin[i & 1][tau];
      float cpost[kHC], ccomb[kHC * kHC];
#pragma unroll
      for (int j = 0; j < kHC; ++j) cpost[j] = c[j];
#pragma unroll
      for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = c[kHC + j];
      post_8(L, cpost, ccomb, xp);
#pragma unroll
      for (int k = 0; k < kHC; ++k) buf_st(ro, xoff + (u32)(k * d * 2), u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
#pragma unroll
      for (int k = 0; k < kHC; ++k)
        a_lds[i & 1][a_s][k][a_swz(a_lane, a_s & 1)] = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
    };
    // the read row of tile i from its kept X'
    auto read_row = [&](int i, const u32 (&xp)[kHC][4]) __attribute__((always_inline)) {
      const u32 v = valid_of(i);
      const rsrc_t ry = make_rsrc(a.y_out + (v ? tok0(i) : 0) * d, v * (u32)(d * 2));
      const float* cf = bcl[i & 1][tau];
      float pr[kHC];
#pragma unroll
      for (int j = 0; j < kHC; ++j) pr[j] = cf[j];
      u32 yp[4];
      pre_8(xp, pr, yp);
      if constexpr (NORM) {
        const float r = cf[kHC];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          yp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(yp[e2]) * r), gm[2 * e2 + 1] * (bf_hi(yp[e2]) * r));
      }
      buf_st(ry, doff, u32x4{yp[0], yp[1], yp[2], yp[3]});
    };

    issue(0, LS[0]);
    issue(1, LS[1]);
    lds_barrier();                                 // weights, cin of tile 0 in place
    // interval k = j - 1, j = r (mod 8): the register sets are compile-time indices
    auto interval = [&](int j, auto R) __attribute__((always_inline)) {
      constexpr int r = decltype(R)::v;
      read_row(j - 1 - kWLag, XS[r]);
      stream(j, LS[r & 1], XS[r]);
      issue(j + 2, LS[r & 1]);
      lds_barrier();
    };
    for (int j0 = 0; j0 < J; j0 += kWXS) {
      interval(j0, IC<0>{});
      interval(j0 + 1, IC<1>{});
      interval(j0 + 2, IC<2>{});
      interval(j0 + 3, IC<3>{});
      interval(j0 + 4, IC<4>{});
      interval(j0 + 5, IC<5>{});
      interval(j0 + 6, IC<6>{});
      interval(j0 + 7, IC<7>{});
    }
  } else if (wave == kWSW) {
    // ======================================================== exchange wave A
    // Each interval: the read coefficients of tile k-6 (from their owners)
    // into LDS, post_in and comb_in of tile k+2, and the sums of squares and
    // Gram entries of tile k (record words 24..35).  Its global loads are
    // issued an interval before their data is used: in the compute unit's
    // memory pipeline they queue behind the stream waves' loads.
    bool dead = false;
    // post_in and comb_in of tile i: issued early, written to LDS late
    auto cin_load = [&](int i, float (&cv)[5]) __attribute__((always_inline)) {
      const int64_t t0 = tok0(i);
      const int tp = lane >> 2;                      // post_in: lane -> (token lane/4, stream lane%4)
      cv[0] = t0 + tp < a.n ? a.post_in[t0 * kHC + lane] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {                  // comb_in: 256 floats, 4 per lane
        const int e = lane + 64 * r;
        cv[1 + r] = t0 + e / (kHC * kHC) < a.n ? a.comb_in[t0 * kHC * kHC + e] : 0.f;
      }
    };
    auto cin_store = [&](int i, const float (&v)[5]) __attribute__((always_inline)) {
      cin[i & 1][lane >> 2][lane & 3] = v[0];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = lane + 64 * r;
        cin[i & 1][e / (kHC * kHC)][kHC + e % (kHC * kHC)] = v[1 + r];
      }
    };
    const rsrc_t rrec = make_rsrc(a.rec, (u32)kWRecBytes);
    // the read-coefficient words of tile i: lane w holds words w and w + 64 of
    // the tile's 80 (token w / 5, word w % 5)
    const int w0 = lane, w1 = lane + 64;
    auto coef_ok = [&](int i, int w) __attribute__((always_inline)) {
      return i >= 0 && i < cnt && w < kWT * (kHC + 1) && tok0(i) + w / (kHC + 1) < a.n;
    };
    auto coef_ptr = [&](int i, int w) __attribute__((always_inline)) -> const u64* {
      return a.coef + ((size_t)(x * kWRR + (i >= 0 ? i % kWRR : 0)) * kWT + w / (kHC + 1)) * kWCoefW + w % (kHC + 1);
    };
    // requests alternate between two register sets (the loop below is unrolled
    // twice), so that nothing waits for a load before the interval that uses it
    u64 cw[2][2] = {{0, 0}, {0, 0}};
    float cvv[2][5];
    if (cnt > 0) { cin_load(0, cvv[0]); cin_store(0, cvv[0]); }
    if (cnt > 1) cin_load(1, cvv[1]);
    lds_barrier();
    auto xa_interval = [&](int k, auto B) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::v;              // this interval's request set; 1 - b holds the last
      const int ic = k - (kWLag - 1);                // consumed now; ic + 1 requested
      // ---- this interval's requests first (ahead of the stream waves' loads
      // in the CU's memory pipeline), used in the next interval: the read
      // coefficients of tile k-5, post_in and comb_in of tile k+3
      if (coef_ok(ic + 1, w0)) cw[b][0] = get_word(coef_ptr(ic + 1, w0));
      if (coef_ok(ic + 1, w1)) cw[b][1] = get_word(coef_ptr(ic + 1, w1));
      if (k + 3 < cnt) cin_load(k + 3, cvv[b]);
      // ---- last interval's requests: the read coefficients of tile k-6 into
      // LDS (a word not there yet is polled), post_in and comb_in of tile k+2
      if (ic >= 0 && ic < cnt) {
        const u32 tg = tag_of(ic);
        if (coef_ok(ic, w0))
          bcl[ic & 1][w0 / (kHC + 1)][w0 % (kHC + 1)] = settle(coef_ptr(ic, w0), cw[1 - b][0], tg, err, dead);
        if (coef_ok(ic, w1))
          bcl[ic & 1][w1 / (kHC + 1)][w1 % (kHC + 1)] = settle(coef_ptr(ic, w1), cw[1 - b][1], tg, err, dead);
      }
      if (k + 2 < cnt) cin_store(k + 2, cvv[1 - b]);
      // ---- tile k: sum x'^2 and the Gram entries of each token from the A tile
      // (X' of tile k), words 24..35 of its record.  Lane 4*tau + c takes the
      // feature groups c, c+4, .., c+16 of token tau (all four streams each);
      // the four lanes of a token then sum by DPP.
      if (k >= 0 && k < cnt) {
        const int tau = lane >> 2, c = lane & 3;
        float sq[kGram + 1];
#pragma unroll
        for (int q = 0; q <= kGram; ++q) sq[q] = 0.f;
#pragma unroll
        for (int m = 0; m < kWG8 / 4; ++m) {
          const int g = c + 4 * m, gs = g >> 2, gl = (g & 3) * 16 + tau;
          u32x4 xv[kHC];
#pragma unroll
          for (int kk = 0; kk < kHC; ++kk) xv[kk] = a_lds[k & 1][gs][kk][a_swz(gl, gs & 1)];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int kk = 0; kk < kHC; ++kk) sq[0] = dot2_bf16(xv[kk][e], xv[kk][e], sq[0]);
            int q = 1;
#pragma unroll
            for (int j2 = 0; j2 < kHC; ++j2)
#pragma unroll
              for (int l2 = j2; l2 < kHC; ++l2, ++q) sq[q] = dot2_bf16(xv[j2][e], xv[l2][e], sq[q]);
          }
        }
#pragma unroll
        for (int q = 0; q <= kGram; ++q) sq[q] = quad_sum(sq[q]);
        // the token's 12 words (sum x'^2, 10 Gram entries, a pad) in two runs of
        // 16-byte stores: lanes c = 0..3 words 2c, 2c+1, then lanes c = 0, 1
        // words 8 + 2c, 9 + 2c (every lane of a token holds all the sums)
        const u32 tg = tag_of(k);
        const u32 base = (u32)(((((x * kWRR + k % kWRR) * kWS + p) * kWT + tau) * kWRecS + kWSq) * sizeof(u64));
        auto sq_at = [&](int q) __attribute__((always_inline)) {
          float v = 0.f;
#pragma unroll
          for (int qq = 0; qq <= kGram; ++qq) v = q == qq ? sq[qq] : v;
          return v;
        };
        auto put2 = [&](int q) __attribute__((always_inline)) {
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(sq_at(q)), tg, __float_as_uint(sq_at(q + 1)), tg},
                                                 rrec, base + (u32)(q * sizeof(u64)), 0, 16 /* device scope */);
        };
        put2(2 * c);
        if (c < 2) put2(8 + 2 * c);
      }
      lds_barrier();
    };
    // intervals k = -1 .. J-2 (J is even): request set 0 at odd k, 1 at even k
    for (int k = -1; k < J - 1; k += 2) {
      xa_interval(k, IC<0>{});
      xa_interval(k + 1, IC<1>{});
    }
  } else if (wave == kWSW + 2) {
    // ======================================================== projection wave
    // Interval k: the 24 dots of tile k on the matrix cores (X' in the LDS A
    // tile, written by the stream waves in interval k-1; the slice's weight
    // tiles resident in LDS), K-outer so that each A operand is read once;
    // then the tile's dots are published, words 0..23 of the token records
    // (tagged).  It never waits on global memory.
    const rsrc_t rrec = make_rsrc(a.rec, (u32)kWRecBytes);
    const int col = lane & 15, grp = lane >> 4;
    lds_barrier();
    for (int k = -1; k < J - 1; ++k) {
      if (k >= 0 && k < cnt) {
        f32x4 acc[kNT][2];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K step st = 4*s + kk; its A and five B operands are read from LDS two
        // steps ahead of their matrix-core instructions (scheduling barriers
        // keep the reads there)
        constexpr int kSteps = kWSt * kHC, kAhead = 2;
        u32x4 Ab[kAhead + 1], Bb[kAhead + 1][kNT];
        auto fetch = [&](int st, u32x4& Ao, u32x4 (&Bo)[kNT]) __attribute__((always_inline)) {
          const int s = st / kHC, kk = st % kHC;
          Ao = a_lds[k & 1][s][kk][a_swz(lane, s & 1)];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) Bo[nt] = w_lds[s][kk][nt][lane];
        };
#pragma unroll
        for (int st = 0; st < kAhead; ++st) fetch(st, Ab[st], Bb[st]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          if (st + kAhead < kSteps) fetch(st + kAhead, Ab[(st + kAhead) % (kAhead + 1)], Bb[(st + kAhead) % (kAhead + 1)]);
          __builtin_amdgcn_sched_barrier(0);
          const int b = st % (kAhead + 1), h = st & 1;
          const bf16x8 A = __builtin_bit_cast(bf16x8, Ab[b]);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            acc[nt][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, Bb[b][nt]), acc[nt][h], 0,
                                                                0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        const u32 tg = tag_of(k);
        const u32 slot_base = (u32)((((x * kWRR + k % kWRR) * kWS + p) * kWT) * kWRecS * sizeof(u64));
        auto put = [&](int tau, int q, float v) __attribute__((always_inline)) {
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, tag_word(v, tg)), rrec,
                                                slot_base + (u32)((tau * kWRecS + q) * sizeof(u64)), 0,
                                                16 /* device scope */);
        };
        // dots: lane holds rows (tokens) 4*grp + r of column col of each weight tile
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t0 = acc[0][0][r] + acc[0][1][r], t1 = acc[1][0][r] + acc[1][1][r];
          const float t2 = acc[2][0][r] + acc[2][1][r], t3 = acc[3][0][r] + acc[3][1][r];
          const float t4 = acc[4][0][r] + acc[4][1][r];
          const float d0 = (t0 + t1) + t2;                      // row col: hi + mid + lo
          const float d1 = (t3 + row_dpp<0x128>(t3)) + t4;      // row 16 + col (col < 8): hi, mid, lo
          put(4 * grp + r, col, d0);
          if (col < 8) put(4 * grp + r, 16 + col, d1);
        }
      }
      lds_barrier();
    }
  } else {
    // ======================================================== exchange wave B (owner)
    // A slice owns one token of every other tile.  Interval k, owner of a token
    // of tile k-3: its records from all 32 slices (published three intervals
    // ago, requested at the start of the last interval) are checked and summed
    // in slice order, and the read coefficients (pre and the RMSNorm factor)
    // are derived and published at once, with the mixes, pre and post.
    // Interval k, owner of a token of tile k-2 and k-4: the records of tile k-2
    // are requested, and the Sinkhorn comb of the token of tile k-4 runs (only
    // an output, nothing in the call waits for it).
    bool dead = false;
    const rsrc_t rrec = make_rsrc(a.rec, (u32)kWRecBytes);
    auto owned = [&](int i) __attribute__((always_inline)) -> int {   // token of tile i this slice owns, or -1
      const int tau = p - kWT * (i & 1);
      if (i < 0 || i >= cnt || tau < 0 || tau >= kWT || tok0(i) + tau >= a.n) return -1;
      return tau;
    };
    constexpr int kGL = kWS * kWRec / 2 / 64;        // 16-byte loads per lane (9)
    static_assert(kGL * 64 * 2 == kWS * kWRec, "gather covers all record words");
    // chunk c: slice c / 18, compact words 2h, 2h+1 (h = c % 18) at record word
    // 2h (dots, h < 12) or kWSq + 2(h - 12) (the sums)
    auto cword = [&](int c) __attribute__((always_inline)) {
      const int h = c % (kWRec / 2);
      return h < kMix / 2 ? 2 * h : kWSq + 2 * (h - kMix / 2);
    };
    // the split parameters, loaded once: no later parameter load waits behind
    // this wave's device-scope stores (one in-order counter covers both)
    const float s0 = a.hc_scale[0], s1 = a.hc_scale[1], s2 = a.hc_scale[2];
    const float base_m = lane < kMix ? a.hc_base[lane] : 0.f;                  // base[lane]
    const float base_c = lane < kHC * kHC ? a.hc_base[2 * kHC + lane] : 0.f;   // base[8 + lane]
    auto base_at = [&](int q) __attribute__((always_inline)) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, base_m), q));
    };
    // the records of the owned token of tile i, lane: words 2c, 2c+1, c = lane + 64r
    auto goff = [&](int i, int tau, int r) __attribute__((always_inline)) -> u32 {
      const int c = lane + 64 * r, s = c / (kWRec / 2);
      return (u32)(((((x * kWRR + i % kWRR) * kWS + s) * kWT + tau) * kWRecS + cword(c)) * sizeof(u64));
    };
    u32x4 gv[kGL];                                   // requested at the start of the interval before
    lds_barrier();
    for (int k = -1; k < J - 1; ++k) {
      // ---- request the records of tile k-2 (published two intervals ago),
      // first in the interval: summed in the next one
      const int in = k - 2, tn = owned(in);
      if (tn >= 0) {
#pragma unroll
        for (int r = 0; r < kGL; ++r) gv[r] = __builtin_amdgcn_raw_buffer_load_b128(rrec, goff(in, tn, r), 0, 16);
      }
      // ---- tile k-3: check the records, sum, read coefficients, mixes, pre, post
      const int ig = k - 3, tg_tau = owned(ig);
      if (tg_tau >= 0) {
        const u32 tg = tag_of(ig);
        unsigned polls = 0;
        while (!dead) {
          bool ok = true;
#pragma unroll
          for (int r = 0; r < kGL; ++r) ok = ok && gv[r][1] == tg && gv[r][3] == tg;
          if (__all(ok)) break;
          if (++polls > kPollLimit) { if (lane == 0) atomicOr(err, kErrPollTimeout); dead = true; break; }
          __builtin_amdgcn_s_sleep(2);
#pragma unroll
          for (int r = 0; r < kGL; ++r) gv[r] = __builtin_amdgcn_raw_buffer_load_b128(rrec, goff(ig, tg_tau, r), 0, 16);
        }
#pragma unroll
        for (int r = 0; r < kGL; ++r) {
          const int c = lane + 64 * r;
          *reinterpret_cast<f32x2*>(&gsc[(2 * c) / kWRec][(2 * c) % kWRec]) =
              f32x2{__uint_as_float(gv[r][0]), __uint_as_float(gv[r][2])};
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        // lane q < 36 sums word q over the slices in slice order (all reads first)
        float sacc = 0.f;
        if (lane < kWRec) {
          float v[kWS];
#pragma unroll
          for (int s = 0; s < kWS; ++s) v[s] = gsc[s][lane];
          sacc = v[0];
#pragma unroll
          for (int s = 1; s < kWS; ++s) sacc = sacc + v[s];
          tot[ig & 1][lane] = sacc;                  // for the comb, next interval
        }
        // the words the read needs, as wave-uniform values
        auto word = [&](int q) __attribute__((always_inline)) {
          return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sacc), q));
        };
        const int64_t t = tok0(ig) + tg_tau;
        const float rx = 1.0f / sqrtf(word(kMix) / (float)(kHC * d) + a.norm_eps);
        float pre[kHC];
#pragma unroll
        for (int l = 0; l < kHC; ++l) pre[l] = sigmoidf_((word(l) * rx) * s0 + base_at(l)) + a.hc_eps;
        float rn = 1.f;
        if constexpr (NORM) {
          // sum_i y_i^2 = p^T G p over the whole row
          double yy = 0.0;
          int q = 0;
#pragma unroll
          for (int l = 0; l < kHC; ++l)
#pragma unroll
            for (int l2 = l; l2 < kHC; ++l2, ++q)
              yy += (l == l2 ? 1.0 : 2.0) * (double)pre[l] * (double)pre[l2] * (double)word(kMix + 1 + q);
          rn = 1.0f / sqrtf((float)(yy / (double)d) + a.rms_eps);
        }
        u64* cw = a.coef + ((size_t)(x * kWRR + ig % kWRR) * kWT + tg_tau) * kWCoefW;
        if (lane <= kHC) put_word(cw + lane, tag_word(lane == 0 ? pre[0] : lane == 1 ? pre[1] : lane == 2 ? pre[2]
                                                        : lane == 3 ? pre[3] : rn, tg));
        if (a.mixes_out && lane < kMix) a.mixes_out[t * kMix + lane] = sacc * rx;
        if (lane < kHC) {
          const float pj = lane == 0 ? pre[0] : lane == 1 ? pre[1] : lane == 2 ? pre[2] : pre[3];
          a.pre_out[t * kHC + lane] = pj;
        } else if (lane < 2 * kHC) {
          a.post_out[t * kHC + lane - kHC] = 2.0f * sigmoidf_((sacc * rx) * s1 + base_m);
        }
      }
      // ---- tile k-4: the comb, softmax (+eps) along the rows, a column step,
      // then iters-1 rounds of (row, column)
      const int ih = k - 4, th = owned(ih);
      if (th >= 0 && lane < kHC * kHC) {
        const float* rc = tot[ih & 1];
        const float rx = 1.0f / sqrtf(rc[kMix] / (float)(kHC * d) + a.norm_eps);
        float A = (rc[2 * kHC + lane] * rx) * s2 + base_c;
        const float mxr = quad_max(A);
        A = expf(A - mxr);
        A = A * __builtin_amdgcn_rcpf(quad_sum(A)) + a.hc_eps;
        A = A * __builtin_amdgcn_rcpf(col4_sum(A) + a.hc_eps);
        for (int it = 1; it < a.iters; ++it) {
          A = A * __builtin_amdgcn_rcpf(quad_sum(A) + a.hc_eps);
          A = A * __builtin_amdgcn_rcpf(col4_sum(A) + a.hc_eps);
        }
        a.comb_out[(tok0(ih) + th) * kHC * kHC + lane] = A;
      }
      lds_barrier();
    }
  }
  // ---- the last workgroup out advances the epoch for the next call
  if (threadIdx.x == 0) {
    const u32 done = __hip_atomic_fetch_add(a.ctrl + kWDoneWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (u32)kWGrid - 1u) {
      for (int i = 0; i < kWX; ++i)
        __hip_atomic_store(a.ctrl + kWEpochWord + 16 * i, epoch + 2u + (u32)a.maxcnt, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctrl + kWDoneWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ======================================================= decode boundary
// decode_kernel<POST, READ>: the boundary for few tokens in one launch, the
// finalize (split + Sinkhorn) done by the last feature slice of each token tile
// to finish ("Source layer, pairs pooled": Block.forward at decode, the read
// taking the given pre; "Reading weights" for the split).  No workgroup waits
// for another, so the launch needs no co-residency.
//
// Work items are (tile of kDT = 16 tokens, slice of kDF = 256 features of each
// stream), one workgroup each.  A workgroup streams its item (hc_post, X'
// stored, the read row y = sum_j pre_j X'_j stored), projects X' on the
// matrix cores with all of its weight tiles loaded into registers at the start,
// and writes the item's per-token record (24 dots, sum x'^2) to the workspace
// as tagged words (value, tile epoch).  It then counts itself in on the tile's
// arrival word; the slice that arrives last sums the S records of each token in
// slice order (the same bits whichever slice it is), waiting for any word not
// yet visible, and derives mixes, pre/post and the Sinkhorn comb.
//
// Words carry the workspace's call epoch (+1): every workgroup reads it at the
// start, and it advances only once every tile's last slice is known, so the
// tags grow from call to call whatever n and d are (a captured graph stays
// valid across replays).  A tile's arrival word and the tiles-done word are
// reset by their last arriver, found as the arrival whose count before it is
// S-1 (tiles-1) modulo S (tiles): exactly one in any run of S (tiles).  The
// record words must not hold the current tag before the first call: a zeroed
// workspace never does.
constexpr int kDT = 16;                      // tokens per tile
constexpr int kDF = 256;                     // features per slice and stream
constexpr int kDSteps = kDF / kStepF;        // 32-feature steps per slice (8)
constexpr int kDThreads = 256;               // 4 waves: 2 steps each in the projection
constexpr int kDRec = 25;                    // record words per token: 24 dots, sum x'^2
constexpr int kDMaxN = 128;                  // decode schedule up to this many tokens (measured crossover)
constexpr int kDTiles = kDMaxN / kDT;        // tiles at most (the region is sized for them)
constexpr int kDArriveBytes = 256;           // arrival, epoch and tiles-done words: head of the decode region
static_assert(kDArriveBytes >= (kDTiles + 2) * (int)sizeof(unsigned long long), "arrival words");

struct DecArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const float* pre_in;
  const u32x4* fn;
  const float* hc_base;
  const float* hc_scale;
  hc_bf16* x_out;
  hc_bf16* y_out;
  hc_bf16* x_mean;    // mean over the streams of X' (MTP tap), or NULL
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  int xtok, xstr;     // elements per token / per stream of x (hc*d, d; or d, 0 when expanded)
  u64* rec;           // [tiles][S][kDT][kDRec] tagged words
  u64* arrive;        // [kDTiles] arrival words, then the epoch word and the tiles-done word
  u32* err;           // sticky error mask (a wait timed out)
  int tiles;
  int64_t n;
  int d, S, iters;
  float hc_eps, norm_eps;
};

template <bool POST, bool READ>
__global__ void __launch_bounds__(kDThreads) decode_kernel(const DecArgs a) {
  __shared__ u32x4 a_lds[kDSteps][kHC][64];            // X' in A layout (32 KB)
  __shared__ float red[kDThreads / 64][kDT][32];       // per-wave dots
  __shared__ float ssq[4][kDT];                        // sum x'^2 per chunk
  __shared__ float tot[kDT][kDRec];                    // the tile's summed records (last slice)
  __shared__ float s_cf[kMix + 3];                     // hc_base, hc_scale (read by the last slice)
  __shared__ u32 s_tag, s_last;

  const int S = a.S, d = a.d;
  // the split's parameters, requested now so that the last slice's derive does
  // not wait for them
  if (a.pre_out && threadIdx.x < kMix + 3)
    s_cf[threadIdx.x] = threadIdx.x < kMix ? a.hc_base[threadIdx.x] : a.hc_scale[threadIdx.x - kMix];
  // XCD-aware numbering: consecutive workgroups land on different XCDs, so
  // they are renumbered XCD by XCD and taken slice-major, the workgroups of an
  // XCD sharing few slices (their weight tiles stay in that XCD's L2)
  const int G = gridDim.x;
  const int lin = (G & 7) ? blockIdx.x : (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int slice = lin / a.tiles, tile = lin % a.tiles;
  const int64_t t0 = (int64_t)tile * kDT;
  const int fs = slice * kDF;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = (threadIdx.x >> 3) & (kDT - 1);        // token of the tile
  const int fl = (threadIdx.x & 7) * 8;                // first feature within the chunk
  const int half = threadIdx.x >> 7;                   // chunk 2p + half in pass p
  const bool tv = t0 + m < a.n;
  const unsigned lt = tv ? (unsigned)m : 0u;

  // ---- the call's epoch
  u64* arw = a.arrive + tile;
  u64* epw = a.arrive + kDTiles;
  u64* donew = a.arrive + kDTiles + 1;
  if (threadIdx.x == 0) s_tag = (u32)get_word(epw) + 1u;   // words carry epoch + 1

  // ---- all loads up front: the weight tiles of this wave's two steps, the
  // streams of both passes and the token's coefficients
  bf16x8 B[2][kHC][kNT];
  {
    const int gstep = fs / kStepF + 2 * wave;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int k = 0; k < kHC; ++k)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          B[st][k][nt] = __builtin_bit_cast(bf16x8, a.fn[((size_t)((gstep + st) * kHC + k) * kNT + nt) * 64 + lane]);
  }
  u32x4 r[2][kHC + 1];
  const hc_bf16* xrow = a.x + (t0 + lt) * a.xtok;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int f = fs + (2 * p + half) * kCF + fl;
#pragma unroll
    for (int j = 0; j < kHC; ++j) r[p][j] = ld_stream(reinterpret_cast<const u32x4*>(xrow + (j * a.xstr + f)));
    r[p][kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(a.delta + (t0 + lt) * d + f)) : u32x4{0u, 0u, 0u, 0u};
  }
  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    cpost[j] = POST ? a.post_in[(t0 + lt) * kHC + j] : 0.f;
    cpre[j] = READ ? a.pre_in[(t0 + lt) * kHC + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = POST ? a.comb_in[(t0 + lt) * kHC * kHC + j] : 0.f;

  // ---- streams: X', the read row, sum x'^2, the A tile
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = 2 * p + half;
    const int f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    if constexpr (POST) {
      post_8(r[p], cpost, ccomb, xp);
      if (tv) {
#pragma unroll
        for (int k = 0; k < kHC; ++k)
          st_stream(reinterpret_cast<u32x4*>(a.x_out + (t0 + lt) * kHC * d + k * d + f),
                    u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
      }
    } else {
#pragma unroll
      for (int k = 0; k < kHC; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[k][e] = r[p][k][e];
    }
    if (a.x_mean && tv) st_stream(reinterpret_cast<u32x4*>(a.x_mean + (t0 + lt) * d + f), mean_8(xp));
    if constexpr (READ) {
      u32 yp[4];
      pre_8(xp, cpre, yp);
      if (tv) st_stream(reinterpret_cast<u32x4*>(a.y_out + (t0 + lt) * d + f), u32x4{yp[0], yp[1], yp[2], yp[3]});
    }
    float sx = 0.f;
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sx = dot2_bf16(xp[k][e], xp[k][e], sx);
      // step 2c + fl/32 of the slice; matrix-core lane (fl/8 % 4) * 16 + token
      a_lds[2 * c + (fl >> 5)][k][((fl >> 3) & 3) * 16 + m] = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
    }
    sx = oct_sum(sx);
    if ((threadIdx.x & 7) == 0) ssq[c][m] = sx;
  }
  __syncthreads();

  // ---- projection: wave w takes steps 2w, 2w+1 of the slice
  f32x4 acc[kAcc];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int k = 0; k < kHC; ++k)
      mfma_step(__builtin_bit_cast(bf16x8, a_lds[2 * wave + st][k][lane]), B[st][k], acc);
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[wave][4 * (lane >> 4) + rr][t * 16 + (lane & 15)] = acc[t][rr];
  __syncthreads();

  // ---- this slice's record of the tile, then count in
  const u32 tag = s_tag;
  u64* rt = a.rec + (size_t)tile * S * kDT * kDRec;
  for (int idx = threadIdx.x; idx < kDT * kDRec; idx += kDThreads) {
    const int tm = idx / kDRec, q = idx % kDRec;
    float v;
    if (q < kMix) {
      auto col = [&](int w, int cq) { return cq < 16 ? red[w][tm][cq] : red[w][tm][cq] + red[w][tm][cq + 8]; };
      v = ((col(0, q) + col(1, q)) + col(2, q)) + col(3, q);
    } else {
      v = ((ssq[0][tm] + ssq[1][tm]) + ssq[2][tm]) + ssq[3][tm];
    }
    put_word(rt + ((size_t)slice * kDT + tm) * kDRec + q, tag_word(v, tag));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const u64 before = __hip_atomic_fetch_add(arw, (u64)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before % (u64)S == (u64)(S - 1);
    if (s_last) {
      put_word(arw, 0ull);                       // every slice of the tile has counted in
      // every workgroup of the call has read the epoch once every tile's last
      // slice is known: the last of those advances it for the next call
      const u64 b2 = __hip_atomic_fetch_add(donew, (u64)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b2 % (u64)a.tiles == (u64)(a.tiles - 1)) {
        put_word(donew, 0ull);
        put_word(epw, (u64)s_tag);               // epoch + 1
      }
    }
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the last slice: sum the S records of each token in slice order; a
  // thread's words of all slices are requested together (one round trip)
  bool dead = false;
  constexpr int kPairs = (kDT * kDRec + kDThreads - 1) / kDThreads;   // (token, word) pairs per thread
  constexpr int kBatch = 32;                                          // slices in flight per pair
  for (int b0 = 0; b0 < S; b0 += kBatch) {
    u64 w[kPairs][kBatch];
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int idx = threadIdx.x + i * kDThreads;
      const u64* p0 = rt + (size_t)(idx / kDRec) * kDRec + idx % kDRec;   // slice b at + b * kDT * kDRec
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        w[i][b] = (idx < kDT * kDRec && b0 + b < S) ? get_word(p0 + (size_t)(b0 + b) * kDT * kDRec) : 0ull;
    }
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int idx = threadIdx.x + i * kDThreads;
      if (idx >= kDT * kDRec) continue;
      const int tm = idx / kDRec, q = idx % kDRec;
      const u64* p0 = rt + (size_t)tm * kDRec + q;
      float s = b0 == 0 ? 0.f : tot[tm][q];
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (b0 + b < S) {
          const float v = settle(p0 + (size_t)(b0 + b) * kDT * kDRec, w[i][b], tag, a.err, dead);
          s = b0 + b == 0 ? v : s + v;
        }
      tot[tm][q] = s;
    }
  }
  __syncthreads();
  // ---- derive: 4 lanes (a quad) per token, lane j holding comb row j
  if (threadIdx.x < kDT * kHC) {
    const int tm = threadIdx.x >> 2, j = threadIdx.x & 3;
    const int64_t t = t0 + tm;
    const bool valid = t < a.n;
    const float* rec = tot[tm];
    const float rx = 1.0f / sqrtf(rec[kMix] / (float)(kHC * d) + a.norm_eps);
    if (valid && a.mixes_out) {
#pragma unroll
      for (int i = 0; i < kMix / kHC; ++i) a.mixes_out[t * kMix + i * kHC + j] = rec[i * kHC + j] * rx;
    }
    if (a.pre_out) {
      const float s0 = s_cf[kMix], s1 = s_cf[kMix + 1], s2 = s_cf[kMix + 2];
      const float pre = sigmoidf_((rec[j] * rx) * s0 + s_cf[j]) + a.hc_eps;
      const float post = 2.0f * sigmoidf_((rec[kHC + j] * rx) * s1 + s_cf[kHC + j]);
      float A[kHC];
      float mxr = -INFINITY;
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        const int q = 2 * kHC + j * kHC + k;
        A[k] = (rec[q] * rx) * s2 + s_cf[q];
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
      if (valid) {
        a.pre_out[t * kHC + j] = pre;
        a.post_out[t * kHC + j] = post;
        *reinterpret_cast<f32x4*>(a.comb_out + t * kHC * kHC + j * kHC) = f32x4{A[0], A[1], A[2], A[3]};
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

bool hc_known(int hc) { return hc == 2 || hc == kHC || hc == 8; }

int check_hd(int hc, int d) {
  if (!hc_known(hc)) return fail(HC_ENOTSUP, "hc=%d: hc must be 2, 4 or 8", hc);
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
size_t split_records_bytes(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return (size_t)tiles * stream_slices(n, d) * kTT * kRec * 4;
}
bool fused_shape(int d) { return d % kFF == 0 && d >= kFMinD && d <= kMaxD; }
size_t fused_records_bytes(int64_t n, int d) {
  if (!fused_shape(d)) return 0;
  const int64_t tiles = (n + kFT - 1) / kFT;
  return (size_t)tiles * (d / kFF) * kFT * kFRec * sizeof(u64);
}
// decode schedule: given pre (or no read), no RMSNorm, few tokens.  Its region
// has a fixed place and size for a width d (whatever n), so a record slot only
// ever holds words of the same tile.
bool decode_shape(int64_t n, int d) { return n <= kDMaxN && d % kDF == 0; }
size_t decode_region_bytes(int d) {
  if (d % kDF != 0) return 0;
  return kDArriveBytes + (size_t)kDTiles * (d / kDF) * kDT * kDRec * sizeof(u64);
}
// slice-resident schedule (hc = 4, d = 5120): record ring, flags, read-coefficient words.
// Its region has a fixed place for a width d and nothing else writes there.
bool sweep_shape(int d) { return d == kWD; }
size_t sweep_region_bytes(int d) { return sweep_shape(d) ? kWRecBytes + kWCoefBytes : 0; }
size_t fixed_region_bytes(int d) { return kCtrlBytes + decode_region_bytes(d) + sweep_region_bytes(d); }
// [control block][decode arrival words + records][slice-resident ring][single-launch records][two-kernel records]
size_t workspace_bytes(int64_t n, int d) {
  return fixed_region_bytes(d) + fused_records_bytes(n, d) + split_records_bytes(n, d);
}

template <bool POST, int RM, bool NORM>
hipError_t launch_stream_t(const StreamArgs& a, unsigned grid, hipStream_t st) {
  StreamArgs copy = a;
  void* args[] = {&copy};
  const void* fn = a.x_mean ? reinterpret_cast<const void*>(&stream_kernel<POST, RM, NORM, true>)
                            : reinterpret_cast<const void*>(&stream_kernel<POST, RM, NORM, false>);
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads),
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
  s.rec = reinterpret_cast<float*>(static_cast<char*>(ws) + fixed_region_bytes(s.d) + fused_records_bytes(s.n, s.d));
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
  f.stok = post ? kHC * s.d : s.xtok;   // X' as written, or x as given (expanded: stride 0)
  f.sstr = post ? s.d : s.xstr;
  const unsigned grid2 = (unsigned)(tiles * f.S2);
  if (rm == kFreshPre) e = norm ? launch_finish_t<kFreshPre, true>(f, grid2, st) : launch_finish_t<kFreshPre, false>(f, grid2, st);
  else if (rm == kGivenPre && norm) e = launch_finish_t<kGivenPre, true>(f, grid2, st);
  else e = launch_finish_t<kNoRead, false>(f, grid2, st);
  return launched(e, what);
}

// ---- decode boundary
template <bool POST, bool READ>
hipError_t launch_decode_t(const DecArgs& a, unsigned grid, hipStream_t st) {
  DecArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<POST, READ>), dim3(grid), dim3(kDThreads), args,
                         0, st);
}
int launch_decode(bool post, bool read, DecArgs a, void* ws, size_t ws_bytes, hipStream_t st, const char* what) {
  const size_t need = workspace_bytes(a.n, a.d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  a.S = a.d / kDF;
  const int64_t tiles = (a.n + kDT - 1) / kDT;
  char* base = static_cast<char*>(ws) + kCtrlBytes;
  a.arrive = reinterpret_cast<u64*>(base);
  a.rec = reinterpret_cast<u64*>(base + kDArriveBytes);
  a.err = static_cast<u32*>(ws) + kErrWord;
  a.tiles = (int)tiles;
  const unsigned grid = (unsigned)(tiles * a.S);
  hipError_t e;
  switch ((post ? 2 : 0) | (read ? 1 : 0)) {
    case 0: e = launch_decode_t<false, false>(a, grid, st); break;
    case 1: e = launch_decode_t<false, true>(a, grid, st); break;
    case 2: e = launch_decode_t<true, false>(a, grid, st); break;
    default: e = launch_decode_t<true, true>(a, grid, st); break;
  }
  return launched(e, what);
}

// ---- single-launch boundary
template <bool POST, int RM, bool NORM>
hipError_t launch_fused_t(const FusedArgs& a, unsigned grid, hipStream_t st) {
  FusedArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fused_kernel<POST, RM, NORM>), dim3(grid), dim3(kFThreads),
                         args, 0, st);
}
const void* fused_fn(bool post, int rm, bool norm) {
  switch ((post ? 4 : 0) | (rm == kFreshPre ? 2 : 0) | (norm ? 1 : 0)) {
    case 0: return reinterpret_cast<const void*>(&fused_kernel<false, kGivenPre, false>);
    case 1: return reinterpret_cast<const void*>(&fused_kernel<false, kGivenPre, true>);
    case 2: return reinterpret_cast<const void*>(&fused_kernel<false, kFreshPre, false>);
    case 3: return reinterpret_cast<const void*>(&fused_kernel<false, kFreshPre, true>);
    case 4: return reinterpret_cast<const void*>(&fused_kernel<true, kGivenPre, false>);
    case 5: return reinterpret_cast<const void*>(&fused_kernel<true, kGivenPre, true>);
    case 6: return reinterpret_cast<const void*>(&fused_kernel<true, kFreshPre, false>);
    default: return reinterpret_cast<const void*>(&fused_kernel<true, kFreshPre, true>);
  }
}
// Workgroups of a variant that can be resident at once on the current device
// (compute units x workgroups per unit), queried once per device and variant.
int fused_capacity(bool post, int rm, bool norm) {
  constexpr int kDevs = 64;
  static int cache[kDevs][8];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  const int v = (post ? 4 : 0) | (rm == kFreshPre ? 2 : 0) | (norm ? 1 : 0);
  int c = __atomic_load_n(&cache[dev][v], __ATOMIC_RELAXED);
  if (c == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_fn(post, rm, norm), kFThreads, 0) != hipSuccess)
      return 0;
    c = cus * occ > 0 ? cus * occ : -1;
    __atomic_store_n(&cache[dev][v], c, __ATOMIC_RELAXED);
  }
  return c > 0 ? c : 0;
}

int launch_fused(bool post, int rm, bool norm, FusedArgs f, void* ws, size_t ws_bytes, hipStream_t st,
                 const char* what) {
  const size_t need = workspace_bytes(f.n, f.d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  f.S = f.d / kFF;
  const int64_t tiles = (f.n + kFT - 1) / kFT;
  const int64_t items = tiles * f.S;
  const int cap = fused_capacity(post, rm, norm);
  const int64_t g = std::min<int64_t>(items, (int64_t)(cap / f.S) * f.S);
  if (g < f.S) return fail(HC_ENOTSUP, "%s: the device holds %d resident workgroups, %d are needed", what, cap, f.S);
  f.tiles = (int)tiles;
  f.items = (int)items;
  f.rounds = (int)((items + g - 1) / g);
  f.ctrl = static_cast<u32*>(ws);
  f.rec = reinterpret_cast<u64*>(static_cast<char*>(ws) + fixed_region_bytes(f.d));
  const unsigned grid = (unsigned)g;
  hipError_t e;
  switch ((post ? 4 : 0) | (rm == kFreshPre ? 2 : 0) | (norm ? 1 : 0)) {
    case 0: e = launch_fused_t<false, kGivenPre, false>(f, grid, st); break;
    case 1: e = launch_fused_t<false, kGivenPre, true>(f, grid, st); break;
    case 2: e = launch_fused_t<false, kFreshPre, false>(f, grid, st); break;
    case 3: e = launch_fused_t<false, kFreshPre, true>(f, grid, st); break;
    case 4: e = launch_fused_t<true, kGivenPre, false>(f, grid, st); break;
    case 5: e = launch_fused_t<true, kGivenPre, true>(f, grid, st); break;
    case 6: e = launch_fused_t<true, kFreshPre, false>(f, grid, st); break;
    default: e = launch_fused_t<true, kFreshPre, true>(f, grid, st); break;
  }
  return launched(e, what);
}

// The slice-resident schedule needs its whole grid resident: one workgroup on
// each of the 256 compute units (8 XCDs x 32).  Checked once per device.
bool sweep_device_ok(bool norm) {
  constexpr int kDevs = 64;
  static int cache[kDevs][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return false;
  int c = __atomic_load_n(&cache[dev][norm], __ATOMIC_RELAXED);
  if (c == 0) {
    int cus = 0, occ = 0;
    const void* fn = norm ? reinterpret_cast<const void*>(&sweep_kernel<true>)
                          : reinterpret_cast<const void*>(&sweep_kernel<false>);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kWThreads, 0) != hipSuccess)
      return false;
    c = (cus == kWGrid && occ >= 1) ? 1 : -1;
    __atomic_store_n(&cache[dev][norm], c, __ATOMIC_RELAXED);
  }
  return c > 0;
}

int launch_sweep(bool norm, SweepArgs a, void* ws, size_t ws_bytes, hipStream_t st, const char* what) {
  const size_t need = workspace_bytes(a.n, kWD);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  if (!sweep_device_ok(norm))
    return fail(HC_ENOTSUP, "%s: the slice-resident schedule needs %d resident workgroups (one per compute unit)",
                what, kWGrid);
  const int64_t tiles = (a.n + kWT - 1) / kWT;
  a.ntiles = (int)tiles;
  a.maxcnt = (int)((tiles + kWX - 1) / kWX);
  char* base = static_cast<char*>(ws);
  a.ctrl = static_cast<u32*>(ws);
  a.rec = reinterpret_cast<u64*>(base + kCtrlBytes + decode_region_bytes(kWD));
  a.coef = reinterpret_cast<u64*>(reinterpret_cast<char*>(a.rec) + kWRecBytes);
  void* args[] = {&a};
  const void* fn = norm ? reinterpret_cast<const void*>(&sweep_kernel<true>)
                        : reinterpret_cast<const void*>(&sweep_kernel<false>);
  return launched(hipLaunchKernel(fn, dim3(kWGrid), dim3(kWThreads), args, 0, st), what);
}

template <bool POST, bool PRE, bool NORM, int TPW, int HC = kHC>
hipError_t launch_row_t(const RowArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.n + kWaves * TPW - 1) / (kWaves * TPW));
  // without the RMSNorm, few tokens: the 512-feature chunks of a row go to
  // several workgroups, aiming at about 512 of them
  const int nch = (a.d + kRowChunk - 1) / kRowChunk;
  const unsigned gy = NORM ? 1u : (unsigned)std::max(1, std::min<int>(nch, (int)((512 + grid - 1) / grid)));
  RowArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&row_kernel<POST, PRE, NORM, TPW, HC>), dim3(grid, gy),
                         dim3(kThreads), args, 0, st);
}

// hc other than 4: one token per wave, every stage combination
template <int HC>
hipError_t launch_row_hc(int key, const RowArgs& a, hipStream_t st) {
  switch (key) {
    case 0b100: return launch_row_t<true, false, false, 1, HC>(a, st);
    case 0b010: return launch_row_t<false, true, false, 1, HC>(a, st);
    case 0b110: return launch_row_t<true, true, false, 1, HC>(a, st);
    case 0b011: return launch_row_t<false, true, true, 1, HC>(a, st);
    default: return launch_row_t<true, true, true, 1, HC>(a, st);
  }
}

int launch_row(bool post, bool pre, bool norm, const RowArgs& a, hipStream_t st, const char* what, int hc = kHC) {
  const bool wide = norm && a.d > kRowChunk * kRowMaxChunks;
  if (norm && a.d > kRowChunk * kRowMaxChunks * 2)
    return fail(HC_ENOTSUP, "%s: RMSNorm of the read row supports d <= %d", what, kRowChunk * kRowMaxChunks * 2);
  const int key = (post ? 4 : 0) | (pre ? 2 : 0) | (norm ? 1 : 0);
  if (key != 0b100 && key != 0b010 && key != 0b110 && key != 0b011 && key != 0b111)
    return fail(HC_EINVAL, "%s: unsupported stage combination", what);
  hipError_t e;
  if (hc != kHC) {
    e = hc == 2 ? launch_row_hc<2>(key, a, st) : launch_row_hc<8>(key, a, st);
    return launched(e, what);
  }
  const bool few = a.n < 2048;                     // one token per wave: more workgroups
  switch (key) {
    case 0b100: e = few ? launch_row_t<true, false, false, 1>(a, st) : launch_row_t<true, false, false, 2>(a, st); break;
    case 0b010: e = few ? launch_row_t<false, true, false, 1>(a, st) : launch_row_t<false, true, false, 2>(a, st); break;
    case 0b110: e = few ? launch_row_t<true, true, false, 1>(a, st) : launch_row_t<true, true, false, 2>(a, st); break;
    case 0b011: e = wide ? launch_row_t<false, true, true, 1>(a, st) : launch_row_t<false, true, true, 2>(a, st); break;
    case 0b111: e = wide ? launch_row_t<true, true, true, 1>(a, st) : launch_row_t<true, true, true, 2>(a, st); break;
    default: return fail(HC_EINVAL, "%s: unsupported stage combination", what);
  }
  return launched(e, what);
}

// ------------------------------------------------------ hc other than 4
int gen_recw(int hc) { return hc == 2 ? GShape<2>::RECW : GShape<8>::RECW; }
int gen_nct(int hc) { return hc == 2 ? GShape<2>::NCT : GShape<8>::NCT; }

// slices of the flattened feature range: the largest divisor of hc*d/64 (a
// slice is whole 64-feature chunks) giving at most about 512 workgroups, 64
// slices at most
int gen_slices(int64_t n, int hc, int d) {
  const int64_t groups = (n + kGTok - 1) / kGTok;
  const int chunks = hc * d / kGChunk;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(64, (512 + groups - 1) / groups));
  int best = 1;
  for (int s = 1; s <= want; ++s)
    if (chunks % s == 0) best = s;
  return best;
}

// workspace of the hc != 4 path: the per-slice records, placed after the
// control block and the decode region of the same d so that a workspace
// shared with hc = 4 calls keeps their words intact
size_t gen_rec_offset(int d) { return fixed_region_bytes(d); }
size_t generic_ws_bytes(int64_t n, int hc, int d) {
  return gen_rec_offset(d) + (size_t)gen_slices(n, hc, d) * n * gen_recw(hc) * 4;
}

int check_generic_ws(int64_t n, int hc, int d, const void* ws, size_t ws_bytes, const char* what) {
  const size_t need = generic_ws_bytes(n, hc, d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  if ((n + kGTok - 1) / kGTok * gen_slices(n, hc, d) > INT32_MAX)
    return fail(HC_ENOTSUP, "%s: n=%lld is too large", what, (long long)n);
  return HC_OK;
}

// projection + split for hc 2 or 8: records into the workspace, then one
// token per lane sums them and derives mixes / pre, post, comb
int launch_mixes_generic(int hc, const hc_bf16* x, int xtok, int xstr, const void* fn, int64_t n, int d,
                         void* ws, GFinArgs f, hipStream_t st, const char* what) {
  GMixArgs m{};
  m.x = x; m.fn = static_cast<const u32x4*>(fn); m.n = n; m.xtok = xtok; m.xstr = xstr; m.d = d;
  m.S = gen_slices(n, hc, d);
  m.Fs = hc * d / m.S;
  m.rec = reinterpret_cast<float*>(static_cast<char*>(ws) + gen_rec_offset(d));
  void* margs[] = {&m};
  const dim3 mgrid((unsigned)((n + kGTok - 1) / kGTok * m.S));
  hipError_t e = hipLaunchKernel(hc == 2 ? reinterpret_cast<const void*>(&gmix_kernel<2>)
                                         : reinterpret_cast<const void*>(&gmix_kernel<8>),
                                 mgrid, dim3(kGThreads), margs, 0, st);
  int rc = launched(e, what);
  if (rc) return rc;
  f.rec = m.rec; f.n = n; f.S = m.S; f.K = hc * d;
  void* fargs[] = {&f};
  const int64_t tpb = 256 / hc;                   // tokens per workgroup: hc lanes each
  e = hipLaunchKernel(hc == 2 ? reinterpret_cast<const void*>(&gfinish_kernel<2>)
                              : reinterpret_cast<const void*>(&gfinish_kernel<8>),
                      dim3((unsigned)((n + tpb - 1) / tpb)), dim3(256), fargs, 0, st);
  return launched(e, what);
}

int launch_split(int hc, const float* mixes, const float* scale, const float* base, int64_t n, int iters,
                 float eps, float* pre, float* post, float* comb, hipStream_t st) {
  const int64_t tpb = 256 / hc;                   // tokens per workgroup: hc lanes each
  const dim3 grid((unsigned)((n + tpb - 1) / tpb)), block(256);
  if (hc == 2)
    hipLaunchKernelGGL(split_kernel<2>, grid, block, 0, st, mixes, scale, base, n, iters, eps, pre, post, comb);
  else if (hc == 8)
    hipLaunchKernelGGL(split_kernel<8>, grid, block, 0, st, mixes, scale, base, n, iters, eps, pre, post, comb);
  else
    hipLaunchKernelGGL(split_kernel<kHC>, grid, block, 0, st, mixes, scale, base, n, iters, eps, pre, post, comb);
  return launched(hipGetLastError(), "split_kernel");
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
  if (!hc_known(hc) || d <= 0 || d % kCF != 0 || d > kMaxD) return 0;
  if (hc != kHC) return (size_t)(hc * d / 32) * gen_nct(hc) * 64 * 16;
  return (size_t)(d / kStepF) * kHC * kNT * 64 * 16;
}

int hc_fn_pack(const float* hc_fn, int hc, int d, void* fn_packed, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  HC_REQ(hc_fn);
  HC_REQ(fn_packed);
  if ((rc = check_device())) return rc;
  if (hc != kHC) {
    const int recs = (hc * d / 32) * gen_nct(hc) * 64;
    if (hc == 2)
      hipLaunchKernelGGL(gpack_kernel<2>, dim3((recs + 255) / 256), dim3(256), 0, (hipStream_t)stream, hc_fn,
                         hc * d, reinterpret_cast<u32x4*>(fn_packed), recs);
    else
      hipLaunchKernelGGL(gpack_kernel<8>, dim3((recs + 255) / 256), dim3(256), 0, (hipStream_t)stream, hc_fn,
                         hc * d, reinterpret_cast<u32x4*>(fn_packed), recs);
    return launched(hipGetLastError(), "gpack_kernel");
  }
  const int records = (d / kStepF) * kHC * kNT * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((records + 255) / 256), dim3(256), 0, (hipStream_t)stream, hc_fn, d,
                     reinterpret_cast<u32x4*>(fn_packed), records);
  return launched(hipGetLastError(), "pack_kernel");
}

size_t hc_workspace_bytes(int64_t n, int hc, int d) {
  if (!hc_known(hc) || d <= 0 || d % kCF != 0 || d > kMaxD || n < 0) return 0;
  if (n == 0) return 0;
  if (hc != kHC) return generic_ws_bytes(n, hc, d);
  return workspace_bytes(n, d);
}

int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base, int64_t n, int hc,
                      int iters, float hc_eps, float* pre, float* post, float* comb, void* stream) {
  g_err[0] = 0;
  int rc;
  if (!hc_known(hc)) return fail(HC_ENOTSUP, "hc=%d: hc must be 2, 4 or 8", hc);
  if ((rc = check_n(n))) return rc;
  if (iters < 1) return fail(HC_EINVAL, "iters=%d: at least one Sinkhorn round is needed", iters);
  HC_REQ(mixes); HC_REQ(hc_scale); HC_REQ(hc_base); HC_REQ(pre); HC_REQ(post); HC_REQ(comb);
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  return launch_split(hc, mixes, hc_scale, hc_base, n, iters, hc_eps, pre, post, comb, (hipStream_t)stream);
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
  if (hc != kHC && (rc = check_generic_ws(n, hc, d, workspace, workspace_bytes, "hc_mixes"))) return rc;
  if ((rc = check_device())) return rc;
  if (hc != kHC) {
    const hipStream_t st = (hipStream_t)stream;
    GFinArgs f{};
    f.hc_scale = hc_scale; f.hc_base = hc_base; f.mixes_out = mixes; f.iters = iters; f.norm_eps = norm_eps;
    f.hc_eps = hc_eps;
    if (split) { f.pre_out = pre; f.post_out = post; f.comb_out = comb; }
    return launch_mixes_generic(hc, x, hc * d, d, fn_packed, n, d, workspace, f, st, "hc_mixes");
  }
  if (decode_shape(n, d)) {
    DecArgs a{};
    a.n = n; a.d = d; a.x = x; a.fn = reinterpret_cast<const u32x4*>(fn_packed); a.mixes_out = mixes;
    a.xtok = kHC * d; a.xstr = d;
    a.hc_scale = hc_scale; a.hc_base = hc_base; a.iters = iters; a.hc_eps = hc_eps; a.norm_eps = norm_eps;
    if (split) { a.pre_out = pre; a.post_out = post; a.comb_out = comb; }
    return launch_decode(false, false, a, workspace, workspace_bytes, (hipStream_t)stream, "hc_mixes");
  }
  StreamArgs s{};
  s.n = n; s.d = d; s.x = x; s.fn = reinterpret_cast<const u32x4*>(fn_packed);
  s.xtok = kHC * d; s.xstr = d;
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
  a.n = n; a.d = d; a.x = x; a.pre_in = pre_mix; a.y_out = y; a.xtok = hc * d; a.xstr = d;
  return launch_row(false, true, false, a, (hipStream_t)stream, "hc_pre", hc);
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
  a.xtok = hc * d; a.xstr = d;
  return launch_row(true, false, false, a, (hipStream_t)stream, "hc_post", hc);
}

size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d) { return hc_workspace_bytes(n, hc, d); }

static int boundary_phases(const hc_boundary_args* p, void* stream, int phases) {
  g_err[0] = 0;
  if (!p) return fail(HC_EINVAL, "args must not be NULL");
  constexpr size_t kNoFlags = offsetof(hc_boundary_args, flags);   // callers of the field-less struct
  if (p->struct_size < kNoFlags)
    return fail(HC_EINVAL, "struct_size=%u, expected %zu", p->struct_size, sizeof(hc_boundary_args));
  const uint32_t flags = p->struct_size >= kNoFlags + sizeof(uint32_t) ? p->flags : 0u;
  constexpr size_t kNoMean = offsetof(hc_boundary_args, x_mean_out);   // callers of the struct without it
  hc_bf16* const x_mean = p->struct_size >= kNoMean + sizeof(void*) ? p->x_mean_out : nullptr;
  if (flags & ~(HC_BOUNDARY_SINGLE_LAUNCH | HC_BOUNDARY_X_EXPANDED | HC_BOUNDARY_SLICE_RESIDENT))
    return fail(HC_EINVAL, "flags=%#x: unknown bits", flags);
  if ((flags & HC_BOUNDARY_SINGLE_LAUNCH) && (flags & HC_BOUNDARY_SLICE_RESIDENT))
    return fail(HC_EINVAL, "flags=%#x: pick one schedule", flags);
  const bool expanded = (flags & HC_BOUNDARY_X_EXPANDED) != 0;
  int rc = check_hd(p->hc, p->d);
  if (rc) return rc;
  if ((rc = check_n(p->n))) return rc;
  const bool post = p->delta != nullptr;
  const bool mix = p->fn_packed != nullptr;
  const bool fresh = p->pre_in == nullptr;
  const bool norm = p->gamma != nullptr;
  HC_REQ(p->x); HC_REQ(p->y_out); HC_OPT(p->delta); HC_OPT(p->pre_in); HC_OPT(p->gamma); HC_OPT(x_mean);
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
  if (flags & HC_BOUNDARY_SINGLE_LAUNCH) {
    if (p->hc != kHC) return fail(HC_ENOTSUP, "the single-launch schedule needs hc=4");
    if (expanded || x_mean) return fail(HC_ENOTSUP, "the single-launch schedule takes neither expanded streams nor x_mean_out");
    if (phases != 3) return fail(HC_EINVAL, "the single-launch schedule has no halves (use hc_boundary)");
    if (!mix) return fail(HC_EINVAL, "the single-launch schedule needs fn_packed");
    if (!fused_shape(p->d)) return fail(HC_ENOTSUP, "single launch: d=%d must be a multiple of %d, at least %d", p->d, kFF, kFMinD);
    if (p->n > kFusedMaxN) return fail(HC_ENOTSUP, "single launch: n=%lld is too large", (long long)p->n);
  }
  if (flags & HC_BOUNDARY_SLICE_RESIDENT) {
    if (p->hc != kHC || !sweep_shape(p->d))
      return fail(HC_ENOTSUP, "the slice-resident schedule needs hc=4 and d=%d", kWD);
    if (expanded || x_mean) return fail(HC_ENOTSUP, "the slice-resident schedule takes neither expanded streams nor x_mean_out");
    if (phases != 3) return fail(HC_EINVAL, "the slice-resident schedule has no halves (use hc_boundary)");
    if (!mix || !post || !fresh)
      return fail(HC_ENOTSUP, "the slice-resident schedule needs delta and fn_packed, and pre_in NULL");
    if (p->n > kFusedMaxN) return fail(HC_ENOTSUP, "slice-resident: n=%lld is too large", (long long)p->n);
  }
  if (p->n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  const hipStream_t st = (hipStream_t)stream;
  const int xtok = expanded ? p->d : p->hc * p->d;   // expanded: every stream reads x
  const int xstr = expanded ? 0 : p->d;

  if (!mix) {  // stack exit: write, read (+ norm); no projection; one kernel, the first phase
    if (!(phases & 1)) return HC_OK;
    RowArgs r{};
    r.n = p->n; r.d = p->d; r.x = p->x; r.delta = p->delta; r.post_in = p->post_in; r.comb_in = p->comb_in;
    r.pre_in = p->pre_in; r.gamma = p->gamma; r.x_out = p->x_out; r.y_out = p->y_out; r.rms_eps = p->rms_eps;
    r.xtok = xtok; r.xstr = xstr; r.x_mean = x_mean;
    return launch_row(post, true, norm, r, st, "hc_boundary (exit)", p->hc);
  }
  if (flags & HC_BOUNDARY_SLICE_RESIDENT) {
    SweepArgs w{};
    w.n = p->n; w.x = p->x; w.delta = p->delta; w.post_in = p->post_in; w.comb_in = p->comb_in;
    w.fn = reinterpret_cast<const u32x4*>(p->fn_packed); w.gamma = p->gamma; w.hc_base = p->hc_base;
    w.hc_scale = p->hc_scale; w.x_out = p->x_out; w.y_out = p->y_out; w.mixes_out = p->mixes_out;
    w.pre_out = p->pre_out; w.post_out = p->post_out; w.comb_out = p->comb_out; w.iters = p->iters;
    w.hc_eps = p->hc_eps; w.norm_eps = p->norm_eps; w.rms_eps = p->rms_eps;
    return launch_sweep(norm, w, p->workspace, p->workspace_bytes, st, "hc_boundary");
  }
  if (flags & HC_BOUNDARY_SINGLE_LAUNCH) {
    FusedArgs f{};
    f.n = p->n; f.d = p->d; f.x = p->x; f.delta = p->delta; f.post_in = p->post_in; f.comb_in = p->comb_in;
    f.pre_in = p->pre_in; f.fn = reinterpret_cast<const u32x4*>(p->fn_packed); f.gamma = p->gamma;
    f.hc_base = p->hc_base; f.hc_scale = p->hc_scale; f.x_out = p->x_out; f.y_out = p->y_out;
    f.mixes_out = p->mixes_out; f.pre_out = p->pre_out; f.post_out = p->post_out; f.comb_out = p->comb_out;
    f.iters = p->iters; f.hc_eps = p->hc_eps; f.norm_eps = p->norm_eps; f.rms_eps = p->rms_eps;
    return launch_fused(post, fresh ? kFreshPre : kGivenPre, norm, f, p->workspace, p->workspace_bytes, st,
                        "hc_boundary");
  }
  if (p->hc != kHC) {
    // hc 2 or 8: the write, the projection, the split and the read as separate
    // launches; begin does the write (and a read from a given pre), end the rest
    const int hc = p->hc, d = p->d;
    if ((rc = check_generic_ws(p->n, hc, d, p->workspace, p->workspace_bytes, "hc_boundary"))) return rc;
    RowArgs r{};
    r.n = p->n; r.d = d; r.x = p->x; r.delta = p->delta; r.post_in = p->post_in; r.comb_in = p->comb_in;
    r.gamma = p->gamma; r.x_out = p->x_out; r.y_out = p->y_out; r.rms_eps = p->rms_eps;
    r.xtok = xtok; r.xstr = xstr;
    if ((phases & 1) && (post || !fresh)) {
      RowArgs w = r;
      w.pre_in = fresh ? nullptr : p->pre_in;
      w.x_mean = x_mean;
      if ((rc = launch_row(post, !fresh, !fresh && norm, w, st, "hc_boundary (write)", hc))) return rc;
    }
    if (phases & 2) {
      const hc_bf16* src = post ? p->x_out : p->x;    // X'
      const int stok = post ? hc * d : xtok, sstr = post ? d : xstr;
      GFinArgs f{};
      f.hc_scale = p->hc_scale; f.hc_base = p->hc_base; f.mixes_out = p->mixes_out; f.pre_out = p->pre_out;
      f.post_out = p->post_out; f.comb_out = p->comb_out; f.iters = p->iters; f.norm_eps = p->norm_eps;
      f.hc_eps = p->hc_eps;
      if ((rc = launch_mixes_generic(hc, src, stok, sstr, p->fn_packed, p->n, d, p->workspace, f, st,
                                     "hc_boundary")))
        return rc;
      if (fresh) {
        RowArgs rd = r;
        rd.x = src; rd.xtok = stok; rd.xstr = sstr; rd.delta = nullptr; rd.post_in = nullptr; rd.comb_in = nullptr;
        rd.x_out = nullptr; rd.pre_in = p->pre_out; rd.x_mean = post ? nullptr : x_mean;
        return launch_row(false, true, norm, rd, st, "hc_boundary (read)", hc);
      }
    }
    return HC_OK;
  }
  if (phases == 3 && !fresh && !norm && decode_shape(p->n, p->d)) {
    DecArgs a{};
    a.n = p->n; a.d = p->d; a.x = p->x; a.delta = p->delta; a.post_in = p->post_in; a.comb_in = p->comb_in;
    a.pre_in = p->pre_in; a.fn = reinterpret_cast<const u32x4*>(p->fn_packed); a.hc_base = p->hc_base;
    a.hc_scale = p->hc_scale; a.x_out = p->x_out; a.y_out = p->y_out; a.mixes_out = p->mixes_out;
    a.pre_out = p->pre_out; a.post_out = p->post_out; a.comb_out = p->comb_out; a.iters = p->iters;
    a.hc_eps = p->hc_eps; a.norm_eps = p->norm_eps; a.xtok = xtok; a.xstr = xstr; a.x_mean = x_mean;
    return launch_decode(post, true, a, p->workspace, p->workspace_bytes, st, "hc_boundary");
  }
  StreamArgs s{};
  s.n = p->n; s.d = p->d; s.x = p->x; s.delta = p->delta; s.post_in = p->post_in; s.comb_in = p->comb_in;
  s.pre_in = p->pre_in; s.fn = reinterpret_cast<const u32x4*>(p->fn_packed); s.x_out = p->x_out;
  s.y_out = p->y_out; s.xtok = xtok; s.xstr = xstr; s.x_mean = x_mean;
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
