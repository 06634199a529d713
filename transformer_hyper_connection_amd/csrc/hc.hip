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
//   stream_kernel<RM, NORM, MEAN> + finish_kernel<RM, NORM>  everything that
//       derives mixes and writes X' (the sublayer boundary) at any n: 64-token
//       tiles x feature slices, about one workgroup per compute unit; the
//       24-wide projection on the matrix cores with the weight tiles shared
//       through LDS; the per-slice sums meet in the workspace, and the finish
//       derives the coefficients and writes the read row.
//   proj_kernel<RM, NORM, MEAN> + finish_kernel<RM, NORM>  the same with no
//       write (hc_mixes, block entry): 128-token workgroups, half the weight
//       traffic per token.
//   exchange_kernel<POST, MEAN, YK>  a given pre with the RMSNorm in one launch
//       (tiles of 4 to 8 slices of YK chunks): the slices of a tile exchange
//       their per-token sums as tagged words; the read row stays in registers.
//   xfew_kernel<POST, MEAN, READ, NORM, YK>  the same for few token tiles
//       (decode, short prefill: up to 2048 tokens at d = 5120), a given pre
//       or no read, with or without the RMSNorm: slices of 1 to 10 chunks, an
//       owner slice per token derives it and publishes its RMS factor.
//   sweep_row_kernel<POST, PRE, HC>, sweep_norm_kernel<POST, CPW, HC>  streams
//       only (hc_post, hc_pre, the stack exit) as a sweep through memory in
//       address order: a (token, 512-feature chunk) per wave, or a token per
//       workgroup with the RMSNorm.
//   row_kernel<POST, PRE, NORM, TPW, HC>  streams only where the sweeps do
//       not apply: whole token rows per wave, 1 KB per load or store.
//   split16_kernel, split_kernel<HC>  hc_split_sinkhorn: 16 lanes per token at
//       hc = 4 up to 8192 tokens (derive_16), else hc lanes per token.
//   pack_kernel     fp32 projection weight -> bf16 hi/mid/lo terms in tile order.
// hc = 2 and 8: the sweeps, row_kernel and split_kernel instantiated for that
//   hc, and gpack_kernel / gmix_kernel / gfinish_kernel<HC>, the projection on
//   the matrix cores with per-slice records and their finish (gstream_kernel<2>
//   fuses the write into the projection at hc = 2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <utility>
#include <cstdarg>
#include <cstdint>
#include <cstddef>
#include <cstdio>
#include <cstring>

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

// records [d/32 steps][kHC streams][kNT tiles][64 lanes] of the weight, then
// [d/32 steps][kNT tiles][64 lanes] of the weight summed over the four stream
// blocks (the projection of four identical streams, the expanded block entry:
// the sum taken in fp64 and rounded to fp32 once, then split the same way)
__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ fn, int d,
                                                   u32x4* __restrict__ out, int records) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= records) return;
  const int main_records = (d / kStepF) * kHC * kNT * 64;
  const bool summed = idx >= main_records;
  const int ridx = summed ? idx - main_records : idx;
  const int lane = ridx & 63;
  const int nt = (ridx >> 6) % kNT;
  const int k = summed ? 0 : (ridx / (64 * kNT)) % kHC;
  const int step = summed ? ridx / (64 * kNT) : ridx / (64 * kNT * kHC);
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
    for (int h = 0; h < 2; ++h) {
      float x = 0.f;
      if (q >= 0 && summed) {
        double sum = 0.0;
#pragma unroll
        for (int kk = 0; kk < kHC; ++kk) sum += (double)fn[(size_t)q * (kHC * d) + (size_t)kk * d + f0 + 2 * e2 + h];
        x = (float)sum;
      } else if (q >= 0) {
        x = fn[(size_t)q * (kHC * d) + (size_t)k * d + f0 + 2 * e2 + h];
      }
      v[h] = q < 0 ? 0.f : split_term(x, part);
    }
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

  // The A operand comes straight from memory in the matrix-core layout: 64
  // bytes of each of 16 token rows per instruction, the two steps' halves of
  // a 128-byte line back to back.  Plain (cached) loads, so that the two
  // halves meet in L2 as one line fill; nontemporal ones measured slower
  // (hc = 8: 314 against 306 us per boundary).
  auto load_a = [&](int ch, u32x4 (&A)[2][2]) {
    const int c = c0 + ch * kGChunk;              // a chunk never crosses a stream (d % 64 == 0)
    const int j = c / a.d, i = c - j * a.d + kg;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int st = 0; st < 2; ++st) A[ti][st] = *reinterpret_cast<const u32x4*>(xr[ti] + j * a.xstr + i + 32 * st);
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

// The stream-only calls without the RMSNorm ("Write the streams"; "Source
// layer, pairs pooled": Block.hc_post, Block.hc_pre; also the write of a
// boundary at hc other than 4, and a read after it without the RMSNorm): one
// unit of work per wave, a (token, 512-feature chunk) pair, four waves per
// workgroup, units and workgroups in address order (token-major), so that the
// chip sweeps the streams front to back (a sweep in address order streams
// faster than the same bytes walked as many concurrent rows).  Each unit is
// row_kernel's chunk: the same loads, arithmetic and stores.
constexpr int kSweepWaves = 4;
template <bool POST, bool PRE, int HC = kHC>
__global__ void __launch_bounds__(kSweepWaves * 64) sweep_row_kernel(const RowArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d = a.d;
  const int nch = (d + kRowChunk - 1) / kRowChunk;
  const int64_t u = (int64_t)blockIdx.x * kSweepWaves + wave;
  const int64_t t = u / nch;
  if (t >= a.n) return;                          // a whole wave: no barrier in this kernel
  const int c = (int)(u - t * nch);
  const int f0 = c * kRowChunk + lane * 8;
  const bool act = f0 < d;
  const int f = act ? f0 : 0;                    // idle lanes of a partial chunk read feature 0 and never store
  float cpost[HC], ccomb[HC * HC], cpre[HC];
#pragma unroll
  for (int j = 0; j < HC; ++j) {
    cpost[j] = POST ? a.post_in[t * HC + j] : 0.f;
    cpre[j] = PRE ? a.pre_in[t * HC + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < HC * HC; ++j) ccomb[j] = POST ? a.comb_in[t * HC * HC + j] : 0.f;
  u32x4 r[HC + 1];
  row_load<POST, HC>(r, reinterpret_cast<const u32x4*>(a.x + t * a.xtok),
                     reinterpret_cast<const u32x4*>(POST ? a.delta + t * d : a.x), a.xstr, f);
  u32 xp[HC][4];
  if constexpr (POST) {
    post_8<HC>(r, cpost, ccomb, xp);
    if (act) {
      u32x4* xo = reinterpret_cast<u32x4*>(a.x_out + t * HC * d);
#pragma unroll
      for (int k = 0; k < HC; ++k) st_stream(xo + (k * d + f) / 8, u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
    }
  } else {
#pragma unroll
    for (int k = 0; k < HC; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) xp[k][e] = r[k][e];
  }
  if (a.x_mean && act) st_stream(reinterpret_cast<u32x4*>(a.x_mean + t * d) + f / 8, mean_8<HC>(xp));
  if constexpr (PRE) {
    u32 yp[4];
    pre_8<HC>(xp, cpre, yp);
    if (act) st_stream(reinterpret_cast<u32x4*>(a.y_out + t * d) + f / 8, u32x4{yp[0], yp[1], yp[2], yp[3]});
  }
}

// The same sweep for the calls with the RMSNorm of the read row at hc = 4
// ("Final RMSNorm"; the stack exit, a read of given streams): a workgroup per
// token, W = blockDim / 64 waves, wave w taking the chunks w, w + W, ... (at
// most CPW), the read row kept in registers until the token's sum y^2 is
// summed over the waves (in wave order) through LDS.
constexpr int kSweepNormMaxW = 10;
template <bool POST, int CPW, int HC = kHC>
__global__ void __launch_bounds__(kSweepNormMaxW * 64) sweep_norm_kernel(const RowArgs a) {
  __shared__ float red[kSweepNormMaxW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int d = a.d;
  const int nch = (d + kRowChunk - 1) / kRowChunk;
  const int64_t t = blockIdx.x;
  float cpost[HC], ccomb[HC * HC], cpre[HC];
#pragma unroll
  for (int j = 0; j < HC; ++j) {
    cpost[j] = POST ? a.post_in[t * HC + j] : 0.f;
    cpre[j] = a.pre_in[t * HC + j];
  }
#pragma unroll
  for (int j = 0; j < HC * HC; ++j) ccomb[j] = POST ? a.comb_in[t * HC * HC + j] : 0.f;
  u32x4 r[CPW][HC + 1];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave + W * i;
    const int f0 = c * kRowChunk + lane * 8;
    const int f = c < nch && f0 < d ? f0 : 0;
    row_load<POST, HC>(r[i], reinterpret_cast<const u32x4*>(a.x + t * a.xtok),
                       reinterpret_cast<const u32x4*>(POST ? a.delta + t * d : a.x), a.xstr, f);
  }
  u32 ykeep[CPW][4];
  float ssy = 0.f;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave + W * i;
    const int f0 = c * kRowChunk + lane * 8;
    const bool act = c < nch && f0 < d;
    u32 xp[HC][4];
    if constexpr (POST) {
      post_8<HC>(r[i], cpost, ccomb, xp);
      if (act) {
        u32x4* xo = reinterpret_cast<u32x4*>(a.x_out + t * HC * d);
#pragma unroll
        for (int k = 0; k < HC; ++k) st_stream(xo + (k * d + f0) / 8, u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
      }
    } else {
#pragma unroll
      for (int k = 0; k < HC; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[k][e] = r[i][k][e];
    }
    if (a.x_mean && act) st_stream(reinterpret_cast<u32x4*>(a.x_mean + t * d) + f0 / 8, mean_8<HC>(xp));
    pre_8<HC>(xp, cpre, ykeep[i]);
    if (act) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ssy = dot2_bf16(ykeep[i][e], ykeep[i][e], ssy);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ssy += __shfl_xor(ssy, o);
  if (lane == 0) red[wave] = ssy;
  __syncthreads();
  float sy = red[0];
  for (int w = 1; w < W; ++w) sy += red[w];
  const float ry = 1.0f / sqrtf(sy / (float)d + a.rms_eps);
  u32x4* yo = reinterpret_cast<u32x4*>(a.y_out + t * d);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave + W * i;
    const int f0 = c * kRowChunk + lane * 8;
    if (c < nch && f0 < d) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + f0);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + f0 + 4);
      const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      u32 zp[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        zp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(ykeep[i][e2]) * ry), gm[2 * e2 + 1] * (bf_hi(ykeep[i][e2]) * ry));
      st_stream(yo + f0 / 8, u32x4{zp[0], zp[1], zp[2], zp[3]});
    }
  }
}

// hc = 2 with a write and a fresh pre: the write and the projection in one
// pass ("Write the streams"; "Source layer, pairs pooled", Block.hc_mixes on
// X'), so X' is not read back for the projection (only for the read, which
// needs the pre the projection gives).  Slices of the feature range of d (all
// hc streams of a feature together), 128 tokens per workgroup; per 64-feature
// chunk each lane loads, for each of its two row tiles and two 32-feature
// steps, its 8 features of the hc stream rows and of Delta in the matrix-core
// A layout, forms X' (the fp32 sequence of Block.hc_post), stores it, and uses
// it as the A operand against the weight tiles of its stream (staged through a
// double-buffered LDS area, one chunk ahead).  The records are gmix_kernel's.
// (hc = 8 would need 240 KB of weight tiles per chunk, more than LDS holds.)
struct GStreamArgs {
  const hc_bf16* x;
  const hc_bf16* delta;
  const float* post_in;
  const float* comb_in;
  const u32x4* fn;     // packed as for gmix_kernel
  hc_bf16* x_out;
  hc_bf16* x_mean;     // mean over the streams of X' (MTP tap), or NULL
  float* rec;          // [S][n][RECW]
  int64_t n;
  int xtok, xstr;      // elements per token / per stream of x
  int d, S, Fs;        // slices of the feature range of d, Fs features each
};

template <int HC, bool MEAN>
__global__ void __launch_bounds__(kGThreads, 2) gstream_kernel(const GStreamArgs a) {
  using G = GShape<HC>;
  constexpr int NCT = G::NCT, RT = G::RT;
  constexpr int BREC = HC * 2 * NCT * 64;       // 16-byte weight records per chunk: [stream][step][tile][lane]
  constexpr int BPT = (BREC + kGThreads - 1) / kGThreads;
  __shared__ u32x4 w_lds[2][BREC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slice = blockIdx.x % a.S, group = blockIdx.x / a.S;
  const int64_t tw = (int64_t)group * kGTok + wave * 32;
  const int d = a.d;
  int64_t tr[2];
  bool tv[2];
  float cpost[2][HC], ccomb[2][HC * HC];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t t = tw + 16 * ti + (lane & 15);
    tv[ti] = t < a.n;
    tr[ti] = tv[ti] ? t : 0;                       // rows past n read token 0 and are never stored
#pragma unroll
    for (int j = 0; j < HC; ++j) cpost[ti][j] = a.post_in[tr[ti] * HC + j];
#pragma unroll
    for (int j = 0; j < HC * HC; ++j) ccomb[ti][j] = a.comb_in[tr[ti] * HC * HC + j];
  }
  const int kg = 8 * (lane >> 4);
  const int c0 = slice * a.Fs;
  const int nch = a.Fs / kGChunk;

  auto load_src = [&](int ch, u32x4 (&R)[2][2][HC + 1]) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int f = c0 + ch * kGChunk + 32 * st + kg;
        const hc_bf16* xr = a.x + tr[ti] * a.xtok + f;
        // plain (cached) loads: the two steps' 64-byte halves of a line meet in L2 as one fill
#pragma unroll
        for (int k = 0; k < HC; ++k) R[ti][st][k] = *reinterpret_cast<const u32x4*>(xr + k * a.xstr);
        R[ti][st][HC] = *reinterpret_cast<const u32x4*>(a.delta + tr[ti] * d + f);
      }
  };
  auto load_b = [&](int ch, u32x4 (&Bs)[BPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
      const int idx = threadIdx.x + kGThreads * r;
      if (idx < BREC) {
        const int k = idx / (2 * NCT * 64), rem = idx % (2 * NCT * 64);   // rem = (step, tile, lane)
        const int step = (k * d + c0 + ch * kGChunk) / 32 + rem / (NCT * 64);
        Bs[r] = a.fn[(size_t)step * NCT * 64 + rem % (NCT * 64)];
      }
    }
  };
  auto store_b = [&](int buf, const u32x4 (&Bs)[BPT]) __attribute__((always_inline)) {
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
  u32x4 cur[2][2][HC + 1], nxt[2][2][HC + 1], Bs[BPT];
  load_b(0, Bs);
  load_src(0, cur);
  store_b(0, Bs);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const bool more = ch + 1 < nch;
    if (more) {
      load_b(ch + 1, Bs);
      load_src(ch + 1, nxt);
    }
    const u32x4* wb = w_lds[ch & 1];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32 xp[HC][4];
        post_8<HC>(cur[ti][st], cpost[ti], ccomb[ti], xp);
        const int f = c0 + ch * kGChunk + 32 * st + kg;
        if (tv[ti]) {
#pragma unroll
          for (int k = 0; k < HC; ++k)
            *reinterpret_cast<u32x4*>(a.x_out + (tr[ti] * HC + k) * d + f) = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
          if constexpr (MEAN) st_stream(reinterpret_cast<u32x4*>(a.x_mean + tr[ti] * d + f), mean_8<HC>(xp));
        }
#pragma unroll
        for (int k = 0; k < HC; ++k) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ss[ti] = dot2_bf16(xp[k][e], xp[k][e], ss[ti]);
          const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]});
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            acc[ti][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A, __builtin_bit_cast(bf16x8, wb[((k * 2 + st) * NCT + ct) * 64 + lane]), acc[ti][ct], 0, 0, 0);
        }
      }
    if (more) store_b((ch + 1) & 1, Bs);
    __syncthreads();                              // next weights in place; this chunk's reads done
    if (more) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int k = 0; k <= HC; ++k) cur[ti][st][k] = nxt[ti][st][k];
    }
  }

  // the records, as gmix_kernel writes them
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

// ======================================================= workgroup exchange
// Words that one workgroup leaves for another travel through the workspace as
// 64-bit (tag, value) pairs written and read with device scope: a word is valid
// when its tag is the current call's, so no ordering between words is needed.
// A reader polls a bounded number of times; a timeout sets a sticky bit in the
// workspace's error mask (read back by hc_workspace_status) instead of hanging.
typedef unsigned long long u64;
constexpr int kCtrlBytes = 8192;             // control block at the head of the workspace
constexpr int kErrWord = 1040;               // u32 index: sticky error mask (byte 4160)
constexpr int kCtlXEpoch = 16;               // u64 index: read-row exchanges' call epoch
constexpr int kCtlXDone = 17;                // u64 index: read-row exchanges' workgroups-done count
constexpr unsigned kPollLimit = 1u << 14;    // polls of one word (about 1 us each) before a wait gives up
enum : unsigned { kErrPollTimeout = 1u };

__device__ __forceinline__ u64 tag_word(float v, u32 tag) { return ((u64)tag << 32) | __float_as_uint(v); }
__device__ __forceinline__ void put_word(u64* p, u64 w) { __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 get_word(const u64* p) { return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// The low half of the call epoch word (a 32-bit load: no dead half register
// for the allocator to reuse while the load is in flight).
__device__ __forceinline__ u32 epoch_low(const u64* ctl) {
  return __hip_atomic_load(reinterpret_cast<u32*>(const_cast<u64*>(ctl + kCtlXEpoch)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until each of the words w[i] (at ptr(i), those with use(i)) holds the
// call's tag: every round checks all of them and reloads all the stale ones
// at once, so the wait ends one round trip after the last of them became
// visible (polling them one after another costs a round trip per stale word).
// After kPollLimit rounds it gives up: it sets the error mask and dead, and a
// later wait of this lane gives up at once, so the call finishes quickly with
// wrong values rather than polling on.
template <int N, typename P, typename U>
__device__ __forceinline__ void settle_all(u64 (&w)[N], P ptr, U use, u32 tag, u32* err, bool& dead) {
  for (unsigned polls = 0; !dead; ++polls) {
    bool stale = false;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= use(i) && (u32)(w[i] >> 32) != tag;
    if (!stale) break;
    if (polls >= kPollLimit) {
      atomicOr(err, kErrPollTimeout);
      dead = true;
      break;
    }
    __builtin_amdgcn_s_sleep(8);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (use(i) && (u32)(w[i] >> 32) != tag) w[i] = get_word(ptr(i));
  }
}

// Lane exchanges inside a 16-lane row for the 16-lanes-per-token derive: lane
// i <- lane i ^ 4 (reverse the quad, then mirror the half row) and lane i <-
// lane i ^ 8 (rotate the row by 8).
__device__ __forceinline__ float xor4_16(float v) { return quad_perm<0x141>(quad_perm<0x1B>(v)); }
__device__ __forceinline__ float xor8_16(float v) { return quad_perm<0x128>(v); }
// Sum over the lanes k, k+4, k+8, k+12 of a 16-lane row (a comb column): a
// butterfly, so every lane of the column gets the same bits.
__device__ __forceinline__ float col_sum16(float v) {
  const float u = v + xor4_16(v);
  return u + xor8_16(u);
}

// The split and Sinkhorn of one token, 16 lanes per token ("Reading weights"
// kernel panel and reading-weight equation): lane 4j+k of the token's 16-lane
// row holds comb element (j, k), so a Sinkhorn row sum is a quad sum and a
// column sum a butterfly over the four quads, one element per lane (a short
// dependency chain: the derive is on the critical path of the one-launch
// exchange).  Lanes k = 0 and k = 1 of quad j also form pre_j and post_j.  r
// points at the token's summed words (24 dots, sum x'^2).  Every lane of the
// row calls it; the outputs are written if valid (pre/post/comb only if
// pre_out).
__device__ __forceinline__ void derive_16(const float* r, float rx, int j, int k, bool valid, int64_t t,
                                          const float* hc_scale, const float* hc_base, int iters, float eps,
                                          float* mixes_out, float* pre_out, float* post_out, float* comb_out) {
  constexpr int HC = 4, MIX = 24;
  const bool odd = k & 1;
  const float mpq = r[odd ? HC + j : j] * rx;           // lane k = 0: pre mix j; k = 1: post mix j
  const float mc = r[2 * HC + 4 * j + k] * rx;
  if (valid && mixes_out) {
    mixes_out[t * MIX + 2 * HC + 4 * j + k] = mc;
    if (k < 2) mixes_out[t * MIX + k * HC + j] = mpq;
  }
  if (!pre_out) return;
  const float u = odd ? mpq * hc_scale[1] + hc_base[HC + j] : mpq * hc_scale[0] + hc_base[j];
  const float sg = sigmoidf_(u);
  const float g = odd ? 2.0f * sg : sg + eps;           // post_j / pre_j
  float a = mc * hc_scale[2] + hc_base[2 * HC + 4 * j + k];
  float mx = fmaxf(a, quad_perm<0xB1>(a));
  mx = fmaxf(mx, quad_perm<0x4E>(mx));
  a = expf(a - mx);
  a = a * __builtin_amdgcn_rcpf(quad_sum(a)) + eps;     // row softmax + eps
  a = a * __builtin_amdgcn_rcpf(col_sum16(a) + eps);    // column step
  for (int it = 1; it < iters; ++it) {
    a = a * __builtin_amdgcn_rcpf(quad_sum(a) + eps);
    a = a * __builtin_amdgcn_rcpf(col_sum16(a) + eps);
  }
  if (!valid) return;
  if (k == 0) pre_out[t * HC + j] = g;
  if (k == 1) post_out[t * HC + j] = g;
  comb_out[t * HC * HC + 4 * j + k] = a;
}

// hc_split_sinkhorn at hc = 4 ("Reading weights" kernel panel): 16 lanes per
// token (derive_16, one comb element per lane), 16 tokens per workgroup; the
// shorter dependency chain per Sinkhorn round than hc lanes per token.
__global__ void __launch_bounds__(256) split16_kernel(const float* __restrict__ mixes, const float* __restrict__ scale,
                                                      const float* __restrict__ base, int64_t n, int iters, float eps,
                                                      float* __restrict__ pre, float* __restrict__ post,
                                                      float* __restrict__ comb) {
  const int q = threadIdx.x & 15;
  const int64_t tq = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = tq < n;
  const int64_t t = valid ? tq : 0;   // lanes past n compute on token 0 and store nothing
  derive_16(mixes + t * kMix, 1.0f, q >> 2, q & 3, valid, t, scale, base, iters, eps, nullptr, pre, post, comb);
}

// ====================================================== boundary: two kernels
// Everything that derives mixes (hc_mixes, block entry, sublayer boundary)
// can run as two ordinary launches; the boundary between them is the only
// device-wide synchronisation.  The first is the stream kernel when X' is
// written, else the projection kernel (proj_kernel, below: the same records
// from 128-token workgroups).
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
  // the read-row exchange (exchange_kernel: given pre + RMSNorm in one launch)
  u64* ctl;           // workspace control block (epoch, done count)
  u64* xw;            // [tiles][S][kTT][kXW] tagged words
  u32* err;           // sticky error mask
  const float* gamma;
  const float* hc_base;
  const float* hc_scale;
  float* mixes_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  int iters;
  float hc_eps, norm_eps, rms_eps;
};
constexpr int kXW = kMix + 2;            // exchanged words per token and slice: 24 dots, sum x'^2, sum y^2

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
// calls without it carry none of its registers.
// (Its 112 KB of LDS allow one workgroup, two waves per SIMD, per compute
// unit; the register budget says so, else the compiler aims at three.)
template <int RM, bool NORM, bool MEAN>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
stream_kernel(const StreamArgs a) {
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
  const hc_bf16* db = a.delta + t0 * d;
  hc_bf16* xob = a.x_out + t0 * kHC * d;
  hc_bf16* yb = RM == kGivenPre ? a.y_out + t0 * d : nullptr;

  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    cpost[j] = a.post_in[(t0 + lt) * kHC + j];
    cpre[j] = RM == kGivenPre ? a.pre_in[(t0 + lt) * kHC + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = a.comb_in[(t0 + lt) * kHC * kHC + j];

  u32x4 cur[kHC + 1];
  u32x4 wst[kNT];  // this wave's share (5 of 40 blocks) of the next chunk's weight tiles
  f32x4 acc[kAcc];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the projection's running sums: each chunk's matrix-core partial sums (fp32)
  // are added here in fp64 and the fp32 accumulators restart, so fp32 rounding
  // builds up over one chunk only, whatever the slice width (a slice can be the
  // whole 20480-long row, and the dot of a heavy-tailed row cancels strongly).
  double acc64[kAcc][4];
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc64[t][i] = 0.0;
  auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kAcc; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[t][i] += (double)acc[t][i];
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  float ssx = 0.f, ssy = 0.f;
  float gram[kGram];
#pragma unroll
  for (int g = 0; g < kGram; ++g) gram[g] = 0.f;

  auto load_wst = [&](int c, u32x4 (&dst)[kNT]) __attribute__((always_inline)) {
    const int gstep = (fs + c * kCF) / 32;
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;          // (st, k, nt) = blk / 20, (blk / 5) % 4, blk % 5
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      dst[i] = a.fn[((size_t)((gstep + st) * kHC + k) * kNT + nt) * 64 + lane];
    }
  };
  auto store_wst = [&](int buf, const u32x4 (&src)[kNT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      w_lds[buf][st][k][nt][lane] = src[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int j = 0; j < kHC; ++j) dst[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * (unsigned)a.xtok + j * (unsigned)a.xstr + f)));
    dst[kHC] = ld_stream(reinterpret_cast<const u32x4*>(db + (lt * d + f)));
  };
  auto stream_phase = [&](int c, const u32x4 (&src)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    post_8(src, cpost, ccomb, xp);
    if (tv) {
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        u32x4* p = reinterpret_cast<u32x4*>(xob + (lt * kHC * d + k * d + f));
        const u32x4 v = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
        if constexpr (RM == kFreshPre) st_keep(p, v); else st_stream(p, v);
      }
    }
    // unconditional: a lane past n works on the tile's first token (lt = 0) and
    // stores the same bits as that token's lane
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
  auto matrix_phase = [&](int buf) __attribute__((always_inline)) {
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
  auto chunk = [&](int c, bool more) __attribute__((always_inline)) {
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
    flush();
    lds_barrier();                 // matrix phase done before the A tiles are rewritten
    if (more) {
#pragma unroll
      for (int j = 0; j <= kHC; ++j) cur[j] = nxt[j];
    }
  };
  load_wst(0, wst);
  load_stream(0, cur);
  store_wst(0, wst);
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
  float* red = reinterpret_cast<float*>(&w_lds[0][0][0][0][0]);   // [4 rb][2 steps][16][32] | extra
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      red[((rb * 2 + hw) * 16 + 4 * (lane >> 4) + rr) * 32 + t * 16 + (lane & 15)] = (float)acc64[t][rr];
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

// ---------------------------------------------------------------------------
// proj_kernel: the stream kernel's work when nothing is written back (hc_mixes,
// the block entry): per-slice records of the projection dots, sum x^2 and the
// norm sums, in the stream kernel's record layout, for the finish kernel.
// Its cost is the weight tiles, not the streams: every workgroup reads its
// slice's tiles (from L2) once, so a workgroup takes 128 tokens (two record
// tiles), half the weight traffic per token of a 64-token tile.  Wave w owns
// row block w (16 tokens) in both phases:
//   stream phase: two groups of 8 tokens, 8 lanes a token, 8 features a lane;
//     the row block's A tiles are written to LDS, where only wave w reads
//     them; the sums accumulate in registers;
//   matrix phase: both 32-feature steps x 4 streams x 5 tiles against the
//     chunk's weight tiles, which all waves stage (double buffered), so one
//     barrier per chunk.
// Streams and weights run two chunks ahead in register pairs.  Each chunk's
// fp32 matrix-core sums are added in fp64, rounded once at the end.
constexpr int kPTT = 128;                 // tokens per workgroup

template <int RM, bool NORM, bool MEAN>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
proj_kernel(const StreamArgs a) {
  static_assert(!NORM || RM != kNoRead, "RMSNorm needs the read row");
  __shared__ u32x4 w_lds[2][2][kHC][kNT][64];          // weight tiles, double buffered (80 KB)
  __shared__ u32x4 a_lds[kWaves][2][kHC][64];          // A tiles per row block (64 KB)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // = row block
  const int d = a.d, S = a.S, F = a.F;
  const int nch = F / kCF;
  const int tiles2 = (a.tiles + 1) / 2;
  const int lin = (gridDim.x & 7) ? blockIdx.x : (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int slice = lin / tiles2;
  const int tile2 = lin % tiles2;
  const int fs = slice * F;

  const int hl = lane >> 3;
  const int fl = (lane & 7) * 8;
  const int a_st = fl >> 5, a_g = (fl >> 3) & 3;
  constexpr int kUsed = rec_used<RM, NORM>();
  constexpr int kQuads = (kUsed + 3) / 4;

  const int64_t t0 = (int64_t)tile2 * kPTT;           // < n: the first token of the workgroup is real
  bool tv[2];
  int64_t tm64[2];
  const hc_bf16* xr[2];
  float cpre[2][kHC];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int m = wave * 16 + p * 8 + hl;
    tv[p] = t0 + m < a.n;
    tm64[p] = t0 + m;
    const int64_t tr = tv[p] ? t0 + m : t0;          // a token past n reads the first token
    xr[p] = a.x + tr * a.xtok;
#pragma unroll
    for (int j = 0; j < kHC; ++j) cpre[p][j] = RM == kGivenPre ? a.pre_in[tr * kHC + j] : 0.f;
  }

  f32x4 acc[kAcc];
  double acc64[kAcc][4];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc64[t][i] = 0.0;
  }
  float ssx[2] = {0.f, 0.f}, ssy[2] = {0.f, 0.f};
  float gram[2][kGram];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int g = 0; g < kGram; ++g) gram[p][g] = 0.f;

  auto load_wst = [&](int c, u32x4 (&dst)[kNT]) __attribute__((always_inline)) {
    const int gstep = (fs + c * kCF) / 32;
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;          // (st, k, nt) = blk / 20, (blk / 5) % 4, blk % 5
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      dst[i] = a.fn[((size_t)((gstep + st) * kHC + k) * kNT + nt) * 64 + lane];
    }
  };
  auto store_wst = [&](int buf, const u32x4 (&src)[kNT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kHC * kNT), k = (blk / kNT) % kHC, nt = blk % kNT;
      w_lds[buf][st][k][nt][lane] = src[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[2][kHC]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < kHC; ++j) dst[p][j] = ld_stream(reinterpret_cast<const u32x4*>(xr[p] + (j * (unsigned)a.xstr + f)));
  };
  auto stream_phase = [&](int c, const u32x4 (&src)[2][kHC]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32 xp[kHC][4];
#pragma unroll
      for (int k = 0; k < kHC; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[k][e] = src[p][k][e];
      if constexpr (MEAN) {
        if (tv[p]) st_stream(reinterpret_cast<u32x4*>(a.x_mean + tm64[p] * d + f), mean_8(xp));
      }
      const int a_lane = a_g * 16 + p * 8 + hl;
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ssx[p] = dot2_bf16(xp[k][e], xp[k][e], ssx[p]);
        a_lds[wave][a_st][k][a_swz(a_lane, a_st)] = u32x4{xp[k][0], xp[k][1], xp[k][2], xp[k][3]};
      }
      if constexpr (RM == kGivenPre) {
        u32 yp[4];
        pre_8(xp, cpre[p], yp);
        if constexpr (NORM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ssy[p] = dot2_bf16(yp[e], yp[e], ssy[p]);
        }
        if (tv[p]) {
          u32x4* q = reinterpret_cast<u32x4*>(a.y_out + tm64[p] * d + f);
          const u32x4 v = u32x4{yp[0], yp[1], yp[2], yp[3]};
          if constexpr (NORM) st_keep(q, v); else st_stream(q, v);
        }
      }
      if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int g = 0;
#pragma unroll
          for (int j = 0; j < kHC; ++j)
#pragma unroll
            for (int l = j; l < kHC; ++l, ++g) gram[p][g] = dot2_bf16(xp[j][e], xp[l][e], gram[p][g]);
        }
      }
    }
  };
  auto matrix_phase = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int k = 0; k < kHC; ++k) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, a_lds[wave][st][k][a_swz(lane, st)]);
        bf16x8 B[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) B[nt] = __builtin_bit_cast(bf16x8, w_lds[buf][st][k][nt][lane]);
        mfma_step(A, B, acc);
      }
#pragma unroll
    for (int t = 0; t < kAcc; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[t][i] += (double)acc[t][i];
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // one chunk: chunk c+1's weights were requested two chunks ago and go to
  // LDS after the barrier (which also ends every wave's reads of that buffer,
  // chunk c-1's); chunk c+2's weights, then its streams, are requested once
  // chunk c's stream registers are free
  auto step = [&](int c, auto ISSUE, auto STORE, u32x4 (&s)[2][kHC], u32x4 (&wfree)[kNT],
                  const u32x4 (&wnext)[kNT]) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    stream_phase(c, s);
    if constexpr (decltype(ISSUE)::v) {
      __builtin_amdgcn_sched_barrier(0);
      load_wst(c + 2, wfree);
      __builtin_amdgcn_sched_barrier(0);
      load_stream(c + 2, s);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    if constexpr (decltype(STORE)::v) store_wst((c + 1) & 1, wnext);
    matrix_phase(c & 1);
  };

  {
    u32x4 sA[2][kHC], sB[2][kHC], wA[kNT], wB[kNT];
    const int c1 = nch > 1 ? 1 : 0;                   // a single chunk loads chunk 0 twice (unused)
    load_wst(0, wA);
    __builtin_amdgcn_sched_barrier(0);
    load_stream(0, sA);
    __builtin_amdgcn_sched_barrier(0);
    load_wst(c1, wB);
    __builtin_amdgcn_sched_barrier(0);
    load_stream(c1, sB);
    __builtin_amdgcn_sched_barrier(0);
    store_wst(0, wA);
    int c = 0;
    for (; c + 3 < nch; c += 2) {
      step(c, IC<1>{}, IC<1>{}, sA, wA, wB);
      step(c + 1, IC<1>{}, IC<1>{}, sB, wB, wA);
    }
    const int left = nch - c;                         // 1..3: chunk c in sA, c+1 in sB
    if (left == 3) {
      step(c, IC<1>{}, IC<1>{}, sA, wA, wB);
      step(c + 1, IC<0>{}, IC<1>{}, sB, wB, wA);
      step(c + 2, IC<0>{}, IC<0>{}, sA, wA, wB);
    } else if (left == 2) {
      step(c, IC<0>{}, IC<1>{}, sA, wA, wB);
      step(c + 1, IC<0>{}, IC<0>{}, sB, wB, wA);
    } else {
      step(c, IC<0>{}, IC<0>{}, sA, wA, wB);
    }
  }

  // ---- per-token records of this slice, in the two record tiles of the workgroup
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      ssx[p] += __shfl_xor(ssx[p], o);
      if constexpr (RM == kGivenPre && NORM) ssy[p] += __shfl_xor(ssy[p], o);
      if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
        for (int g = 0; g < kGram; ++g) gram[p][g] += __shfl_xor(gram[p][g], o);
      }
    }
  lds_barrier();                                      // every wave's last matrix phase done: the weight area is reused
  double* red64 = reinterpret_cast<double*>(&w_lds[0][0][0][0][0]);   // [row block][acc tile][4 rows][64 lanes]
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red64[((wave * kAcc + t) * 4 + i) * 64 + lane] = acc64[t][i];
  float* extra = reinterpret_cast<float*>(red64 + kWaves * kAcc * 4 * 64);   // [kRec - kMix][kPTT]
  if ((lane & 7) == 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int m = wave * 16 + p * 8 + hl;
      extra[m] = ssx[p];
      if constexpr (RM == kGivenPre && NORM) extra[kPTT + m] = ssy[p];
      if constexpr (RM == kFreshPre && NORM) {
#pragma unroll
        for (int g = 0; g < kGram; ++g) extra[(1 + g) * kPTT + m] = gram[p][g];
      }
    }
  }
  lds_barrier();
  for (int idx = threadIdx.x; idx < kPTT * kQuads; idx += kThreads) {
    const int tm = idx / kQuads, q0 = (idx % kQuads) * 4;
    const int tile = 2 * tile2 + (tm >> 6);
    if (tile >= a.tiles) continue;                    // the second record tile of a call's last 64 tokens
    // token tm's accumulator element: row block tm / 16, row tm % 4 of lanes 16 ((tm % 16) / 4) + column;
    // rows 16..23 sit in columns q - 16 and q - 8 of the second tile
    const double* e = red64 + ((tm >> 4) * kAcc * 4 + (tm & 3)) * 64 + 16 * ((tm & 15) >> 2);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + i;
      if (q < 16) v[i] = (float)e[q];
      else if (q < kMix) v[i] = (float)(e[4 * 64 + q - 16] + e[4 * 64 + q - 8]);
      else v[i] = q < kUsed ? extra[(q - kMix) * kPTT + tm] : 0.f;
    }
    float* rec = a.rec + (((size_t)tile * S + slice) * kTT + (tm & 63)) * kRec;
    *reinterpret_cast<f32x4*>(rec + q0) = f32x4{v[0], v[1], v[2], v[3]};
  }
}

// ---------------------------------------------------------------------------
// exchange_kernel: the boundary with a given pre and the RMSNorm in one launch
// ("Source layer, pairs pooled", Block.forward; "Final RMSNorm").  The RMSNorm
// of the read row needs sum y^2 over the whole row, which the S feature slices
// of a token tile each hold a part of.  Each lane keeps its slice of y in
// registers (the chunk loop unrolled at compile time) instead of storing it;
// the slices of a tile exchange their per-token sums (24 dots, sum x'^2,
// sum y^2) as tagged words in the workspace; every slice sums the S parts of
// sum y^2 of each of its tokens in slice order (the same bits in every slice)
// and writes z = gamma * (y * r); the owner slice of a token (token m with
// m % S == slice) sums all of the token's words in slice order and derives
// its mixes, pre/post and comb.  The owners' words are summed first, so that
// the derive (one wave) runs while the other waves' z stores drain.
// Per 64-feature chunk the streaming is that of the stream kernel (X' stored,
// its A tile and the matrix-core projection, sum x'^2 and sum y^2).  Every
// workgroup of a call must be resident at once (one per compute unit, at most
// 256); a wait that times out sets the error mask instead of hanging.
constexpr int kXS = 8;                    // slices per tile at most on this path

// SUMW (the block entry from the expanded embedding: no write, four identical
// streams): each lane loads its row once, and the projection takes the
// weight summed over the stream blocks (the tiles hc_fn_pack appends) against
// one stream's A tile, a quarter of the weight tiles and matrix-core work.
template <bool POST, bool MEAN, int YK, bool SUMW = false>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
exchange_kernel(const StreamArgs a) {
  static_assert(!(SUMW && POST), "summed weights only for four identical streams (no write)");
  constexpr int kPK = SUMW ? 1 : kHC;           // stream blocks of the projection
  __shared__ u32x4 w_lds[2][2][kHC][kNT][64];          // weight tiles, double buffered (80 KB)
  __shared__ u32x4 a_lds[4][2][kHC][64];               // X' in A layout per row block (32 KB)
  __shared__ float red[4][2][16][32];                  // projection sums per (row block, step) (16 KB)
  __shared__ float ssum[kTT];                          // sum x'^2 per token
  __shared__ float tot[kTT / 4 * kXW];                 // the owned tokens' words, summed over the slices
  __shared__ f32x4 g_slice[YK * kCF / 4];              // gamma of the slice
  __shared__ float s_cf[kMix + 3];                     // hc_base, hc_scale (read by the derive)
  __shared__ u32 s_tag;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave >> 1, hw = wave & 1;   // row block, half (stream phase) / step (matrix phase)
  const int d = a.d, S = a.S;
  // XCD-aware: consecutive blocks land on different XCDs; renumbered so that
  // each XCD holds a contiguous run, slice-major (an XCD's L2 holds the
  // weights of few slices)
  const int lin = (gridDim.x & 7) ? blockIdx.x : (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int slice = lin / a.tiles, tile = lin % a.tiles;
  const int fs = slice * (YK * kCF);
  const int hl = lane >> 3, fl = (lane & 7) * 8;
  const int m = rb * 16 + hw * 8 + hl;          // token within the tile
  const int a_st = fl >> 5, a_g = (fl >> 3) & 3;
  const int a_lane = a_g * 16 + hw * 8 + hl;
  const int nown = (kTT - slice + S - 1) / S;   // owned tokens: slice, slice + S, ... (S >= 4: at most 16)
  const int pr = threadIdx.x;                   // (owned token, word) pair of this thread
  const bool has_pair = pr < nown * kXW;
  const int ptm = has_pair ? slice + S * (pr / kXW) : 0, pq = has_pair ? pr % kXW : 0;

  // (Issuing these after the first chunk's loads, as xfew_kernel does,
  // measured no faster here, where the first loads of every workgroup queue.)
  if (threadIdx.x == 0) s_tag = epoch_low(a.ctl) + 1u;   // words carry epoch + 1
  if (threadIdx.x < YK * kCF / 4) g_slice[threadIdx.x] = reinterpret_cast<const f32x4*>(a.gamma + fs)[threadIdx.x];
  // the split's parameters, requested now so that the derive does not wait for them
  if (a.pre_out && threadIdx.x >= kThreads - (kMix + 3)) {
    const int i = threadIdx.x - (kThreads - (kMix + 3));
    s_cf[i] = i < kMix ? a.hc_base[i] : a.hc_scale[i - kMix];
  }

  const int64_t t0 = (int64_t)tile * kTT;
  const bool tv = t0 + m < a.n;
  const unsigned lt = tv ? (unsigned)m : 0u;   // a token past n reads the tile's first token
  const hc_bf16* xb = a.x + t0 * a.xtok;
  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    cpost[j] = POST ? a.post_in[(t0 + lt) * kHC + j] : 0.f;
    cpre[j] = a.pre_in[(t0 + lt) * kHC + j];
  }
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = POST ? a.comb_in[(t0 + lt) * kHC * kHC + j] : 0.f;

  // the chunk's 2 x kPK x kNT weight tiles, kPK x kNT / 4 per wave
  constexpr int kWB = (2 * kPK * kNT + kWaves - 1) / kWaves;
  const u32x4* fsum = SUMW ? a.fn + (size_t)(d / kStepF) * kHC * kNT * 64 : nullptr;   // stream-summed tiles
  auto load_wst = [&](int c, u32x4 (&dst)[kNT]) __attribute__((always_inline)) {
    const int gstep = (fs + c * kCF) / 32;
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      const int blk = wave + i * kWaves;          // (st, k, nt) = blk / (5 kPK), (blk / 5) % kPK, blk % 5
      const int st = blk / (kPK * kNT), kk = (blk / kNT) % kPK, nt = blk % kNT;
      if constexpr (SUMW) {
        if (blk < 2 * kPK * kNT) dst[i] = fsum[((size_t)(gstep + st) * kNT + nt) * 64 + lane];
      } else {
        dst[i] = a.fn[((size_t)((gstep + st) * kHC + kk) * kNT + nt) * 64 + lane];   // 40 blocks, 5 per wave
      }
    }
  };
  auto store_wst = [&](int buf, const u32x4 (&src)[kNT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kPK * kNT), kk = (blk / kNT) % kPK, nt = blk % kNT;
      if (!SUMW || blk < 2 * kPK * kNT) w_lds[buf][st][kk][nt][lane] = src[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
    if constexpr (SUMW) {
      dst[0] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * (unsigned)a.xtok + f)));
#pragma unroll
      for (int j = 1; j < kHC; ++j) dst[j] = dst[0];
    } else {
#pragma unroll
      for (int j = 0; j < kHC; ++j)
        dst[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * (unsigned)a.xtok + j * (unsigned)a.xstr + f)));
    }
    dst[kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(a.delta + (t0 + lt) * d + f)) : u32x4{0u, 0u, 0u, 0u};
  };
  float ssx = 0.f, ssy = 0.f;
  f32x4 acc[kAcc];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32 ykeep[YK][4];                             // this lane's read row, chunk by chunk
  u32 xlast[kHC][4];                            // X' of the last chunk, stored after the sums are published
  auto store_x = [&](int c, const u32 (&xp)[kHC][4]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
    if (tv) {
      hc_bf16* xob = a.x_out + (t0 + lt) * kHC * d;
#pragma unroll
      for (int j = 0; j < kHC; ++j)
        st_stream(reinterpret_cast<u32x4*>(xob + (j * d + f)), u32x4{xp[j][0], xp[j][1], xp[j][2], xp[j][3]});
    }
  };
  auto stream_phase = [&](int c, const u32x4 (&src)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    if constexpr (POST) {
      post_8(src, cpost, ccomb, xp);
      if (c + 1 < YK) {
        store_x(c, xp);
      } else {
#pragma unroll
        for (int j = 0; j < kHC; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) xlast[j][e] = xp[j][e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[j][e] = src[j][e];
    }
    // unconditional: a lane past n stores the same bits as its tile's first token
    if constexpr (MEAN) st_stream(reinterpret_cast<u32x4*>(a.x_mean + (t0 + lt) * d + f), mean_8(xp));
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ssx = dot2_bf16(xp[j][e], xp[j][e], ssx);
      if (j < kPK) a_lds[rb][a_st][j][a_swz(a_lane, a_st)] = u32x4{xp[j][0], xp[j][1], xp[j][2], xp[j][3]};
    }
    u32 yp[4];
    pre_8(xp, cpre, yp);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ssy = dot2_bf16(yp[e], yp[e], ssy);
      ykeep[c][e] = yp[e];
    }
  };
  auto matrix_phase = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPK; ++j) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, a_lds[rb][hw][j][a_swz(lane, hw)]);
      bf16x8 B[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) B[nt] = __builtin_bit_cast(bf16x8, w_lds[buf][hw][j][nt][lane]);
      mfma_step(A, B, acc);
    }
  };

  // the chunks: the next chunk's weights, then its streams, are requested
  // before this chunk's work; two barriers (A tiles and weights in place; the
  // matrix phase done before the A tiles are rewritten)
  if constexpr (SUMW) {
    // little to load per chunk (one row, a quarter of the weight tiles): the
    // row kP chunks ahead and the weight tiles two chunks ahead, in rings
    // indexed by the (compile-time) chunk number, so the chunks do not wait
    // on a memory round trip each
    constexpr int kP = 4;
    u32x4 hq[kP], wq[2][kNT];
    load_wst(0, wq[0]);
#pragma unroll
    for (int c = 0; c < kP && c < YK; ++c) {
      u32x4 t[kHC + 1];
      load_stream(c, t);
      hq[c] = t[0];
    }
    store_wst(0, wq[0]);
    if constexpr (YK > 1) load_wst(1, wq[1]);
    lds_barrier();
    auto chunk = [&]<int C>(IC<C>) __attribute__((always_inline)) {
      if constexpr (C + 2 < YK) load_wst(C + 2, wq[C & 1]);   // its slot's tiles were stored a chunk ago
      u32x4 src[kHC + 1];
#pragma unroll
      for (int j = 0; j < kHC; ++j) src[j] = hq[C % kP];
      src[kHC] = u32x4{0u, 0u, 0u, 0u};
      stream_phase(C, src);
      if constexpr (C + kP < YK) {
        u32x4 t[kHC + 1];
        load_stream(C + kP, t);
        hq[C % kP] = t[0];
      }
      lds_barrier();
      if constexpr (C + 1 < YK) store_wst((C + 1) & 1, wq[(C + 1) & 1]);
      matrix_phase(C & 1);
      lds_barrier();
    };
    [&]<int... C>(std::integer_sequence<int, C...>) __attribute__((always_inline)) {
      (chunk(IC<C>{}), ...);
    }(std::make_integer_sequence<int, YK>{});
  } else {
    u32x4 cur[kHC + 1], wst[kNT];
    load_wst(0, wst);
    load_stream(0, cur);
    store_wst(0, wst);
    lds_barrier();
    auto chunk = [&]<int C>(IC<C>) __attribute__((always_inline)) {
      constexpr bool kMore = C + 1 < YK;
      u32x4 nxt[kHC + 1];
      if constexpr (kMore) {
        load_wst(C + 1, wst);
        load_stream(C + 1, nxt);
      }
      stream_phase(C, cur);
      lds_barrier();
      if constexpr (kMore) store_wst((C + 1) & 1, wst);
      matrix_phase(C & 1);
      lds_barrier();
      if constexpr (kMore) {
#pragma unroll
        for (int j = 0; j <= kHC; ++j) cur[j] = nxt[j];
      }
    };
    [&]<int... C>(std::integer_sequence<int, C...>) __attribute__((always_inline)) {
      (chunk(IC<C>{}), ...);
    }(std::make_integer_sequence<int, YK>{});
  }

  // ---- this slice's sums of every token of the tile, as tagged words: sum y^2
  // (every slice of the tile waits for it) straight from the lanes, the rest
  // through LDS, then the last chunk's X'
  const u32 tag = s_tag;
  u64* tilew = a.xw + (size_t)tile * S * kTT * kXW;
  u64* mine = tilew + (size_t)slice * kTT * kXW;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    ssx += __shfl_xor(ssx, o);
    ssy += __shfl_xor(ssy, o);
  }
  if ((lane & 7) == 0) put_word(mine + m * kXW + kMix + 1, tag_word(ssy, tag));
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[rb][hw][4 * (lane >> 4) + rr][t * 16 + (lane & 15)] = acc[t][rr];
  if ((lane & 7) == 0) ssum[m] = ssx;
  lds_barrier();
  for (int i = threadIdx.x; i < kTT * (kXW - 1); i += kThreads) {
    const int tm = i / (kXW - 1), q = i % (kXW - 1);
    const int idx = tm * kXW + q;
    float v;
    if (q < kMix) {
      const float* r0 = red[tm >> 4][0][tm & 15];
      const float* r1 = red[tm >> 4][1][tm & 15];
      v = q < 16 ? r0[q] + r1[q] : (r0[q] + r0[q + 8]) + (r1[q] + r1[q + 8]);
    } else {
      v = ssum[tm];
    }
    put_word(mine + idx, tag_word(v, tag));
  }
  if constexpr (POST) store_x(YK - 1, xlast);
  // ---- every word this workgroup waits for, in one round trip: sum y^2 of
  // this lane's token and, for the owned (token, word) pair of this thread,
  // that word, from every slice; each summed in slice order
  // words 0 .. kXS-1: sum y^2 of this lane's token; kXS ..: the owned pair
  auto wptr = [&](int i) {
    return i < kXS ? tilew + ((size_t)i * kTT + m) * kXW + kMix + 1 : tilew + ((size_t)(i - kXS) * kTT + ptm) * kXW + pq;
  };
  auto wuse = [&](int i) { return i < kXS ? i < S : has_pair && i - kXS < S; };
  u64 wv[2 * kXS];
#pragma unroll
  for (int i = 0; i < 2 * kXS; ++i) wv[i] = wuse(i) ? get_word(wptr(i)) : 0ull;
  bool dead = false;
  settle_all(wv, wptr, wuse, tag, a.err, dead);
  if (has_pair) {
    float tr = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kXS; ++s2)
      if (s2 < S) {
        const float v = __uint_as_float((u32)wv[kXS + s2]);
        tr = s2 == 0 ? v : tr + v;
      }
    tot[pr] = tr;
  }
  float ty = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < kXS; ++s2)
    if (s2 < S) {
      const float v = __uint_as_float((u32)wv[s2]);
      ty = s2 == 0 ? v : ty + v;
    }
  const float ry = 1.0f / sqrtf(ty / (float)d + a.rms_eps);
  __syncthreads();
  // every word of this call read: count this workgroup done.  A thread of the
  // last wave (no derive work) issues it, and awaits the count only at its end.
  constexpr int kDoneThread = kThreads - 1;
  u64 before = 0;
  if (threadIdx.x == kDoneThread)
    before = __hip_atomic_fetch_add(a.ctl + kCtlXDone, (u64)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // ---- the owned tokens' mixes, pre/post and comb: 16 lanes per token (up to
  // four waves, which write their part of z after it, while the others' z stores
  // drain)
  if ((int)threadIdx.x < 16 * nown) {
    const int k = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int tm = slice + S * k;
    const float* r = &tot[k * kXW];
    const float rx = 1.0f / sqrtf(r[kMix] / (float)(kHC * d) + a.norm_eps);
    derive_16(r, rx, q >> 2, q & 3, t0 + tm < a.n, t0 + tm, s_cf + kMix, s_cf, a.iters, a.hc_eps,
              a.mixes_out, a.pre_out, a.post_out, a.comb_out);
  }
  // ---- z = gamma * (y * r) from the kept read row
#pragma unroll
  for (int c = 0; c < YK; ++c) {
    const int f = fs + c * kCF + fl;
    const f32x4 g0 = g_slice[(c * kCF + fl) / 4];
    const f32x4 g1 = g_slice[(c * kCF + fl) / 4 + 1];
    const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    u32 zp[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      zp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(ykeep[c][e2]) * ry), gm[2 * e2 + 1] * (bf_hi(ykeep[c][e2]) * ry));
    if (tv) st_stream(reinterpret_cast<u32x4*>(a.y_out + (t0 + lt) * d + f), u32x4{zp[0], zp[1], zp[2], zp[3]});
  }
  // the last workgroup to count itself done advances the call epoch
  if (threadIdx.x == kDoneThread && before % (u64)gridDim.x == (u64)(gridDim.x - 1)) {
    put_word(a.ctl + kCtlXDone, 0ull);
    put_word(a.ctl + kCtlXEpoch, (u64)tag);
  }
}

// ---------------------------------------------------------------------------
// xfew_kernel: the boundary for few token tiles (decode, short prefill) in one
// launch ("Source layer, pairs pooled", Block.forward; "Final RMSNorm";
// "Reading weights" for the split).  A workgroup owns (64-token tile, slice of
// YK 64-feature chunks of every stream), with YK from 1 up so small that the
// tiles x slices workgroups fill the compute units (S = d / 64 / YK slices per
// tile, at least 8).  Per chunk the streaming and the matrix-core projection
// are those of exchange_kernel (X' stored, the read row kept in registers).
// The owner slice of a token (token m with m % S == slice) sums each of the
// token's words (24 dots, sum x'^2, with the RMSNorm sum y^2) over the slices
// in G interleaved groups (slices g, g + G, ...) and then the G group sums in
// order, derives its mixes, pre/post and comb with 16 lanes (derive_16) and,
// with the RMSNorm, publishes the token's factor r = rsqrt(mean y^2 + eps) as
// one more tagged word (in the slot of its own sum y^2 word of the token,
// which only it reads, with the complement of the call's tag); every slice
// then scales its part of the read row by the r of its tokens (two hops, but
// a slice reads 64 words instead of 64 x S).  Without the RMSNorm the read row is stored as it is formed, and without
// a read (READ false: the mixes alone) there is none.  Tokens of a tile past n
// take no part in the exchange.  Every workgroup of a call must be resident
// at once (at most 256, one per compute unit); a wait that times out sets the
// error mask instead of hanging.
constexpr int kXFMinD = 256, kXFMaxD = 8192;    // widths of the schedule
constexpr int kXFMinS = 4;                   // slices per tile at least
constexpr int kXFMaxOwn = kTT / kXFMinS;     // owned tokens per slice at most (16)
constexpr int kXFGroups = 20;                // partial sums per owned word at most
constexpr int kXFOLoads = 8;                 // owned words per thread at most (S <= 8 G for every S)
constexpr int kXFMixesMaxN = 2048;           // hc_mixes takes the schedule up to this many tokens

template <bool POST, bool MEAN, bool READ, bool NORM, int YK>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
xfew_kernel(const StreamArgs a) {
  static_assert(!NORM || READ, "the RMSNorm is of the read row");
  constexpr int kOW = NORM ? kXW : kXW - 1;             // owned words per token: 24 dots, sum x'^2 (, sum y^2)
  __shared__ u32x4 w_lds[2][2][kHC][kNT][64];          // weight tiles, double buffered (80 KB)
  __shared__ u32x4 a_lds[4][2][kHC][64];               // X' in A layout per row block (32 KB)
  __shared__ float red[4][2][16][32];                  // projection sums per (row block, step) (16 KB)
  __shared__ float ssum[2][kTT];                       // sum x'^2, sum y^2 per token
  __shared__ float part[kThreads];                     // owned words: group sums, [pair][group]
  __shared__ float tot[kXFMaxOwn][kXW];                // owned words summed over the slices
  __shared__ f32x4 g_slice[NORM ? YK * kCF / 4 : 1];   // gamma of the slice
  __shared__ float s_cf[kMix + 3];                     // hc_base, hc_scale (read by the derive)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave >> 1, hw = wave & 1;   // row block, half (stream phase) / step (matrix phase)
  const int d = a.d, S = a.S;
  // XCD-aware: renumbered so that each XCD holds a contiguous run, slice-major
  // (the tiles of a slice share its weight tiles in one L2)
  const int lin = (gridDim.x & 7) ? blockIdx.x : (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int slice = lin / a.tiles, tile = lin % a.tiles;
  const int fs = slice * (YK * kCF);
  const int hl = lane >> 3, fl = (lane & 7) * 8;
  const int m = rb * 16 + hw * 8 + hl;                 // token within the tile
  const int a_st = fl >> 5, a_g = (fl >> 3) & 3;
  const int a_lane = a_g * 16 + hw * 8 + hl;

  // The call's tag, the slice's gamma and the split's parameters are
  // requested by every lane without a branch, and written to LDS only once
  // the first chunk's loads are in flight (a load inside a branch, with its
  // wait, holds every later load of the wave behind it: a round trip at the
  // start of a call that is all latency).
  const u32 tag = epoch_low(a.ctl) + 1u;   // words carry epoch + 1 (one value for every lane)
  f32x4 gv = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (NORM) gv = reinterpret_cast<const f32x4*>(a.gamma + fs)[min((int)threadIdx.x, YK * kCF / 4 - 1)];
  const int cfi = max((int)threadIdx.x - (kThreads - (kMix + 3)), 0);
  const float cfv = *(!a.pre_out ? reinterpret_cast<const float*>(a.ctl) : cfi < kMix ? a.hc_base + cfi : a.hc_scale + (cfi - kMix));
  auto stage_params = [&]() __attribute__((always_inline)) {
    if (NORM && threadIdx.x < YK * kCF / 4) g_slice[threadIdx.x] = gv;
    if (threadIdx.x >= kThreads - (kMix + 3)) s_cf[cfi] = cfv;   // read by the derive only with pre_out
  };
  const int64_t t0 = (int64_t)tile * kTT;
  const int nval = (int)min<int64_t>(kTT, a.n - t0);  // valid tokens of the tile
  const bool tv = m < nval;
  const unsigned lt = tv ? (unsigned)m : 0u;           // a token past n reads the tile's first token
  const hc_bf16* xb = a.x + t0 * a.xtok;
  float cpost[kHC], ccomb[kHC * kHC], cpre[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    cpost[j] = POST ? a.post_in[(t0 + lt) * kHC + j] : 0.f;
    cpre[j] = READ ? a.pre_in[(t0 + lt) * kHC + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHC * kHC; ++j) ccomb[j] = POST ? a.comb_in[(t0 + lt) * kHC * kHC + j] : 0.f;

  // the chunk's 2 x 4 x 5 weight tiles, 5 per wave
  auto load_wst = [&](int c, u32x4 (&dst)[kNT]) __attribute__((always_inline)) {
    const int gstep = (fs + c * kCF) / kStepF;
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      const int st = blk / (kHC * kNT), kk = (blk / kNT) % kHC, nt = blk % kNT;
      dst[i] = a.fn[((size_t)((gstep + st) * kHC + kk) * kNT + nt) * 64 + lane];
    }
  };
  auto store_wst = [&](int buf, const u32x4 (&src)[kNT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      const int blk = wave + i * kWaves;
      w_lds[buf][blk / (kHC * kNT)][(blk / kNT) % kHC][blk % kNT][lane] = src[i];
    }
  };
  auto load_stream = [&](int c, u32x4 (&dst)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
#pragma unroll
    for (int j = 0; j < kHC; ++j)
      dst[j] = ld_stream(reinterpret_cast<const u32x4*>(xb + (lt * (unsigned)a.xtok + j * (unsigned)a.xstr + f)));
    dst[kHC] = POST ? ld_stream(reinterpret_cast<const u32x4*>(a.delta + (t0 + lt) * d + f)) : u32x4{0u, 0u, 0u, 0u};
  };
  float ssx = 0.f, ssy = 0.f;
  f32x4 acc[kAcc];
#pragma unroll
  for (int t = 0; t < kAcc; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32 ykeep[NORM ? YK : 1][4];                         // the read row, chunk by chunk (RMSNorm)
  u32 xlast[kHC][4];                                   // X' of the last chunk, stored after the words
  auto store_x = [&](int c, const u32 (&xp)[kHC][4]) __attribute__((always_inline)) {
    if (tv) {
      hc_bf16* xob = a.x_out + (t0 + lt) * kHC * d + fs + c * kCF + fl;
#pragma unroll
      for (int j = 0; j < kHC; ++j)
        st_stream(reinterpret_cast<u32x4*>(xob + j * d), u32x4{xp[j][0], xp[j][1], xp[j][2], xp[j][3]});
    }
  };
  auto stream_phase = [&](int c, const u32x4 (&src)[kHC + 1]) __attribute__((always_inline)) {
    const unsigned f = fs + c * kCF + fl;
    u32 xp[kHC][4];
    if constexpr (POST) {
      post_8(src, cpost, ccomb, xp);
      if (c + 1 < YK) {
        store_x(c, xp);
      } else {
#pragma unroll
        for (int j = 0; j < kHC; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) xlast[j][e] = xp[j][e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[j][e] = src[j][e];
    }
    if constexpr (MEAN) {
      if (tv) st_stream(reinterpret_cast<u32x4*>(a.x_mean + (t0 + lt) * d + f), mean_8(xp));
    }
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ssx = dot2_bf16(xp[j][e], xp[j][e], ssx);
      a_lds[rb][a_st][j][a_swz(a_lane, a_st)] = u32x4{xp[j][0], xp[j][1], xp[j][2], xp[j][3]};
    }
    if constexpr (READ) {
      u32 yp[4];
      pre_8(xp, cpre, yp);
      if constexpr (NORM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ssy = dot2_bf16(yp[e], yp[e], ssy);
          ykeep[c][e] = yp[e];
        }
      } else if (tv) {
        st_stream(reinterpret_cast<u32x4*>(a.y_out + (t0 + lt) * d + f), u32x4{yp[0], yp[1], yp[2], yp[3]});
      }
    }
  };
  auto matrix_phase = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, a_lds[rb][hw][j][a_swz(lane, hw)]);
      bf16x8 B[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) B[nt] = __builtin_bit_cast(bf16x8, w_lds[buf][hw][j][nt][lane]);
      mfma_step(A, B, acc);
    }
  };
  // the chunks: the next chunk's weights, then its streams, are requested
  // before this chunk's work; two barriers (A tiles and weights in place; the
  // matrix phase done before the A tiles are rewritten)
  {
    u32x4 cur[kHC + 1], wst[kNT];
    load_wst(0, wst);
    load_stream(0, cur);
    stage_params();
    store_wst(0, wst);
    lds_barrier();
    auto chunk = [&]<int C>(IC<C>) __attribute__((always_inline)) {
      constexpr bool kMore = C + 1 < YK;
      u32x4 nxt[kHC + 1];
      if constexpr (kMore) {
        load_wst(C + 1, wst);
        load_stream(C + 1, nxt);
      }
      stream_phase(C, cur);
      lds_barrier();
      if constexpr (kMore) store_wst((C + 1) & 1, wst);
      matrix_phase(C & 1);
      if constexpr (kMore) {
        lds_barrier();
#pragma unroll
        for (int j = 0; j <= kHC; ++j) cur[j] = nxt[j];
      }
    };
    [&]<int... C>(std::integer_sequence<int, C...>) __attribute__((always_inline)) {
      (chunk(IC<C>{}), ...);
    }(std::make_integer_sequence<int, YK>{});
  }

  // ---- the words of the valid tokens, through LDS
  u64* tilew = a.xw + (size_t)tile * S * kTT * kXW;
  u64* mine = tilew + (size_t)slice * kTT * kXW;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    ssx += __shfl_xor(ssx, o);
    if constexpr (NORM) ssy += __shfl_xor(ssy, o);
  }
#pragma unroll
  for (int t = 0; t < kAcc; ++t)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[rb][hw][4 * (lane >> 4) + rr][t * 16 + (lane & 15)] = acc[t][rr];
  if ((lane & 7) == 0) {
    ssum[0][m] = ssx;
    ssum[1][m] = ssy;
  }
  lds_barrier();
  for (int i = threadIdx.x; i < nval * kOW; i += kThreads) {
    const int tm = i / kOW, q = i % kOW;
    float v;
    if (q < kMix) {
      const float* r0 = red[tm >> 4][0][tm & 15];
      const float* r1 = red[tm >> 4][1][tm & 15];
      v = q < 16 ? r0[q] + r1[q] : (r0[q] + r0[q + 8]) + (r1[q] + r1[q + 8]);
    } else {
      v = ssum[q - kMix][tm];
    }
    put_word(mine + tm * kXW + q, tag_word(v, tag));
  }
  if constexpr (POST) store_x(YK - 1, xlast);   // so that the words do not queue behind these stores

  // ---- the owned tokens' words from every slice, in one round trip
  const int nown = slice < nval ? (nval - 1 - slice) / S + 1 : 0;   // owned tokens slice, slice + S, ...
  const int npairs = nown * kOW;
  // slices summed in slice order when a thread can load them all (as the
  // two-launch finish does), else in G interleaved groups
  const int G = npairs && S > kXFOLoads ? min(kXFGroups, kThreads / npairs) : 1;
  const bool has_o = (int)threadIdx.x < npairs * G;
  const int opr = has_o ? threadIdx.x / G : 0, og = has_o ? threadIdx.x % G : 0;
  const int ok = opr / kOW, oq = opr % kOW;
  const int otm = slice + S * ok;
  auto wptr = [&](int i) { return tilew + ((size_t)(og + G * i) * kTT + otm) * kXW + oq; };
  auto wuse = [&](int i) { return has_o && og + G * i < S; };
  u64 wv[kXFOLoads];
#pragma unroll
  for (int i = 0; i < kXFOLoads; ++i) wv[i] = wuse(i) ? get_word(wptr(i)) : 0ull;
  bool dead = false;
  settle_all(wv, wptr, wuse, tag, a.err, dead);
  if (has_o) {
    float po = 0.f;
#pragma unroll
    for (int i = 0; i < kXFOLoads; ++i)
      if (og + G * i < S) {
        const float v = __uint_as_float((u32)wv[i]);
        po = i == 0 ? v : po + v;
      }
    part[opr * G + og] = po;
  }
  __syncthreads();
  if ((int)threadIdx.x < npairs) {
    const int k = threadIdx.x / kOW, q = threadIdx.x % kOW;
    float v = part[threadIdx.x * G];
    for (int g = 1; g < G; ++g) v += part[threadIdx.x * G + g];
    tot[k][q] = v;
  }
  __syncthreads();
  constexpr int kDoneThread = kThreads - 1;
  // the factor of token tm: its owner's sum y^2 slot, tagged ~tag
  auto rword = [&](int tm) { return tilew + ((size_t)(tm % S) * kTT + tm) * kXW + kMix + 1; };
  if constexpr (NORM) {   // the owned tokens' factors, for every slice of the tile
    if ((int)threadIdx.x < nown) {
      const int tm = slice + S * threadIdx.x;
      put_word(rword(tm), tag_word(1.0f / sqrtf(tot[threadIdx.x][kXW - 1] / (float)d + a.rms_eps), ~tag));
    }
  }
  // ---- the owned tokens' mixes, pre/post and comb: 16 lanes per token
  if ((int)threadIdx.x < 16 * nown) {
    const int k = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int tm = slice + S * k;
    const float* r = tot[k];
    const float rx = 1.0f / sqrtf(r[kMix] / (float)(kHC * d) + a.norm_eps);
    derive_16(r, rx, q >> 2, q & 3, true, t0 + tm, s_cf + kMix, s_cf, a.iters, a.hc_eps,
              a.mixes_out, a.pre_out, a.post_out, a.comb_out);
  }
  // ---- z = gamma * (y * r) for the slice, r from the token's owner
  if constexpr (NORM) {
    u64 rv[1] = {tv ? get_word(rword(m)) : 0ull};
    settle_all(rv, [&](int) { return rword(m); }, [&](int) { return tv; }, ~tag, a.err, dead);
    if (tv) {
      const float ry = __uint_as_float((u32)rv[0]);
#pragma unroll
      for (int c = 0; c < YK; ++c) {
        const f32x4 g0 = g_slice[(c * kCF + fl) / 4];
        const f32x4 g1 = g_slice[(c * kCF + fl) / 4 + 1];
        const float gm[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        u32 zp[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          zp[e2] = pack_bf16(gm[2 * e2] * (bf_lo(ykeep[c][e2]) * ry), gm[2 * e2 + 1] * (bf_hi(ykeep[c][e2]) * ry));
        st_stream(reinterpret_cast<u32x4*>(a.y_out + (t0 + lt) * d + fs + c * kCF + fl), u32x4{zp[0], zp[1], zp[2], zp[3]});
      }
    }
    __syncthreads();   // every factor word of this workgroup read before it counts itself done
  }
  // every word of this call read: count this workgroup done; the last one
  // advances the call epoch
  if (threadIdx.x == kDoneThread) {
    const u64 before = __hip_atomic_fetch_add(a.ctl + kCtlXDone, (u64)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before % (u64)gridDim.x == (u64)(gridDim.x - 1)) {
      put_word(a.ctl + kCtlXDone, 0ull);
      put_word(a.ctl + kCtlXEpoch, (u64)tag);
    }
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

// The library's own workspace for hc_boundary_static, one copy per GPU the
// library runs on (held until the process ends).  Zero when the code object
// is loaded, as a fresh caller workspace must be; every call leaves it valid
// for the next (the tagged words' call epochs only grow).  Host code uses the
// per-device address from hipGetSymbolAddress, never the name itself.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// one 32-bit word set to zero (a kernel rather than a memset, so that it may
// sit in a captured graph)
__global__ void clear_word_kernel(u32* w) {
  if (threadIdx.x == 0) *w = 0u;
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

// The device address of the static scratch on the current device, looked up
// once per device (nullptr and HC_EHIP detail on failure).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
void* static_scratch(int* rc) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = fail(HC_ENODEV, "no current HIP device: %s", hipGetErrorName(e));
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *rc = fail(HC_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorName(e));
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);   // the same value whichever thread wins
  }
  *rc = HC_OK;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) share a byte (both non-empty)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

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
// slices of the projection kernel (128-token workgroups)
int proj_slices(int64_t n, int d) {
  const int64_t tiles2 = (n + 2 * kTT - 1) / (2 * kTT);
  return divisor_at_least(d / kCF, std::min<int64_t>((256 + tiles2 - 1) / tiles2, kMaxSlices));
}
int read_slices(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return divisor_at_least(d / kCF, std::min<int64_t>((512 + tiles - 1) / tiles, kMaxSlices));
}
size_t split_records_bytes(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  return (size_t)tiles * std::max(stream_slices(n, d), proj_slices(n, d)) * kTT * kRec * 4;
}
// Workspace layout, the same for every (n, hc, d), so that one workspace
// serves calls of any shape and no region of one call lies on the persistent
// words of another:
//   [control block, kCtrlBytes]  error mask, the read-row exchanges' epoch and
//                                done words
//   [read-row exchange words]    [kXMaxGroups][kTT][kXW] tagged words (both
//                                exchange kernels)
//   [per-slice records]          two-launch schedule (hc = 4) or hc = 2, 8;
//                                plain floats, rewritten by every call
// Tagged words carry the exchanges' call epoch + 1 (the few-tile exchange's
// RMS factor words its complement); the epoch only grows, so a word left by an
// earlier call (of any shape) never holds a current tag.
constexpr int kXMaxGroups = 256;             // (tile, slice) groups (= workgroups) of one read-row exchange at most
constexpr size_t kXRegionBytes = (size_t)kXMaxGroups * kTT * kXW * sizeof(u64);
constexpr size_t kXOffset = kCtrlBytes;
constexpr size_t kRecOffset = kXOffset + kXRegionBytes;
constexpr int64_t kXPart = (int64_t)kXMaxGroups / 4 * kTT;   // tokens of the largest exchange (4 slices a tile)
// The per-slice records a call of n tokens can need: its own, and, since a
// call beyond kXPart tokens may run as parts of kXPart tokens and a rest (any
// shorter count, whose slices can be more), those of every shorter call.
size_t records_bytes(int64_t n, int d) {
  size_t b = split_records_bytes(n, d);
  if (n > kXPart)
    for (int64_t t = 1; t <= kXPart / kTT; ++t) b = std::max(b, split_records_bytes(t * kTT, d));
  return b;
}
size_t workspace_bytes(int64_t n, int d) { return kRecOffset + records_bytes(n, d); }

// without POST the 128-token projection kernel, with it the stream kernel
template <bool POST, int RM, bool NORM>
hipError_t launch_stream_t(const StreamArgs& a, unsigned grid, hipStream_t st) {
  StreamArgs copy = a;
  void* args[] = {&copy};
  const void* fn;
  if constexpr (POST) {
    fn = a.x_mean ? reinterpret_cast<const void*>(&stream_kernel<RM, NORM, true>)
                  : reinterpret_cast<const void*>(&stream_kernel<RM, NORM, false>);
  } else {
    fn = a.x_mean ? reinterpret_cast<const void*>(&proj_kernel<RM, NORM, true>)
                  : reinterpret_cast<const void*>(&proj_kernel<RM, NORM, false>);
  }
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
}
// the given-pre boundary with the RMSNorm in one launch (read row kept, slice YK chunks wide)
template <bool POST, int YK>
hipError_t launch_exchange_t(const StreamArgs& a, unsigned grid, hipStream_t st) {
  StreamArgs copy = a;
  void* args[] = {&copy};
  const void* fn;
  if constexpr (POST) {
    fn = a.x_mean ? reinterpret_cast<const void*>(&exchange_kernel<true, true, YK>)
                  : reinterpret_cast<const void*>(&exchange_kernel<true, false, YK>);
  } else if (a.xstr == 0) {   // the four streams are one row: the stream-summed weight
    fn = a.x_mean ? reinterpret_cast<const void*>(&exchange_kernel<false, true, YK, true>)
                  : reinterpret_cast<const void*>(&exchange_kernel<false, false, YK, true>);
  } else {
    fn = a.x_mean ? reinterpret_cast<const void*>(&exchange_kernel<false, true, YK>)
                  : reinterpret_cast<const void*>(&exchange_kernel<false, false, YK>);
  }
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
}
// the few-tile exchange (decode, short prefill): YK chunks per workgroup
template <bool POST, bool READ, bool NORM, int YK>
hipError_t launch_xfew_yk(const StreamArgs& a, unsigned grid, hipStream_t st) {
  StreamArgs copy = a;
  void* args[] = {&copy};
  const void* fn = a.x_mean ? reinterpret_cast<const void*>(&xfew_kernel<POST, true, READ, NORM, YK>)
                            : reinterpret_cast<const void*>(&xfew_kernel<POST, false, READ, NORM, YK>);
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
}
template <bool POST, bool READ, bool NORM>
hipError_t launch_xfew_t(const StreamArgs& a, int yk, unsigned grid, hipStream_t st) {
  switch (yk) {
    case 1: return launch_xfew_yk<POST, READ, NORM, 1>(a, grid, st);
    case 2: return launch_xfew_yk<POST, READ, NORM, 2>(a, grid, st);
    case 4: return launch_xfew_yk<POST, READ, NORM, 4>(a, grid, st);
    case 5: return launch_xfew_yk<POST, READ, NORM, 5>(a, grid, st);
    case 8: return launch_xfew_yk<POST, READ, NORM, 8>(a, grid, st);
    default: return launch_xfew_yk<POST, READ, NORM, 10>(a, grid, st);
  }
}
// Chunks per workgroup of the few-tile exchange for (n, d): the fewest of 1,
// 2, 4, 5, 8, 10 that divide d / 64 and leave at most 256 workgroups (one per
// compute unit, all resident) with at least 8 slices per tile; 0 if none does.
int xfew_chunks(int64_t n, int d) {
  if (d % kCF || d < kXFMinD || d > kXFMaxD) return 0;
  const int64_t tiles = (n + kTT - 1) / kTT;
  const int nch = d / kCF;
  for (int yk : {1, 2, 4, 5, 8, 10})
    if (nch % yk == 0 && nch / yk >= kXFMinS && tiles * (nch / yk) <= kXMaxGroups) return yk;
  return 0;
}
// The read-row exchange: slices of 10 or 20 chunks (640 or 1280 features), 4
// to kXS slices per tile (the owned (token, word) pairs of a workgroup fit its
// threads), and every workgroup resident at once (at most 256, one per
// compute unit).  The slices are the two-launch schedule's where those fit;
// else, from 20 tiles up (fewer leave too many compute units idle), slices of
// 10 chunks, else of 20.  Returns the slice count, 0 if the shape has no such
// split.  (Shapes the few-tile exchange takes, up to 2048 tokens at d = 5120,
// run that instead: measured at n = 1280 and 1536, 38.2 and 40.2 us against
// 40.4 and 41.7 us; equal at 2048.)
int exchange_slices(int64_t n, int d) {
  const int64_t tiles = (n + kTT - 1) / kTT;
  auto fits = [&](int S) {
    const int yk = S > 0 && d / kCF % S == 0 ? d / kCF / S : 0;
    return (yk == 10 || yk == 20) && S >= 4 && S <= kXS && tiles * S <= kXMaxGroups;
  };
  const int S = stream_slices(n, d);
  if (fits(S)) return S;
  if (d / kCF % 10 == 0 && fits(d / kCF / 10) && tiles >= 20) return d / kCF / 10;
  if (d / kCF % 20 == 0 && fits(d / kCF / 20)) return d / kCF / 20;   // more tiles than 10-chunk slices allow
  return 0;
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
                    hipStream_t st, const char* what, int phases = 3, bool exchange = false) {
  const size_t need = workspace_bytes(s.n, s.d);
  if (!ws) return fail(HC_EINVAL, "%s: workspace must not be NULL (need %zu bytes)", what, need);
  if (!aligned16(ws)) return fail(HC_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need) return fail(HC_EINVAL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
  const int64_t tiles = (s.n + kTT - 1) / kTT;
  if (tiles * kMaxSlices > INT32_MAX) return fail(HC_ENOTSUP, "%s: n=%lld is too large", what, (long long)s.n);
  s.S = stream_slices(s.n, s.d);
  s.F = s.d / s.S;
  s.tiles = (int)tiles;
  s.rec = reinterpret_cast<float*>(static_cast<char*>(ws) + kRecOffset);
  const unsigned grid1 = (unsigned)(tiles * s.S);
  hipError_t e = hipSuccess;
  const int xyk = exchange && phases == 3 && rm != kFreshPre ? xfew_chunks(s.n, s.d) : 0;
  const int xs = exchange && phases == 3 && rm == kGivenPre && norm && !xyk ? exchange_slices(s.n, s.d) : 0;
  if (xyk) {
    // few token tiles: slices of xyk chunks, the tile's slices exchanging their words
    s.S = s.d / kCF / xyk;
    s.F = s.d / s.S;
    s.ctl = static_cast<u64*>(ws);
    s.xw = reinterpret_cast<u64*>(static_cast<char*>(ws) + kXOffset);
    s.err = static_cast<u32*>(ws) + kErrWord;
    s.gamma = f.gamma; s.hc_base = f.hc_base; s.hc_scale = f.hc_scale; s.mixes_out = f.mixes_out;
    s.pre_out = f.pre_out; s.post_out = f.post_out; s.comb_out = f.comb_out; s.iters = f.iters;
    s.hc_eps = f.hc_eps; s.norm_eps = f.norm_eps; s.rms_eps = f.rms_eps;
    if ((size_t)tiles * s.S * kTT * kXW * sizeof(u64) > kXRegionBytes)
      return fail(HC_ENOTSUP, "%s: %lld exchange groups exceed the region", what, (long long)(tiles * s.S));
    const unsigned grid = (unsigned)(tiles * s.S);
    if (rm == kNoRead) e = launch_xfew_t<false, false, false>(s, xyk, grid, st);
    else if (post) e = norm ? launch_xfew_t<true, true, true>(s, xyk, grid, st) : launch_xfew_t<true, true, false>(s, xyk, grid, st);
    else e = norm ? launch_xfew_t<false, true, true>(s, xyk, grid, st) : launch_xfew_t<false, true, false>(s, xyk, grid, st);
    return launched(e, what);
  }
  if (xs) {
    const int yk = s.d / kCF / xs;
    s.S = xs;
    s.F = s.d / xs;
    // the words of every (tile, slice) group stay inside the exchange region
    if ((size_t)tiles * s.S * kTT * kXW * sizeof(u64) > kXRegionBytes)
      return fail(HC_ENOTSUP, "%s: %lld exchange groups exceed the region", what, (long long)(tiles * s.S));
    s.ctl = static_cast<u64*>(ws);
    s.xw = reinterpret_cast<u64*>(static_cast<char*>(ws) + kXOffset);
    s.err = static_cast<u32*>(ws) + kErrWord;
    s.gamma = f.gamma; s.hc_base = f.hc_base; s.hc_scale = f.hc_scale; s.mixes_out = f.mixes_out;
    s.pre_out = f.pre_out; s.post_out = f.post_out; s.comb_out = f.comb_out; s.iters = f.iters;
    s.hc_eps = f.hc_eps; s.norm_eps = f.norm_eps; s.rms_eps = f.rms_eps;
    const unsigned grid = (unsigned)(tiles * s.S);
    if (post) e = yk == 20 ? launch_exchange_t<true, 20>(s, grid, st) : launch_exchange_t<true, 10>(s, grid, st);
    else e = yk == 20 ? launch_exchange_t<false, 20>(s, grid, st) : launch_exchange_t<false, 10>(s, grid, st);
    return launched(e, what);
  }
  if (!post) {                                    // the projection kernel: 128-token workgroups
    s.S = proj_slices(s.n, s.d);
    s.F = s.d / s.S;
  }
  const unsigned gridp = (unsigned)((tiles + 1) / 2 * s.S);
  if (phases & 1) switch ((post ? 8 : 0) | (rm << 1) | (norm ? 1 : 0)) {
    case 0x0: e = launch_stream_t<false, kNoRead, false>(s, gridp, st); break;
    case 0x2: e = launch_stream_t<false, kGivenPre, false>(s, gridp, st); break;
    case 0x3: e = launch_stream_t<false, kGivenPre, true>(s, gridp, st); break;
    case 0x4: e = launch_stream_t<false, kFreshPre, false>(s, gridp, st); break;
    case 0x5: e = launch_stream_t<false, kFreshPre, true>(s, gridp, st); break;
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

// the stream-only calls without the RMSNorm as an address-order sweep; false
// if the grid would not fit (then the row kernel runs)
template <bool POST, bool PRE, int HC = kHC>
bool launch_sweep_t(const RowArgs& a, hipStream_t st, hipError_t& e) {
  const int64_t units = a.n * (int64_t)((a.d + kRowChunk - 1) / kRowChunk);
  const int64_t grid = (units + kSweepWaves - 1) / kSweepWaves;
  if (grid > INT32_MAX) return false;
  RowArgs copy = a;
  void* args[] = {&copy};
  e = hipLaunchKernel(reinterpret_cast<const void*>(&sweep_row_kernel<POST, PRE, HC>), dim3((unsigned)grid),
                      dim3(kSweepWaves * 64), args, 0, st);
  return true;
}
// with the RMSNorm: a workgroup per token, up to kSweepNormMaxW waves, at most
// two chunks per wave (d <= 10240); false if the shape does not fit
template <bool POST, int HC>
bool launch_sweep_norm_t(const RowArgs& a, hipStream_t st, hipError_t& e) {
  const int nch = (a.d + kRowChunk - 1) / kRowChunk;
  const int W = std::min(nch, kSweepNormMaxW);
  const int cpw = (nch + W - 1) / W;
  if (cpw > 2 || a.n > INT32_MAX) return false;
  RowArgs copy = a;
  void* args[] = {&copy};
  const void* fn = cpw == 1 ? reinterpret_cast<const void*>(&sweep_norm_kernel<POST, 1, HC>)
                            : reinterpret_cast<const void*>(&sweep_norm_kernel<POST, 2, HC>);
  e = hipLaunchKernel(fn, dim3((unsigned)a.n), dim3(W * 64), args, 0, st);
  return true;
}
template <int HC>
bool launch_sweep_hc(int key, const RowArgs& a, hipStream_t st, hipError_t& e) {
  switch (key) {
    case 0b100: return launch_sweep_t<true, false, HC>(a, st, e);
    case 0b010: return launch_sweep_t<false, true, HC>(a, st, e);
    case 0b110: return launch_sweep_t<true, true, HC>(a, st, e);
    // with the RMSNorm only at hc = 4 (at hc = 2 and 8 the read after the
    // projection measured slower as a sweep: 65.3 against 63.6 and 303.7
    // against 289.8 us per boundary at n = 4096)
    case 0b011:
      if constexpr (HC == kHC) return launch_sweep_norm_t<false, HC>(a, st, e);
      return false;
    case 0b111:
      if constexpr (HC == kHC) return launch_sweep_norm_t<true, HC>(a, st, e);
      return false;
    default: return false;
  }
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
  {   // the address-order sweep where the shape fits it
    const bool ok = hc == 2 ? launch_sweep_hc<2>(key, a, st, e)
                  : hc == 8 ? launch_sweep_hc<8>(key, a, st, e) : launch_sweep_hc<kHC>(key, a, st, e);
    if (ok) return launched(e, what);
  }
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

// slices of the fused hc = 2 write and projection: of the feature range of d
int fused_slices(int64_t n, int d) {
  const int64_t groups = (n + kGTok - 1) / kGTok;
  const int chunks = d / kGChunk;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(64, (512 + groups - 1) / groups));
  int best = 1;
  for (int s = 1; s <= want; ++s)
    if (chunks % s == 0) best = s;
  return best;
}

// workspace of the hc != 4 path: the per-slice records (of the projection
// kernel or, at hc = 2, of the fused write and projection), placed after the
// control block and the exchange words so that a workspace shared with
// hc = 4 calls keeps their words intact
size_t gen_rec_offset(int) { return kRecOffset; }
size_t generic_ws_bytes(int64_t n, int hc, int d) {
  const int S = hc == 2 ? std::max(gen_slices(n, hc, d), fused_slices(n, d)) : gen_slices(n, hc, d);
  return gen_rec_offset(d) + (size_t)S * n * gen_recw(hc) * 4;
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
// the finish of the hc != 4 projection: f.rec, f.n, f.S and f.K set
int launch_gfinish(int hc, GFinArgs f, hipStream_t st, const char* what) {
  void* fargs[] = {&f};
  const int64_t tpb = 256 / hc;                   // tokens per workgroup: hc lanes each
  const hipError_t e = hipLaunchKernel(hc == 2 ? reinterpret_cast<const void*>(&gfinish_kernel<2>)
                                               : reinterpret_cast<const void*>(&gfinish_kernel<8>),
                                       dim3((unsigned)((f.n + tpb - 1) / tpb)), dim3(256), fargs, 0, st);
  return launched(e, what);
}

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
  return launch_gfinish(hc, f, st, what);
}

// hc = 2, a write with a fresh pre: the fused write and projection (phase 1), the finish (phase 2)
int launch_stream_generic(const hc_boundary_args* p, int xtok, int xstr, hc_bf16* x_mean, GFinArgs f,
                          hipStream_t st, const char* what, int phases) {
  GStreamArgs g{};
  g.x = p->x; g.delta = p->delta; g.post_in = p->post_in; g.comb_in = p->comb_in;
  g.fn = static_cast<const u32x4*>(p->fn_packed); g.x_out = p->x_out; g.x_mean = x_mean;
  g.n = p->n; g.xtok = xtok; g.xstr = xstr; g.d = p->d;
  g.S = fused_slices(p->n, p->d);
  g.Fs = p->d / g.S;
  g.rec = reinterpret_cast<float*>(static_cast<char*>(p->workspace) + gen_rec_offset(p->d));
  if (phases & 1) {
    void* args[] = {&g};
    const dim3 grid((unsigned)((p->n + kGTok - 1) / kGTok * g.S));
    const hipError_t e = hipLaunchKernel(x_mean ? reinterpret_cast<const void*>(&gstream_kernel<2, true>)
                                                : reinterpret_cast<const void*>(&gstream_kernel<2, false>),
                                         grid, dim3(kGThreads), args, 0, st);
    const int rc = launched(e, what);
    if (rc || !(phases & 2)) return rc;
  }
  f.rec = g.rec; f.n = p->n; f.S = g.S; f.K = 2 * p->d;
  return launch_gfinish(2, f, st, what);
}

constexpr int64_t kSplit16MaxN = 8192;   // hc_split_sinkhorn at hc = 4 takes 16 lanes per token up to here
int launch_split(int hc, const float* mixes, const float* scale, const float* base, int64_t n, int iters,
                 float eps, float* pre, float* post, float* comb, hipStream_t st) {
  const int64_t tpb = 256 / hc;                   // tokens per workgroup: hc lanes each
  const dim3 grid((unsigned)((n + tpb - 1) / tpb)), block(256);
  if (hc == 2)
    hipLaunchKernelGGL(split_kernel<2>, grid, block, 0, st, mixes, scale, base, n, iters, eps, pre, post, comb);
  else if (hc == 8)
    hipLaunchKernelGGL(split_kernel<8>, grid, block, 0, st, mixes, scale, base, n, iters, eps, pre, post, comb);
  else if (n <= kSplit16MaxN)   // latency-bound: the shorter chain wins (n = 4096: 3.1 against 3.5 us)
    hipLaunchKernelGGL(split16_kernel, dim3((unsigned)((n + 15) / 16)), block, 0, st, mixes, scale, base, n, iters, eps,
                       pre, post, comb);
  else                          // throughput-bound: 4x fewer lanes (n = 32768: 5.0 against 6.4 us)
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
  return (size_t)(d / kStepF) * (kHC + 1) * kNT * 64 * 16;   // + the stream-summed tiles
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
  const int records = (d / kStepF) * (kHC + 1) * kNT * 64;
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
  StreamArgs s{};
  s.n = n; s.d = d; s.x = x; s.fn = reinterpret_cast<const u32x4*>(fn_packed);
  s.xtok = kHC * d; s.xstr = d;
  FinishArgs f{};
  f.mixes_out = mixes; f.norm_eps = norm_eps; f.hc_scale = hc_scale; f.hc_base = hc_base; f.iters = iters;
  f.hc_eps = hc_eps;
  if (split) { f.pre_out = pre; f.post_out = post; f.comb_out = comb; }
  return launch_boundary(false, kNoRead, false, s, f, workspace, workspace_bytes, (hipStream_t)stream, "hc_mixes", 3,
                         n <= kXFMixesMaxN);
}

int hc_pre(const hc_bf16* x, const float* pre_mix, int64_t n, int hc, int d, hc_bf16* y, void* stream) {
  g_err[0] = 0;
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  HC_REQ(x); HC_REQ(pre_mix); HC_REQ(y);
  if (overlap(y, (size_t)n * d * 2, x, (size_t)n * hc * d * 2)) return fail(HC_EINVAL, "y overlaps x");
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
  {
    const size_t sb = (size_t)n * hc * d * 2, rb = (size_t)n * d * 2;
    if (overlap(x_out, sb, x, sb)) return fail(HC_EINVAL, "x_out overlaps x");
    if (overlap(x_out, sb, delta, rb)) return fail(HC_EINVAL, "x_out overlaps delta");
  }
  if (n == 0) return HC_OK;
  if ((rc = check_device())) return rc;
  RowArgs a{};
  a.n = n; a.d = d; a.delta = delta; a.x = x; a.post_in = post; a.comb_in = comb; a.x_out = x_out;
  a.xtok = hc * d; a.xstr = d;
  return launch_row(true, false, false, a, (hipStream_t)stream, "hc_post", hc);
}

size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d) { return hc_workspace_bytes(n, hc, d); }

int hc_workspace_layout(int64_t n, int hc, int d, size_t regions[6]) {
  g_err[0] = 0;
  if (!regions) return fail(HC_EINVAL, "regions must not be NULL");
  int rc = check_hd(hc, d);
  if (rc) return rc;
  if ((rc = check_n(n))) return rc;
  regions[0] = 0;            regions[1] = kCtrlBytes;
  regions[2] = kXOffset;     regions[3] = kXRegionBytes;
  regions[4] = kRecOffset;
  regions[5] = n == 0 ? 0 : (hc == kHC ? records_bytes(n, d) : generic_ws_bytes(n, hc, d) - kRecOffset);
  return HC_OK;
}

int hc_workspace_status(void* workspace, size_t workspace_bytes, int clear, uint32_t* mask, void* stream) {
  g_err[0] = 0;
  HC_REQ(workspace);
  if (!mask) return fail(HC_EINVAL, "mask must not be NULL");
  if (workspace_bytes < (size_t)kCtrlBytes)
    return fail(HC_EINVAL, "workspace has %zu bytes, the control block alone is %d", workspace_bytes, kCtrlBytes);
  int rc;
  if ((rc = check_device())) return rc;
  const hipStream_t st = (hipStream_t)stream;
  u32* word = static_cast<u32*>(workspace) + kErrWord;
  hipError_t e = hipMemcpyAsync(mask, word, sizeof(u32), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(HC_EHIP, "reading the error mask: %s", hipGetErrorName(e));
  if (clear) {
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, st, word);
    return launched(hipGetLastError(), "clear_word_kernel");
  }
  return HC_OK;
}

static int boundary_phases(const hc_boundary_args* p, void* stream, int phases) {
  g_err[0] = 0;
  if (!p) return fail(HC_EINVAL, "args must not be NULL");
  constexpr size_t kNoFlags = offsetof(hc_boundary_args, flags);   // callers of the field-less struct
  if (p->struct_size < kNoFlags)
    return fail(HC_EINVAL, "struct_size=%u, expected %zu", p->struct_size, sizeof(hc_boundary_args));
  const uint32_t flags = p->struct_size >= kNoFlags + sizeof(uint32_t) ? p->flags : 0u;
  constexpr size_t kNoMean = offsetof(hc_boundary_args, x_mean_out);   // callers of the struct without it
  hc_bf16* const x_mean = p->struct_size >= kNoMean + sizeof(void*) ? p->x_mean_out : nullptr;
  if (flags & ~(HC_BOUNDARY_X_EXPANDED | HC_BOUNDARY_TWO_LAUNCH))
    return fail(HC_EINVAL, "flags=%#x: unknown bits", flags);
  const bool expanded = (flags & HC_BOUNDARY_X_EXPANDED) != 0;
  int rc = check_hd(p->hc, p->d);
  if (rc) return rc;
  if ((rc = check_n(p->n))) return rc;
  const bool post = p->delta != nullptr;
  const bool mix = p->fn_packed != nullptr;
  const bool fresh = p->pre_in == nullptr;
  const bool norm = p->gamma != nullptr;
  HC_REQ(p->x); HC_REQ(p->y_out); HC_OPT(p->delta); HC_OPT(p->pre_in); HC_OPT(p->gamma); HC_OPT(x_mean);
  if (post) { HC_REQ(p->post_in); HC_REQ(p->comb_in); HC_REQ(p->x_out); }
  if (mix) {
    HC_REQ(p->fn_packed); HC_REQ(p->hc_base); HC_REQ(p->hc_scale);
    HC_REQ(p->pre_out); HC_REQ(p->post_out); HC_REQ(p->comb_out); HC_OPT(p->mixes_out);
    if (p->iters < 1) return fail(HC_EINVAL, "iters=%d: at least one Sinkhorn round is needed", p->iters);
  }
  if (fresh && !mix) return fail(HC_EINVAL, "pre_in is NULL but no mixes are derived (fn_packed is NULL)");
  if (norm && p->d > kRowChunk * kRowMaxChunks * 2)
    return fail(HC_ENOTSUP, "RMSNorm of the read row supports d <= %d", kRowChunk * kRowMaxChunks * 2);
  {  // the outputs may not overlap the streams they are formed from, nor each other
    const size_t n = (size_t)p->n, hc = (size_t)p->hc, d = (size_t)p->d;
    const size_t xb = n * (expanded ? 1 : hc) * d * 2, sb = n * hc * d * 2, rb = n * d * 2;
    if (post && overlap(p->x_out, sb, p->x, xb)) return fail(HC_EINVAL, "x_out overlaps x");
    if (post && overlap(p->x_out, sb, p->delta, rb)) return fail(HC_EINVAL, "x_out overlaps delta");
    if (overlap(p->y_out, rb, p->x, xb)) return fail(HC_EINVAL, "y_out overlaps x");
    if (post && overlap(p->y_out, rb, p->x_out, sb)) return fail(HC_EINVAL, "y_out overlaps x_out");
    if (overlap(p->y_out, rb, p->delta, rb)) return fail(HC_EINVAL, "y_out overlaps delta");
    if (x_mean && overlap(x_mean, rb, p->y_out, rb)) return fail(HC_EINVAL, "x_mean_out overlaps y_out");
    if (x_mean && overlap(x_mean, rb, p->x, xb)) return fail(HC_EINVAL, "x_mean_out overlaps x");
    if (x_mean && post && overlap(x_mean, rb, p->x_out, sb)) return fail(HC_EINVAL, "x_mean_out overlaps x_out");
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
  if (p->hc != kHC) {
    // hc 2 or 8: the write, the projection, the split and the read as separate
    // launches; begin does the write (and a read from a given pre), end the rest
    const int hc = p->hc, d = p->d;
    if ((rc = check_generic_ws(p->n, hc, d, p->workspace, p->workspace_bytes, "hc_boundary"))) return rc;
    RowArgs r{};
    r.n = p->n; r.d = d; r.x = p->x; r.delta = p->delta; r.post_in = p->post_in; r.comb_in = p->comb_in;
    r.gamma = p->gamma; r.x_out = p->x_out; r.y_out = p->y_out; r.rms_eps = p->rms_eps;
    r.xtok = xtok; r.xstr = xstr;
    if (hc == 2 && post && fresh) {
      // the write and the projection in one pass (begin); the finish and the read (end)
      GFinArgs f{};
      f.hc_scale = p->hc_scale; f.hc_base = p->hc_base; f.mixes_out = p->mixes_out; f.pre_out = p->pre_out;
      f.post_out = p->post_out; f.comb_out = p->comb_out; f.iters = p->iters; f.norm_eps = p->norm_eps;
      f.hc_eps = p->hc_eps;
      if ((rc = launch_stream_generic(p, xtok, xstr, x_mean, f, st, "hc_boundary", phases))) return rc;
      if (!(phases & 2)) return HC_OK;
      RowArgs rd = r;
      rd.x = p->x_out; rd.xtok = hc * d; rd.xstr = d; rd.delta = nullptr; rd.post_in = nullptr;
      rd.comb_in = nullptr; rd.x_out = nullptr; rd.pre_in = p->pre_out; rd.x_mean = nullptr;
      return launch_row(false, true, norm, rd, st, "hc_boundary (read)", hc);
    }
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
  const bool two = (flags & HC_BOUNDARY_TWO_LAUNCH) != 0;
  // Consecutive calls on parts of kXPart tokens, then the rest as its own call
  // (whatever schedule suits it): a given pre with the RMSNorm beyond one
  // exchange's reach (one launch a part), and a fresh pre from 4 kXPart tokens
  // on (where the two launches' slices are a whole row: measured at n = 32768,
  // 871 against 965 us with the RMSNorm; at n = 8192 the parts are no faster)
  const bool split_given = !fresh && norm && p->n > kXPart;
  const bool split_fresh = fresh && p->n >= 4 * kXPart;
  if (phases == 3 && !two && (split_given || split_fresh) && exchange_slices(kXPart, p->d)) {
    hc_boundary_args q{};
    memcpy(&q, p, std::min<size_t>(p->struct_size, sizeof q));
    q.struct_size = sizeof q;
    q.x_mean_out = x_mean;
    q.flags = flags;
    for (int64_t t0 = 0; t0 < p->n; t0 += kXPart) {
      const int64_t m = std::min<int64_t>(kXPart, p->n - t0);
      q.n = m;
      q.x = p->x + t0 * xtok;
      q.delta = post ? p->delta + t0 * p->d : nullptr;
      q.post_in = post ? p->post_in + t0 * kHC : nullptr;
      q.comb_in = post ? p->comb_in + t0 * kHC * kHC : nullptr;
      q.pre_in = fresh ? nullptr : p->pre_in + t0 * kHC;
      q.x_out = post ? p->x_out + t0 * kHC * p->d : nullptr;
      q.y_out = p->y_out + t0 * p->d;
      q.x_mean_out = x_mean ? x_mean + t0 * p->d : nullptr;
      q.mixes_out = p->mixes_out ? p->mixes_out + t0 * kMix : nullptr;
      q.pre_out = p->pre_out + t0 * kHC;
      q.post_out = p->post_out + t0 * kHC;
      q.comb_out = p->comb_out + t0 * kHC * kHC;
      if ((rc = boundary_phases(&q, stream, 3))) return rc;
    }
    return HC_OK;
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
                         "hc_boundary", phases, !two);
}

int hc_boundary(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 3); }

int hc_boundary_static(const hc_boundary_args* p, void* stream) {
  g_err[0] = 0;
  if (!p) return fail(HC_EINVAL, "args must not be NULL");
  if (p->struct_size < offsetof(hc_boundary_args, flags))
    return fail(HC_EINVAL, "struct_size=%u, expected %zu", p->struct_size, sizeof(hc_boundary_args));
  hc_boundary_args a{};
  memcpy(&a, p, std::min<size_t>(p->struct_size, sizeof a));
  a.struct_size = (uint32_t)std::min<size_t>(p->struct_size, sizeof a);
  int rc = check_hd(a.hc, a.d);
  if (rc) return rc;
  if ((rc = check_n(a.n))) return rc;
  const size_t need = hc_workspace_bytes(a.n, a.hc, a.d);
  if (a.fn_packed && need > kStaticScratchBytes)
    return fail(HC_ENOTSUP, "n=%lld, hc=%d, d=%d needs %zu workspace bytes; the static workspace holds %zu",
                (long long)a.n, a.hc, a.d, need, kStaticScratchBytes);
  if (a.n == 0) return boundary_phases(&a, stream, 3);
  if ((rc = check_device())) return rc;
  a.workspace = static_scratch(&rc);
  if (!a.workspace) return rc;
  a.workspace_bytes = kStaticScratchBytes;
  return boundary_phases(&a, stream, 3);
}
int hc_boundary_begin(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 1); }
int hc_boundary_end(const hc_boundary_args* p, void* stream) { return boundary_phases(p, stream, 2); }

}  // extern "C"
