// Router: fp64 logits, top-k selection with (logit desc, index asc) order,
// gate weights, and the token x expert lists (counting sort by expert, tokens
// rising inside an expert) plus the expert union.
#include <float.h>
#include <algorithm>
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"
#include "mfma_plan.hpp"
#include "route_small.hpp"

namespace moeq {

constexpr int kLogitTok = 16;       // tokens per logits tile
constexpr int kSmallT = 256;        // single-workgroup selection + lists up to this many tokens
constexpr int kTopkParT = 24;       // from this many tokens the top-k has a launch of its own
constexpr int kChunkT = 128;        // tokens per chunk of the multi-kernel lists path
constexpr int kMfmaRouteT = 256;    // from this many tokens the logits run on fp64 matrix cores

// logits[t, e] = sum_i W[e, i] * x[t, i] (+ bias[e]) in fp64.  The fp32*fp32
// products are exact in fp64, so fma and mul+add agree; only the summation
// order differs from a sequential sum.  One workgroup per expert: each of its
// four waves sums a quarter of the row (all loads of a step in flight), then
// the four partials are added in wave order.  Extra workgroups past the
// experts quantise x to q8_K (one wave per 256-block), so the router and the
// activation quantisation share one launch.
__global__ __launch_bounds__(256) void k_logits(const float* __restrict__ x, const float* __restrict__ W,
                                                const float* __restrict__ bias, int64_t T, int64_t H,
                                                int64_t E, double* __restrict__ logits,
                                                uint8_t* __restrict__ xq) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  if ((int64_t)blockIdx.x >= E) {
    if (xq != nullptr && blockIdx.y == 0) quantize_block_wave(x, H, (int64_t)(blockIdx.x - E) * 4 + wave, T * (H / 256), xq);
    return;
  }
  __shared__ double part[4][kLogitTok];
  const int64_t e = blockIdx.x;
  const int64_t n4 = H / 4, q4 = (n4 + 3) / 4;             // float4s per wave
  const int64_t i0 = wave * q4, i1 = (i0 + q4) < n4 ? (i0 + q4) : n4;
  const float4* w4 = reinterpret_cast<const float4*>(W + e * H);
  for (int64_t t0 = (int64_t)blockIdx.y * kLogitTok; t0 < T; t0 += (int64_t)gridDim.y * kLogitTok) {
    const int nt = (int)((T - t0) < kLogitTok ? (T - t0) : kLogitTok);
    double acc[kLogitTok];
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t) acc[t] = 0.0;
    for (int64_t i = i0 + lane; i < i1; i += 4 * kWave) {
      // Every load is issued, a unit past the wave's range reloading unit 0
      // and left out of the sums by a select after its FMAs: a conditional
      // load would leave register copies that wait for it before the next
      // loads go out.
      bool uv[4];
      int64_t iu[4];
      float4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uv[u] = i + u * kWave < i1;
        iu[u] = uv[u] ? i + u * kWave : i;
        w[u] = w4[iu[u]];
      }
      // four tokens at a time (a token past the tile reloads the tile's
      // last one): all their activation loads go out before the first FMA
#pragma unroll
      for (int tg = 0; tg < kLogitTok; tg += 4) {
        if (tg < nt) {
          float4 xv[4][4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const float* xr = x + (t0 + (tg + tt < nt ? tg + tt : nt - 1)) * H;
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[tt][u] = gld_f4(xr + 4 * iu[u]);
          }
          __builtin_amdgcn_sched_barrier(0);
          // the weights' fp64 conversions stay here, after this group's
          // loads (shared by the groups, they would be hoisted to the
          // weight loads and wait there)
          float4 wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            wv[u] = w[u];
            asm volatile("" : "+v"(wv[u].x), "+v"(wv[u].y), "+v"(wv[u].z), "+v"(wv[u].w));
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (tg + tt >= nt) continue;
            double a = acc[tg + tt];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              double b = fma((double)wv[u].x, (double)xv[tt][u].x, a);
              b = fma((double)wv[u].y, (double)xv[tt][u].y, b);
              b = fma((double)wv[u].z, (double)xv[tt][u].z, b);
              b = fma((double)wv[u].w, (double)xv[tt][u].w, b);
              a = uv[u] ? b : a;
            }
            acc[tg + tt] = a;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t) {
      if (t < nt) {                          // only the tile's tokens (one at decode)
        const double v = wave_sum(acc[t]);
        if (lane == 0) part[wave][t] = v;
      }
    }
    __syncthreads();
    if (threadIdx.x < nt) {
      const int t = threadIdx.x;
      double v = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
      if (bias) v += (double)bias[e];
      logits[(t0 + t) * E + e] = v;
    }
    __syncthreads();
  }
}

// One token through the RMS pre-norm of a stack of layers: the same logits
// as k_logits on xn = fl32((x * r) * g), r from the whole row
// (row_rms_scale), and q8_K(xn) from the workgroups past the experts, with
// no normalised copy written: every wave forms the xn elements it uses.  The
// per-lane unit order, the wave sums and the order of the four partials are
// k_logits' for one token (H <= 4096: one pass of up to four float4 units per
// lane), so the logits are bit-identical to k_rms_norm followed by k_logits.
// The router row's loads go out before the norm's row sum.
__global__ __launch_bounds__(256) void k_logits_norm1(const float* __restrict__ x, const float* __restrict__ g,
                                                      double eps, const float* __restrict__ W,
                                                      const float* __restrict__ bias, int64_t H, int64_t E,
                                                      double* __restrict__ logits, uint8_t* __restrict__ xq) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const float4 ones = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  if ((int64_t)blockIdx.x >= E) {
    const int64_t blk = (int64_t)(blockIdx.x - E) * 4 + wave;
    if (blk >= H / 256) return;
    const int64_t i = blk * 256 + 4 * lane;
    const float4 v = gld_f4(x + i);
    const float4 gv = g ? gld_f4(g + i) : ones;
    const double r = row_rms_scale(x, H, eps);
    quantize_block_vals(norm4(v, r, gv), xq + blk * kQ8KBytes);
    return;
  }
  __shared__ double part[4];
  const int64_t e = blockIdx.x;
  const int64_t n4 = H / 4, q4 = (n4 + 3) / 4;             // float4 units per wave (<= 256)
  const int64_t i0 = wave * q4, i1 = (i0 + q4) < n4 ? (i0 + q4) : n4;
  const float4* w4 = reinterpret_cast<const float4*>(W + e * H);
  bool uv[4];
  int64_t iu[4];
  float4 w[4], xv[4], gv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + lane + u * kWave;
    uv[u] = i < i1;
    iu[u] = uv[u] ? i : i0;
    w[u] = w4[iu[u]];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    xv[u] = gld_f4(x + 4 * iu[u]);
    gv[u] = g ? gld_f4(g + 4 * iu[u]) : ones;
  }
  const double r = row_rms_scale(x, H, eps);
  double a = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 xn = norm4(xv[u], r, gv[u]);
    double b = fma((double)w[u].x, (double)xn.x, a);
    b = fma((double)w[u].y, (double)xn.y, b);
    b = fma((double)w[u].z, (double)xn.z, b);
    b = fma((double)w[u].w, (double)xn.w, b);
    a = uv[u] ? b : a;
  }
  const double v = wave_sum(a);
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = ((part[0] + part[1]) + part[2]) + part[3];
    if (bias) t += (double)bias[e];
    logits[e] = t;
  }
}

// Logits of many tokens as a dense contraction on fp64 matrix cores:
// v_mfma_f64_16x16x4f64 on exact fp64 copies of the fp32 operands, so every
// product is exact and only the order of the fp64 additions differs from a
// sequential sum (as in k_logits).  Workgroup tile 64 tokens x 64 experts,
// wave tile 32 x 32 (2 x 2 MFMA blocks); K staged through LDS 32 at a time.
// Operand lanes: A lane l = x[m = l%16][k = l/16], B lane l = W[n = l%16][k = l/16]
// (the same k on both sides); result lane l, value r = logit[4*r + l/16][l%16].
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int kRt = 64, kRe = 64, kRk = 32, kRpad = 36;

__global__ __launch_bounds__(256) void k_logits_mfma(const float* __restrict__ x, const float* __restrict__ W,
                                                     const float* __restrict__ bias, int64_t T, int64_t H,
                                                     int64_t E, double* __restrict__ logits) {
  // two LDS stages: block k0 is written while the MFMAs of block k0 - 32 may
  // still read the other stage, and the global loads of the next block are in
  // flight during this block's MFMAs (one barrier per block)
  __shared__ float xs[2][kRt][kRpad];
  __shared__ float ws[2][kRe][kRpad];
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int64_t t0 = (int64_t)blockIdx.x * kRt, e0 = (int64_t)blockIdx.y * kRe;
  const int wt = (wave & 1) * 32, we = (wave >> 1) * 32;
  const int m16 = lane & 15, kq = lane >> 4;
  v4d acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v4d){0.0, 0.0, 0.0, 0.0};
  float4 xv[2], wv[2];
  auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;
      const int64_t kc = k0 + 4 * c4;
      const int64_t tr = t0 + row, er = e0 + row;
      const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
      xv[i] = (tr < T && kc < H) ? gld_f4(x + tr * H + kc) : zero;
      wv[i] = (er < E && kc < H) ? gld_f4(W + er * H + kc) : zero;
    }
  };
  fetch(0);
  int buf = 0;
  for (int64_t k0 = 0; k0 < H; k0 += kRk, buf ^= 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;
      *reinterpret_cast<float4*>(&xs[buf][row][4 * c4]) = xv[i];
      *reinterpret_cast<float4*>(&ws[buf][row][4 * c4]) = wv[i];
    }
    __syncthreads();
    if (k0 + kRk < H) fetch(k0 + kRk);
#pragma unroll
    for (int kk = 0; kk < kRk / 4; ++kk) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = (double)xs[buf][wt + 16 * i + m16][4 * kk + kq];
        b[i] = (double)ws[buf][we + 16 * i + m16][4 * kk + kq];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t e = e0 + we + 16 * j + m16;
      if (e >= E) continue;
      const double bv = bias ? (double)bias[e] : 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wt + 16 * i + 4 * r + kq;
        if (t < T) logits[t * E + e] = acc[i][j][r] + bv;
      }
    }
}

// ------------------------------------------------------------------
// Many tokens without a logits output: an approximate contraction on bf16
// matrix cores, then exact fp64 logits of the few experts that can still be
// among the k (the router logits in fp32 with fp64 rescoring near the k-th:
// the selection and the gate weights come from exact fp64 logits, so ids and
// weights are those of the fp64 router).
//
// Operands: every fp32 value v is split as hi = bf16(v), lo = bf16(v - hi)
// (round to nearest even; v - hi is exact), and the contraction sums
// hi*hi + hi*lo + lo*hi with exact bf16 products into fp32, moved into an fp64
// sum every kSegK elements of K.  Error of one logit (first order, u = 2^-24):
//   split:        |v - hi - lo| <= 2^-18 |v|, |lo| <= 2^-9 |v| (1 + 2^-8), so
//                 the dropped terms are below 3.1 * 2^-18 * sum |x_i w_i|
//   accumulation: 3 * kSegK products per segment summed in fp32 (any order):
//                 below 3.1 * kSegK * u * sum |x_i w_i|
//   the fp32 result: u |sum|; the fp64 segment sums: negligible
// and sum |x_i w_i| <= ||x|| ||w_e|| (Cauchy-Schwarz).  The bound is doubled
// (kRouteGamma below) and also covers a rounding of the matrix unit's sums
// toward zero.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSegK = 256;                       // fp32 accumulation segment of K
constexpr double kRouteGamma = 2.0 * (3.1 * 3.814697265625e-06 + 3.1 * kSegK * 5.9604644775390625e-08 +
                                      2.0 * 5.9604644775390625e-08);
constexpr int kGt = 128, kGe = 128, kGk = 32, kGpad = 40;   // tile rows, K chunk, LDS row (bf16)
constexpr int kRescoreMaxE = 1024;   // experts of the rescoring selection (16 logits per lane)
constexpr int kRescoreMaxB = 8;      // 256-blocks of a token row held in registers (H <= 2048)

__device__ __forceinline__ uint32_t bf16_bits_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split of four values into hi / lo bf16 pairs, packed two per word.
__device__ __forceinline__ void split4(float4 v, uint2& hi, uint2& lo) {
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = bf16_bits_rne(f[i]);
    l[i] = bf16_bits_rne(f[i] - bf16_bits_to_f32(h[i]));
  }
  hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// One pass over the rows of x ([T, H]) and of the router weights ([E, H]),
// one wave per row: the bf16 hi / lo planes of every row, the fp64 Euclidean
// norm of every row, and (x rows) q8_K of the row.
__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ x, int64_t T,
                                                      const float* __restrict__ W, int64_t E, int64_t H,
                                                      uint16_t* __restrict__ xhl, uint16_t* __restrict__ whl,
                                                      double* __restrict__ nx, double* __restrict__ nw,
                                                      uint8_t* __restrict__ xq) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T + E) return;
  const bool isx = row < T;
  const int64_t r = isx ? row : row - T;
  const float* src = (isx ? x : W) + r * H;
  uint16_t* hi = (isx ? xhl : whl) + r * H;
  uint16_t* lo = hi + (isx ? T : E) * H;
  const int lane = lane_id();
  double ss = 0.0;
  for (int64_t b = 0; b < H / 256; ++b) {
    const int64_t i = b * 256 + 4 * lane;
    const float4 v = gld_f4(src + i);
    ss = fma((double)v.x, (double)v.x, ss);
    ss = fma((double)v.y, (double)v.y, ss);
    ss = fma((double)v.z, (double)v.z, ss);
    ss = fma((double)v.w, (double)v.w, ss);
    uint2 h, l;
    split4(v, h, l);
    *reinterpret_cast<uint2*>(hi + i) = h;
    *reinterpret_cast<uint2*>(lo + i) = l;
    if (isx && xq != nullptr) quantize_block_vals(v, xq + (r * (H / 256) + b) * kQ8KBytes);
  }
  ss = wave_sum(ss);
  if (lane == 0) (isx ? nx : nw)[r] = sqrt(ss);
}

// Approximate logits[t, e] = sum_i x[t, i] W[e, i] (no bias) in fp32, from the
// bf16 planes: v_mfma_f32_32x32x16_bf16 on 128-token x 128-expert workgroup
// tiles, 8 waves of 32 tokens x 64 experts, K staged through two LDS stages 32
// at a time.  Operand lanes: A lane l = x[m = l % 32][k = 8 (l / 32) .. +7],
// B lane l = W[n = l % 32][same k]; result lane l, value r =
// logit[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__global__ __launch_bounds__(512) void k_logits_bf16x3(const uint16_t* __restrict__ xhl,
                                                       const uint16_t* __restrict__ whl, int64_t T, int64_t H,
                                                       int64_t E, float* __restrict__ approx) {
  __shared__ __align__(16) uint16_t As[2][2][kGt][kGpad];   // [stage][hi, lo][token][k]
  __shared__ __align__(16) uint16_t Bs[2][2][kGe][kGpad];   // [stage][hi, lo][expert][k]
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int64_t t0 = (int64_t)blockIdx.x * kGt, e0 = (int64_t)blockIdx.y * kGe;
  const int wt = (wave & 3) * 32, we = (wave >> 2) * 64;
  // staging: 2 planes x 128 rows x 4 pieces of 8 bf16, for A and for B: two
  // 16-byte pieces of each per thread
  uint4 av[2], bv[2];
  auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 512 * q, pl = idx >> 9, row = (idx >> 2) & 127, c = idx & 3;
      const int64_t tr = t0 + row, er = e0 + row;
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      av[q] = tr < T ? gld_u4(xhl + (pl * T + tr) * H + k0 + 8 * c) : z;
      bv[q] = er < E ? gld_u4(whl + (pl * E + er) * H + k0 + 8 * c) : z;
    }
  };
  f32x16 acc[2];
  double sum[2][16];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    acc[n] = (f32x16){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[n][r] = 0.0;
  }
  fetch(0);
  int buf = 0;
  for (int64_t k0 = 0; k0 < H; k0 += kGk, buf ^= 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 512 * q, pl = idx >> 9, row = (idx >> 2) & 127, c = idx & 3;
      *reinterpret_cast<uint4*>(&As[buf][pl][row][8 * c]) = av[q];
      *reinterpret_cast<uint4*>(&Bs[buf][pl][row][8 * c]) = bv[q];
    }
    __syncthreads();
    if (k0 + kGk < H) fetch(k0 + kGk);
#pragma unroll
    for (int ks = 0; ks < kGk / 16; ++ks) {
      const int kk = 16 * ks + 8 * (lane >> 5);
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&As[buf][0][wt + (lane & 31)][kk]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&As[buf][1][wt + (lane & 31)][kk]);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Bs[buf][0][we + 32 * n + (lane & 31)][kk]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Bs[buf][1][we + 32 * n + (lane & 31)][kk]);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[n], 0, 0, 0);
      }
    }
    if ((k0 + kGk) % kSegK == 0 || k0 + kGk >= H) {      // end of a segment: into the fp64 sums
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sum[n][r] += (double)acc[n][r];
          acc[n][r] = 0.f;
        }
    }
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int64_t e = e0 + we + 32 * n + (lane & 31);
    if (e >= E) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + wt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (t < T) approx[t * E + e] = (float)sum[n][r];
    }
  }
}

// Per token (one wave): from the approximate logits a_e (+ bias, in fp64) and
// the bound eps_e = gamma ||x_t|| ||W_e|| (|exact - a_e| <= eps_e), the lower
// bound L = the k-th largest of a_e - eps_e; every expert of the top k has
// exact logit >= exact k-th >= L, so it is among the candidates a_e + eps_e
// >= L (an expert tied with the k-th too).  The candidates' logits are then
// computed exactly (fp64, + bias), the others set to -inf, and the register
// top-k and gating run on them: the same ids and weights as from all exact
// logits.  A non-finite bound makes every expert a candidate.
template <int NPER>
__global__ __launch_bounds__(256) void k_topk_rescore(const float* __restrict__ approx, const double* __restrict__ nx,
                                                      const double* __restrict__ nw, const float* __restrict__ x,
                                                      const float* __restrict__ W, const float* __restrict__ bias,
                                                      int64_t T, int64_t E, int64_t H, int k, int gating,
                                                      float scale, int32_t* __restrict__ ids,
                                                      float* __restrict__ wout) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const double xn = nx[t];
  double a[NPER], eps[NPER];
  int vi[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int64_t e = lane + (int64_t)kWave * i;
    const int64_t ec = e < E ? e : E - 1;
    const double av = (double)approx[t * E + ec] + (bias ? (double)bias[ec] : 0.0);
    const double ev = kRouteGamma * xn * nw[ec] + 1e-300;
    a[i] = e < E ? av : -INFINITY;
    eps[i] = e < E ? ev : 0.0;
    vi[i] = e < E ? (int)e : INT_MAX;
  }
  // L: k rounds of a wave arg-max over each lane's sorted lower bounds
  double lb[NPER];
  int li[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) { lb[i] = a[i] - eps[i]; li[i] = vi[i]; }
#pragma unroll
  for (int p = 0; p < NPER; ++p)
#pragma unroll
    for (int q = NPER - 1; q > p; --q) {
      double hv = lb[q - 1];
      int hi = li[q - 1];
      better(hv, hi, lb[q], li[q]);
      const bool sw = hi != li[q - 1];
      const double lv = sw ? lb[q - 1] : lb[q];
      const int lj = sw ? li[q - 1] : li[q];
      lb[q - 1] = hv; li[q - 1] = hi; lb[q] = lv; li[q] = lj;
    }
  int head = 0;
  double L = -INFINITY;
  for (int s = 0; s < k; ++s) {
    double best = lb[0];
    int bi = li[0];
#pragma unroll
    for (int j = 1; j < NPER; ++j) {
      best = head == j ? lb[j] : best;
      bi = head == j ? li[j] : bi;
    }
    best = head < NPER ? best : -INFINITY;
    bi = head < NPER ? bi : INT_MAX;
    const int mine = bi;
    wave_argmax(best, bi);
    head += (mine == bi) ? 1 : 0;
    L = best;
  }
  const bool all = !(L > -INFINITY) || !(xn < INFINITY);   // a non-finite bound: every expert
  // the candidate list, in (i, lane) order: lane l's element i sits at
  // position base_i + (candidates of set i below lane l)
  // per wave: E fp64 exact logits, then E int32 candidate ids (dynamic LDS)
  extern __shared__ __align__(8) uint8_t rlds[];
  double* exw = reinterpret_cast<double*>(rlds) + (threadIdx.x >> 6) * E;
  int* clw = reinterpret_cast<int*>(rlds + 4 * E * sizeof(double)) + (threadIdx.x >> 6) * E;
  int pos[NPER];
  bool cand[NPER];
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int64_t e = lane + (int64_t)kWave * i;
    cand[i] = e < E && (all || !(a[i] + eps[i] < L));
    const uint64_t m = __ballot(cand[i]);
    pos[i] = n + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (cand[i]) clw[pos[i]] = (int)e;
    n += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the list is in LDS before any lane reads it
  __builtin_amdgcn_wave_barrier();
  // the token's row in registers (H / 256 float4 per lane; a unit past the row
  // reloads unit 0 and is left out of the sums)
  const int nb = (int)(H / 256);
  const float* xr = x + t * H;
  float4 xv[kRescoreMaxB];
#pragma unroll
  for (int b = 0; b < kRescoreMaxB; ++b) xv[b] = gld_f4(xr + (b < nb ? b : 0) * 256 + 4 * lane);
  // exact logits, two candidates at a time (all weight loads of both issued
  // before the first FMA)
  for (int c = 0; c < n; c += 2) {
    const int e0 = clw[c], e1 = clw[c + 1 < n ? c + 1 : c];
    const float* w0 = W + (int64_t)e0 * H;
    const float* w1 = W + (int64_t)e1 * H;
    float4 u0[kRescoreMaxB], u1[kRescoreMaxB];
#pragma unroll
    for (int b = 0; b < kRescoreMaxB; ++b) {
      const int bb = b < nb ? b : 0;
      u0[b] = gld_f4(w0 + bb * 256 + 4 * lane);
      u1[b] = gld_f4(w1 + bb * 256 + 4 * lane);
    }
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int b = 0; b < kRescoreMaxB; ++b) {
      double d0 = fma((double)u0[b].x, (double)xv[b].x, s0);
      d0 = fma((double)u0[b].y, (double)xv[b].y, d0);
      d0 = fma((double)u0[b].z, (double)xv[b].z, d0);
      d0 = fma((double)u0[b].w, (double)xv[b].w, d0);
      double d1 = fma((double)u1[b].x, (double)xv[b].x, s1);
      d1 = fma((double)u1[b].y, (double)xv[b].y, d1);
      d1 = fma((double)u1[b].z, (double)xv[b].z, d1);
      d1 = fma((double)u1[b].w, (double)xv[b].w, d1);
      s0 = b < nb ? d0 : s0;
      s1 = b < nb ? d1 : s1;
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      exw[c] = s0 + (bias ? (double)bias[e0] : 0.0);
      if (c + 1 < n) exw[c + 1] = s1 + (bias ? (double)bias[e1] : 0.0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  double v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) v[i] = cand[i] ? exw[pos[i]] : -INFINITY;
  int my_i;
  float my_w;
  topk_wave_vals<NPER>(v, vi, E, k, gating, scale, my_i, my_w);
  if (lane < k) {
    gst_i32(ids + t * k + lane, my_i);
    gst_f32(wout + t * k + lane, my_w);
  }
}

template <int NPER>
__device__ __forceinline__ void topk_row_wave(const double* __restrict__ row, int64_t E, int k, int gating, float scale,
                              int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* ids_lds) {
  int my_i;
  float my_w;
  topk_wave_regs<NPER>(row, E, k, gating, scale, my_i, my_w);
  const int lane = lane_id();
  if (lane < k) {
    gst_i32(ids_out + lane, my_i);
    gst_f32(w_out + lane, my_w);
    if (ids_lds) ids_lds[lane] = my_i;
  }
}

// Exclusive scan over a block of blockDim.x threads (a multiple of 64).
__device__ int block_exclusive_scan(int v, int* tmp /* >= 16 ints */, int* total) {
  const int lane = lane_id(), w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < nw ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, kWave);
      if (lane >= o) s += y;
    }
    if (lane < nw) tmp[16 + lane] = s;   // inclusive prefix of wave sums
  }
  __syncthreads();
  const int before = w == 0 ? 0 : tmp[16 + w - 1];
  *total = tmp[16 + nw - 1];
  return before + x - v;
}

// counts[E] -> offsets[E+1] and the active list; `cnt` lives in LDS.  With
// loff / lact (LDS [E+1] each) the offsets and the list are also kept there.
__device__ void offsets_and_union(int* cnt, int64_t E, int32_t* offsets, int32_t* active,
                                  int* scan_tmp, int* base_out /* LDS [E] or null */, int* loff = nullptr,
                                  int* lact = nullptr) {
  const int per = (int)((E + blockDim.x - 1) / blockDim.x);
  const int64_t e0 = (int64_t)threadIdx.x * per;
  int local = 0, flags = 0;
  for (int i = 0; i < per; ++i) {
    const int64_t e = e0 + i;
    if (e < E) { local += cnt[e]; flags += cnt[e] > 0; }
  }
  int tot, ftot;
  int run = block_exclusive_scan(local, scan_tmp, &tot);
  int frun = block_exclusive_scan(flags, scan_tmp + 32, &ftot);
  for (int i = 0; i < per; ++i) {
    const int64_t e = e0 + i;
    if (e < E) {
      const int c = cnt[e];   // read before base_out (which may alias cnt) is written
      offsets[e] = run;
      if (base_out) base_out[e] = run;
      if (loff) loff[e] = run;
      if (c > 0) {
        if (lact) lact[1 + frun] = (int32_t)e;
        active[1 + frun++] = (int32_t)e;
      }
      run += c;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = tot;
    active[0] = ftot;
    if (loff) loff[E] = tot;
    if (lact) lact[0] = ftot;
  }
}

// T <= kSmallT: top-k for every token, then the lists, in one workgroup.
template <int NPER>
__global__ __launch_bounds__(1024) void k_select_small(const double* __restrict__ logits, int64_t T, int64_t E,
                                                       int k, int gating, float scale, int32_t* __restrict__ ids,
                                                       float* __restrict__ w, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ pairs, int32_t* __restrict__ active,
                                                       MfmaPlan plan, int ids_in) {
  extern __shared__ int lds[];
  int* ids_s = lds;                                           // [T*k]
  int* cnt = ids_s + T * k;                                   // [E]
  int* scan_tmp = cnt + E;                                    // [64]
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (ids_in) {   // ids and weights already written by k_topk (one wave per token)
    for (int64_t p = threadIdx.x; p < T * k; p += blockDim.x) ids_s[p] = gld_i32(ids + p);
  } else {
    for (int64_t t = wv; t < T; t += nw)
      topk_row_wave<NPER>(logits + t * E, E, k, gating, scale, ids + t * k, w + t * k, ids_s + t * k);
  }
  if (T * k <= kSmallPairs) {
    int* skey = ids_s + T * k;                                // [64]
    int* lact = skey + kSmallPairs;                           // [65]
    int* loff = lact + kSmallPairs + 1;                       // [E + 1]
    int* ebase = loff + E + 1;                                // [E + 1] tile-list scratch
    __syncthreads();
    small_lists(ids_s, (int)(T * k), E, offsets, pairs, active, skey, loff, lact);
    if (plan.tiles != nullptr) {
      __syncthreads();
      mfma_plan_block(lact, loff, plan, ebase);
    }
    return;
  }
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < T * k; p += blockDim.x) atomicAdd(&cnt[ids_s[p]], 1);
  __syncthreads();
  offsets_and_union(cnt, E, offsets, active, scan_tmp, cnt);   // cnt becomes the write cursor
  __syncthreads();
  if (wv == 0) {
    const int lane = lane_id();
    for (int64_t t = 0; t < T; ++t) {
      if (lane < k) {
        const int e = ids_s[t * k + lane];
        // The experts of one token are distinct, and one wave's LDS atomics
        // complete in issue order, so positions rise with t inside an expert.
        const int pos = atomicAdd(&cnt[e], 1);
        pairs[pos] = (int32_t)(t * k + lane);
      }
    }
  }
  if (plan.tiles != nullptr) {   // the MFMA tile lists of the FFN that follows
    __syncthreads();
    mfma_plan_block(active, offsets, plan, cnt);   // cnt and scan_tmp (E + 64 ints) are free here
  }
}

// ---- multi-kernel path for large T
template <int NPER>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int64_t T, int64_t E, int k,
                                              int gating, float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_row_wave<NPER>(logits + t * E, E, k, gating, scale, ids + t * k, w + t * k, nullptr);
}

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int64_t T, int k, int64_t E,
                                              int32_t* __restrict__ hist) {
  extern __shared__ int cnt[];
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * kChunkT;
  const int64_t t1 = (t0 + kChunkT) < T ? (t0 + kChunkT) : T;
  for (int64_t p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) atomicAdd(&cnt[ids[p]], 1);
  __syncthreads();
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) hist[blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ hist, int64_t nchunks, int64_t E,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                               MfmaPlan plan) {
  extern __shared__ int lds[];
  int* tot = lds;              // [E]
  int* scan_tmp = tot + E;     // [64]
  int* loff = scan_tmp + 64;   // [E + 1] offsets and union for the tile lists
  int* lact = loff + E + 1;    // [E + 1]
  // the chunk counts of an expert are read kScanBatch at a time, all loads of
  // a batch in flight before the first is used
  constexpr int kScanBatch = 16;
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int64_t c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) h[j] = c0 + j < nchunks ? gld_i32(hist + (c0 + j) * E + e) : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) s += h[j];
    }
    tot[e] = s;
  }
  __syncthreads();
  offsets_and_union(tot, E, offsets, active, scan_tmp, tot, loff, lact);   // tot becomes the offsets
  __syncthreads();
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tot[e];
    for (int64_t c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) h[j] = c0 + j < nchunks ? gld_i32(hist + (c0 + j) * E + e) : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (c0 + j < nchunks) gst_i32(hist + (c0 + j) * E + e, run);
        run += h[j];
      }
    }
  }
  if (plan.tiles != nullptr) {   // the MFMA tile lists of the FFN that follows (from the LDS copies)
    __syncthreads();
    mfma_plan_block(lact, loff, plan, tot);   // tot and scan_tmp (E + 64 ints) are free here
  }
}

__global__ __launch_bounds__(64) void k_scatter(const int32_t* __restrict__ ids, int64_t T, int k, int64_t E,
                                                const int32_t* __restrict__ base, int32_t* __restrict__ pairs) {
  extern __shared__ int cur[];
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) cur[e] = base[blockIdx.x * E + e];
  __syncthreads();
  const int lane = lane_id();
  const int64_t t0 = (int64_t)blockIdx.x * kChunkT;
  const int64_t t1 = (t0 + kChunkT) < T ? (t0 + kChunkT) : T;
  // ids of 8 tokens in flight at once; the LDS atomics still go out token by
  // token (one wave: they complete in issue order, so positions rise with t)
  for (int64_t t = t0; t < t1; t += 8) {
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (lane < k && t + j < t1) ? gld_i32(ids + (t + j) * k + lane) : -1;
    int pos[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pos[j] = e[j] >= 0 ? atomicAdd(&cur[e[j]], 1) : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pos[j] >= 0) gst_i32(pairs + pos[j], (int32_t)((t + j) * k + lane));
  }
}

__global__ void k_empty_lists(int64_t E, int32_t* offsets, int32_t* active) {
  for (int64_t e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
  if (threadIdx.x == 0) active[0] = 0;
}

// Logits of a chunk of kSplitT to kMfmaRouteT - 1 tokens on fp64 matrix
// cores, with K split over the grid so that the launch fills the chip: the
// per-expert kernel above re-reads every token row once per expert (a
// 200-token chunk at hidden 4096 moves about 0.8 GB from L2 that way), and a
// 64 x 64 tile over the whole of K leaves all but a few CUs idle.
// Workgroup (token tile of 16, expert tile of 64, K slice z): each wave one
// 16 x 16 block, v_mfma_f64_16x16x4f64 on exact fp64 copies of the fp32
// operands.  Lane l loads 16 bytes of its row (token or expert l % 16) at
// k0 + 4 (l / 16); step j of the four MFMAs takes component j, so the four
// steps cover k0 .. k0 + 15 once each, with the same k on both operands.  A
// row past T or E reloads the last row and its results are dropped.  The
// slice's sums go to part[z][t][e]; k_logits_sum adds the slices.
constexpr int kSplitT = 40;          // from this many tokens (below kMfmaRouteT) the split-K logits
constexpr int kSplitMax = 16;        // K slices at most
constexpr int kSplitTok = 16, kSplitExp = 64;

struct LogitSplit { int64_t slices, kc; };
__host__ __device__ inline LogitSplit logit_split(int64_t T, int64_t E, int64_t H) {
  const int64_t tiles = ((T + kSplitTok - 1) / kSplitTok) * ((E + kSplitExp - 1) / kSplitExp);
  int64_t sl = (512 + tiles - 1) / tiles;
  sl = sl < 1 ? 1 : (sl > kSplitMax ? kSplitMax : sl);
  int64_t kc = (H + sl - 1) / sl;
  kc = (kc + 15) / 16 * 16;
  return LogitSplit{(H + kc - 1) / kc, kc};
}
inline bool logit_split_ok(int64_t T, int64_t H) { return T >= kSplitT && T < kMfmaRouteT && H % 16 == 0; }

__global__ __launch_bounds__(256) void k_logits_split(const float* __restrict__ x, const float* __restrict__ W,
                                                      int64_t T, int64_t H, int64_t E, int64_t kc,
                                                      double* __restrict__ part) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t t0 = (int64_t)blockIdx.x * kSplitTok, e0 = (int64_t)blockIdx.y * kSplitExp + 16 * wave;
  const int64_t kb = (int64_t)blockIdx.z * kc, ke = (kb + kc) < H ? (kb + kc) : H;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t tr = (t0 + r16) < T ? (t0 + r16) : T - 1;
  const int64_t er = (e0 + r16) < E ? (e0 + r16) : E - 1;
  const float* xr = x + tr * H + 4 * kq;
  const float* wr = W + er * H + 4 * kq;
  v4d acc = (v4d){0.0, 0.0, 0.0, 0.0};
  // four 16-wide K steps per round: all eight loads out before the MFMAs
  for (int64_t k0 = kb; k0 < ke; k0 += 64) {
    float4 xv[4], wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = (k0 + 16 * u) < ke ? (k0 + 16 * u) : k0;
      xv[u] = gld_f4(xr + k);
      wv[u] = gld_f4(wr + k);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (k0 + 16 * u >= ke) break;   // uniform over the wave
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[u].x, (double)wv[u].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[u].y, (double)wv[u].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[u].z, (double)wv[u].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[u].w, (double)wv[u].w, acc, 0, 0, 0);
    }
  }
  // result lane l, value r: token 4 r + l / 16, expert l % 16
  const int64_t e = e0 + r16;
  double* pz = part + (int64_t)blockIdx.z * T * E;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + 4 * r + kq;
    if (t < T && e < E) pz[t * E + e] = acc[r];
  }
}

// logits[t, e] = ((part[0] + part[1]) + ...) + bias[e], slices in order;
// workgroups past the outputs quantise x to q8_K (one wave per 256-block).
__global__ __launch_bounds__(256) void k_logits_sum(const double* __restrict__ part, int64_t slices, int64_t T,
                                                    int64_t E, const float* __restrict__ bias,
                                                    double* __restrict__ logits, const float* __restrict__ x,
                                                    int64_t H, uint8_t* __restrict__ xq) {
  const int64_t nout = T * E, nb = (nout + 255) / 256;
  if ((int64_t)blockIdx.x >= nb) {
    quantize_block_wave(x, H, ((int64_t)blockIdx.x - nb) * 4 + (threadIdx.x >> 6), T * (H / 256), xq);
    return;
  }
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nout) return;
  double p[kSplitMax];
#pragma unroll
  for (int z = 0; z < kSplitMax; ++z) p[z] = z < slices ? part[z * nout + i] : 0.0;
  double v = p[0];
#pragma unroll
  for (int z = 1; z < kSplitMax; ++z)
    if (z < slices) v += p[z];
  if (bias) v += (double)bias[i % E];
  logits[i] = v;
}

size_t logit_part_bytes(int64_t T, int64_t E, int64_t H) {
  return logit_split_ok(T, H) ? (size_t)logit_split(T, E, H).slices * T * E * sizeof(double) : 0;
}

int launch_logits(int64_t T, int64_t H, int64_t E, const float* x, const float* W, const float* bias,
                  double* logits, void* xq, hipStream_t s, void* part) {
  if (part != nullptr && logit_split_ok(T, H)) {
    const LogitSplit sp = logit_split(T, E, H);
    dim3 g((unsigned)((T + kSplitTok - 1) / kSplitTok), (unsigned)((E + kSplitExp - 1) / kSplitExp),
           (unsigned)sp.slices);
    hipLaunchKernelGGL(k_logits_split, g, dim3(256), 0, s, x, W, T, H, E, sp.kc, (double*)part);
    if (hipGetLastError() != hipSuccess) return -1;
    const int64_t nq = xq ? (T * (H / 256) + 3) / 4 : 0;
    hipLaunchKernelGGL(k_logits_sum, dim3((unsigned)((T * E + 255) / 256 + nq)), dim3(256), 0, s,
                       (const double*)part, sp.slices, T, E, bias, logits, x, H, (uint8_t*)xq);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (T >= kMfmaRouteT) {
    // many tokens: the router is a dense contraction (matrix cores); q8_K(x)
    // in its own launch
    dim3 g((unsigned)((T + kRt - 1) / kRt), (unsigned)((E + kRe - 1) / kRe));
    hipLaunchKernelGGL(k_logits_mfma, g, dim3(256), 0, s, x, W, bias, T, H, E, logits);
    if (hipGetLastError() != hipSuccess) return -1;
    return xq ? launch_quantize_q8K(x, T, H, xq, s) : 0;
  }
  const int64_t nq = xq ? (T * (H / 256) + 3) / 4 : 0;
  const int64_t tiles = (T + kLogitTok - 1) / kLogitTok;
  dim3 g1((unsigned)(E + nq), (unsigned)(tiles < 64 ? tiles : 64));
  hipLaunchKernelGGL(k_logits, g1, dim3(256), 0, s, x, W, bias, T, H, E, logits, (uint8_t*)xq);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_logits_norm1(int64_t H, int64_t E, const float* x, const float* g, double eps, const float* W,
                        const float* bias, double* logits, void* xq, hipStream_t s) {
  if (H > kNorm1MaxH) return -1;
  const int64_t nq = (H / 256 + 3) / 4;
  hipLaunchKernelGGL(k_logits_norm1, dim3((unsigned)(E + nq)), dim3(256), 0, s, x, g, eps, W, bias, H, E, logits,
                     (uint8_t*)xq);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Route workspace: the logits (fp64 [T, E]; the fast path keeps its fp32
// approximations there), the chunk histograms (more than kSmallT tokens), and
// for the fast path the bf16 hi / lo planes of x and W and their row norms.
struct RouteLayout {
  size_t off_hist, off_xhl, off_whl, off_nx, off_nw, off_part, total;
};
// (up to 1024 experts: 16 logits per lane in registers; the token row in
// registers: H <= 2048)
bool fast_route_ok(int64_t T, int64_t E, int64_t H) {
  return T > kSmallT && H % 256 == 0 && H <= 256 * kRescoreMaxB && E <= kRescoreMaxE;
}
RouteLayout route_layout(int64_t T, int64_t E, int64_t H) {
  RouteLayout L{};
  size_t o = align256((size_t)T * E * sizeof(double));
  L.off_hist = o;
  if (T > kSmallT) o += align256((size_t)((T + kChunkT - 1) / kChunkT) * E * sizeof(int32_t));
  if (fast_route_ok(T, E, H)) {
    L.off_xhl = o; o += align256((size_t)2 * T * H * sizeof(uint16_t));
    L.off_whl = o; o += align256((size_t)2 * E * H * sizeof(uint16_t));
    L.off_nx = o;  o += align256((size_t)T * sizeof(double));
    L.off_nw = o;  o += align256((size_t)E * sizeof(double));
  }
  L.off_part = o; o += align256(logit_part_bytes(T, E, H));
  L.total = o;
  return L;
}
size_t route_part_off(int64_t T, int64_t E, int64_t H) { return route_layout(T, E, H).off_part; }

size_t route_ws_bytes(int64_t T, int64_t E, int64_t H) { return route_layout(T, E, H).total; }

// The token x expert lists of more than kSmallT tokens from their ids: chunk
// histograms, one scan (offsets, union, MFMA tile lists), the scatter.
int lists_many(int64_t T, int k, int64_t E, const int32_t* ids, int32_t* offsets, int32_t* pairs, int32_t* active,
               uint8_t* hist_ws, hipStream_t s, const MfmaPlan& pl) {
  const int64_t nch = (T + kChunkT - 1) / kChunkT;
  int32_t* hist = reinterpret_cast<int32_t*>(hist_ws);
  hipLaunchKernelGGL(k_hist, dim3((unsigned)nch), dim3(256), (size_t)E * sizeof(int), s, ids, T, k, E, hist);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), (size_t)(3 * E + 66) * sizeof(int), s, hist, nch, E, offsets,
                     active, pl);
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)nch), dim3(64), (size_t)E * sizeof(int), s, ids, T, k, E, hist, pairs);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_route(int64_t T, int64_t H, int64_t E, int k, int gating, float scale, const float* x,
                 const float* W, const float* bias, double* logits, int32_t* ids, float* w,
                 int32_t* offsets, int32_t* pairs, int32_t* active, void* xq, void* ws, hipStream_t s,
                 const MfmaPlan* plan, bool have_logits) {
  const MfmaPlan pl = plan != nullptr ? *plan : MfmaPlan{0, 0, nullptr, nullptr, nullptr, nullptr, kThinRows};
  if (T == 0) {
    hipLaunchKernelGGL(k_empty_lists, dim3(1), dim3(256), 0, s, E, offsets, active);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  uint8_t* wsb = (uint8_t*)ws;
  const RouteLayout RL = route_layout(T, E, H);
  if (logits == nullptr && gating != 1 && fast_route_ok(T, E, H)) {
    // fast path: bf16 planes, norms and q8_K(x) in one pass; the approximate
    // contraction; selection with exact rescoring; then the lists as below
    uint16_t* xhl = reinterpret_cast<uint16_t*>(wsb + RL.off_xhl);
    uint16_t* whl = reinterpret_cast<uint16_t*>(wsb + RL.off_whl);
    double* nx = reinterpret_cast<double*>(wsb + RL.off_nx);
    double* nw = reinterpret_cast<double*>(wsb + RL.off_nw);
    float* approx = reinterpret_cast<float*>(wsb);
    hipLaunchKernelGGL(k_router_split, dim3((unsigned)((T + E + 3) / 4)), dim3(256), 0, s, x, T, W, E, H, xhl, whl,
                       nx, nw, (uint8_t*)xq);
    hipLaunchKernelGGL(k_logits_bf16x3, dim3((unsigned)((T + kGt - 1) / kGt), (unsigned)((E + kGe - 1) / kGe)),
                       dim3(512), 0, s, xhl, whl, T, H, E, approx);
    const size_t lds = (size_t)4 * E * (sizeof(double) + sizeof(int));
#define MOEQ_RESCORE(N) hipLaunchKernelGGL(k_topk_rescore<N>, dim3((unsigned)((T + 3) / 4)), dim3(256), lds, s, \
                                            approx, nx, nw, x, W, bias, T, E, H, k, gating, scale, ids, w)
    if (E <= 256) MOEQ_RESCORE(4);
    else if (E <= 512) MOEQ_RESCORE(8);
    else MOEQ_RESCORE(16);
#undef MOEQ_RESCORE
    return lists_many(T, k, E, ids, offsets, pairs, active, wsb + RL.off_hist, s, pl);
  }
  double* lg = logits ? logits : reinterpret_cast<double*>(wsb);
  if (have_logits && (logits == nullptr || T > kSmallT)) return -2;
  if (!have_logits) {
    if (int rc = launch_logits(T, H, E, x, W, bias, lg, xq, s, wsb + RL.off_part)) return rc;
  }
  if (T <= kSmallT) {
    size_t lds = (size_t)(T * k + 2 * E + 2 * kSmallPairs + 3) * sizeof(int);   // either list path
    // up to 64 pairs: one wave per token and one for the lists, so fewer
    // waves (cheaper barriers); more pairs: block scans over 1024 threads
    const unsigned nt = T * k <= kSmallPairs ? (unsigned)(64 * std::min<int64_t>(16, std::max<int64_t>(4, T))) : 1024u;
    // from kTopkParT tokens the top-k runs one wave per token in its own launch
    // (the selection workgroup would take the tokens 16 at a time)
    const int ids_in = T >= kTopkParT ? 1 : 0;
    if (ids_in) {
#define MOEQ_TOPK(N) hipLaunchKernelGGL(k_topk<N>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, lg, T, E, k, \
                                         gating, scale, ids, w)
      if (E <= 256) MOEQ_TOPK(4);
      else if (E <= 512) MOEQ_TOPK(8);
      else if (E <= 1024) MOEQ_TOPK(16);
      else MOEQ_TOPK(64);
#undef MOEQ_TOPK
    }
#define MOEQ_SEL(N) hipLaunchKernelGGL(k_select_small<N>, dim3(1), dim3(nt), lds, s, lg, T, E, k, gating, \
                                        scale, ids, w, offsets, pairs, active, pl, ids_in)
    if (E <= 256) MOEQ_SEL(4);
    else if (E <= 512) MOEQ_SEL(8);
    else if (E <= 1024) MOEQ_SEL(16);
    else MOEQ_SEL(64);
#undef MOEQ_SEL
  } else {
#define MOEQ_TOPK(N) hipLaunchKernelGGL(k_topk<N>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, lg, T, E, k, \
                                         gating, scale, ids, w)
    if (E <= 256) MOEQ_TOPK(4);
    else if (E <= 512) MOEQ_TOPK(8);
    else if (E <= 1024) MOEQ_TOPK(16);
    else MOEQ_TOPK(64);
#undef MOEQ_TOPK
    return lists_many(T, k, E, ids, offsets, pairs, active, wsb + RL.off_hist, s, pl);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
