// Router: fp64 logits, top-k selection with (logit desc, index asc) order,
// gate weights, and the token x expert lists (counting sort by expert, tokens
// rising inside an expert) plus the expert union.
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"

namespace moeq {

constexpr int kLogitTok = 16;       // tokens per logits tile
constexpr int kSmallT = 256;        // single-workgroup selection + lists up to this many tokens
constexpr int kChunkT = 256;        // tokens per chunk of the multi-kernel lists path

// logits[t, e] = sum_i W[e, i] * x[t, i] (+ bias[e]) in fp64.  The fp32*fp32
// products are exact in fp64, so fma and mul+add agree; only the summation
// order differs from a sequential sum.  One wave per expert, 16 tokens per tile.
__global__ __launch_bounds__(256) void k_logits(const float* __restrict__ x, const float* __restrict__ W,
                                                const float* __restrict__ bias, int64_t T, int64_t H,
                                                int64_t E, double* __restrict__ logits) {
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lane = lane_id();
  const int64_t t0 = (int64_t)blockIdx.y * kLogitTok;
  const int nt = (int)((T - t0) < kLogitTok ? (T - t0) : kLogitTok);
  double acc[kLogitTok];
#pragma unroll
  for (int t = 0; t < kLogitTok; ++t) acc[t] = 0.0;
  const float4* w4 = reinterpret_cast<const float4*>(W + e * H);
  const int64_t n4 = H / 4;
  for (int64_t i = lane; i < n4; i += kWave) {
    const float4 w = w4[i];
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t) {
      if (t < nt) {
        const float4 xv = reinterpret_cast<const float4*>(x + (t0 + t) * H)[i];
        double a = acc[t];
        a = fma((double)w.x, (double)xv.x, a);
        a = fma((double)w.y, (double)xv.y, a);
        a = fma((double)w.z, (double)xv.z, a);
        a = fma((double)w.w, (double)xv.w, a);
        acc[t] = a;
      }
    }
  }
  const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
  for (int t = 0; t < kLogitTok; ++t) {
    double v = group_sum(acc[t], kWave);
    if (lane == 0 && t < nt) logits[(t0 + t) * E + e] = bias ? v + b : v;
  }
}

// Top-k of one logits row by one wave; writes ids and gate weights.  The k
// winners are found one at a time: each lane scans its stripe (elements lane,
// lane+64, ...), skipping taken ones, then a butterfly keeps the larger logit,
// the lower index on a tie.
__device__ void topk_row_wave(const double* __restrict__ row, int64_t E, int k, int gating, float scale,
                              int32_t* __restrict__ ids_out, float* __restrict__ w_out, double* sel_v,
                              int* sel_i, int32_t* ids_lds) {
  const int lane = lane_id();
  const int nper = (int)((E + kWave - 1) / kWave);
  uint64_t taken = 0;
  for (int s = 0; s < k; ++s) {
    double best = -INFINITY;
    int bi = INT_MAX;
    for (int i = 0; i < nper; ++i) {
      const int64_t e = lane + (int64_t)kWave * i;
      if (e < E && !((taken >> i) & 1ull)) {
        const double v = row[e];
        if (v > best || (v == best && (int)e < bi)) { best = v; bi = (int)e; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(best, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1ull << (bi / kWave);
    if (lane == 0) { sel_v[s] = best; sel_i[s] = bi; }
  }
  // softmax-all needs the partition function over every logit.
  double zall = 0.0;
  if (gating == 1) {
    const double mx = __shfl(sel_v[0], 0, kWave);
    double part = 0.0;
    for (int i = 0; i < nper; ++i) {
      const int64_t e = lane + (int64_t)kWave * i;
      if (e < E) part += exp(row[e] - mx);
    }
    zall = group_sum(part, kWave);
  }
  if (lane == 0) {
    const double mx = sel_v[0];
    double z = 0.0;
    if (gating == 0) {
      for (int s = 0; s < k; ++s) z += exp(sel_v[s] - mx);
    } else if (gating == 1) {
      z = zall;
    } else {
      for (int s = 0; s < k; ++s) z += 1.0 / (1.0 + exp(-sel_v[s]));
    }
    for (int s = 0; s < k; ++s) {
      const double num = gating == 2 ? 1.0 / (1.0 + exp(-sel_v[s])) : exp(sel_v[s] - mx);
      ids_out[s] = sel_i[s];
      w_out[s] = (float)(num / z * (double)scale);
      if (ids_lds) ids_lds[s] = sel_i[s];
    }
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

// counts[E] -> offsets[E+1] and the active list; `cnt` lives in LDS.
__device__ void offsets_and_union(int* cnt, int64_t E, int32_t* offsets, int32_t* active,
                                  int* scan_tmp, int* base_out /* LDS [E] or null */) {
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
      if (c > 0) active[1 + frun++] = (int32_t)e;
      run += c;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = tot;
    active[0] = ftot;
  }
}

// T <= kSmallT: top-k for every token, then the lists, in one workgroup.
__global__ __launch_bounds__(1024) void k_select_small(const double* __restrict__ logits, int64_t T, int64_t E,
                                                       int k, int gating, float scale, int32_t* __restrict__ ids,
                                                       float* __restrict__ w, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ pairs, int32_t* __restrict__ active) {
  extern __shared__ double lds_d[];
  double* sel_v = lds_d;                                      // [16][32]
  int* sel_i = reinterpret_cast<int*>(sel_v + 16 * 32);       // [16][32]
  int* ids_s = sel_i + 16 * 32;                               // [T*k]
  int* cnt = ids_s + T * k;                                   // [E]
  int* scan_tmp = cnt + E;                                    // [64]
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int64_t t = wv; t < T; t += nw)
    topk_row_wave(logits + t * E, E, k, gating, scale, ids + t * k, w + t * k, sel_v + 32 * wv,
                  sel_i + 32 * wv, ids_s + t * k);
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
}

// ---- multi-kernel path for large T
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int64_t T, int64_t E, int k,
                                              int gating, float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ w) {
  __shared__ double sel_v[4][32];
  __shared__ int sel_i[4][32];
  const int wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= T) return;
  topk_row_wave(logits + t * E, E, k, gating, scale, ids + t * k, w + t * k, sel_v[wv], sel_i[wv], nullptr);
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
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ active) {
  extern __shared__ int lds[];
  int* tot = lds;              // [E]
  int* scan_tmp = tot + E;     // [64]
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int64_t c = 0; c < nchunks; ++c) s += hist[c * E + e];
    tot[e] = s;
  }
  __syncthreads();
  offsets_and_union(tot, E, offsets, active, scan_tmp, tot);   // tot becomes the offsets
  __syncthreads();
  for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tot[e];
    for (int64_t c = 0; c < nchunks; ++c) {
      const int h = hist[c * E + e];
      hist[c * E + e] = run;
      run += h;
    }
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
  for (int64_t t = t0; t < t1; ++t) {
    if (lane < k) {
      const int e = ids[t * k + lane];
      const int pos = atomicAdd(&cur[e], 1);
      pairs[pos] = (int32_t)(t * k + lane);
    }
  }
}

__global__ void k_empty_lists(int64_t E, int32_t* offsets, int32_t* active) {
  for (int64_t e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
  if (threadIdx.x == 0) active[0] = 0;
}

size_t route_ws_bytes(int64_t T, int64_t E) {
  size_t b = align256((size_t)T * E * sizeof(double));
  if (T > kSmallT) b += align256((size_t)((T + kChunkT - 1) / kChunkT) * E * sizeof(int32_t));
  return b;
}

int launch_route(int64_t T, int64_t H, int64_t E, int k, int gating, float scale, const float* x,
                 const float* W, const float* bias, double* logits, int32_t* ids, float* w,
                 int32_t* offsets, int32_t* pairs, int32_t* active, void* ws, hipStream_t s) {
  if (T == 0) {
    hipLaunchKernelGGL(k_empty_lists, dim3(1), dim3(256), 0, s, E, offsets, active);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  uint8_t* wsb = (uint8_t*)ws;
  double* lg = logits ? logits : reinterpret_cast<double*>(wsb);
  dim3 g1((unsigned)((E + 3) / 4), (unsigned)((T + kLogitTok - 1) / kLogitTok));
  hipLaunchKernelGGL(k_logits, g1, dim3(256), 0, s, x, W, bias, T, H, E, lg);
  if (T <= kSmallT) {
    size_t lds = (size_t)(T * k + E + 64) * sizeof(int) + 16 * 32 * (sizeof(double) + sizeof(int));
    hipLaunchKernelGGL(k_select_small, dim3(1), dim3(1024), lds, s, lg, T, E, k, gating, scale, ids, w,
                       offsets, pairs, active);
  } else {
    const int64_t nch = (T + kChunkT - 1) / kChunkT;
    int32_t* hist = reinterpret_cast<int32_t*>(wsb + align256((size_t)T * E * sizeof(double)));
    hipLaunchKernelGGL(k_topk, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, lg, T, E, k, gating, scale,
                       ids, w);
    hipLaunchKernelGGL(k_hist, dim3((unsigned)nch), dim3(256), (size_t)E * sizeof(int), s, ids, T, k, E, hist);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), (size_t)(E + 64) * sizeof(int), s, hist, nch, E, offsets,
                       active);
    hipLaunchKernelGGL(k_scatter, dim3((unsigned)nch), dim3(64), (size_t)E * sizeof(int), s, ids, T, k, E,
                       hist, pairs);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
