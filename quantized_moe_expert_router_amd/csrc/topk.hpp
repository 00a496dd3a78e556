// Top-k routing of one logits row by one wave (shared by the router kernels
// and the one-token FFN kernel, which routes inline).
#pragma once
#include <limits.h>

#include "common.hpp"

namespace moeq {

// Order-preserving key of (fp32 rounding of v, index): for elements whose
// fp32 values differ, the larger key comes first under (logit desc, index
// asc) -- rounding to fp32 never reverses an order, it can only merge values.
__device__ __forceinline__ uint64_t topk_key(double v, int i) {
  uint32_t u = __float_as_uint((float)v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(~(uint32_t)i);
}
__device__ __forceinline__ uint64_t as_u64(double d) { return __builtin_bit_cast(uint64_t, d); }
__device__ __forceinline__ double as_f64(uint64_t u) { return __builtin_bit_cast(double, u); }

// Wave-wide maximum of a 32-bit unsigned value; every lane gets it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  auto mx = [](uint32_t a, int b) { return a > (uint32_t)b ? a : (uint32_t)b; };
  x = mx(x, dpp_all_i<kDppXor1>((int)x));
  x = mx(x, dpp_all_i<kDppXor2>((int)x));
  x = mx(x, dpp_all_i<kDppRowRor4>((int)x));
  x = mx(x, dpp_all_i<kDppRowRor8>((int)x));
  x = mx(x, dpp_i<kDppRowBcast15, 0xA>((int)x, (int)x));
  x = mx(x, dpp_i<kDppRowBcast31, 0xC>((int)x, (int)x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Selection on the fp32 keys: k + 1 rounds of a one-compare arg-max over the
// lanes' sorted key lists.  The result is the exact (fp64) selection when the
// first k + 1 winners have pairwise different fp32 values: then every order
// among them, and between the k-th and everything not selected, is the same
// in fp64.  Returns false (nothing decided) otherwise -- equal fp32 values
// among them, e.g. exact ties -- and the caller runs the fp64 rounds.
template <int NPER>
__device__ __forceinline__ bool topk_fast(const double* v, const int* vi, int k, double& my_v, int& my_i) {
  const int lane = lane_id();
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) key[i] = topk_key(v[i], vi[i]);
  // the lane's keys in descending order (insertion network)
#pragma unroll
  for (int a = 1; a < NPER; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const uint64_t k0 = key[b - 1], k1 = key[b];
      key[b - 1] = k1 > k0 ? k1 : k0;
      key[b] = k1 > k0 ? k0 : k1;
    }
  // rounds: every lane offers the fp32 half of its first unused key (0 once
  // all are used); the round's maximum is a 32-bit wave max, and the lowest
  // lane holding it gives up its head and names the index.  Two heads with
  // the same fp32 value cannot both be decided here: the other one wins the
  // next round with the same value (or, in round k, is not a winner).
  int head = 0;
  uint32_t cf = (uint32_t)(key[0] >> 32), ci = (uint32_t)key[0];
  uint32_t prev_f = 0;
  bool clear = true;
  for (int s = 0; s <= k; ++s) {
    const uint32_t f = wave_max_u32(cf);
    clear = clear && (s == 0 || f != prev_f);
    prev_f = f;
    const int w = __builtin_ctzll(__ballot(cf == f));
    const int idx = (int)~(uint32_t)__builtin_amdgcn_readlane((int)ci, w);
    my_i = lane == s ? idx : my_i;
    head += lane == w ? 1 : 0;
    uint64_t c = 0;
#pragma unroll
    for (int j = NPER - 1; j >= 0; --j) c = head == j ? key[j] : c;
    cf = (uint32_t)(c >> 32);
    ci = (uint32_t)c;
  }
  // the winners' fp64 logits: element e sits in lane e % 64, slot e / 64
  const int src = my_i & (kWave - 1), slot = my_i >> 6;
  double val = 0.0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const double t = __shfl(v[i], src, kWave);
    val = slot == i ? t : val;
  }
  if (lane < k) my_v = val;
  return clear;
}

// Top-k of one logits row by one wave, logits held in registers (NPER per
// lane, element lane + 64*i), under (logit desc, index asc).  The fp32-key
// selection above decides nearly every row; rows it leaves open take rounds
// of an fp64 DPP arg-max over the first remaining element of every lane.
// Lane s < k ends holding the s-th winner (id) and its gate weight: computed
// in fp64 in parallel over the k lanes and normalised by a fixed-order wave
// sum.
// The same on logits already in registers: v[i], vi[i] = logit and index of
// element lane + 64*i (-inf and INT_MAX past E).  Elements known not to be
// among the winners may hold -inf with their index (softmax over all E then
// needs every logit).
template <int NPER>
__device__ __forceinline__ void topk_wave_vals(const double* v, const int* vi, int64_t E, int k, int gating,
                                               float scale, int& my_i, float& my_w) {
  const int lane = lane_id();
  double my_v = 0.0;
  my_i = 0;
  if constexpr (NPER <= 8) {
    if (!topk_fast<NPER>(v, vi, k, my_v, my_i)) {
      // Sort copies of the lane's few logits first (same order), so a round
      // only needs the lane's head: the first of its elements not yet taken.
      double sv[NPER];
      int si[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) { sv[i] = v[i]; si[i] = vi[i]; }
#pragma unroll
      for (int a = 0; a < NPER; ++a)
#pragma unroll
        for (int b = NPER - 1; b > a; --b) {
          double hv = sv[b - 1];
          int hi = si[b - 1];
          better(hv, hi, sv[b], si[b]);              // the first of the pair moves up
          const bool sw = hi != si[b - 1];
          const double lv = sw ? sv[b - 1] : sv[b];
          const int li = sw ? si[b - 1] : si[b];
          sv[b - 1] = hv; si[b - 1] = hi; sv[b] = lv; si[b] = li;
        }
      int head = 0;
      for (int s = 0; s < k; ++s) {
        double best = sv[0];
        int bi = si[0];
#pragma unroll
        for (int j = 1; j < NPER; ++j) {
          best = head == j ? sv[j] : best;
          bi = head == j ? si[j] : bi;
        }
        best = head < NPER ? best : -INFINITY;
        bi = head < NPER ? bi : INT_MAX;
        const int mine = bi;
        wave_argmax(best, bi);
        head += (mine == bi) ? 1 : 0;
        my_v = lane == s ? best : my_v;
        my_i = lane == s ? bi : my_i;
      }
    }
  } else {
    uint64_t taken = 0;
    for (int s = 0; s < k; ++s) {
      double best = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const bool free = !((taken >> i) & 1ull);
        better(best, bi, free ? v[i] : -INFINITY, free ? vi[i] : INT_MAX);
      }
      wave_argmax(best, bi);
      if ((bi & (kWave - 1)) == lane) taken |= 1ull << (bi / kWave);
      my_v = lane == s ? best : my_v;
      my_i = lane == s ? bi : my_i;
    }
  }
  const double mx = readlane_d(my_v, 0);
  double num = 0.0;
  if (lane < k) num = gating == 2 ? 1.0 / (1.0 + exp(-my_v)) : exp(my_v - mx);
  double z;
  if (gating == 1) {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int64_t e = lane + (int64_t)kWave * i;
      if (e < E) part += exp(v[i] - mx);
    }
    z = wave_sum(part);
  } else {
    z = wave_sum(num);
  }
  my_w = (float)(num / z * (double)scale);
}

template <int NPER>
__device__ __forceinline__ void topk_wave_regs(const double* __restrict__ row, int64_t E, int k, int gating, float scale,
                               int& my_i, float& my_w) {
  const int lane = lane_id();
  double v[NPER];
  int vi[NPER];
  // every load is issued (an element past E reloads element E - 1) before
  // the first wait; then the elements past E become -inf
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int64_t e = lane + (int64_t)kWave * i;
    v[i] = gld_f64(row + (e < E ? e : E - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int64_t e = lane + (int64_t)kWave * i;
    v[i] = e < E ? v[i] : -INFINITY;
    vi[i] = e < E ? (int)e : INT_MAX;
  }
  topk_wave_vals<NPER>(v, vi, E, k, gating, scale, my_i, my_w);
}

}  // namespace moeq
