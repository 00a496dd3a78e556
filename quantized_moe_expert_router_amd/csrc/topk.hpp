// Top-k routing of one logits row by one wave (shared by the router kernels
// and the one-token FFN kernel, which routes inline).
#pragma once
#include <limits.h>

#include "common.hpp"

namespace moeq {

// Top-k of one logits row by one wave, logits held in registers (NPER per
// lane, element lane + 64*i).  Each round takes the first remaining element
// under (logit desc, index asc) with a DPP arg-max.  Lane s < k ends holding
// the s-th winner (id) and its gate weight: computed in fp64 in parallel over
// the k lanes and normalised by a fixed-order wave sum.
template <int NPER>
__device__ void topk_wave_regs(const double* __restrict__ row, int64_t E, int k, int gating, float scale,
                               int& my_i, float& my_w) {
  const int lane = lane_id();
  double v[NPER];
  int vi[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int64_t e = lane + (int64_t)kWave * i;
    v[i] = e < E ? gld_f64(row + e) : -INFINITY;
    vi[i] = e < E ? (int)e : INT_MAX;
  }
  double my_v = 0.0;
  my_i = 0;
  if constexpr (NPER <= 8) {
    // Sort the lane's few logits first (same order), so a round only needs
    // the lane's head: the first of its elements not yet taken.
#pragma unroll
    for (int a = 0; a < NPER; ++a)
#pragma unroll
      for (int b = NPER - 1; b > a; --b) {
        double hv = v[b - 1];
        int hi = vi[b - 1];
        better(hv, hi, v[b], vi[b]);               // the first of the pair moves up
        const bool sw = hi != vi[b - 1];
        const double lv = sw ? v[b - 1] : v[b];
        const int li = sw ? vi[b - 1] : vi[b];
        v[b - 1] = hv; vi[b - 1] = hi; v[b] = lv; vi[b] = li;
      }
    int head = 0;
    for (int s = 0; s < k; ++s) {
      double best = v[0];
      int bi = vi[0];
#pragma unroll
      for (int j = 1; j < NPER; ++j) {
        best = head == j ? v[j] : best;
        bi = head == j ? vi[j] : bi;
      }
      best = head < NPER ? best : -INFINITY;
      bi = head < NPER ? bi : INT_MAX;
      const int mine = bi;
      wave_argmax(best, bi);
      head += (mine == bi) ? 1 : 0;
      my_v = lane == s ? best : my_v;
      my_i = lane == s ? bi : my_i;
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

}  // namespace moeq
