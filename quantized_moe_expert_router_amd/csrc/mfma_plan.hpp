// Tile lists of the int8 MFMA path, built by one wave (of the planning
// kernel, or at the tail of the routing kernel inside the whole-layer call).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace moeq {

constexpr int kTileT = 32;         // activation rows (tokens / pairs) per tile
constexpr int kThinRows = 8;       // experts with at most this many rows get one 8-row tile

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Routed experts whose row count exceeds `thr`: experts with at most
// kThinRows rows get one 8-row tile, the others 32-row tiles; a tile is
// (expert, first row, rows, list offset), experts in union order (absent
// experts too: their down tiles write zero rows).  Wave 0 of the workgroup
// builds both lists with no barrier (active / offsets may have been written
// by this workgroup before a barrier).  Lane l takes union entries
// l*per .. l*per+per-1 to count tiles and write the 8-row ones; the 32-row
// tiles are then written by all lanes, each a contiguous share of the list
// (a hot expert's hundreds of tiles would otherwise fall to one lane): its
// first tile's expert by binary search over the experts' first-tile indices
// (ebase, LDS scratch of at least union size + 1 entries), then a walk.
constexpr int kPlanMaxE = 4096;
__device__ void mfma_plan_block(const int32_t* __restrict__ active, const int32_t* __restrict__ offsets,
                                const MfmaPlan& p, int* ebase) {
  if (threadIdx.x >= kWave) return;
  const int lane = lane_id();
  const int na = active[0];
  const int per = (na + kWave - 1) / kWave;
  const int s0 = lane * per;
  int local = 0, tlocal = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < na) {
      const int e = active[1 + s];
      const int ne = offsets[e + 1] - offsets[e];
      if (ne > p.thr) {
        if (ne <= kThinRows) ++tlocal;
        else local += (ne + kTileT - 1) / kTileT;
      }
    }
  }
  const int inc = wave_incl_scan(local), tinc = wave_incl_scan(tlocal);
  int base = inc - local, tbase = tinc - tlocal;
  if (lane == kWave - 1) {
    *p.count = inc < p.max_tiles ? inc : p.max_tiles;
    *p.thin_count = tinc;
    ebase[na] = inc;
  }
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < na) {
      const int e = active[1 + s];
      const int ne = offsets[e + 1] - offsets[e];
      ebase[s] = base;
      if (ne > p.thr && ne <= kThinRows) {
        p.thin[tbase++] = make_int4(e, 0, ne, offsets[e]);
      } else if (ne > p.thr) {
        base += (ne + kTileT - 1) / kTileT;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int tot_all = __builtin_amdgcn_readlane(inc, kWave - 1);
  const int total = tot_all < p.max_tiles ? tot_all : p.max_tiles;
  const int B = (total + kWave - 1) / kWave;
  const int t_begin = lane * B, t_end = t_begin + B < total ? t_begin + B : total;
  if (t_begin < t_end) {
    int lo = 0, hi = na;            // the last expert s with ebase[s] <= t_begin (its range is not empty)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ebase[mid] <= t_begin) lo = mid;
      else hi = mid - 1;
    }
    int s = lo;
    for (int t = t_begin; t < t_end; ++t) {
      while (ebase[s + 1] <= t) ++s;
      const int e = active[1 + s];
      const int ne = offsets[e + 1] - offsets[e];
      const int t0 = (t - ebase[s]) * kTileT;
      p.tiles[t] = make_int4(e, t0, ne - t0 < kTileT ? ne - t0 : kTileT, offsets[e]);
    }
  }
}

}  // namespace moeq
