// Tile lists of the int8 MFMA path, built by one wave (of the planning
// kernel, or at the tail of the routing kernel inside the whole-layer call).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace moeq {

constexpr int kTileT = 32;         // activation rows (tokens / pairs) per tile
constexpr int kThinRows = 8;       // rows of the tiles of experts with few rows

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

// The counting half of mfma_plan_block, by wave 0: tile counts, the 8-row
// tiles (ceil(rows / 8) per expert, consecutive), each expert's first 32-row
// tile index in ebase (ebase[na] = total), and the two counts.
__device__ __forceinline__ void plan_count(const int32_t* __restrict__ active, const int32_t* __restrict__ offsets,
                                           const MfmaPlan& p, int* ebase, int na) {
  const int lane = lane_id();
  const int per = (na + kWave - 1) / kWave;
  const int s0 = lane * per;
  int local = 0, tlocal = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < na) {
      const int e = active[1 + s];
      const int ne = offsets[e + 1] - offsets[e];
      if (ne > p.thr) {
        if (ne <= p.thin_max) tlocal += (ne + kThinRows - 1) / kThinRows;
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
      if (ne > p.thr && ne <= p.thin_max) {
        for (int t0 = 0; t0 < ne; t0 += kThinRows)
          p.thin[tbase++] = make_int4(e, t0, ne - t0 < kThinRows ? ne - t0 : kThinRows, offsets[e]);
      } else if (ne > p.thr) {
        base += (ne + kTileT - 1) / kTileT;
      }
    }
  }
}

// Routed experts whose row count exceeds `thr`: experts with at most
// p.thin_max rows get 8-row tiles, the others 32-row tiles; a tile is
// (expert, first row, rows, list offset), experts in union order (absent
// experts too: their down tiles write zero rows).  Every thread of the
// workgroup calls it (active / offsets may have been written by this
// workgroup before a barrier).  Wave 0 counts: lane l takes union entries
// l*per .. l*per+per-1 to count tiles and write the 8-row ones, and records
// each expert's first-tile index (ebase, LDS scratch of at least union size
// + 1 entries).  After a barrier the 32-row tiles are written by every thread
// of the workgroup, each a contiguous share of the list (a hot expert's
// hundreds of tiles would otherwise fall to one lane): its first tile's
// expert by binary search over ebase, then a walk.
constexpr int kPlanMaxE = 4096;
__device__ void mfma_plan_block(const int32_t* __restrict__ active, const int32_t* __restrict__ offsets,
                                const MfmaPlan& p, int* ebase) {
  const int na = active[0];
  if (threadIdx.x < kWave) plan_count(active, offsets, p, ebase, na);
  __syncthreads();
  const int tot_all = ebase[na];
  const int total = tot_all < p.max_tiles ? tot_all : p.max_tiles;
  const int nthr = (int)blockDim.x;
  const int B = (total + nthr - 1) / nthr;
  const int t_begin = (int)threadIdx.x * B, t_end = t_begin + B < total ? t_begin + B : total;
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
