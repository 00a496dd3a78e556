// Routing of a small chunk (at most 64 token x slot pairs) inside one
// workgroup: the pair lists and the expert union from the selected experts
// held in LDS.  The routing kernel uses it, and so do the first gate/up tiles
// of small chunks, which route inline from the logits (every workgroup routes
// for itself; one of them also writes the routing outputs).
#pragma once
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_plan.hpp"
#include "topk.hpp"

namespace moeq {

// Lists of at most 64 (token, slot) pairs p = t*k + slot, from their experts
// in LDS: ordered by expert and, inside an expert, by p (the counting-sort
// order), pair p's list position is its rank by the key (expert, p) -- keys
// are distinct, so the ranks are a permutation.  Wave 0 ranks the pairs
// (keys broadcast lane by lane), writes the sorted keys, and takes the union
// as the first key of every expert in that order; then every thread finds
// offsets[e] (the pairs with a smaller expert) by binary search in the sorted
// keys.  Sorted keys, union and offsets go to LDS (skey, lact, loff); the
// pair list, union and offsets also go to memory unless those pointers are
// null.  With lpos, union entry i's first sorted position goes to lpos[i]
// (lpos[union size] = P); a null loff skips the offsets (offsets must then be
// null too).  Ends without a barrier after the offsets.
constexpr int kSmallPairs = 64;
__device__ __forceinline__ void small_lists(const int* ids_s, int P, int64_t E, int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ pairs, int32_t* __restrict__ active, int* skey,
                                            int* loff, int* lact, int* lpos = nullptr) {
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    const int key = lane < P ? ((ids_s[lane] << 6) | lane) : INT_MAX;
    int rank = 0;
    for (int q = 0; q < P; ++q) rank += __builtin_amdgcn_readlane(key, q) < key;
    if (lane < P) {
      skey[rank] = key;
      if (pairs) gst_i32(pairs + rank, lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int ex = lane < P ? skey[lane] >> 6 : -1;
    const int prev = lane > 0 && lane < P ? skey[lane - 1] >> 6 : -1;
    const bool first = lane < P && ex != prev;
    const uint64_t bal = __ballot(first);
    const int idx = __popcll(bal & ((1ull << lane) - 1ull));
    if (first) {
      lact[1 + idx] = ex;
      if (lpos) lpos[idx] = lane;
      if (active) gst_i32(active + 1 + idx, ex);
    }
    if (lane == 0) {
      lact[0] = __popcll(bal);
      if (lpos) lpos[__popcll(bal)] = P;
      if (active) gst_i32(active, __popcll(bal));
    }
  }
  __syncthreads();
  if (loff == nullptr) return;
  for (int64_t e = threadIdx.x; e <= E; e += blockDim.x) {
    const int ke = (int)e << 6;
    int lo = 0, hi = P;                     // first sorted position whose key is >= (e, 0)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (skey[mid] < ke) lo = mid + 1;
      else hi = mid;
    }
    loff[e] = lo;
    if (offsets) gst_i32(offsets + e, lo);
  }
}

// Inline routing of a chunk of 2..8 tokens with at most 64 pairs by the
// fp32-h gate/up tiles of the int8 MFMA path (every routed expert then has at
// most 8 rows: one 8-row tile each, tile j = the j-th expert of the union in
// expert order).  The layer call launches the router logits (fp64) and
// q8_K(x), then these tiles in place of the selection launch.
constexpr int kSmallRouteMaxT = 8;
constexpr int64_t kSmallRouteMaxE = 512;   // top-k in registers: at most 8 logits per lane
struct SmallRoute {
  const double* logits;   // [T, E] fp64
  int64_t E;
  int gating;
  float scale;
  int32_t* ids;           // routing outputs, written by workgroup (0, 0)
  float* w;
  int32_t* offsets;
  int32_t* pairs;
  int32_t* active;
  MfmaPlan plan;          // the 8-row tile list the down launch reads, written by the same workgroup
};
int launch_mfma_route_gateup(int fmt, dim3 grid, const MfmaArgs& a, const SmallRoute& r, hipStream_t s);
// The same with the shared expert's nsh fp32-h tiles (sa) in the first
// workgroups of every grid row (format pairs as mfma_hf2_pair).
int launch_mfma_route_gateup2(int fmt_r, int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa,
                              const SmallRoute& r, int nsh, hipStream_t s);

// The routing of a small chunk by one workgroup (every thread calls it; the
// LDS arrays hold kSmallPairs, kSmallPairs, kSmallPairs + 1, kSmallPairs + 1,
// E + 1 and kSmallPairs + 1 ints): each wave takes tokens wave, wave + waves,
// ... and selects their experts from the logits; then the sorted pairs and
// the union in LDS.  Workgroup (0, 0) also forms the offsets of every expert
// and writes the ids, gate weights, lists and the MFMA tile lists to memory.
// The workgroup's tile is union entry j (blockIdx.x unless the launch also
// holds other tiles; the writer is the workgroup of entry 0 in grid row 0):
// its expert e, rows n and list offset; false when the union has no such
// entry.
template <int NPER>
__device__ __forceinline__ bool route_small_tile(const SmallRoute& r, int64_t T, int k, int* ids_s, int* skey,
                                                 int* lact, int* lpos, int* loff, int* ebase, int j, int& e, int& n,
                                                 int64_t& list_off) {
  const int lane = lane_id(), wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const bool writer = j == 0 && blockIdx.y == 0;
  for (int64_t t = wv; t < T; t += nw) {
    int my_i;
    float my_w;
    topk_wave_regs<NPER>(r.logits + t * r.E, r.E, k, r.gating, r.scale, my_i, my_w);
    if (lane < k) {
      ids_s[t * k + lane] = my_i;
      if (writer) {
        gst_i32(r.ids + t * k + lane, my_i);
        gst_f32(r.w + t * k + lane, my_w);
      }
    }
  }
  __syncthreads();
  small_lists(ids_s, (int)(T * k), r.E, writer ? r.offsets : nullptr, writer ? r.pairs : nullptr,
              writer ? r.active : nullptr, skey, writer ? loff : nullptr, lact, lpos);
  __syncthreads();
  if (writer) mfma_plan_block(lact, loff, r.plan, ebase);
  const int na = lact[0];
  if (j >= na) return false;
  e = lact[1 + j];
  list_off = lpos[j];
  n = lpos[j + 1] - lpos[j];
  return true;
}

}  // namespace moeq
