// Shared device helpers of libmoeq (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;
constexpr int kQ8KBytes = 292;   // f32 d | i8 q[256] | i16 bsums[16]

enum FmtId : int { FQ4K = 1, FQ6K = 2, FQ2K = 3, FQ80 = 4, FQ3K = 5, FQ5K = 6, FQ40 = 7, FQ51 = 8 };

__device__ __forceinline__ int dot4(int a, int b, int acc) {
  return __builtin_amdgcn_sdot4(a, b, acc, false);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  uint16_t b = (uint16_t)bits16;
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// Accesses through the global address space (global_load / global_store).
// Pointers read from tables or argument structs are generic to the compiler,
// and generic (flat) accesses also count against the LDS wait counter: a wait
// for an LDS read would then also wait for every weight load in flight.
#define MOEQ_GLOBAL __attribute__((address_space(1)))
typedef unsigned int g_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int g_u32x2 __attribute__((ext_vector_type(2)));
typedef float g_f32x4 __attribute__((ext_vector_type(4)));
// 16-byte aligned
__device__ __forceinline__ uint4 gld_u4(const void* p) {
  const g_u32x4 v = *(const MOEQ_GLOBAL g_u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 8-byte aligned
__device__ __forceinline__ uint2 gld_u2(const void* p) {
  const g_u32x2 v = *(const MOEQ_GLOBAL g_u32x2*)p;
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 gld_f4(const void* p) {
  const g_f32x4 v = *(const MOEQ_GLOBAL g_f32x4*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t gld_u32(const void* p) { return *(const MOEQ_GLOBAL uint32_t*)p; }
__device__ __forceinline__ uint32_t gld_u16(const void* p) { return *(const MOEQ_GLOBAL uint16_t*)p; }
__device__ __forceinline__ float gld_f32(const void* p) { return *(const MOEQ_GLOBAL float*)p; }
__device__ __forceinline__ double gld_f64(const void* p) { return *(const MOEQ_GLOBAL double*)p; }
__device__ __forceinline__ uint64_t gld_u64(const void* p) { return *(const MOEQ_GLOBAL uint64_t*)p; }
__device__ __forceinline__ int32_t gld_i32(const void* p) { return *(const MOEQ_GLOBAL int32_t*)p; }
__device__ __forceinline__ void gst_f32(void* p, float v) { *(MOEQ_GLOBAL float*)p = v; }
__device__ __forceinline__ void gst_f4(void* p, float4 v) {   // 16-byte aligned
  *(MOEQ_GLOBAL g_f32x4*)p = g_f32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void gst_u32(void* p, uint32_t v) { *(MOEQ_GLOBAL uint32_t*)p = v; }
__device__ __forceinline__ void gst_i32(void* p, int32_t v) { *(MOEQ_GLOBAL int32_t*)p = v; }
__device__ __forceinline__ void gst_i16(void* p, int16_t v) { *(MOEQ_GLOBAL int16_t*)p = v; }

// ---- DPP cross-lane moves (register to register, no LDS round trip).
// Control codes of the gfx9 DPP encoding.
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within a 16-lane row
constexpr int kDppHalfMirror = 0x141;    // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
// Full-row patterns write every lane: no "old" operand needed.
template <int CTRL>
__device__ __forceinline__ int dpp_all_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ double dpp_all_d(double v) {
  int2 x = *reinterpret_cast<int2*>(&v), r;
  r.x = __builtin_amdgcn_mov_dpp(x.x, CTRL, 0xF, 0xF, false);
  r.y = __builtin_amdgcn_mov_dpp(x.y, CTRL, 0xF, 0xF, false);
  return *reinterpret_cast<double*>(&r);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_d(double old, double v) {
  int2 o = *reinterpret_cast<int2*>(&old), x = *reinterpret_cast<int2*>(&v), r;
  r.x = __builtin_amdgcn_update_dpp(o.x, x.x, CTRL, ROW_MASK, 0xF, false);
  r.y = __builtin_amdgcn_update_dpp(o.y, x.y, CTRL, ROW_MASK, 0xF, false);
  return *reinterpret_cast<double*>(&r);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  int2 x = *reinterpret_cast<int2*>(&v), r;
  r.x = __builtin_amdgcn_readlane(x.x, lane);
  r.y = __builtin_amdgcn_readlane(x.y, lane);
  return *reinterpret_cast<double*>(&r);
}

// (value, index) that comes first under (value desc, index asc); branch-free
// (selects, no exec-mask branches).
__device__ __forceinline__ void better(double& v, int& i, double ov, int oi) {
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}

// Wave-wide arg-max under (value desc, index asc); every lane gets the winner.
// Each step combines a lane with a partner from another lane set; lanes a
// DPP move does not write keep their own value (neutral for the max).
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  better(v, i, dpp_all_d<kDppXor1>(v), dpp_all_i<kDppXor1>(i));
  better(v, i, dpp_all_d<kDppXor2>(v), dpp_all_i<kDppXor2>(i));
  better(v, i, dpp_all_d<kDppRowRor4>(v), dpp_all_i<kDppRowRor4>(i));
  better(v, i, dpp_all_d<kDppRowRor8>(v), dpp_all_i<kDppRowRor8>(i));
  better(v, i, dpp_d<kDppRowBcast15, 0xA>(v, v), dpp_i<kDppRowBcast15, 0xA>(i, i));
  better(v, i, dpp_d<kDppRowBcast31, 0xC>(v, v), dpp_i<kDppRowBcast31, 0xC>(i, i));
  v = readlane_d(v, 63);
  i = __builtin_amdgcn_readlane(i, 63);
}

template <int CTRL>
__device__ __forceinline__ float dpp_all_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// fp64 sum over aligned groups of `width` lanes (a power of two <= 64, uniform
// across the wave).  The total is valid in the group's last lane (in every
// lane of the group for width <= 16); the addition order is fixed.
__device__ __forceinline__ double group_sum_dpp(double v, int width) {
  if (width >= 2) v += dpp_all_d<kDppXor1>(v);
  if (width >= 4) v += dpp_all_d<kDppXor2>(v);
  if (width >= 8) v += dpp_all_d<kDppHalfMirror>(v);
  if (width >= 16) v += dpp_all_d<kDppRowMirror>(v);
  if (width >= 32) v += dpp_d<kDppRowBcast15, 0xA>(0.0, v);
  if (width >= 64) v += dpp_d<kDppRowBcast31, 0xC>(0.0, v);
  return v;
}

// Max over aligned groups of GW lanes (GW = 4 or 8); every lane of the group
// gets the result.
template <int GW>
__device__ __forceinline__ float group_max_dpp(float v) {
  v = fmaxf(v, dpp_all_f<kDppXor1>(v));
  v = fmaxf(v, dpp_all_f<kDppXor2>(v));
  if constexpr (GW >= 8) v = fmaxf(v, dpp_all_f<kDppHalfMirror>(v));
  static_assert(GW == 4 || GW == 8, "group width");
  return v;
}

// Max over the whole wave, broadcast to every lane.
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_all_f<kDppXor1>(v));
  v = fmaxf(v, dpp_all_f<kDppXor2>(v));
  v = fmaxf(v, dpp_all_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_all_f<kDppRowMirror>(v));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                    __builtin_bit_cast(int, v),
                                                                    kDppRowBcast15, 0xA, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                    __builtin_bit_cast(int, v),
                                                                    kDppRowBcast31, 0xC, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Wave-wide fp64 sum; every lane gets the total.  The order of additions is
// fixed by the lane pattern, so the result is deterministic.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_all_d<kDppXor1>(v);
  v += dpp_all_d<kDppXor2>(v);
  v += dpp_all_d<kDppRowRor4>(v);
  v += dpp_all_d<kDppRowRor8>(v);
  v += dpp_d<kDppRowBcast15, 0xA>(0.0, v);
  v += dpp_d<kDppRowBcast31, 0xC>(0.0, v);
  return readlane_d(v, 63);
}

// SiLU in fp64: z / (1 + e^-z).
__device__ __forceinline__ double silu64(double z) { return z / (1.0 + exp(-z)); }

// q8_K of one value given the block's inverse scale: clamp(rint(x*id), -127, 127).
__device__ __forceinline__ int q8_code(float x, float id) {
  float v = __builtin_rintf(__fmul_rn(x, id));
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int)v;
}

// q8_K of one 256-block held by one wave (4 consecutive elements per lane),
// identical to the definition: amax, then id = 127/amax (correctly rounded),
// q = rint(x*id) clamped to +-127, d = amax/127, per-16 sums; amax == 0 or
// an infinite id gives a zero block.
__device__ __forceinline__ void quantize_block_vals(float4 v, uint8_t* __restrict__ o) {
  const int lane = lane_id();
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = wave_max_f(amax);
  const float id = amax == 0.0f ? 0.0f : __fdiv_rn(127.0f, amax);
  const bool zero = amax == 0.0f || __builtin_isinf(id);
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (!zero) { q0 = q8_code(v.x, id); q1 = q8_code(v.y, id); q2 = q8_code(v.z, id); q3 = q8_code(v.w, id); }
  gst_u32(o + 4 + 4 * lane,
          (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24));
  int s = q0 + q1 + q2 + q3;
  s += dpp_all_i<kDppXor1>(s);
  s += dpp_all_i<kDppXor2>(s);
  if ((lane & 3) == 0) gst_i16(o + 260 + 2 * (lane >> 2), (int16_t)s);
  if (lane == 0) gst_f32(o, zero ? 0.0f : __fdiv_rn(amax, 127.0f));
}

// q8_K of 256-block g of a row-major fp32 matrix with `cols` columns, by one
// wave.
__device__ __forceinline__ void quantize_block_wave(const float* __restrict__ x, int64_t cols, int64_t g,
                                                    int64_t nblocks, uint8_t* __restrict__ out) {
  if (g >= nblocks) return;
  const int64_t nb = cols / 256, row = g / nb, b = g % nb;
  quantize_block_vals(gld_f4(x + row * cols + b * 256 + 4 * lane_id()), out + g * kQ8KBytes);
}

// RMS pre-norm of one token's residual row (the MoE block's input in a stack
// of layers): r = 1 / sqrt(mean(x^2) + eps) in fp64, by one wave over `cols`
// (a multiple of 256) fp32 values; every lane gets r.  Lane l adds the exact
// fp64 squares of elements 256m + 4l .. 256m + 4l + 3 for m = 0, 1, ... in
// that order, then the lanes' sums add in wave_sum's fixed order, so every
// wave that computes r for the same row gets the same bits.
__device__ __forceinline__ double row_rms_scale(const float* __restrict__ row, int64_t cols, double eps) {
  constexpr int U = 8;                      // loads in flight per lane
  const int lane = lane_id();
  double ss = 0.0;
  for (int64_t base = 0; base < cols; base += (int64_t)U * 4 * kWave) {
    float4 v[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {           // a unit past the row reloads unit 0, left out below
      const int64_t i = base + 4 * lane + (int64_t)u * 4 * kWave;
      ok[u] = i < cols;
      v[u] = gld_f4(row + (ok[u] ? i : 4 * lane));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double t = fma((double)v[u].x, (double)v[u].x, ss);
      t = fma((double)v[u].y, (double)v[u].y, t);
      t = fma((double)v[u].z, (double)v[u].z, t);
      t = fma((double)v[u].w, (double)v[u].w, t);
      ss = ok[u] ? t : ss;
    }
  }
  ss = wave_sum(ss);
  return 1.0 / sqrt(ss / (double)cols + eps);
}
// Normalised element: fl32((x * r) * g), both products in fp64.
__device__ __forceinline__ float norm_elem(float x, double r, float g) {
  return (float)(((double)x * r) * (double)g);
}
__device__ __forceinline__ float4 norm4(float4 v, double r, float4 g) {
  return make_float4(norm_elem(v.x, r, g.x), norm_elem(v.y, r, g.y), norm_elem(v.z, r, g.z), norm_elem(v.w, r, g.w));
}

__host__ __device__ constexpr size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace moeq
