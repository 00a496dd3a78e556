// Shared device helpers of libmoeq (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;
constexpr int kQ8KBytes = 292;   // f32 d | i8 q[256] | i16 bsums[16]

enum FmtId : int { FQ4K = 1, FQ6K = 2, FQ2K = 3, FQ80 = 4 };

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

// Butterfly sum over groups of `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ double group_sum(double v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float group_max(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// SiLU in fp64: z / (1 + e^-z).
__device__ __forceinline__ double silu64(double z) { return z / (1.0 + exp(-z)); }

// q8_K of one value given the block's inverse scale: clamp(rint(x*id), -127, 127).
__device__ __forceinline__ int q8_code(float x, float id) {
  float v = __builtin_rintf(__fmul_rn(x, id));
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int)v;
}

__host__ __device__ constexpr size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace moeq
