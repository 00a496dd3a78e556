// Measured ceilings of the two rooflines the expert kernels are read against:
// a streaming read of a large buffer (HBM bandwidth with the plain 16-byte
// global loads the kernels use) and a loop of independent int8 MFMAs on
// registers (matrix-core throughput with no memory traffic).  Each kernel
// leaves a result the caller can check, so no load or MFMA can be dropped.
#include "common.hpp"
#include "ceilings.hpp"

namespace moeq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kCeilThreads = 256;

// Every 16-byte word of p[0 .. n16) is read once: thread t of the grid reads
// words t, t + S, t + 2S, ... (S = the grid's thread count), four loads in
// flight per step.  The wrapping 64-bit sum of the 32-bit words a workgroup
// read goes to out[blockIdx.x].
__global__ __launch_bounds__(kCeilThreads) void k_ceiling_read(const uint4* __restrict__ p, int64_t n16,
                                                              uint64_t* __restrict__ out) {
  __shared__ uint64_t part[kCeilThreads];
  const int64_t S = (int64_t)gridDim.x * kCeilThreads;
  int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
  uint64_t s = 0;
  for (; i + 3 * S < n16; i += 4 * S) {
    const uint4 a = gld_u4(p + i), b = gld_u4(p + i + S), c = gld_u4(p + i + 2 * S), d = gld_u4(p + i + 3 * S);
    s += (uint64_t)a.x + a.y + a.z + a.w;
    s += (uint64_t)b.x + b.y + b.z + b.w;
    s += (uint64_t)c.x + c.y + c.z + c.w;
    s += (uint64_t)d.x + d.y + d.z + d.w;
  }
  for (; i < n16; i += S) {
    const uint4 a = gld_u4(p + i);
    s += (uint64_t)a.x + a.y + a.z + a.w;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int j = 0; j < kCeilThreads; ++j) t += part[j];
    out[blockIdx.x] = t;
  }
}

// Four independent accumulation chains of v_mfma_i32_32x32x32_i8 per wave on
// the byte pattern `bytes` (both operands), iters steps.  With bytes of 1
// every step adds 32 to each result, so wave w of workgroup b writes
// 4 * 32 * iters (mod 2^32) to out[4 b + w].
__global__ __launch_bounds__(kCeilThreads) void k_ceiling_mfma_i8(int64_t iters, int32_t bytes,
                                                                 int32_t* __restrict__ out) {
  const v4i a = {bytes, bytes, bytes, bytes};
  v16i c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c3, 0, 0, 0);
  }
  if (lane_id() == 0) {
    const uint32_t v = (uint32_t)c0[0] + (uint32_t)c1[0] + (uint32_t)c2[0] + (uint32_t)c3[0];
    gst_i32(out + 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6), (int32_t)v);
  }
}

}  // namespace

int launch_ceiling_read(const void* buf, int64_t bytes, int n_blocks, uint64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_ceiling_read, dim3((unsigned)n_blocks), dim3(kCeilThreads), 0, s,
                     (const uint4*)buf, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_ceiling_mfma_i8(int64_t iters, int n_blocks, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_ceiling_mfma_i8, dim3((unsigned)n_blocks), dim3(kCeilThreads), 0, s, iters,
                     (int32_t)0x01010101, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
