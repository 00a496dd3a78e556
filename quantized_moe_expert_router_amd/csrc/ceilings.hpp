// Launchers of the measured-ceiling kernels (HBM streaming read; int8 MFMA
// loop), at most kCeilMaxBlocks workgroups each.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moeq {

constexpr int32_t kCeilMaxBlocks = 1 << 22;
int launch_ceiling_read(const void* buf, int64_t bytes, int n_blocks, uint64_t* out, hipStream_t s);
int launch_ceiling_mfma_i8(int64_t iters, int n_blocks, int32_t* out, hipStream_t s);

}  // namespace moeq
