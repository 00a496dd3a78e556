// q8_K activation quantisation and the one-time exchange->packed weight repack.
#include "formats.hpp"
#include "launch.hpp"

namespace moeq {

__global__ __launch_bounds__(256) void k_quantize_q8K(const float* __restrict__ x, int64_t rows,
                                                      int64_t cols, uint8_t* __restrict__ out) {
  quantize_block_wave(x, cols, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), rows * (cols / 256), out);
}

int launch_quantize_q8K(const float* x, int64_t rows, int64_t cols, void* out, hipStream_t s) {
  int64_t nblk = rows * (cols / 256);
  if (nblk == 0) return 0;
  int64_t grid = (nblk + 3) / 4;
  hipLaunchKernelGGL(k_quantize_q8K, dim3((unsigned)grid), dim3(256), 0, s, x, rows, cols,
                     (uint8_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// RMS pre-norm, one wave per token row: out = fl32((x * r) * g) with
// r = 1 / sqrt(mean(x^2) + eps) in fp64; g null means all ones.
__global__ __launch_bounds__(256) void k_rms_norm(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                  const float* __restrict__ g, double eps, float* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * cols;
  const double r = row_rms_scale(xr, cols, eps);
  for (int64_t i = 4 * lane_id(); i < cols; i += 4 * kWave) {
    const float4 gv = g ? gld_f4(g + i) : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    const float4 v = norm4(gld_f4(xr + i), r, gv);
    *reinterpret_cast<float4*>(out + row * cols + i) = v;
  }
}

int launch_rms_norm(const float* x, int64_t rows, int64_t cols, const float* g, double eps, float* out,
                    hipStream_t s) {
  if (rows == 0) return 0;
  hipLaunchKernelGGL(k_rms_norm, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, rows, cols, g, eps, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------ repack

__device__ __forceinline__ int q4k_code(const uint8_t* b, int e) {   // exchange Q4_K element
  int g = e >> 6, i = e & 63;
  uint8_t v = b[16 + 32 * g + (i & 31)];
  return i < 32 ? (v & 15) : (v >> 4);
}
__device__ __forceinline__ int q2k_code(const uint8_t* b, int e) {
  int h = e >> 7, r = e & 127, s = r >> 5, i = r & 31;
  return (b[20 + 32 * h + i] >> (2 * s)) & 3;
}
__device__ __forceinline__ int q6k_low4(const uint8_t* b, int e) {
  int h = e >> 7, r = e & 127;
  uint8_t v = b[18 + 64 * h + (r & 63)];
  return r < 64 ? (v & 15) : (v >> 4);
}
__device__ __forceinline__ int q6k_high2(const uint8_t* b, int e) {
  int h = e >> 7, r = e & 127, s = r >> 5, i = r & 31;
  return (b[146 + 32 * h + i] >> (2 * s)) & 3;
}

// exchange Q3_K element: low pair (as Q2_K's quants, after a 14-byte head) and high bit
__device__ __forceinline__ int q3k_low2(const uint8_t* b, int e) {
  int h = e >> 7, r = e & 127, s = r >> 5, i = r & 31;
  return (b[14 + 32 * h + i] >> (2 * s)) & 3;
}
__device__ __forceinline__ int q3k_high(const uint8_t* b, int e) { return (b[78 + (e & 31)] >> (e >> 5)) & 1; }
// six-bit value j of the scale stream starting at p
__device__ __forceinline__ int stream6(const uint8_t* p, int j) {
  int v = 0;
  for (int bit = 0; bit < 6; ++bit) v |= ((p[(6 * j + bit) >> 3] >> ((6 * j + bit) & 7)) & 1) << bit;
  return v;
}
// exchange Q5_K element bit 4 (the plane after the Q4_K bytes)
__device__ __forceinline__ int q5k_high(const uint8_t* b, int e) { return (b[144 + (e & 31)] >> (e >> 5)) & 1; }

__device__ __forceinline__ void st_u32(uint8_t* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }

template <int FMT>
__global__ __launch_bounds__(256) void k_pack(const uint8_t* __restrict__ aos, int64_t n_mats,
                                              int64_t rows, int64_t cols, uint8_t* __restrict__ packed,
                                              size_t mat_bytes, int64_t sb_bytes_aos) {
  const int64_t nb = cols / 256, nsb = rows * nb;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_mats * nsb) return;
  const int64_t mat = gid / nsb, sbi = gid % nsb;
  const uint8_t* src = aos + gid * sb_bytes_aos;   // (mat*rows + r)*nb + s == gid
  uint8_t* m = packed + mat * mat_bytes;
  if (FMT == FQ4K || FMT == FQ5K) {
    for (int j = 0; j < 8; ++j)
      for (int w = 0; w < 4; ++w) {
        uint32_t v = 0;
        for (int bb = 0; bb < 4; ++bb) {
          int b = 4 * w + bb;
          v |= (uint32_t)(q4k_code(src, 32 * j + b) | (q4k_code(src, 32 * j + 16 + b) << 4)) << (8 * bb);
        }
        st_u32(m + sbi * 128 + 16 * j + 4 * w, v);
      }
    uint8_t* ph = m + align256(nsb * 128) + (FMT == FQ5K ? align256(nsb * 32) : 0) + sbi * 16;
    for (int i = 0; i < 16; ++i) ph[i] = src[i];
    if (FMT == FQ5K) {
      uint8_t* px = m + align256(nsb * 128);
      for (int j = 0; j < 8; ++j) {
        uint32_t v = 0;
        for (int w = 0; w < 4; ++w)
          for (int b = 0; b < 4; ++b)
            v |= (uint32_t)(q5k_high(src, 32 * j + 4 * w + b) << (8 * b + w)) |
                 (uint32_t)(q5k_high(src, 32 * j + 16 + 4 * w + b) << (8 * b + 4 + w));
        st_u32(px + sbi * 32 + 4 * (4 * (j & 1) + (j >> 1)), v);
      }
    }
  } else if (FMT == FQ3K) {
    uint8_t* px = m + align256(nsb * 64);
    uint8_t* ps = px + align256(nsb * 32);
    uint8_t* pd = ps + align256(nsb * 16);
    for (int j = 0; j < 8; ++j) {
      for (int t = 0; t < 2; ++t) {
        uint32_t v = 0;
        for (int i = 0; i < 4; ++i)
          for (int b = 0; b < 4; ++b) v |= (uint32_t)q3k_low2(src, 16 * (2 * j + t) + 4 * i + b) << (8 * b + 2 * i);
        st_u32(m + sbi * 64 + 8 * j + 4 * t, v);
      }
      uint32_t v = 0;
      for (int i = 0; i < 8; ++i)
        for (int b = 0; b < 4; ++b) v |= (uint32_t)q3k_high(src, 32 * j + 4 * i + b) << (8 * b + i);
      st_u32(px + sbi * 32 + 4 * j, v);
    }
    for (int j = 0; j < 16; ++j) ps[sbi * 16 + j] = (uint8_t)(int8_t)(stream6(src + 2, j) - 32);
    pd[sbi * 2] = src[0];
    pd[sbi * 2 + 1] = src[1];
  } else if (FMT == FQ6K) {
    uint8_t* px = m + align256(nsb * 128);
    uint8_t* ps = px + align256(nsb * 64);
    uint8_t* pd = ps + align256(nsb * 16);
    for (int j = 0; j < 8; ++j) {
      for (int w = 0; w < 4; ++w) {
        uint32_t v = 0;
        for (int bb = 0; bb < 4; ++bb) {
          int b = 4 * w + bb;
          v |= (uint32_t)(q6k_low4(src, 32 * j + b) | (q6k_low4(src, 32 * j + 16 + b) << 4)) << (8 * bb);
        }
        st_u32(m + sbi * 128 + 16 * j + 4 * w, v);
      }
      for (int a = 0; a < 2; ++a) {
        uint32_t v = 0;
        for (int s = 0; s < 4; ++s)
          for (int b = 0; b < 4; ++b)
            v |= (uint32_t)q6k_high2(src, 32 * j + 4 * (4 * a + s) + b) << (8 * b + 2 * s);
        st_u32(px + sbi * 64 + 8 * j + 4 * a, v);
      }
    }
    for (int i = 0; i < 16; ++i) ps[sbi * 16 + i] = src[2 + i];
    pd[sbi * 2] = src[0];
    pd[sbi * 2 + 1] = src[1];
  } else if (FMT == FQ2K) {
    // tiled (32-row units); see the Q2_K plane description
    const int64_t row = sbi / nb, sb = sbi % nb, u = (row >> 5) * nb + sb;
    const int r = (int)(row & 31);
    uint8_t* U = m + u * kQ2KUnit;
    for (int g = 0; g < 2; ++g)
      for (int p = 0; p < 8; ++p) {
        const int j = 2 * p + g;                // sub-block of step p, half g
        uint32_t v = 0;
        for (int i = 0; i < 4; ++i)
          for (int b = 0; b < 4; ++b) v |= (uint32_t)q2k_code(src, 16 * j + 4 * i + b) << (8 * b + 2 * i);
        st_u32(U + 1024 * (p >> 2) + 16 * (32 * g + r) + 4 * (p & 3), v);
      }
    for (int i = 0; i < 16; ++i) U[kQ2KScales + 16 * r + i] = src[4 + i];
    for (int i = 0; i < 4; ++i) U[kQ2KD + 4 * r + i] = src[i];
  } else if (FMT == FQ40 || FMT == FQ51) {
    // eight 18- or 24-byte blocks per super-block: the quant bytes as they are,
    // Q5_1's bit-4 word rearranged for v_dot4, and the scales
    const int bb = FMT == FQ40 ? 18 : 24, qo = FMT == FQ40 ? 2 : 8;
    uint8_t* p2 = m + align256(nsb * 128);
    for (int b = 0; b < 8; ++b) {
      const uint8_t* blk = src + bb * b;
      for (int i = 0; i < 16; ++i) m[sbi * 128 + 16 * b + i] = blk[qo + i];
      if (FMT == FQ40) {
        p2[sbi * 16 + 2 * b] = blk[0];
        p2[sbi * 16 + 2 * b + 1] = blk[1];
      } else {
        const uint32_t qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) | ((uint32_t)blk[6] << 16) |
                            ((uint32_t)blk[7] << 24);
        uint32_t v = 0;
        for (int w = 0; w < 4; ++w)
          for (int c = 0; c < 4; ++c)
            v |= (((qh >> (4 * w + c)) & 1u) << (8 * c + w)) | (((qh >> (16 + 4 * w + c)) & 1u) << (8 * c + 4 + w));
        st_u32(p2 + sbi * 64 + 8 * b, v);
        for (int i = 0; i < 4; ++i) p2[sbi * 64 + 8 * b + 4 + i] = blk[i];
      }
    }
  } else {  // Q8_0: eight 34-byte blocks per super-block
    uint8_t* pd = m + align256(nsb * 256);
    for (int b = 0; b < 8; ++b) {
      const uint8_t* blk = src + 34 * b;
      for (int i = 0; i < 32; ++i) m[sbi * 256 + 32 * b + i] = blk[2 + i];
      pd[sbi * 16 + 2 * b] = blk[0];
      pd[sbi * 16 + 2 * b + 1] = blk[1];
    }
  }
}

int launch_pack(int fmt, const void* aos, int64_t n_mats, int64_t rows, int64_t cols, void* packed,
                hipStream_t s) {
  const int64_t total = n_mats * rows * (cols / 256);
  if (total == 0) return 0;
  const size_t mb = packed_bytes_of(fmt, rows, cols);
  const unsigned grid = (unsigned)((total + 255) / 256);
  const uint8_t* a = (const uint8_t*)aos;
  uint8_t* p = (uint8_t*)packed;
  switch (fmt) {
    case FQ4K: hipLaunchKernelGGL(k_pack<FQ4K>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)144); break;
    case FQ6K: hipLaunchKernelGGL(k_pack<FQ6K>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)210); break;
    case FQ2K: hipLaunchKernelGGL(k_pack<FQ2K>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)84); break;
    case FQ80: hipLaunchKernelGGL(k_pack<FQ80>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)272); break;
    case FQ3K: hipLaunchKernelGGL(k_pack<FQ3K>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)110); break;
    case FQ5K: hipLaunchKernelGGL(k_pack<FQ5K>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)176); break;
    case FQ40: hipLaunchKernelGGL(k_pack<FQ40>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)144); break;
    case FQ51: hipLaunchKernelGGL(k_pack<FQ51>, dim3(grid), dim3(256), 0, s, a, n_mats, rows, cols, p, mb, (int64_t)192); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// --------------------------------------------------------------- subdots

template <int FMT>
__global__ __launch_bounds__(256) void k_subdots(const uint8_t* __restrict__ w, int64_t rows, int64_t cols,
                                                 const uint8_t* __restrict__ xq, int64_t n_x,
                                                 int32_t* __restrict__ out) {
  using L = Fmt<FMT>;
  const int64_t cpr = cols / L::WPC, nb = cols / 256;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_x * rows * cpr) return;
  const int64_t c = gid % cpr, r = (gid / cpr) % rows, n = gid / (cpr * rows);
  int xw[L::XDW], bs[L::NBS], is[L::SPC];
  double dx;
  load_x_chunk<FMT>(xq + n * nb * kQ8KBytes, (int)c, xw, bs, dx);
  typename L::W wv = L::load(w, rows, nb, r, c / L::CPS, (int)(c % L::CPS));
  L::isums(wv, xw, bs, is);
  // sub-block order of the row (a chunk's sub-blocks need not be adjacent)
  for (int i = 0; i < L::SPC; ++i)
    out[(n * rows + r) * (cpr * L::SPC) + (c / L::CPS) * (L::CPS * L::SPC) + L::sub_of((int)(c % L::CPS), i)] = is[i];
}

int launch_subdots(int fmt, const void* w, int64_t rows, int64_t cols, const void* xq, int64_t n_x,
                   int32_t* out, hipStream_t s) {
  const Geo g = geo_of(fmt);
  const int64_t total = n_x * rows * (cols / g.wpc);
  if (total == 0) return 0;
  const unsigned grid = (unsigned)((total + 255) / 256);
  const uint8_t* W = (const uint8_t*)w;
  const uint8_t* X = (const uint8_t*)xq;
  switch (fmt) {
    case FQ4K: hipLaunchKernelGGL(k_subdots<FQ4K>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ6K: hipLaunchKernelGGL(k_subdots<FQ6K>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ2K: hipLaunchKernelGGL(k_subdots<FQ2K>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ80: hipLaunchKernelGGL(k_subdots<FQ80>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ3K: hipLaunchKernelGGL(k_subdots<FQ3K>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ5K: hipLaunchKernelGGL(k_subdots<FQ5K>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ40: hipLaunchKernelGGL(k_subdots<FQ40>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    case FQ51: hipLaunchKernelGGL(k_subdots<FQ51>, dim3(grid), dim3(256), 0, s, W, rows, cols, X, n_x, out); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
