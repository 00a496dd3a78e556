// Packed (kernel-side) layouts of the quantised weight formats, their per-lane
// dot routines and the exchange->packed repack.
//
// A packed matrix of nsb = rows * cols/256 super-blocks is a set of planes, each
// contiguous over super-blocks in row-major order and 256-byte aligned.  A wave
// lane works on one "chunk" of a super-block: 16 contiguous bytes of the main
// quant plane, so a wave reads 1 KiB of quants per load instruction, fully
// coalesced.  The element order inside a chunk is chosen so that one 32-bit
// word, after a mask or a shift, holds four consecutive elements of one
// sub-block, matching four consecutive q8_K bytes of the activation: one
// v_dot4_i32_i8.
//
//   Q4_K  plane Q 128 B/sb: chunk j (sub-block j, 32 elements), byte b =
//           elem 32j+b (low nibble) | elem 32j+16+b (high nibble)
//         plane H  16 B/sb: the exchange header as is (d, dmin, 12 B scales)
//   Q6_K  plane L 128 B/sb: chunk j (elements 32j..32j+31, sub-blocks 2j, 2j+1),
//           byte b = low4(32j+b) | low4(32j+16+b) << 4
//         plane X  64 B/sb: chunk j = 2 words; word a, byte b, bits 2s..2s+1 =
//           high2(elem 32j + 4(4a+s) + b)
//         plane S  16 B/sb: int8 scales;  plane D 2 B/sb: fp16 d
//   Q2_K  tiled: unit u = (row / 32) * nb + sb (32 rows x one super-block),
//         2688 contiguous bytes at 2688 u, so a wave reading the 32 rows of a
//         unit reads whole lines of one stretch (and the matrix-core tiles
//         read it with every load instruction contiguous); inside the unit:
//         codes 2048 B: 16 B at 1024 k + 16 (32 g + row % 32) = the words of
//           steps 4k..4k+3 of half g; step p of half g is sub-block 2p + g,
//           its word holds element 4i + b of the sub-block at bits 8b + 2i.
//           A lane chunk j = 2k + g is that 16 B piece: sub-blocks
//           8k + g + 2t, t = 0..3
//         scales 512 B at 2048: the row's 16 bytes (sc | m << 4) at 16 (row % 32)
//         d 128 B at 2560: d, dmin at 4 (row % 32)
//   Q8_0  plane Q 256 B/sb: chunk b = the 32 int8 quants of block b
//         plane D  16 B/sb: eight fp16 d
//   Q3_K  plane L  64 B/sb: chunk j = 2 words; word t = sub-block 2j+t, bits
//           8b+2i = low pair of its element 4i+b
//         plane X  32 B/sb: chunk j = 1 word, bit 8b+i = high bit of chunk
//           element 4i+b (i = 0..7)
//         plane S  16 B/sb: int8 scales (sc_j, the stored value - 32);
//         plane D 2 B/sb: fp16 d
//   Q5_K  plane Q 128 B/sb: Q4_K's, on the low nibbles
//         plane X  32 B/sb: one word per chunk j, at word 4 (j % 2) + j / 2 (the
//           even chunks first: a matrix-core lane half reads its four words
//           at once); bits 8b+i / 8b+4+i = bit 4 of chunk elements 4i+b /
//           16+4i+b (the two nibbles of word i, byte b)
//         plane H  16 B/sb: the exchange header as is (d, dmin, 12 B scales)
//   Q4_0  plane Q 128 B/sb: chunk b = the 16 quant bytes of 32-block b as is
//           (byte i = element i low nibble, element 16+i high nibble)
//         plane D  16 B/sb: eight fp16 d
//   Q5_1  plane Q 128 B/sb: as Q4_0
//         plane XD 64 B/sb: two words per block: the bit-4 word (bits 8b+i /
//           8b+4+i = bit 4 of block elements 4i+b / 16+4i+b, as a Q5_K
//           chunk's word), then fp16 d | fp16 m << 16
#pragma once
#include "common.hpp"

namespace moeq {

template <int FMT> struct Fmt;

// Q2_K unit: 32 rows x one super-block (codes, then scales, then d)
constexpr int kQ2KUnit = 2688, kQ2KScales = 2048, kQ2KD = 2560;

// Host-side geometry shared by every format.
struct Geo {
  int wpc;          // weights per lane chunk
  int nplanes;
  int pb[4];        // bytes per super-block of each plane
  int tile;         // rows per layout unit (the row count is padded to it)
};

__host__ __device__ inline Geo geo_of(int fmt) {
  switch (fmt) {
    case FQ4K: return Geo{32, 2, {128, 16, 0, 0}, 1};
    case FQ6K: return Geo{32, 4, {128, 64, 16, 2}, 1};
    case FQ2K: return Geo{64, 1, {84, 0, 0, 0}, 32};   // one plane of 2688-byte units
    case FQ80: return Geo{32, 2, {256, 16, 0, 0}, 1};
    case FQ3K: return Geo{32, 4, {64, 32, 16, 2}, 1};
    case FQ5K: return Geo{32, 3, {128, 32, 16, 0}, 1};
    case FQ40: return Geo{32, 2, {128, 16, 0, 0}, 1};
    case FQ51: return Geo{32, 2, {128, 64, 0, 0}, 1};
  }
  return Geo{0, 0, {0, 0, 0, 0}, 1};
}

__host__ __device__ inline size_t packed_bytes_of(int fmt, int64_t rows, int64_t cols) {
  Geo g = geo_of(fmt);
  const int64_t prow = (rows + g.tile - 1) / g.tile * g.tile;
  size_t nsb = (size_t)prow * (size_t)(cols / 256), tot = 0;
  for (int p = 0; p < g.nplanes; ++p) tot += align256(nsb * g.pb[p]);
  return tot;
}

// ---------------------------------------------------------------- Q4_K
// Every format: load(m, rows, nb, row, sb, j) reads lane chunk j of super-block
// sb of a row; chunk j covers sub-blocks sub_of(j, t); its activation dword i
// sits at byte xoff(j, i) of the q8_K block and its block sum t at bsidx(j, t).
// Row-major formats: chunk j is elements j*WPC .. (j+1)*WPC - 1.
template <int WPC_> struct RowMajor {
  __device__ static constexpr int xoff(int j, int i) { return j * WPC_ + 4 * i; }
  __device__ static constexpr int bsidx(int j, int t) { return ((j * WPC_) >> 4) + t; }
};

template <> struct Fmt<FQ4K> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 1;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 q; uint4 h; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int j) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    W w;
    w.q = gld_u4(m + sbi * 128 + 16 * j);
    w.h = gld_u4(m + align256(nsb * 128) + sbi * 16);
    return w;
  }
  __device__ static void isums(const W& w, const int* xw, const int*, int* is) {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = dot4((int)(q[i] & 0x0F0F0F0Fu), xw[i], s);
      s = dot4((int)((q[i] >> 4) & 0x0F0F0F0Fu), xw[4 + i], s);
    }
    is[0] = s;
  }
  __device__ static double term(const W& w, int j, const int* is, const int* bs, double dx) {
    uint64_t lo = (uint64_t)w.h.y | ((uint64_t)w.h.z << 32);   // stream bits 0..63
    uint64_t hi = (uint64_t)w.h.z | ((uint64_t)w.h.w << 32);   // stream bits 32..95
    int sc = (int)((lo >> (6 * j)) & 63);
    int mn = (int)((hi >> (16 + 6 * j)) & 63);
    double d = half_bits_to_float(w.h.x & 0xFFFF), dmin = half_bits_to_float(w.h.x >> 16);
    int s1 = sc * is[0], s2 = mn * (bs[0] + bs[1]);
    return dx * (d * (double)s1 - dmin * (double)s2);
  }
};

// ---------------------------------------------------------------- Q6_K
template <> struct Fmt<FQ6K> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 2;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 l; uint2 x; uint32_t sc; uint32_t d; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int j) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    W w;
    const uint8_t* px = m + align256(nsb * 128);
    const uint8_t* ps = px + align256(nsb * 64);
    const uint8_t* pd = ps + align256(nsb * 16);
    w.l = gld_u4(m + sbi * 128 + 16 * j);
    w.x = gld_u2(px + sbi * 64 + 8 * j);
    w.sc = gld_u16(ps + sbi * 16 + 2 * j);
    w.d = gld_u16(pd + sbi * 2);
    return w;
  }
  __device__ static void isums(const W& w, const int* xw, const int* bs, int* is) {
    const uint32_t l[4] = {w.l.x, w.l.y, w.l.z, w.l.w};
    int a = 0, b = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t ha = ((w.x.x >> (2 * i)) & 0x03030303u) << 4;
      uint32_t hb = ((w.x.y >> (2 * i)) & 0x03030303u) << 4;
      a = dot4((int)((l[i] & 0x0F0F0F0Fu) | ha), xw[i], a);
      b = dot4((int)(((l[i] >> 4) & 0x0F0F0F0Fu) | hb), xw[4 + i], b);
    }
    is[0] = a - 32 * bs[0];   // sum (q - 32) q_x = sum q q_x - 32 sum q_x
    is[1] = b - 32 * bs[1];
  }
  __device__ static double term(const W& w, int, const int* is, const int*, double dx) {
    int sa = (int)(int8_t)(w.sc & 0xFF), sb = (int)(int8_t)(w.sc >> 8);
    int s1 = sa * is[0] + sb * is[1];
    double d = half_bits_to_float(w.d);
    return dx * (d * (double)s1);
  }
};

// ---------------------------------------------------------------- Q2_K
template <> struct Fmt<FQ2K> {
  static constexpr int WPC = 64, CPS = 4, XDW = 16, NBS = 4, SPC = 4;
  __device__ static constexpr int sub_of(int j, int t) { return 8 * (j >> 1) + (j & 1) + 2 * t; }
  __device__ static constexpr int xoff(int j, int i) { return 16 * sub_of(j, i >> 2) + 4 * (i & 3); }
  __device__ static constexpr int bsidx(int j, int t) { return sub_of(j, t); }
  struct W { uint4 q; uint2 sm; uint32_t dd; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int j) {
    const int64_t u = (row >> 5) * nb + sb;
    const int r = (int)(row & 31);
    const uint8_t* U = m + u * kQ2KUnit;
    W w;
    w.q = gld_u4(U + 1024 * (j >> 1) + 16 * (32 * (j & 1) + r));
    w.sm = gld_u2(U + kQ2KScales + 16 * r + 8 * (j >> 1));
    w.dd = gld_u32(U + kQ2KD + 4 * r);
    return w;
  }
  // word t: sub-block sub_of(j, t); element 4i + b at bits 8b + 2i
  __device__ static void isums(const W& w, const int* xw, const int*, int* is) {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      int acc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot4((int)((q[t] >> (2 * i)) & 0x03030303u), xw[4 * t + i], acc);
      is[t] = acc;
    }
  }
  __device__ static double term(const W& w, int j, const int* is, const int* bs, double dx) {
    int s1 = 0, s2 = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int byte = (j & 1) + 2 * t;                 // sub-block byte inside the 8 loaded
      const uint32_t v = ((t < 2 ? w.sm.x : w.sm.y) >> (8 * (byte & 3))) & 0xFF;
      s1 += (int)(v & 15) * is[t];
      s2 += (int)(v >> 4) * bs[t];
    }
    double d = half_bits_to_float(w.dd & 0xFFFF), dmin = half_bits_to_float(w.dd >> 16);
    return dx * (d * (double)s1 - dmin * (double)s2);
  }
};

// ---------------------------------------------------------------- Q8_0
template <> struct Fmt<FQ80> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 1;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 q0, q1; uint32_t d; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int b) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    W w;
    const uint8_t* pd = m + align256(nsb * 256);
    w.q0 = gld_u4(m + sbi * 256 + 32 * b);
    w.q1 = gld_u4(m + sbi * 256 + 32 * b + 16);
    w.d = gld_u16(pd + sbi * 16 + 2 * b);
    return w;
  }
  __device__ static void isums(const W& w, const int* xw, const int*, int* is) {
    const uint32_t q[8] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w, w.q1.x, w.q1.y, w.q1.z, w.q1.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4((int)q[i], xw[i], s);
    is[0] = s;
  }
  __device__ static double term(const W& w, int, const int* is, const int*, double dx) {
    double d = half_bits_to_float(w.d);
    return dx * (d * (double)is[0]);
  }
};

// ---------------------------------------------------------------- Q3_K
template <> struct Fmt<FQ3K> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 2;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint2 l; uint32_t x; uint32_t sc; uint32_t d; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int j) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    const uint8_t* px = m + align256(nsb * 64);
    const uint8_t* ps = px + align256(nsb * 32);
    const uint8_t* pd = ps + align256(nsb * 16);
    W w;
    w.l = gld_u2(m + sbi * 64 + 8 * j);
    w.x = gld_u32(px + sbi * 32 + 4 * j);
    w.sc = gld_u16(ps + sbi * 16 + 2 * j);
    w.d = gld_u16(pd + sbi * 2);
    return w;
  }
  // q = low pair | high bit << 2 (0..7), four elements per word
  __device__ static void isums(const W& w, const int* xw, const int* bs, int* is) {
    const uint32_t l[2] = {w.l.x, w.l.y};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int a = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = ((l[t] >> (2 * i)) & 0x03030303u) | (((w.x >> (4 * t + i)) & 0x01010101u) << 2);
        a = dot4((int)q, xw[4 * t + i], a);
      }
      is[t] = a - 4 * bs[t];   // sum (q - 4) q_x
    }
  }
  __device__ static double term(const W& w, int, const int* is, const int*, double dx) {
    const int sa = (int)(int8_t)(w.sc & 0xFF), sb = (int)(int8_t)(w.sc >> 8);
    const double d = half_bits_to_float(w.d);
    return dx * (d * (double)(sa * is[0] + sb * is[1]));
  }
};

// ---------------------------------------------------------------- Q5_K
template <> struct Fmt<FQ5K> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 1;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 q; uint32_t x; uint4 h; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int j) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    const uint8_t* px = m + align256(nsb * 128);
    const uint8_t* ph = px + align256(nsb * 32);
    W w;
    w.q = gld_u4(m + sbi * 128 + 16 * j);
    w.x = gld_u32(px + sbi * 32 + 4 * (4 * (j & 1) + (j >> 1)));
    w.h = gld_u4(ph + sbi * 16);
    return w;
  }
  // q = nibble | bit 4 (0..31)
  __device__ static void isums(const W& w, const int* xw, const int*, int* is) {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (q[i] & 0x0F0F0F0Fu) | (((w.x >> i) & 0x01010101u) << 4);
      const uint32_t hi = ((q[i] >> 4) & 0x0F0F0F0Fu) | (((w.x >> (4 + i)) & 0x01010101u) << 4);
      s = dot4((int)lo, xw[i], s);
      s = dot4((int)hi, xw[4 + i], s);
    }
    is[0] = s;
  }
  __device__ static double term(const W& w, int j, const int* is, const int* bs, double dx) {
    const uint64_t lo = (uint64_t)w.h.y | ((uint64_t)w.h.z << 32);
    const uint64_t hi = (uint64_t)w.h.z | ((uint64_t)w.h.w << 32);
    const int sc = (int)((lo >> (6 * j)) & 63);
    const int mn = (int)((hi >> (16 + 6 * j)) & 63);
    const double d = half_bits_to_float(w.h.x & 0xFFFF), dmin = half_bits_to_float(w.h.x >> 16);
    return dx * (d * (double)(sc * is[0]) - dmin * (double)(mn * (bs[0] + bs[1])));
  }
};

// ---------------------------------------------------------------- Q4_0
template <> struct Fmt<FQ40> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 1;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 q; uint32_t d; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int b) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    W w;
    w.q = gld_u4(m + sbi * 128 + 16 * b);
    w.d = gld_u16(m + align256(nsb * 128) + sbi * 16 + 2 * b);
    return w;
  }
  // sum (q - 8) q_x = sum q q_x - 8 (the block's activation sum)
  __device__ static void isums(const W& w, const int* xw, const int* bs, int* is) {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = dot4((int)(q[i] & 0x0F0F0F0Fu), xw[i], s);
      s = dot4((int)((q[i] >> 4) & 0x0F0F0F0Fu), xw[4 + i], s);
    }
    is[0] = s - 8 * (bs[0] + bs[1]);
  }
  __device__ static double term(const W& w, int, const int* is, const int*, double dx) {
    return dx * (half_bits_to_float(w.d) * (double)is[0]);
  }
};

// ---------------------------------------------------------------- Q5_1
template <> struct Fmt<FQ51> : RowMajor<32> {
  static constexpr int WPC = 32, CPS = 8, XDW = 8, NBS = 2, SPC = 1;
  __device__ static constexpr int sub_of(int j, int t) { return j * SPC + t; }
  struct W { uint4 q; uint32_t x; uint32_t dm; };
  __device__ static W load(const uint8_t* m, int64_t rows, int64_t nb, int64_t row, int64_t sb, int b) {
    const size_t nsb = (size_t)(rows * nb), sbi = (size_t)(row * nb + sb);
    W w;
    w.q = gld_u4(m + sbi * 128 + 16 * b);
    const uint2 xd = gld_u2(m + align256(nsb * 128) + sbi * 64 + 8 * b);
    w.x = xd.x;
    w.dm = xd.y;
    return w;
  }
  // q = nibble | bit 4 (0..31)
  __device__ static void isums(const W& w, const int* xw, const int*, int* is) {
    const uint32_t q[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (q[i] & 0x0F0F0F0Fu) | (((w.x >> i) & 0x01010101u) << 4);
      const uint32_t hi = ((q[i] >> 4) & 0x0F0F0F0Fu) | (((w.x >> (4 + i)) & 0x01010101u) << 4);
      s = dot4((int)lo, xw[i], s);
      s = dot4((int)hi, xw[4 + i], s);
    }
    is[0] = s;
  }
  // d q + m summed against the block: d isum + m bsum
  __device__ static double term(const W& w, int, const int* is, const int* bs, double dx) {
    const double d = half_bits_to_float(w.dm & 0xFFFF), mn = half_bits_to_float(w.dm >> 16);
    return dx * (d * (double)is[0] + mn * (double)(bs[0] + bs[1]));
  }
};

// Element positions inside a lane chunk, in x-word order: word i of a chunk
// holds chunk elements xoff(i)..xoff(i)+3.  For every format here the x words
// are simply the chunk's elements in order (4 per word).

// Load the activation side of one chunk from a q8_K row.
template <int FMT>
__device__ __forceinline__ void load_x_chunk(const uint8_t* xrow, int c, int* xw, int* bs, double& dx) {
  using L = Fmt<FMT>;
  const int j = c % L::CPS;
  const uint8_t* blk = xrow + (size_t)(c / L::CPS) * kQ8KBytes;
  dx = (double)gld_f32(blk);
#pragma unroll
  for (int i = 0; i < L::XDW; ++i) xw[i] = (int)gld_u32(blk + 4 + L::xoff(j, i));
#pragma unroll
  for (int t = 0; t < L::NBS; ++t) bs[t] = (int)(int16_t)gld_u16(blk + 260 + 2 * L::bsidx(j, t));
}

}  // namespace moeq
