// int8 MFMA grouped GEMM for the experts of multi-token calls (verify unions,
// chunks, prefill).  The pages run multi-token work on int8 matrix units with
// the weights kept quantized instead of per-row dot products (Pulsar README,
// 'What it does today', prefill paragraphs: dense int8 GEMM plus a grouped
// MoE that unpacks each expert super-block once per chunk; Strata article,
// long-prompt section: quantized MMQ expert kernels beat expanding to FP16;
// the MoE verify unions already take the int8-MMA path: Pulsar README,
// ThinkingCap paragraph), while a single token stays on the dot-product path.
//
// Tile = one expert x 32 of its rows (tokens, or pairs for down) x 256 weight
// rows: a 512-thread workgroup of 8 waves, each wave 32 weight rows.  The
// activation side (q8_K rows of the tile, one 256-block at a time) is staged
// in LDS once and shared by the 8 waves; each wave reads its weights straight
// from HBM into registers (each weight byte is read once per tile).
//
// MFMA roles: C[m = token][n = weight row] = sum_k A[m][k] * B[k][n] with
// v_mfma_i32_32x32x32_i8, so a lane's 16 results share one weight row
// (n = lane % 32) and its per-row scales stay in that lane.  Lane l holds
// K bytes 16*(l/32) .. +15 of both operands, the same assignment on both
// sides, so only the output layout is fixed by the hardware: lane l, value r
// is C[8*(r/4) + 4*(l/32) + r%4][l%32].
//
// Exactness per super-block (the integer parts of the dequant-dot are exact,
// the combine is fp64):
//   Q4_K  w = d*sc_j*q - dmin*m_j, sc, m < 64, q < 16.  sc*q does not fit in
//         int8, so sc = 8*sh + sl (sh, sl < 8) and two exact int32 sums run
//         over the whole super-block on pre-scaled weights q*sl, q*sh (< 106):
//         S1 = sum_j sc_j isum_j = P_lo + 8*P_hi.
//   Q2_K  w = d*sc_j*q - dmin*m_j, sc*q < 46: one sum on q*sc.
//   Min term S2 = sum_j m_j * bsum_j(x): each block sum is split as
//         64*bh + bl (bl < 64, |bh| <= 64) so one MFMA over [bl | bh] against
//         [m | 0] and one against [0 | m] give S2 = X_l + 64*X_h exactly.
//   Q6_K  w = d*sc_j*(q-32), signed 8-bit sc: one 16-deep MFMA per sub-block
//         (exact int32 dot of q with x), scaled by sc_j in int32; the -32 part
//         is 32 * sum_j sc_j bsum_j, from the same split-sum MFMA pair.
//   Q8_0  w = d_b*q: one MFMA per 32-block, scaled by d_b in fp64.
//   Q4_0  w = d_b*(q-8): as Q8_0 on the bytes q - 8.
//   Q5_1  w = d_b*q + m_b: as Q8_0 on the bytes q, plus one MFMA of the
//         activations against ones for the block sum the min multiplies.
//   Q3_K  w = d*sc_j*(q-4), signed six-bit sc, q < 8: as Q6_K (sc*q does not
//         fit in int8): one 16-deep MFMA per sub-block on the codes q, scaled
//         by sc_j in int32; the -4 part is 4 * sum_j sc_j bsum_j.
//   Q5_K  w = d*sc_j*q - dmin*m_j, q = l + 16h < 32: Q4_K's two pre-scaled
//         sums on the nibbles l plus a third on h*sc_j (< 64), chained on one
//         accumulator: S1 = 8*(2*P_h + P_hi) + P_lo; the min term as Q4_K's.
// term per super-block = d_x * (d * S1 - dmin * S2) in fp64, summed over the
// super-blocks in order; h = fl32(silu(g) * u); y rows in fp32.
#include <type_traits>

#include "formats.hpp"
#include "mfma_plan.hpp"
#include "launch.hpp"
#include "route_small.hpp"

namespace moeq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMfWaves = 8;        // waves per workgroup, 32 weight rows each
constexpr int kMfRows = 32 * kMfWaves;
constexpr int kQsStride = 272;     // LDS bytes per staged row: 256 + 16 (bank spread)

template <int TM>
struct __align__(16) StageLds {
  uint8_t qs[TM][kQsStride];       // q8_K quants of the tile rows, one 256-block
  uint8_t bsp[TM][2][16];          // split block sums: [0] = bl entries, [1] = bh entries
  double dx[TM];                   // q8_K scales (widened once here, not per unit)
};

__device__ __forceinline__ v16i mfma_k32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16i mfma_k16(long a, long b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, c, 0, 0, 0);
}

// Four packed bytes times a small factor s: every byte product stays below
// 256, so two bytes per 16-bit half multiply without carries (v_pk_mul_lo_u16).
__device__ __forceinline__ uint32_t bytes_times(uint32_t v, uint32_t s) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 a = __builtin_bit_cast(u16x2, v);
  const u16x2 b = (u16x2)((unsigned short)s);   // splat: the multiply reads s's low half twice (op_sel)
  return __builtin_bit_cast(uint32_t, a * b);
}

// A fragments come from LDS unconditionally: a lane whose tile row lies beyond
// the staged rows reads a zero row instead (no per-step branch or zeroing).
__device__ __forceinline__ v4i lds_v4(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// Token row m of the lane's results for value r.
__device__ __forceinline__ int out_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// fp64 combine over the lane's results: value r = 4q+i is tile row 8q + 4g + i,
// whose scale is dxs[8q+4g+i]; only the first NQ groups of 8 rows exist in the
// stage (NQ = 4 for 32-row tiles, 1 for 8-row tiles) and groups past the
// tile's n rows are skipped (uniform over the wave).
#define MOEQ_COMBINE(STMT)                                                            \
  _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                   \
    if (8 * q < n) {                                                                  \
      const double2 d01 = *reinterpret_cast<const double2*>(dxs + 8 * q + 4 * g);     \
      const double2 d23 = *reinterpret_cast<const double2*>(dxs + 8 * q + 4 * g + 2); \
      const double dxa[4] = {d01.x, d01.y, d23.x, d23.y};                            \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                \
        const int r = 4 * q + i;                                                      \
        const double dx = dxa[i];                                                     \
        STMT;                                                                         \
      }                                                                               \
    }                                                                                 \
  }

// ------------------------------------------------------------ per-format W side
//
// A trait per weight format:
//   NBSP      entries of the split block sums the min / offset term needs (0: none)
//   Wt        the weight registers of one lane for one super-block
//   load      global loads of lane (row, half g) for super-block sbi
//   mac       MFMAs and the fp64 combine into acc[16]; A fragments from LDS

template <int FMT> struct Mf;

// A wave's 32 weight rows start at a multiple of 32 (lane row r = row % 32),
// so row / 32 is the same in every lane: the (row group, super-block) part of
// an address is put in scalar registers, and each load takes that scalar base
// plus a 32-bit lane offset that never changes (no 64-bit address arithmetic
// per lane and load).
__device__ __forceinline__ int64_t wave_uni(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const uint8_t* wave_uni_ptr(const uint8_t* p) {
  return reinterpret_cast<const uint8_t*>(wave_uni(reinterpret_cast<int64_t>(p)));
}
// super-block index of (row group, sb) of a row-major matrix, and the lane row
struct RowSplit {
  int64_t su;      // (row & ~31) * nbK + sb, the same in every lane
  uint32_t r;      // row & 31
};
__device__ __forceinline__ RowSplit row_split(int64_t row, int64_t nbK, int64_t sb) {
  return RowSplit{wave_uni(row >> 5) * 32 * nbK + sb, (uint32_t)row & 31u};
}

template <> struct Mf<FQ4K> {
  static constexpr int NBSP = 8;   // one sum per 32-sub-block: bsums[2j] + bsums[2j+1]
  struct Wt { uint4 c[4]; uint4 h; };
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int g) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;              // lane super-block offset
    const uint8_t* Wb = wave_uni_ptr(W);
    const uint8_t* qb = Wb + rs.su * 128;
    const uint8_t* hb = Wb + align256(nsb * 128) + rs.su * 16;
    Wt w;
#pragma unroll
    for (int p = 0; p < 4; ++p) w.c[p] = gld_u4(qb + (lr * 128u + 16u * (uint32_t)(2 * p + g)));
    w.h = gld_u4(hb + lr * 16u);
    return w;
  }
  // The exact integer parts of the super-block term for the lane's 16 results:
  // s1 = sum_j sc_j isum_j, s2 = sum_j m_j bsum_j.
  // MFMA 2p+s: lane half g holds sub-block 2p+g, nibble s (elements 64p+32g+16s .. +15).
  struct Ints { v16i s1, s2; };
  __device__ __forceinline__ static Ints ints(const Wt& w, int g, const uint8_t* qrow, const v4i abs) {
    const uint64_t lo = (uint64_t)w.h.y | ((uint64_t)w.h.z << 32);
    const uint64_t hi = (uint64_t)w.h.z | ((uint64_t)w.h.w << 32);
    v16i plo = {0}, phi = {0};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t sc = (uint32_t)(lo >> (6 * (2 * p + g))) & 63;
      const uint32_t c[4] = {w.c[p].x, w.c[p].y, w.c[p].z, w.c[p].w};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4i bl, bh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t q = (c[i] >> (4 * s)) & 0x0F0F0F0Fu;
          bl[i] = (int)bytes_times(q, sc & 7);
          bh[i] = (int)bytes_times(q, sc >> 3);
        }
        const v4i a = lds_v4(qrow + 64 * p + 32 * g + 16 * s);
        plo = mfma_k32(a, bl, plo);
        phi = mfma_k32(a, bh, phi);
      }
    }
    // min term: bytes m_0..m_7 of this row against the split block sums
    uint32_t m0 = 0, m1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m0 |= (uint32_t)((hi >> (16 + 6 * j)) & 63) << (8 * j);
      m1 |= (uint32_t)((hi >> (16 + 6 * (j + 4))) & 63) << (8 * j);
    }
    const v4i bm = {(int)m0, (int)m1, 0, 0}, zero = {0, 0, 0, 0};
    const v16i z16 = {0};
    const v16i xl = mfma_k32(abs, g == 0 ? bm : zero, z16);
    const v16i xh = mfma_k32(abs, g == 1 ? bm : zero, z16);
    return Ints{plo + 8 * phi, xl + 64 * xh};
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i abs, const double* dxs,
                             int n, double* acc) {
    const Ints I = ints(w, g, qrow, abs);
    const double d = half_bits_to_float(w.h.x & 0xFFFF), dmin = half_bits_to_float(w.h.x >> 16);
    MOEQ_COMBINE(acc[r] += dx * (d * (double)I.s1[r] - dmin * (double)I.s2[r]))
  }
};

template <> struct Mf<FQ2K> {
  static constexpr int NBSP = 16;  // one sum per 16-sub-block: bsums[j]
  struct Wt { uint4 c[2]; uint4 sm; uint32_t dd; };
  // Tiled layout (2688-byte 32-row units): lane (half g, row r) reads the two
  // 16 B pieces of its half, each load instruction covering 1 KB contiguously,
  // then the row's scales and d from the same unit.
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int g) {
    const int64_t u = wave_uni(row >> 5) * nbK + sb;
    const uint32_t r = (uint32_t)row & 31u;
    const uint8_t* cb = wave_uni_ptr(W) + u * kQ2KUnit;   // the unit: codes, scales, d
    Wt w;
#pragma unroll
    for (int k = 0; k < 2; ++k) w.c[k] = gld_u4(cb + (1024u * (uint32_t)k + 16u * (32u * (uint32_t)g + r)));
    w.sm = gld_u4(cb + ((uint32_t)kQ2KScales + 16u * r));
    w.dd = gld_u32(cb + ((uint32_t)kQ2KD + 4u * r));
    return w;
  }
  // The exact integer parts of the super-block term: s1 = sum_j sc_j isum_j,
  // s2 = sum_j m_j bsum_j.
  // MFMA p: lane half g holds sub-block 2p+g (elements 32p+16g .. +15), whose
  // 16 codes are word p of the half: element 4i + b at bits 8b + 2i.
  struct Ints { v16i s1, s2; };
  __device__ __forceinline__ static Ints ints(const Wt& w, int g, const uint8_t* qrow, const v4i abs) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t sm[4] = {w.sm.x, w.sm.y, w.sm.z, w.sm.w};
    v16i P = {0};
    const uint32_t words[8] = {w.c[0].x, w.c[0].y, w.c[0].z, w.c[0].w, w.c[1].x, w.c[1].y, w.c[1].z, w.c[1].w};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // sub-block j = 2p+g: byte 2(p&1)+g of word p/2, so steps 2q and 2q+1
      // take the two 16-bit halves of one shift and mask (op_sel picks the half)
      const u16x2 pair = __builtin_bit_cast(u16x2, (sm[p >> 1] >> (8 * g)) & 0x000F000Fu);
      const u16x2 scv = (p & 1) ? pair.yy : pair.xx;
      v4i b;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b[i] = (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, (words[p] >> (2 * i)) & 0x03030303u) * scv);
      P = mfma_k32(lds_v4(qrow + 32 * p + 16 * g), b, P);
    }
    v4i bm;
#pragma unroll
    for (int i = 0; i < 4; ++i) bm[i] = (int)((sm[i] >> 4) & 0x0F0F0F0Fu);
    const v4i zero = {0, 0, 0, 0};
    const v16i z16 = {0};
    const v16i xl = mfma_k32(abs, g == 0 ? bm : zero, z16);
    const v16i xh = mfma_k32(abs, g == 1 ? bm : zero, z16);
    return Ints{P, xl + 64 * xh};
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i abs, const double* dxs,
                             int n, double* acc) {
    const Ints I = ints(w, g, qrow, abs);
    const double d = half_bits_to_float(w.dd & 0xFFFF), dmin = half_bits_to_float(w.dd >> 16);
    MOEQ_COMBINE(acc[r] += dx * (d * (double)I.s1[r] - dmin * (double)I.s2[r]))
  }
};

template <> struct Mf<FQ6K> {
  static constexpr int NBSP = 16;
  struct Wt { uint2 l[8]; uint4 x[4]; uint4 sc; uint32_t d; };
  // Lane half g needs words 2g, 2g+1 of every low-nibble chunk and all of the
  // high-pair row.
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int g) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    Wt w;
    const uint8_t* px = Wb + align256(nsb * 128);
    const uint8_t* ps = px + align256(nsb * 64);
    const uint8_t* pd = ps + align256(nsb * 16);
    const uint8_t* lb = Wb + rs.su * 128;
    const uint8_t* xb = px + rs.su * 64;
#pragma unroll
    for (int j = 0; j < 8; ++j) w.l[j] = gld_u2(lb + (lr * 128u + 16u * (uint32_t)j + 8u * (uint32_t)g));
#pragma unroll
    for (int j = 0; j < 4; ++j) w.x[j] = gld_u4(xb + (lr * 64u + 16u * (uint32_t)j));
    w.sc = gld_u4(ps + rs.su * 16 + lr * 16u);
    w.d = gld_u16(pd + rs.su * 2 + lr * 2u);
    return w;
  }
  // The MFMA part of the super-block term: S1[r] = sum_j sc_j (sum q q_x)
  // with the unsigned codes q, and the offset sum xl + 64 xh = sum_j sc_j bsum_j.
  // One 16-deep MFMA per sub-block jj: lane half g holds elements 16jj+8g .. +7
  // (low nibbles: word i = 2g+t of chunk jj/2, nibble jj%2; high pairs: word
  // jj%2 of chunk jj/2 in the high-pair plane, bits 2i).
  __device__ __forceinline__ static v16i sub_mfma(const Wt& w, int g, const uint8_t* qrow, int jj) {
    const int j = jj >> 1, s = jj & 1;
    const uint32_t l2[2] = {w.l[j].x, w.l[j].y};
    const uint4 xv = w.x[j >> 1];
    const uint32_t xs = (j & 1) ? (s ? xv.w : xv.z) : (s ? xv.y : xv.x);
    uint32_t q[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = 2 * g + t;
      q[t] = ((l2[t] >> (4 * s)) & 0x0F0F0F0Fu) | (((xs >> (2 * i)) & 0x03030303u) << 4);
    }
    const long b = (long)(((uint64_t)q[1] << 32) | q[0]);
    const long a = *reinterpret_cast<const long*>(qrow + 16 * jj + 8 * g);
    const v16i z16 = {0};
    return mfma_k16(a, b, z16);
  }
  // Two-deep pipeline over the sub-blocks: the MFMA of sub-block jj + 1 is
  // issued before the result of jj is scaled.  An empty asm statement that
  // takes the running sums and clobbers memory ends each step: the next
  // step's LDS operand load (and so its MFMA) cannot move above it, and the
  // scaling must be done before it.  Without it the compiler issued all 16
  // MFMAs first and kept every result live (16 registers each), which spilled
  // the 32-row tiles to scratch.
  __device__ __forceinline__ static void raw(const Wt& w, int g, const uint8_t* qrow, const v4i abs, int* S1,
                                             v16i& xl, v16i& xh) {
    const uint32_t scw[4] = {w.sc.x, w.sc.y, w.sc.z, w.sc.w};
    v16i acc = {0};
    v16i prev = sub_mfma(w, g, qrow, 0);
#pragma unroll
    for (int jj = 1; jj <= 16; ++jj) {
      v16i cur;
      if (jj < 16) cur = sub_mfma(w, g, qrow, jj);
      const int sc = (int)(int8_t)((scw[(jj - 1) >> 2] >> (8 * ((jj - 1) & 3))) & 0xFF);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += __mul24(sc, prev[r]);   // |P| < 2^17: 24-bit multiply is exact
      asm volatile("" : "+v"(acc) : : "memory");
      if (jj < 16) prev = cur;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) S1[r] = acc[r];
    const v16i z16 = {0};
    const v4i bm = {(int)scw[0], (int)scw[1], (int)scw[2], (int)scw[3]}, zero = {0, 0, 0, 0};
    xl = mfma_k32(abs, g == 0 ? bm : zero, z16);
    xh = mfma_k32(abs, g == 1 ? bm : zero, z16);
  }
  // The exact integer parts of the super-block term: s1 = sum_j sc_j isum_j
  // (isum over the codes q - 32), s2 = sum_j sc_j bsum_j.
  struct Ints { v16i s1, s2; };
  __device__ __forceinline__ static Ints ints(const Wt& w, int g, const uint8_t* qrow, const v4i abs) {
    int S1[16];
    v16i xl, xh;
    raw(w, g, qrow, abs, S1, xl, xh);
    Ints o;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o.s2[r] = xl[r] + 64 * xh[r];
      o.s1[r] = S1[r] - 32 * o.s2[r];
    }
    return o;
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i abs, const double* dxs,
                             int n, double* acc) {
    int S1[16];
    v16i xl, xh;
    raw(w, g, qrow, abs, S1, xl, xh);
    const double d = half_bits_to_float(w.d);
    MOEQ_COMBINE(acc[r] += dx * (d * (double)(S1[r] - 32 * (xl[r] + 64 * xh[r]))))
  }
};

template <> struct Mf<FQ80> {
  static constexpr int NBSP = 0;
  struct Wt { uint4 q[8]; uint4 d; };
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int g) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    const uint8_t* qb = Wb + rs.su * 256;
    Wt w;
#pragma unroll
    for (int b = 0; b < 8; ++b) w.q[b] = gld_u4(qb + (lr * 256u + 32u * (uint32_t)b + 16u * (uint32_t)g));
    w.d = gld_u4(Wb + align256(nsb * 256) + rs.su * 16 + lr * 16u);
    return w;
  }
  // The exact integer sum of 32-block b of the super-block: isum_b.
  __device__ __forceinline__ static v16i block_ints(const Wt& w, int g, const uint8_t* qrow, int b) {
    const v4i bq = {(int)w.q[b].x, (int)w.q[b].y, (int)w.q[b].z, (int)w.q[b].w};
    const v16i z16 = {0};
    return mfma_k32(lds_v4(qrow + 32 * b + 16 * g), bq, z16);
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i, const double* dxs,
                             int n, double* acc) {
    const uint32_t dw[4] = {w.d.x, w.d.y, w.d.z, w.d.w};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v16i P = block_ints(w, g, qrow, b);
      const double db = half_bits_to_float(dw[b >> 1] >> (16 * (b & 1)));
      MOEQ_COMBINE(acc[r] += (dx * db) * (double)P[r])
    }
  }
};

// Sum over the sub-blocks of sc_j * (the sub-block's exact MFMA dot), for
// a format whose scale does not fit into pre-scaled int8 weights (Q3_K).  Two-deep pipeline: the MFMA of sub-block jj + 1 is issued before
// the result of jj is scaled; the empty asm statement on the running sums
// (with a memory clobber) ends each step, so the next step's LDS operand load
// and MFMA stay behind it and at most two MFMA results are live.
template <class M>
__device__ __forceinline__ v16i sub_scaled_sum(const typename M::Wt& w, int g, const uint8_t* qrow) {
  v16i acc = {0};
  v16i prev = M::sub_mfma(w, g, qrow, 0);
#pragma unroll
  for (int jj = 1; jj <= M::NSUB; ++jj) {
    v16i cur;
    if (jj < M::NSUB) cur = M::sub_mfma(w, g, qrow, jj);
    const int sc = M::sub_scale(w, jj - 1);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += __mul24(sc, prev[r]);   // |sc| < 64, |P| < 2^17: exact
    asm volatile("" : "+v"(acc) : : "memory");
    if (jj < M::NSUB) prev = cur;
  }
  return acc;
}

template <> struct Mf<FQ3K> {
  static constexpr int NBSP = 16, NSUB = 16;
  struct Wt { uint4 l[4]; uint4 x[2]; uint4 sc; uint32_t d; };
  // Every lane loads the row's whole super-block: all 16 low-pair words (one
  // per sub-block), the 8 high-bit words, the scales and d.
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    const uint8_t* px = Wb + align256(nsb * 64);
    const uint8_t* ps = px + align256(nsb * 32);
    const uint8_t* pd = ps + align256(nsb * 16);
    Wt w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w.l[k] = gld_u4(Wb + rs.su * 64 + (lr * 64u + 16u * (uint32_t)k));
#pragma unroll
    for (int k = 0; k < 2; ++k) w.x[k] = gld_u4(px + rs.su * 32 + (lr * 32u + 16u * (uint32_t)k));
    w.sc = gld_u4(ps + rs.su * 16 + lr * 16u);
    w.d = gld_u16(pd + rs.su * 2 + lr * 2u);
    return w;
  }
  __device__ static uint32_t pick(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
  // Sub-block jj (16 elements): lane half g holds its elements 8g .. 8g+7,
  // words i = 2g, 2g+1 of the sub-block's low-pair word, high bits 4(jj%2)+i
  // of chunk jj/2's high word.
  __device__ __forceinline__ static v16i sub_mfma(const Wt& w, int g, const uint8_t* qrow, int jj) {
    const uint32_t lw = pick(w.l[jj >> 2], jj & 3);
    const uint32_t hx = pick(w.x[jj >> 3], (jj >> 1) & 3);
    uint32_t q[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = 2 * g + t;
      q[t] = ((lw >> (2 * i)) & 0x03030303u) | (((hx >> (4 * (jj & 1) + i)) & 0x01010101u) << 2);
    }
    const long b = (long)(((uint64_t)q[1] << 32) | q[0]);
    const long a = *reinterpret_cast<const long*>(qrow + 16 * jj + 8 * g);
    const v16i z16 = {0};
    return mfma_k16(a, b, z16);
  }
  __device__ __forceinline__ static int sub_scale(const Wt& w, int jj) {
    return (int)(int8_t)((pick(w.sc, jj >> 2) >> (8 * (jj & 3))) & 0xFF);
  }
  // The exact integer parts: s1 = sum_j sc_j isum_j over the codes q - 4,
  // s2 = sum_j sc_j bsum_j (split-sum MFMA pair with the int8 scales).
  struct Ints { v16i s1, s2; };
  __device__ __forceinline__ static Ints ints(const Wt& w, int g, const uint8_t* qrow, const v4i abs) {
    const v16i P = sub_scaled_sum<Mf<FQ3K>>(w, g, qrow);
    const v16i z16 = {0};
    const v4i bm = {(int)w.sc.x, (int)w.sc.y, (int)w.sc.z, (int)w.sc.w}, zero = {0, 0, 0, 0};
    const v16i xl = mfma_k32(abs, g == 0 ? bm : zero, z16);
    const v16i xh = mfma_k32(abs, g == 1 ? bm : zero, z16);
    Ints o;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o.s2[r] = xl[r] + 64 * xh[r];
      o.s1[r] = P[r] - 4 * o.s2[r];
    }
    return o;
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i abs, const double* dxs,
                             int n, double* acc) {
    const Ints I = ints(w, g, qrow, abs);
    const double d = half_bits_to_float(w.d);
    MOEQ_COMBINE(acc[r] += dx * (d * (double)I.s1[r]))
  }
};

template <> struct Mf<FQ5K> {
  static constexpr int NBSP = 8;   // one block sum per 32-sub-block, as Q4_K
  struct Wt { uint4 c[4]; uint4 x; uint4 h; };
  // Q4_K's loads (lane half g: chunks 2p+g) plus that half's four bit-4 words
  // (the plane keeps the words of chunks g, g+2, g+4, g+6 together).
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int g) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    const uint8_t* px = Wb + align256(nsb * 128);
    const uint8_t* ph = px + align256(nsb * 32);
    Wt w;
#pragma unroll
    for (int p = 0; p < 4; ++p) w.c[p] = gld_u4(Wb + rs.su * 128 + (lr * 128u + 16u * (uint32_t)(2 * p + g)));
    w.x = gld_u4(px + rs.su * 32 + (lr * 32u + 16u * (uint32_t)g));
    w.h = gld_u4(ph + rs.su * 16 + lr * 16u);
    return w;
  }
  // The exact integer parts: s1 = sum_j sc_j isum_j, s2 = sum_j m_j bsum_j.
  // q = l + 16 h (l the nibble, h bit 4) and sc = 8 sh + sl (sh, sl < 8):
  // sc_j isum_j = sum (l sl) x + 8 sum (l sh) x + 16 sum (h sc) x, every
  // weight byte below 128.  The three sums run as one chain of MFMAs on one
  // accumulator: the h*sc sum, doubled, is the input of the l*sh MFMAs, and
  // that result times 8 the input of the l*sl MFMAs, so
  // s1 = 8 (2 P_h + P_hi) + P_lo with a single running sum.
  // MFMA 2p+s: lane half g holds sub-block 2p+g, nibble s.
  struct Ints { v16i s1, s2; };
  __device__ __forceinline__ static Ints ints(const Wt& w, int g, const uint8_t* qrow, const v4i abs) {
    const uint64_t lo = (uint64_t)w.h.y | ((uint64_t)w.h.z << 32);
    const uint64_t hi = (uint64_t)w.h.z | ((uint64_t)w.h.w << 32);
    const uint32_t hx[4] = {w.x.x, w.x.y, w.x.z, w.x.w};
    v16i acc = {0};
#pragma unroll
    for (int ph = 0; ph < 3; ++ph) {
      if (ph > 0) acc = (ph == 1 ? 2 : 8) * acc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t sc = (uint32_t)(lo >> (6 * (2 * p + g))) & 63;
        const uint32_t c[4] = {w.c[p].x, w.c[p].y, w.c[p].z, w.c[p].w};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          v4i b;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (ph == 0) b[i] = (int)bytes_times((hx[p] >> (4 * s + i)) & 0x01010101u, sc);
            else b[i] = (int)bytes_times((c[i] >> (4 * s)) & 0x0F0F0F0Fu, ph == 1 ? sc >> 3 : sc & 7);
          }
          acc = mfma_k32(lds_v4(qrow + 64 * p + 32 * g + 16 * s), b, acc);
        }
      }
    }
    uint32_t m0 = 0, m1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m0 |= (uint32_t)((hi >> (16 + 6 * j)) & 63) << (8 * j);
      m1 |= (uint32_t)((hi >> (16 + 6 * (j + 4))) & 63) << (8 * j);
    }
    const v4i bm = {(int)m0, (int)m1, 0, 0}, zero = {0, 0, 0, 0};
    const v16i z16 = {0};
    const v16i xl = mfma_k32(abs, g == 0 ? bm : zero, z16);
    const v16i xh = mfma_k32(abs, g == 1 ? bm : zero, z16);
    return Ints{acc, xl + 64 * xh};
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i abs, const double* dxs,
                             int n, double* acc) {
    const Ints I = ints(w, g, qrow, abs);
    const double d = half_bits_to_float(w.h.x & 0xFFFF), dmin = half_bits_to_float(w.h.x >> 16);
    MOEQ_COMBINE(acc[r] += dx * (d * (double)I.s1[r] - dmin * (double)I.s2[r]))
  }
};

// Q4_0 and Q5_1: every lane loads the row's eight 16-byte quant chunks (its
// lane half takes one nibble of each) and the scales, as Q8_0.
__device__ __forceinline__ uint32_t pick4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <> struct Mf<FQ40> {
  static constexpr int NBSP = 0;
  struct Wt { uint4 q[8]; uint4 d; };
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    Wt w;
#pragma unroll
    for (int b = 0; b < 8; ++b) w.q[b] = gld_u4(Wb + rs.su * 128 + (lr * 128u + 16u * (uint32_t)b));
    w.d = gld_u4(Wb + align256(nsb * 128) + rs.su * 16 + lr * 16u);
    return w;
  }
  // The exact integer sum of 32-block b over the codes q - 8: nibble g of the
  // block's words, biased to signed bytes ((v + 0x78) ^ 0x80 = v - 8 for v < 16).
  __device__ __forceinline__ static v16i block_ints(const Wt& w, int g, const uint8_t* qrow, int b) {
    v4i bq;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bq[i] = (int)((((pick4(w.q[b], i) >> (4 * g)) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
    const v16i z16 = {0};
    return mfma_k32(lds_v4(qrow + 32 * b + 16 * g), bq, z16);
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i, const double* dxs,
                             int n, double* acc) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v16i P = block_ints(w, g, qrow, b);
      const double db = half_bits_to_float(pick4(w.d, b >> 1) >> (16 * (b & 1)));
      MOEQ_COMBINE(acc[r] += (dx * db) * (double)P[r])
    }
  }
};

template <> struct Mf<FQ51> {
  static constexpr int NBSP = 0;
  struct Wt { uint4 q[8]; uint4 xd[4]; };   // xd[k]: (bit-4 word, d | m) of blocks 2k, 2k+1
  __device__ static Wt load(const uint8_t* W, int64_t N, int64_t nbK, int64_t row, int64_t sb, int) {
    const size_t nsb = (size_t)(N * nbK);
    const RowSplit rs = row_split(row, nbK, sb);
    const uint32_t lr = rs.r * (uint32_t)nbK;
    const uint8_t* Wb = wave_uni_ptr(W);
    const uint8_t* pxd = Wb + align256(nsb * 128);
    Wt w;
#pragma unroll
    for (int b = 0; b < 8; ++b) w.q[b] = gld_u4(Wb + rs.su * 128 + (lr * 128u + 16u * (uint32_t)b));
#pragma unroll
    for (int k = 0; k < 4; ++k) w.xd[k] = gld_u4(pxd + rs.su * 64 + (lr * 64u + 16u * (uint32_t)k));
    return w;
  }
  // The exact integer sum of 32-block b over the codes q = nibble | bit 4.
  __device__ __forceinline__ static v16i block_ints(const Wt& w, int g, const uint8_t* qrow, int b) {
    const uint32_t hx = pick4(w.xd[b >> 1], 2 * (b & 1));
    v4i bq;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bq[i] = (int)(((pick4(w.q[b], i) >> (4 * g)) & 0x0F0F0F0Fu) | (((hx >> (4 * g + i)) & 0x01010101u) << 4));
    const v16i z16 = {0};
    return mfma_k32(lds_v4(qrow + 32 * b + 16 * g), bq, z16);
  }
  template <int NQ>
  __device__ static void mac(const Wt& w, int g, const uint8_t* qrow, const v4i, const double* dxs,
                             int n, double* acc) {
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const v16i z16 = {0};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v16i P = block_ints(w, g, qrow, b);
      const v16i S = mfma_k32(lds_v4(qrow + 32 * b + 16 * g), ones, z16);   // the block's activation sums
      const uint32_t dmw = pick4(w.xd[b >> 1], 2 * (b & 1) + 1);
      const double db = half_bits_to_float(dmw & 0xFFFF), mb = half_bits_to_float(dmw >> 16);
      MOEQ_COMBINE(acc[r] += dx * (db * (double)P[r] + mb * (double)S[r]))
    }
  }
};

// Formats whose tiles scale each sub-block's MFMA result in int32 (more
// registers per lane): no 8-row ring or fp32-h kernels for them.
template <int F> constexpr bool kSubScaled = F == FQ6K || F == FQ3K;

// ------------------------------------------------------------ staging

// Staging of 256-block sb of the tile's activation rows, in two halves so the
// global loads of block sb+1 overlap the MFMAs of block sb: thread (m, piece)
// loads 16 quant bytes (piece 0 also the scale, piece 1 the 16 block sums)
// into registers, then writes them (and the split block sums) to LDS.
struct StageRegs {
  uint32_t q[4];
  float d;
  uint32_t bs[8];
};
template <int NBSP>
__device__ __forceinline__ StageRegs stage_load(const uint8_t* srow, int64_t sb, int piece) {
  StageRegs r;
  const uint8_t* blk = srow != nullptr ? srow + sb * kQ8KBytes : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.q[i] = blk != nullptr ? gld_u32(blk + 4 + 16 * piece + 4 * i) : 0u;
  r.d = (blk != nullptr && piece == 0) ? gld_f32(blk) : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.bs[i] = (NBSP > 0 && blk != nullptr && piece == 1) ? gld_u32(blk + 260 + 4 * i) : 0u;
  return r;
}
template <int NBSP, int TM>
__device__ __forceinline__ void stage_store(StageLds<TM>& L, const StageRegs& r, int m, int piece) {
  *reinterpret_cast<uint4*>(&L.qs[m][16 * piece]) = make_uint4(r.q[0], r.q[1], r.q[2], r.q[3]);
  if (piece == 0) L.dx[m] = r.d;
  if (NBSP > 0 && piece == 1) {
    int bs[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bs[2 * i] = (int)(int16_t)(r.bs[i] & 0xFFFF);
      bs[2 * i + 1] = (int)(int16_t)(r.bs[i] >> 16);
    }
    uint32_t lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < NBSP; ++j) {
      const int v = NBSP == 8 ? bs[2 * j] + bs[2 * j + 1] : bs[j];
      lo[j >> 2] |= (uint32_t)(v & 63) << (8 * (j & 3));
      hi[j >> 2] |= (uint32_t)((v >> 6) & 255) << (8 * (j & 3));
    }
    *reinterpret_cast<uint4*>(&L.bsp[m][0][0]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(&L.bsp[m][1][0]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

// Staging of fp32 h (the fp32-h variant of the down tiles): thread (m, piece)
// quantises elements 16*piece .. +15 of 256-block sb of tile row m with the
// amax of the block's 16 threads (one 16-lane DPP row), by the same definition
// as quantize_row_lds, and writes codes, scale and split block sums to LDS
// (and, with `view`, the q8_K block to the q8_K(h) rows).  Rows beyond the
// tile (hrow null) stage as zero blocks.
struct StageF { float4 v[4]; };
__device__ __forceinline__ StageF stage_load_f(const float* hrow, int64_t sb, int piece) {
  StageF r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = hrow != nullptr ? gld_f4(hrow + sb * 256 + 16 * piece + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
  return r;
}
template <int NBSP, int TM>
__device__ __forceinline__ void stage_quant(StageLds<TM>& L, const StageF& r, int m, int piece, uint8_t* view) {
  const float v[16] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w,
                       r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w, r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_all_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_all_f<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_all_f<kDppRowRor4>(amax));
  amax = fmaxf(amax, dpp_all_f<kDppRowRor8>(amax));
  const float id = amax == 0.0f ? 0.0f : __fdiv_rn(127.0f, amax);
  const bool zero = amax == 0.0f || __builtin_isinf(id);
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = zero ? 0 : q8_code(v[i], id);
    q[i >> 2] |= (uint32_t)(c & 255) << (8 * (i & 3));
    sum += c;
  }
  const float d = zero ? 0.0f : __fdiv_rn(amax, 127.0f);
  *reinterpret_cast<uint4*>(&L.qs[m][16 * piece]) = make_uint4(q[0], q[1], q[2], q[3]);
  if (piece == 0) L.dx[m] = d;
  if constexpr (NBSP == 16) {
    L.bsp[m][0][piece] = (uint8_t)(sum & 63);
    L.bsp[m][1][piece] = (uint8_t)((sum >> 6) & 255);
  } else if constexpr (NBSP == 8) {
    // entry j = sums of sub-blocks 2j and 2j+1, written by the even thread;
    // the odd thread clears entry 8 + j
    const int pair = sum + dpp_all_i<kDppXor1>(sum);
    const int e = (piece & 1) ? 8 + (piece >> 1) : (piece >> 1);
    L.bsp[m][0][e] = (piece & 1) ? (uint8_t)0 : (uint8_t)(pair & 63);
    L.bsp[m][1][e] = (piece & 1) ? (uint8_t)0 : (uint8_t)((pair >> 6) & 255);
  }
  if (view != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gst_u32(view + 4 + 16 * piece + 4 * i, q[i]);
    gst_i16(view + 260 + 2 * piece, (int16_t)sum);
    if (piece == 0) gst_f32(view, d);
  }
}

// q8_K of one 256-wide fp32 row held in LDS, by one wave (4 values per lane),
// identical to the definition (amax; id = 127/amax correctly rounded;
// q = rint(h*id) clamped; d = amax/127; per-16 sums; amax == 0 or an infinite
// id gives a zero block).
__device__ __forceinline__ void quantize_row_lds(const float* hrow, uint8_t* __restrict__ o) {
  const int lane = lane_id();
  const float4 v = *reinterpret_cast<const float4*>(hrow + 4 * lane);
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

// Staging of the tile's resident activation blocks (all nbK of them) into
// LDS, in rounds of R items per thread: work item i is 256-block i / (16 n),
// row (i / 16) % n, 16-byte piece i % 16, so the 16 items of one (block, row)
// sit in one 16-lane row of a wave.  Only the tile's n real rows are staged:
// rows n .. TM-1 of the stage hold stale LDS, and every output of those MFMA
// rows is dropped (the combine, h and y stores all stop at row n), so their
// values never matter.  QUANT: the rows are fp32 h, quantised to q8_K on the
// way.  The caller splits the first round into its loads and its stores (the
// ring of weight loads goes out in between), then stages the rest.
template <bool QUANT> struct StageRound {
  static constexpr int R = QUANT ? 2 : 4;   // items per thread and round
  typename std::conditional<QUANT, StageF, StageRegs>::type v[R];
};
template <int NBSP, int NT, bool QUANT>
__device__ __forceinline__ void stage_round_load(StageRound<QUANT>& b, const uint8_t* const* srows, int i0,
                                                 int per_blk, int items) {
#pragma unroll
  for (int j = 0; j < StageRound<QUANT>::R; ++j) {
    const int i = i0 + NT * j;
    if (i < items) {
      const int blk = i / per_blk, m = (i - blk * per_blk) >> 4;
      if constexpr (QUANT) b.v[j] = stage_load_f(reinterpret_cast<const float*>(srows[m]), blk, i & 15);
      else b.v[j] = stage_load<NBSP>(srows[m], blk, i & 15);
    }
  }
}
template <int NBSP, int TM, int NT, bool QUANT>
__device__ __forceinline__ void stage_round_store(const StageRound<QUANT>& b, StageLds<TM>* L,
                                                  uint8_t* const* vrows, int i0, int per_blk, int items) {
#pragma unroll
  for (int j = 0; j < StageRound<QUANT>::R; ++j) {
    const int i = i0 + NT * j;
    if (i < items) {
      const int blk = i / per_blk, m = (i - blk * per_blk) >> 4;
      if constexpr (QUANT)
        stage_quant<NBSP, TM>(L[blk], b.v[j], m, i & 15, vrows[m] != nullptr ? vrows[m] + blk * kQ8KBytes : nullptr);
      else
        stage_store<NBSP, TM>(L[blk], b.v[j], m, i & 15);
    }
  }
}
template <int NBSP, int TM, int NT, bool QUANT>
__device__ __forceinline__ void stage_rest(StageLds<TM>* L, const uint8_t* const* srows, uint8_t* const* vrows,
                                           int tid, int per_blk, int items) {
  constexpr int R = StageRound<QUANT>::R;
  for (int i0 = tid + R * NT; i0 < items; i0 += R * NT) {
    StageRound<QUANT> b;
    stage_round_load<NBSP, NT, QUANT>(b, srows, i0, per_blk, items);
    stage_round_store<NBSP, TM, NT, QUANT>(b, L, vrows, i0, per_blk, items);
  }
  __syncthreads();
}

// ------------------------------------------------------------ combine in the shared tiles

// The combine of tokens t0 .. t0+n-1 over columns c0 .. c0+255, by all NT
// threads of a workgroup (four consecutive columns per item): y (=|+=)
// fl32(sum over the k routed staging rows in slot order, then the shared
// staging row, in fp64), the same sum in the same order as k_combine.  A
// shared-expert down tile runs it after staging its own rows of the block,
// when the routed down launches have finished before it.
template <int NT>
__device__ __forceinline__ void combine_block(const float* __restrict__ yp, int64_t T, int64_t H, int k, int64_t t0,
                                              int n, int64_t c0, float* __restrict__ y, int accumulate) {
  constexpr int kRows = 12;                 // staging rows in flight per item
  const bool al = (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  for (int i = threadIdx.x; i < n * 64; i += NT) {
    const int64_t t = t0 + i / 64, c = c0 + 4 * (i % 64);
    const float* base = yp + t * k * H + c;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int s = 0; s < k; s += kRows) {
      float4 v[kRows];
#pragma unroll
      for (int j = 0; j < kRows; ++j)
        if (s + j < k) v[j] = gld_f4(base + (int64_t)(s + j) * H);
#pragma unroll
      for (int j = 0; j < kRows; ++j) {
        if (s + j < k) {
          a0 += (double)v[j].x; a1 += (double)v[j].y; a2 += (double)v[j].z; a3 += (double)v[j].w;
        }
      }
    }
    const float4 v = gld_f4(yp + (T * k + t) * H + c);
    a0 += (double)v.x; a1 += (double)v.y; a2 += (double)v.z; a3 += (double)v.w;
    float* out = y + t * H + c;
    if (accumulate) {
      a0 += (double)gld_f32(out); a1 += (double)gld_f32(out + 1);
      a2 += (double)gld_f32(out + 2); a3 += (double)gld_f32(out + 3);
    }
    if (al) {
      gst_f4(out, make_float4((float)a0, (float)a1, (float)a2, (float)a3));
    } else {
      gst_f32(out, (float)a0); gst_f32(out + 1, (float)a1); gst_f32(out + 2, (float)a2); gst_f32(out + 3, (float)a3);
    }
  }
}

// LDS of the tile code, one object per (type, tag) and kernel: it depends on
// the tile's shape, not on the weight format, so a kernel that runs the tiles
// of two formats (a workgroup takes one or the other) holds one copy.
template <class T, int TAG>
__device__ __forceinline__ T& lds_var() {
  __shared__ __align__(16) T v;
  return v;
}

// The tile of this workgroup (b: its tile index, blockIdx.x unless a kernel
// runs two tile lists): for the shared expert, tokens t0 .. t0+n-1 of
// block row b; for routed experts, tile list entry j (expert e, rows
// t0 .. t0+n-1 of its list at list_off).  32-row tiles run in XCD-aware
// order: workgroup b runs on XCD b % 8, and XCD x takes the x-th contiguous
// eighth of the expert-ordered tile list, so the tiles of one expert run side
// by side on one XCD and share its L2 for the expert's weights (the grid is a
// multiple of 8 covering the list).  Measured at prefill size: gate/up
// fetches 0.84 GB past L2 instead of 1.93 GB, down 0.39 GB instead of
// 0.89 GB (the algorithmic bytes).  8-row tiles have one tile per expert:
// plain order.  False: no tile for this workgroup.
template <int TM>
__device__ __forceinline__ bool pick_tile(const MfmaArgs& a, int b, int& e, int& t0, int& n, int64_t& list_off) {
  e = -1;
  list_off = 0;
  if (a.shared) {
    t0 = b * TM;
    if (t0 >= a.T) return false;
    n = (int)((a.T - t0) < TM ? (a.T - t0) : TM);
    return true;
  }
  const int cnt = *a.count;
  int j = b;
  if constexpr (TM == 32) {
    const int per = (cnt + 7) >> 3;
    j = (b & 7) * per + (b >> 3);
    if ((b >> 3) >= per) return false;
  }
  if (j >= cnt) return false;
  const int4 tl = a.tiles[j];
  e = tl.x; t0 = tl.y; n = tl.z; list_off = tl.w;
  return true;
}

// ------------------------------------------------------------ the kernel
//
// MODE 0 (gate/up): A = q8_K(x) rows of the tile's tokens, W0 = gate, W1 = up;
//   epilogue per 256-row block: h = fl32(silu(g) u) into LDS, then q8_K(h) of
//   the block (one q8_K block per tile row) into hq.
// MODE 1 (down): A = q8_K(h) rows of the tile's pairs, W0 = down; epilogue
//   yp[row] = fl32(gate weight * y).
// TM: activation rows a tile stages (32; or 8 for experts with at most 8 rows,
//   whose MFMA rows 8..31 are zero and whose combine covers only 8 rows).
// RES: the whole activation tile fits in LDS (K up to kRes(TM) 256-blocks), so
//   the k-loop runs without barriers; otherwise the blocks stream through a
//   double-buffered stage (one barrier per block).
// A workgroup covers `rb` consecutive 256-row blocks of its tile (grid.y =
// ceil(blocks / rb)), so the staging and start-up are paid once per rb blocks;
// the weight loads of the next (row block, 256-block, matrix) unit are always
// in flight while the current unit's MFMAs run.
__host__ __device__ constexpr int kRes(int TM) { return TM == 32 ? 8 : 16; }
static_assert(kRes(8) == kHfMaxBlocks, "resident 8-row tiles");

// NW = 16 (gate/up of resident 8-row tiles only): waves 0-7 stream gate and
// waves 8-15 stream up for the same 256 rows, so a CU holds twice the waves;
// g reaches the up waves through LDS for h.
// HF (fp32 h, resident ring tiles only): mode 0 writes h = fl32(silu(g) u) as
// fp32 rows, so a workgroup needs no whole 256-row block for q8_K(h) and may
// cover fewer rows (NW = 4: two gate and two up waves over 64 rows, several
// workgroups per CU, every CU busy on small unions); mode 1 then quantises
// the fp32 rows to q8_K while staging them.
// COMB (shared-expert down tiles that run after the routed down launches):
//   after staging its rows of a row block, the tile also does the combine of
//   its tokens over those columns into y (combine_block), so no separate
//   combine launch is needed.
// RNPER > 0 (fp32-h gate/up of small chunks): the workgroup routes the chunk
//   inline from the logits (route_small_tile, top-k with RNPER logits per
//   lane) and takes its tile and pair rows from that, not from the lists.
template <int FMT, int MODE, bool RES, int TM, int RING, int NW = 8, bool HF = false, bool COMB = false,
          int RNPER = 0>
__device__ __forceinline__ void mfma_tile(const MfmaArgs& a, const SmallRoute* rt = nullptr, int tile_b = -1) {
  static_assert(RNPER == 0 || (MODE == 0 && HF && TM == kThinRows), "inline routing: fp32-h 8-row gate/up");
  static_assert(NW == 8 || (NW == 16 && MODE == 0 && RES && RING > 1) || (NW == 4 && MODE == 0 && HF),
                "split waves: resident gate/up ring");
  static_assert(!HF || (RES && RING > 1), "fp32 h: resident ring tiles");
  constexpr bool SPLIT = MODE == 0 && NW != 8;        // gate and up on separate waves
  constexpr int WPM = SPLIT ? NW / 2 : NW;            // waves per matrix
  constexpr int RB = 32 * WPM;                        // weight rows per row block
  static_assert(MODE == 1 || HF || RB == 256, "q8_K(h) in the epilogue needs whole 256-row blocks");
  constexpr int NT = 64 * NW;
  using M = Mf<FMT>;
  constexpr int NQ = TM / 8;
  auto& L = lds_var<StageLds<TM>[RES ? kRes(TM) : 2], 0>();
  auto& orow = lds_var<int64_t[TM], 1>();
  auto& owt = lds_var<double[TM], 2>();
  auto& srows = lds_var<const uint8_t* [TM], 3>();
  auto& vrows = lds_var<uint8_t* [TM], 4>();            // HF mode 1: q8_K(h) view rows (workgroup row 0 only)
  auto& zrow = lds_var<uint8_t[kQsStride], 5>();        // A rows past the tile height read zeros

  // ---- tile: expert (or the shared expert) and its rows t0 .. t0+n-1
  int e, t0 = 0, n;
  int64_t list_off;
  const int* rkey = nullptr;   // inline routing: sorted pair keys (expert << 6 | pair) in LDS
  if constexpr (RNPER > 0) {
    __shared__ int r_ids[kSmallPairs], r_key[kSmallPairs], r_act[kSmallPairs + 1], r_pos[kSmallPairs + 1];
    __shared__ int r_ebase[kSmallPairs + 1], r_off[kSmallRouteMaxE + 1];
    if (!route_small_tile<RNPER>(*rt, a.T, a.k, r_ids, r_key, r_act, r_pos, r_off, r_ebase,
                                 tile_b >= 0 ? tile_b : (int)blockIdx.x, e, n, list_off))
      return;
    rkey = r_key;
  } else {
    if (!pick_tile<TM>(a, tile_b >= 0 ? tile_b : (int)blockIdx.x, e, t0, n, list_off)) return;
  }
  const int64_t nrb = a.N / RB;
  const int64_t rb0 = (int64_t)blockIdx.y * a.rb;
  const int64_t rb1 = rb0 + a.rb < nrb ? rb0 + a.rb : nrb;
  if (rb0 >= nrb) return;
  const uint8_t *W0, *W1 = nullptr;
  if (a.shared) {
    W0 = a.sh_w0;
    W1 = a.sh_w1;
  } else {
    const void *pg = a.gate[e], *pu = a.up[e], *pd = a.down[e];
    const bool resident = pg != nullptr && pu != nullptr && pd != nullptr;
    W0 = (const uint8_t*)(MODE == 0 ? pg : pd);
    W1 = (const uint8_t*)pu;
    if (!resident) {
      // not resident: its pairs add exactly nothing (their down rows are zero)
      if (MODE == 1) {
        const int64_t cols = (rb1 - rb0) * RB;
        for (int64_t i = threadIdx.x; i < n * cols; i += blockDim.x) {
          const int p = a.pairs[list_off + t0 + i / cols];
          gst_f32(a.yp + (int64_t)p * a.N + rb0 * RB + i % cols, 0.0f);
        }
      }
      return;
    }
  }

  // ---- per-row bookkeeping: source rows, output rows, gate weights
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id(), g = lane >> 5;
  const bool arow = (lane & 31) < TM;                  // the lane's A row is staged
  for (int i = tid; i < kQsStride / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(zrow)[i] = 0u;
  if (tid < TM) {
    int64_t orr = -1, ridx = 0, vidx = 0;
    double wt = 0.0;
    const uint8_t* sr = nullptr;
    uint8_t* vr = nullptr;
    if (tid < n) {
      if (a.shared) {
        ridx = t0 + tid;
        orr = MODE == 0 ? (int64_t)(t0 + tid) : a.T * a.k + t0 + tid;
        wt = a.shared_scale != nullptr ? (double)a.shared_scale[t0 + tid] : 1.0;
      } else {
        const int p = rkey != nullptr ? (rkey[list_off + t0 + tid] & 63) : a.pairs[list_off + t0 + tid];
        ridx = MODE == 0 ? p / a.k : p;
        orr = p;
        wt = MODE == 1 ? (double)a.topk_w[p] : 0.0;
      }
      vidx = a.shared ? t0 + tid : ridx;
      if (HF && MODE == 1) {
        sr = reinterpret_cast<const uint8_t*>(a.hf + ridx * a.hf_stride);
        if (a.hq != nullptr && blockIdx.y == 0) vr = a.hq + vidx * a.hq_stride;
      } else {
        sr = a.src + ridx * a.src_stride;
      }
    }
    orow[tid] = orr;
    owt[tid] = wt;
    srows[tid] = sr;
    vrows[tid] = vr;
  }
  __syncthreads();

  const int64_t nbK = a.K / 256;
  const int64_t lrow = (wave % WPM) * 32 + (lane & 31);        // the lane's weight row inside a row block
  const int wmat = SPLIT ? wave / WPM : 0;                      // split waves: the wave's matrix
  const uint8_t* Wsel = wmat == 0 ? W0 : W1;
  const int64_t nmat = MODE == 0 && !SPLIT ? 2 : 1;   // matrices a wave walks
  constexpr bool RINGP = RES && RING > 1;

  if constexpr (RINGP) {
  // RING weight units in flight per wave (memory-bound tiles): ring slot j
  // holds unit u0 + j, and the loop is unrolled by RING so every slot index
  // is static.  Units run (row block, 256-block, matrix) in the same order in
  // every wave, so the row-block epilogue (with its barriers) is uniform.
  // The fp32-h gate/up tiles (EARLY) fill the ring between the first staging
  // round's loads and its stores, so the weights are in flight while the
  // activations arrive (loads return in order: the activations first).  The
  // other tiles stage first and fill the ring after: with the ring state live
  // through their staging, scalars spill to scratch.  The ring state and its
  // lambdas live in this branch, not at function scope, and capture no kernel
  // argument (either keeps the arguments in scratch).
  constexpr bool Q = HF && MODE == 1, EARLY = HF && MODE == 0;
  const int per_blk = 16 * n, items = (int)nbK * per_blk;
  if constexpr (!EARLY) {
    StageRound<Q> b;
    stage_round_load<M::NBSP, NT, Q>(b, srows, tid, per_blk, items);
    stage_round_store<M::NBSP, TM, NT, Q>(b, L, vrows, tid, per_blk, items);
    stage_rest<M::NBSP, TM, NT, Q>(L, srows, vrows, tid, per_blk, items);
  }
  typename M::Wt ring[RING];
  int64_t l_rb = rb0, l_sb = 0;
  int l_mat = 0;
  auto adv_l = [&]() __attribute__((always_inline)) {
    if (++l_mat == nmat) {
      l_mat = 0;
      if (++l_sb == nbK) { l_sb = 0; ++l_rb; }
    }
  };
  // Every refill is issued, also past the wave's last unit (it then reloads
  // that unit, already in cache, and the slot is never consumed): with the
  // same loads on every path the compiler waits for one unit at a time
  // (vmcnt of the RING-1 units behind it) instead of for all of them.
  const int64_t wN = a.N;
  auto load_unit = [&]() __attribute__((always_inline)) {
    const bool in = l_rb < rb1;
    const int64_t rb = in ? l_rb : rb1 - 1, sb = in ? l_sb : nbK - 1;
    const int mt = in ? l_mat : (int)nmat - 1;
    return M::load(SPLIT ? Wsel : (mt == 0 ? W0 : W1), wN, nbK, rb * RB + lrow, sb, g);
  };
  auto fill_ring = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RING; ++j) { ring[j] = load_unit(); adv_l(); }
  };
  if constexpr (EARLY) {
    StageRound<Q> b;
    stage_round_load<M::NBSP, NT, Q>(b, srows, tid, per_blk, items);
    fill_ring();
    stage_round_store<M::NBSP, TM, NT, Q>(b, L, vrows, tid, per_blk, items);
    stage_rest<M::NBSP, TM, NT, Q>(L, srows, vrows, tid, per_blk, items);
  } else {
    fill_ring();
  }
  static_assert(MODE == 1 || SPLIT || RING % 2 == 0, "gate/up units alternate between the two matrices");
  const int64_t U = (rb1 - rb0) * nbK * nmat;
  double acc0[4 * NQ], acc1[4 * NQ];
#pragma unroll
  for (int r = 0; r < 4 * NQ; ++r) { acc0[r] = 0.0; acc1[r] = 0.0; }
  int64_t c_rb = rb0, c_sb = 0;
  for (int64_t u0 = 0; u0 < U; u0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      if (u0 + j < U) {
        const int mat = MODE == 0 && !SPLIT ? (j & 1) : 0;
        const typename M::Wt& wc = ring[j];
        StageLds<TM>& S = L[c_sb];
        const uint8_t* qrow = arow ? &S.qs[lane & 31][0] : zrow;
        v4i abs = {0, 0, 0, 0};
        if constexpr (M::NBSP > 0) abs = lds_v4(arow ? &S.bsp[lane & 31][g][0] : zrow);
        if (mat == 0) M::template mac<NQ>(wc, g, qrow, abs, S.dx, n, acc0);
        else M::template mac<NQ>(wc, g, qrow, abs, S.dx, n, acc1);
        if (mat == nmat - 1 && ++c_sb == nbK) {
          const int64_t wrow = c_rb * RB + lrow;
          if constexpr (MODE == 0 && HF) {
            // h = fl32(silu(g) u) straight to the fp32 h rows
            if constexpr (SPLIT) {
              auto& gxh = lds_var<double[TM][RB], 6>();
              if (wmat == 0) {
#pragma unroll
                for (int r = 0; r < 4 * NQ; ++r) gxh[out_row(r, g)][lrow] = acc0[r];
              }
              __syncthreads();
              if (wmat == 1) {
#pragma unroll
                for (int r = 0; r < 4 * NQ; ++r) {
                  const int m = out_row(r, g);
                  if (m < n) gst_f32(a.hf + orow[m] * a.hf_stride + wrow, (float)(silu64(gxh[m][lrow]) * acc0[r]));
                }
              }
              __syncthreads();   // gxh is rewritten by the next row block
            } else {
#pragma unroll
              for (int r = 0; r < 4 * NQ; ++r) {
                const int m = out_row(r, g);
                if (m < n) gst_f32(a.hf + orow[m] * a.hf_stride + wrow, (float)(silu64(acc0[r]) * acc1[r]));
              }
            }
          } else if constexpr (MODE == 0) {
            auto& hs2 = lds_var<float[TM][kMfRows + 4], 7>();
            if constexpr (NW == 16) {
              auto& gx = lds_var<double[TM][kMfRows], 8>();
              if (wmat == 0) {
#pragma unroll
                for (int r = 0; r < 4 * NQ; ++r) gx[out_row(r, g)][lrow] = acc0[r];
              }
              __syncthreads();
              if (wmat == 1) {
#pragma unroll
                for (int r = 0; r < 4 * NQ; ++r)
                  hs2[out_row(r, g)][lrow] = (float)(silu64(gx[out_row(r, g)][lrow]) * acc0[r]);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4 * NQ; ++r) hs2[out_row(r, g)][lrow] = (float)(silu64(acc0[r]) * acc1[r]);
            }
            __syncthreads();
            for (int m = wave; m < n; m += NW)
              quantize_row_lds(&hs2[m][0], a.hq + orow[m] * a.hq_stride + c_rb * kQ8KBytes);
            __syncthreads();   // hs2 (and gx) are rewritten by the next row block
          } else {
#pragma unroll
            for (int r = 0; r < 4 * NQ; ++r) {
              const int m = out_row(r, g);
              if (m < n) gst_f32(a.yp + orow[m] * a.N + wrow, (float)(owt[m] * acc0[r]));
            }
            if constexpr (COMB) {
              __syncthreads();   // every wave's staged rows of this block are written
              combine_block<NT>(a.yp, a.T, a.N, a.k, t0, n, c_rb * RB, a.y, a.accumulate);
            }
          }
#pragma unroll
          for (int r = 0; r < 4 * NQ; ++r) { acc0[r] = 0.0; acc1[r] = 0.0; }
          c_sb = 0;
          ++c_rb;
        }
      }
      // the slot is free again: refill it with the unit RING ahead
      ring[j] = load_unit();
      adv_l();
    }
  }
  } else {
  // One unit of weights ahead (few registers, so more waves per SIMD hide the
  // latency); activation blocks resident in LDS, or streamed through a
  // double-buffered stage when K exceeds the resident limit.
  // the first unit's weights, in flight during the staging
  typename M::Wt wn = M::load(Wsel, a.N, nbK, rb0 * RB + lrow, 0, g);
  if constexpr (RES) {
    const int per_blk = 16 * n, items = (int)nbK * per_blk;
    StageRound<false> b;
    stage_round_load<M::NBSP, NT, false>(b, srows, tid, per_blk, items);
    stage_round_store<M::NBSP, TM, NT, false>(b, L, vrows, tid, per_blk, items);
    stage_rest<M::NBSP, TM, NT, false>(L, srows, vrows, tid, per_blk, items);
  }
  const int ms = (tid >> 4) % TM, piece = tid & 15;
  const bool stager = tid < 16 * TM;
  StageRegs sr;
  for (int64_t rb = rb0; rb < rb1; ++rb) {
    const int64_t wrow = rb * kMfRows + lrow;
    double acc0[4 * NQ], acc1[4 * NQ];
#pragma unroll
    for (int r = 0; r < 4 * NQ; ++r) { acc0[r] = 0.0; acc1[r] = 0.0; }
    if constexpr (!RES)
      if (stager) sr = stage_load<M::NBSP>(srows[ms], 0, piece);
    for (int64_t sb = 0; sb < nbK; ++sb) {
      StageLds<TM>& S = RES ? L[sb] : L[sb & 1];
      if constexpr (!RES) {
        if (stager) stage_store<M::NBSP, TM>(S, sr, ms, piece);
        __syncthreads();
      }
      // next unit: up of this block (mode 0), else the next block, else the
      // first block of the next row block
      const bool last_k = sb + 1 == nbK;
      const bool more = !last_k || rb + 1 < rb1;
      const int64_t next_row = last_k ? wrow + kMfRows : wrow, next_sb = last_k ? 0 : sb + 1;
      typename M::Wt wc = wn;
      if constexpr (MODE == 0) {
        wn = M::load(W1, a.N, nbK, wrow, sb, g);
      } else if (more) {
        wn = M::load(W0, a.N, nbK, next_row, next_sb, g);
      }
      if constexpr (!RES)
        if (stager && !last_k) sr = stage_load<M::NBSP>(srows[ms], sb + 1, piece);
      const uint8_t* qrow = arow ? &S.qs[lane & 31][0] : zrow;
      v4i abs = {0, 0, 0, 0};
      if constexpr (M::NBSP > 0) abs = lds_v4(arow ? &S.bsp[lane & 31][g][0] : zrow);
      M::template mac<NQ>(wc, g, qrow, abs, S.dx, n, acc0);
      if constexpr (MODE == 0) {
        wc = wn;
        if (more) wn = M::load(W0, a.N, nbK, next_row, next_sb, g);
        M::template mac<NQ>(wc, g, qrow, abs, S.dx, n, acc1);
      }
    }

    if constexpr (MODE == 0) {
      // h = fl32(silu(g) u) -> LDS, then q8_K per tile row over this row block
      auto& hs = lds_var<float[TM][kMfRows + 4], 9>();
#pragma unroll
      for (int r = 0; r < 4 * NQ; ++r) hs[out_row(r, g)][lrow] = (float)(silu64(acc0[r]) * acc1[r]);
      __syncthreads();
      for (int m = wave; m < n; m += kMfWaves)
        quantize_row_lds(&hs[m][0], a.hq + orow[m] * a.hq_stride + rb * kQ8KBytes);
      __syncthreads();   // hs (and a streamed stage) is rewritten next
    } else {
#pragma unroll
      for (int r = 0; r < 4 * NQ; ++r) {
        const int m = out_row(r, g);
        if (m < n) gst_f32(a.yp + orow[m] * a.N + wrow, (float)(owt[m] * acc0[r]));
      }
      if constexpr (COMB) {
        __syncthreads();   // every wave's staged rows of this block are written
        combine_block<NT>(a.yp, a.T, a.N, a.k, t0, n, rb * kMfRows, a.y, a.accumulate);
      }
      if constexpr (!RES) __syncthreads();   // the streamed stage is rewritten next
    }
  }
  }
}

// 32-row tiles take every register they can use (2 waves per SIMD); 8-row
// tiles are held to 128 registers so two workgroups share a CU (4 waves per
// SIMD), which hides the weight-load latency of these memory-bound tiles
// (except Q6_K, whose per-sub-block scaling needs more registers).
template <int FMT, int MODE, bool RES, int TM>
__global__ __launch_bounds__(512) void k_mfma(MfmaArgs a) { mfma_tile<FMT, MODE, RES, TM, 1>(a); }
// shared-expert down tiles (32 rows) that also do the combine
template <int FMT, bool RES>
__global__ __launch_bounds__(512) void k_mfma_comb(MfmaArgs a) {
  mfma_tile<FMT, 1, RES, 32, 1, 8, false, true>(a);
}
template <int FMT, int MODE, bool RES>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(4, 8))) void k_mfma_thin(
    MfmaArgs a) {
  mfma_tile<FMT, MODE, RES, 8, 1>(a);
}
// 8-row tiles with resident activations and RING weight units in flight per
// wave (the memory-bound verify unions and small chunks).
template <int FMT> constexpr int kRing = (FMT == FQ80 || FMT == FQ40 || FMT == FQ51) ? 2 : 4;
template <int FMT, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 8))) void k_mfma_ring(
    MfmaArgs a) {
  mfma_tile<FMT, MODE, true, 8, kRing<FMT>>(a);
}
// gate/up of the same tiles on 16 waves (gate and up on separate waves)
template <int FMT>
__global__ __launch_bounds__(1024) void k_mfma_ring16(MfmaArgs a) {
  mfma_tile<FMT, 0, true, 8, kRing<FMT>, 16>(a);
}
// fp32-h variant: gate/up over 64 rows on 4 waves (two gate, two up; several
// workgroups per CU), down staging q8_K(h) from the fp32 rows itself.  Two
// units in flight per wave: every wave asks for its first units at once, and
// a shallower ring lets the first units of all waves arrive sooner (the
// stream rate is the same from 2 to 8 units in flight).
template <int FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 8))) void k_mfma_hf_gateup(
    MfmaArgs a) {
  mfma_tile<FMT, 0, true, 8, 2, 4, true>(a);
}
template <int FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 8))) void k_mfma_hf_down(
    MfmaArgs a) {
  mfma_tile<FMT, 1, true, 8, 2, 8, true>(a);
}
// The routed 8-row fp32-h tiles and the shared expert's in one launch (a
// chunk of 9 to 16 tokens, so no auxiliary stream and no fork or join):
// workgroups blockIdx.x < nsh take shared tile blockIdx.x, the others routed
// tile blockIdx.x - nsh; the two formats' tiles share one LDS layout.  The
// shared tiles come first in every grid row, so they are dispatched first.
template <int FR, int FS>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 8))) void
k_mfma_hf_gateup2(MfmaArgs a, MfmaArgs sa, int nsh) {
  if ((int)blockIdx.x < nsh) mfma_tile<FS, 0, true, 8, 2, 4, true>(sa, nullptr, (int)blockIdx.x);
  else mfma_tile<FR, 0, true, 8, 2, 4, true>(a, nullptr, (int)blockIdx.x - nsh);
}
template <int FR, int FS>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 8))) void
k_mfma_hf_down2(MfmaArgs a, MfmaArgs sa, int nsh) {
  if ((int)blockIdx.x < nsh) mfma_tile<FS, 1, true, 8, 2, 8, true>(sa, nullptr, (int)blockIdx.x);
  else mfma_tile<FR, 1, true, 8, 2, 8, true>(a, nullptr, (int)blockIdx.x - nsh);
}
// the same gate/up tiles of a small chunk, routing inline
template <int FMT, int NPER>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 8))) void
k_mfma_hf_gateup_route(MfmaArgs a, SmallRoute r) {
  mfma_tile<FMT, 0, true, 8, 2, 4, true, false, NPER>(a, &r);
}
// and with the shared expert's tiles in the same launch (as k_mfma_hf_gateup2)
template <int FR, int FS, int NPER>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 8))) void
k_mfma_hf_gateup_route2(MfmaArgs a, MfmaArgs sa, SmallRoute r, int nsh) {
  if ((int)blockIdx.x < nsh) mfma_tile<FS, 0, true, 8, 2, 4, true>(sa, nullptr, (int)blockIdx.x);
  else mfma_tile<FR, 0, true, 8, 2, 4, true, false, NPER>(a, &r, (int)blockIdx.x - nsh);
}

// ------------------------------------------------------------ integer hook
//
// The exact integer parts of every super-block term, computed by the same
// MFMA code the tiles run (Mf<F>::ints, Mf<Q8_0>::block_ints) on the same LDS
// staging of the activation rows: for a packed matrix W [N, K] and n_x q8_K
// rows, out[x][row][sb][0..7] holds (S1, S2, 0, 0, 0, 0, 0, 0) for Q4_K and
// Q2_K (S1 = sum_j sc_j isum_j, S2 = sum_j m_j bsum_j), for Q6_K (S1 over the
// codes q - 32, S2 = sum_j sc_j bsum_j), and the eight 32-block sums isum_b
// for Q8_0, Q4_0 (over q - 8) and Q5_1 (over q).  Grid (ceil(n_x / 32), N / 256): 32 activation rows and 8 waves
// of 32 weight rows per workgroup, one 256-block staged at a time.
template <int FMT>
__global__ __launch_bounds__(512) void k_mfma_ints(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                   const uint8_t* __restrict__ xq, int64_t n_x,
                                                   int32_t* __restrict__ out) {
  using M = Mf<FMT>;
  __shared__ StageLds<32> S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id(), g = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int n = (int)((n_x - t0) < 32 ? (n_x - t0) : 32);
  const int64_t nbK = K / 256;
  const int64_t row = (int64_t)blockIdx.y * kMfRows + wave * 32 + (lane & 31);
  const int ms = tid >> 4, piece = tid & 15;          // staging: tile row ms (0..31), 16-byte piece
  const uint8_t* srow = ms < n ? xq + (t0 + ms) * nbK * kQ8KBytes : nullptr;
  for (int64_t sb = 0; sb < nbK; ++sb) {
    const StageRegs sr = stage_load<M::NBSP>(srow, sb, piece);
    __syncthreads();                                  // the previous block's readers are done
    stage_store<M::NBSP, 32>(S, sr, ms, piece);
    __syncthreads();
    const typename M::Wt w = M::load(W, N, nbK, row, sb, g);
    const uint8_t* qrow = &S.qs[lane & 31][0];
    int32_t* o = out + (t0 * N + row) * nbK * 8 + sb * 8;
    const int64_t mstride = N * nbK * 8;
    if constexpr (FMT == FQ80 || FMT == FQ40 || FMT == FQ51) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const v16i P = M::block_ints(w, g, qrow, b);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = out_row(r, g);
          if (m < n) o[m * mstride + b] = P[r];
        }
      }
    } else {
      const v4i abs = lds_v4(&S.bsp[lane & 31][g][0]);
      const typename M::Ints I = M::ints(w, g, qrow, abs);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = out_row(r, g);
        if (m < n) {
          *reinterpret_cast<int4*>(o + m * mstride) = make_int4(I.s1[r], I.s2[r], 0, 0);
          *reinterpret_cast<int4*>(o + m * mstride + 4) = make_int4(0, 0, 0, 0);
        }
      }
    }
  }
}

int launch_mfma_ints(int fmt, const void* W, int64_t N, int64_t K, const void* xq, int64_t n_x, int32_t* out,
                     hipStream_t s) {
  const dim3 grid((unsigned)((n_x + 31) / 32), (unsigned)(N / kMfRows));
  const uint8_t* w8 = (const uint8_t*)W;
  const uint8_t* x8 = (const uint8_t*)xq;
  switch (fmt) {
    case FQ4K: hipLaunchKernelGGL(k_mfma_ints<FQ4K>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ6K: hipLaunchKernelGGL(k_mfma_ints<FQ6K>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ2K: hipLaunchKernelGGL(k_mfma_ints<FQ2K>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ80: hipLaunchKernelGGL(k_mfma_ints<FQ80>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ3K: hipLaunchKernelGGL(k_mfma_ints<FQ3K>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ5K: hipLaunchKernelGGL(k_mfma_ints<FQ5K>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ40: hipLaunchKernelGGL(k_mfma_ints<FQ40>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    case FQ51: hipLaunchKernelGGL(k_mfma_ints<FQ51>, grid, dim3(512), 0, s, w8, N, K, x8, n_x, out); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Tile lists of the routed experts (one workgroup; see mfma_plan.hpp).
__global__ __launch_bounds__(64) void k_mfma_plan(const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ offsets, MfmaPlan p) {
  __shared__ int ebase[kPlanMaxE + 1];
  mfma_plan_block(active, offsets, p, ebase);
}

int launch_mfma_plan(const int32_t* active, const int32_t* offsets, const MfmaPlan& p, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_plan, dim3(1), dim3(64), 0, s, active, offsets, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {

// Kernel choice for one (format, mode, tile height): 8-row tiles of the
// formats with pre-scaled int8 weights (not Q6_K or Q3_K, whose
// per-sub-block scaling needs more registers) run the ring kernels when their
// activations fit in LDS, gate/up of Q2_K and Q8_0 on 16 waves; everything
// else runs the one-unit-ahead tiles.
template <int F, int MD, int TM>
void launch_tile(dim3 grid, const MfmaArgs& a, int64_t nbK, bool hf, hipStream_t s) {
  if constexpr (TM == 8 && !kSubScaled<F>) {
    if (hf) {
      if constexpr (MD == 0) hipLaunchKernelGGL((k_mfma_hf_gateup<F>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_mfma_hf_down<F>), grid, dim3(512), 0, s, a);
    } else if (nbK <= kRes(TM)) {
      if constexpr (MD == 0 && (F == FQ2K || F == FQ80))
        hipLaunchKernelGGL((k_mfma_ring16<F>), grid, dim3(1024), 0, s, a);
      else
        hipLaunchKernelGGL((k_mfma_ring<F, MD>), grid, dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_mfma_thin<F, MD, false>), grid, dim3(512), 0, s, a);
    }
  } else if (MD == 1 && TM == 32 && a.y != nullptr) {
    if (nbK <= kRes(TM)) hipLaunchKernelGGL((k_mfma_comb<F, true>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_mfma_comb<F, false>), grid, dim3(512), 0, s, a);
  } else {
    if (nbK <= kRes(TM)) hipLaunchKernelGGL((k_mfma<F, MD, true, TM>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_mfma<F, MD, false, TM>), grid, dim3(512), 0, s, a);
  }
}

template <int F>
void launch_fmt(int mode, bool thin, bool hf, dim3 grid, const MfmaArgs& a, int64_t nbK, hipStream_t s) {
  if (mode == 0) {
    if (thin) launch_tile<F, 0, 8>(grid, a, nbK, hf, s);
    else launch_tile<F, 0, 32>(grid, a, nbK, false, s);
  } else {
    if (thin) launch_tile<F, 1, 8>(grid, a, nbK, hf, s);
    else launch_tile<F, 1, 32>(grid, a, nbK, false, s);
  }
}

}  // namespace

int launch_mfma_route_gateup(int fmt, dim3 grid, const MfmaArgs& a, const SmallRoute& r, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  if (a.T < 2 || a.T > kSmallRouteMaxT || a.T * a.k > kSmallPairs || r.E > kSmallRouteMaxE) return -2;
  if (a.K / 256 > kRes(8) || a.hf == nullptr || a.shared) return -2;
#define MOEQ_RG(F, N) hipLaunchKernelGGL((k_mfma_hf_gateup_route<F, N>), grid, dim3(256), 0, s, a, r)
#define MOEQ_RG_FMT(F) \
  if (r.E <= 256) MOEQ_RG(F, 4); \
  else MOEQ_RG(F, 8);
  switch (fmt) {
    case FQ4K: MOEQ_RG_FMT(FQ4K) break;
    case FQ2K: MOEQ_RG_FMT(FQ2K) break;
    case FQ80: MOEQ_RG_FMT(FQ80) break;
    case FQ5K: MOEQ_RG_FMT(FQ5K) break;
    case FQ40: MOEQ_RG_FMT(FQ40) break;
    case FQ51: MOEQ_RG_FMT(FQ51) break;
    default: return -2;
  }
#undef MOEQ_RG_FMT
#undef MOEQ_RG
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Format pairs of the two-list fp32-h kernels: a shared expert in Q8_0 or
// in the routed experts' format.
namespace {
constexpr bool hf_fmt(int f) { return f == FQ4K || f == FQ2K || f == FQ80 || f == FQ5K || f == FQ40 || f == FQ51; }
template <int FR, int FS>
void launch_hf2_pair(int mode, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, int nsh, hipStream_t s) {
  if (mode == 0) hipLaunchKernelGGL((k_mfma_hf_gateup2<FR, FS>), grid, dim3(256), 0, s, a, sa, nsh);
  else hipLaunchKernelGGL((k_mfma_hf_down2<FR, FS>), grid, dim3(512), 0, s, a, sa, nsh);
}
template <int FR>
int launch_hf2_fr(int mode, int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, int nsh, hipStream_t s) {
  if (fmt_s == FQ80) launch_hf2_pair<FR, FQ80>(mode, grid, a, sa, nsh, s);
  else if (fmt_s == FR) launch_hf2_pair<FR, FR>(mode, grid, a, sa, nsh, s);
  else return -2;
  return 0;
}
}  // namespace

bool mfma_hf2_pair(int fmt_r, int fmt_s) { return hf_fmt(fmt_r) && (fmt_s == FQ80 || fmt_s == fmt_r); }

namespace {
template <int FR, int FS>
void launch_route2_pair(dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, const SmallRoute& r, int nsh,
                        hipStream_t s) {
  if (r.E <= 256) hipLaunchKernelGGL((k_mfma_hf_gateup_route2<FR, FS, 4>), grid, dim3(256), 0, s, a, sa, r, nsh);
  else hipLaunchKernelGGL((k_mfma_hf_gateup_route2<FR, FS, 8>), grid, dim3(256), 0, s, a, sa, r, nsh);
}
template <int FR>
int launch_route2_fr(int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, const SmallRoute& r, int nsh,
                     hipStream_t s) {
  if (fmt_s == FQ80) launch_route2_pair<FR, FQ80>(grid, a, sa, r, nsh, s);
  else if (fmt_s == FR) launch_route2_pair<FR, FR>(grid, a, sa, r, nsh, s);
  else return -2;
  return 0;
}
}  // namespace

int launch_mfma_route_gateup2(int fmt_r, int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa,
                              const SmallRoute& r, int nsh, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  if (a.T < 2 || a.T > kSmallRouteMaxT || a.T * a.k > kSmallPairs || r.E > kSmallRouteMaxE) return -2;
  if (!mfma_hf2_pair(fmt_r, fmt_s) || !a.hf || !sa.hf || a.shared || !sa.shared) return -2;
  if (a.K / 256 > kRes(8) || sa.K / 256 > kRes(8)) return -2;
  int rc;
  switch (fmt_r) {
    case FQ4K: rc = launch_route2_fr<FQ4K>(fmt_s, grid, a, sa, r, nsh, s); break;
    case FQ2K: rc = launch_route2_fr<FQ2K>(fmt_s, grid, a, sa, r, nsh, s); break;
    case FQ80: rc = launch_route2_fr<FQ80>(fmt_s, grid, a, sa, r, nsh, s); break;
    case FQ5K: rc = launch_route2_fr<FQ5K>(fmt_s, grid, a, sa, r, nsh, s); break;
    case FQ40: rc = launch_route2_fr<FQ40>(fmt_s, grid, a, sa, r, nsh, s); break;
    case FQ51: rc = launch_route2_fr<FQ51>(fmt_s, grid, a, sa, r, nsh, s); break;
    default: return -2;
  }
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mfma_hf2(int mode, int fmt_r, int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, int nsh,
                    hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  if (!mfma_hf2_pair(fmt_r, fmt_s) || !a.hf || !sa.hf || a.K / 256 > kRes(8) || sa.K / 256 > kRes(8)) return -2;
  int rc;
  switch (fmt_r) {
    case FQ4K: rc = launch_hf2_fr<FQ4K>(mode, fmt_s, grid, a, sa, nsh, s); break;
    case FQ2K: rc = launch_hf2_fr<FQ2K>(mode, fmt_s, grid, a, sa, nsh, s); break;
    case FQ80: rc = launch_hf2_fr<FQ80>(mode, fmt_s, grid, a, sa, nsh, s); break;
    case FQ5K: rc = launch_hf2_fr<FQ5K>(mode, fmt_s, grid, a, sa, nsh, s); break;
    case FQ40: rc = launch_hf2_fr<FQ40>(mode, fmt_s, grid, a, sa, nsh, s); break;
    case FQ51: rc = launch_hf2_fr<FQ51>(mode, fmt_s, grid, a, sa, nsh, s); break;
    default: return -2;
  }
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mfma(int fmt, int mode, bool thin, bool hf, dim3 grid, const MfmaArgs& a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  const int64_t nbK = a.K / 256;
  // the fp32-h kernels: resident 8-row tiles of the pre-scaled formats
  // (checked by the caller too)
  if (hf && (!thin || fmt_sub_scaled(fmt) || nbK > kRes(8) || a.hf == nullptr)) return -2;
  switch (fmt) {
    case FQ4K: launch_fmt<FQ4K>(mode, thin, hf, grid, a, nbK, s); break;
    case FQ6K: launch_fmt<FQ6K>(mode, thin, false, grid, a, nbK, s); break;
    case FQ2K: launch_fmt<FQ2K>(mode, thin, hf, grid, a, nbK, s); break;
    case FQ80: launch_fmt<FQ80>(mode, thin, hf, grid, a, nbK, s); break;
    case FQ3K: launch_fmt<FQ3K>(mode, thin, false, grid, a, nbK, s); break;
    case FQ5K: launch_fmt<FQ5K>(mode, thin, hf, grid, a, nbK, s); break;
    case FQ40: launch_fmt<FQ40>(mode, thin, hf, grid, a, nbK, s); break;
    case FQ51: launch_fmt<FQ51>(mode, thin, hf, grid, a, nbK, s); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
