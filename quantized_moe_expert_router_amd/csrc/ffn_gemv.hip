// Expert-grouped dequant GEMV for decode and verify rows (a few tokens per
// expert).  Each expert's weights are read once for all of its tokens (rows
// that share an expert share one weight read: Pulsar README, ThinkingCap
// paragraph; the per-chunk expert union: DeepSeek-V4-Flash paragraph).
//
// Work item = (expert slot of the union, block of output rows).  A wave covers
// rps = 64/lpr rows per step, lpr lanes per row, each lane one or more 16-byte
// quant chunks at fixed column positions, so the activation chunks it needs
// stay in registers for every row it visits.  Integer sub-block dots are
// exact (v_dot4_i32_i8); the per-super-block scale/min combine and all sums
// are fp64; the only fp32 roundings are h = fl32(silu(g) u), the q8_K
// arithmetic and y.
//
// gate/up: h[pair, f] = fl32(silu(g) * u) with g, u the fp64 dots.
// down:    q8_K(h) is rebuilt in registers by every wave that needs it (it is a
//          pure function of h, so all waves agree bit for bit); each work item
//          writes fl32(w * (W_d h^)) (the fp64 row dot times the gate weight,
//          rounded once) to the pair's staging row.  A separate k_combine
//          launch then sums the staged rows of every token in fp64, slot
//          order and the shared expert last, and rounds y.
#include "one_token.hpp"

namespace moeq {

struct Slot {
  int valid, shared, e, n;
  int64_t list_off;
};

// Slot of the union (or the shared expert); experts with more than gemv_max
// rows belong to the MFMA path and are not valid here.
__device__ __forceinline__ Slot decode_slot(int slot, int mode, int max_union, const int32_t* active,
                                            const int32_t* offsets, int64_t T, int gemv_max) {
  Slot s{0, 0, -1, 0, 0};
  if (mode == kModeShared || (mode == kModeBoth && slot == max_union)) {
    s.valid = T <= gemv_max; s.shared = 1; s.n = (int)T;
    return s;
  }
  if (slot >= active[0]) return s;
  s.e = active[1 + slot];
  s.list_off = offsets[s.e];
  s.n = offsets[s.e + 1] - offsets[s.e];
  s.valid = s.n > 0 && s.n <= gemv_max;
  return s;
}

// token i of a slot: (token index, pair row)
__device__ __forceinline__ void slot_token(const Slot& s, int i, const int32_t* pairs, int64_t T, int k,
                                           int& tok, int64_t& prow) {
  if (s.shared) { tok = i; prow = T * k + i; return; }
  const int p = pairs[s.list_off + i];
  tok = p / k;
  prow = p;
}

template <int FMT, int TT, int CPL, int UNR>
__global__ __launch_bounds__(256) void k_gateup(GateUpArgs a) {
  using L = Fmt<FMT>;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int lpr = a.lpr, rps = kWave / lpr, rig = lane / lpr, lir = lane % lpr;
  const int64_t nb = a.H / 256, xrow = nb * kQ8KBytes;
  int xw[TT][CPL][L::XDW], bs[TT][CPL][L::NBS];
  double dx[TT][CPL];
  if (TT == 1) {
    // One token: its activation chunks do not depend on the routing, so their
    // loads are issued before the slot lookup.
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lir + lpr * c;
      if (ch < a.cpr) {
        load_x_chunk<FMT>(a.xq, ch, xw[0][c], bs[0][c], dx[0][c]);
      } else {
#pragma unroll
        for (int q = 0; q < L::XDW; ++q) xw[0][c][q] = 0;
#pragma unroll
        for (int q = 0; q < L::NBS; ++q) bs[0][c][q] = 0;
        dx[0][c] = 0.0;
      }
    }
  }
  const Slot sl = decode_slot(blockIdx.y, a.mode, a.max_union, a.active, a.offsets, a.T, a.gemv_max);
  if (!sl.valid) return;
  const uint8_t* Wg = sl.shared ? a.sh_gate : (const uint8_t*)a.gate[sl.e];
  const uint8_t* Wu = sl.shared ? a.sh_up : (const uint8_t*)a.up[sl.e];
  if (Wg == nullptr || Wu == nullptr) return;   // not resident: its pairs add nothing
  if (!sl.shared && a.down[sl.e] == nullptr) return;
  const int64_t row0 = (int64_t)blockIdx.x * (4 * a.steps * rps) + (int64_t)wave * a.steps * rps + rig;

  for (int tile = 0; tile < sl.n; tile += TT) {
    int tok[TT];
    int64_t prow[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      tok[i] = -1; prow[i] = 0;
      if (tile + i < sl.n) slot_token(sl, tile + i, a.pairs, a.T, a.k, tok[i], prow[i]);
      if (TT == 1) continue;   // already loaded (token 0)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lir + lpr * c;
        if (tok[i] >= 0 && ch < a.cpr) {
          load_x_chunk<FMT>(a.xq + tok[i] * xrow, ch, xw[i][c], bs[i][c], dx[i][c]);
        } else {
#pragma unroll
          for (int q = 0; q < L::XDW; ++q) xw[i][c][q] = 0;
#pragma unroll
          for (int q = 0; q < L::NBS; ++q) bs[i][c][q] = 0;
          dx[i][c] = 0.0;
        }
      }
    }
    for (int st = 0; st < a.steps; st += UNR) {
      typename L::W wg[UNR][CPL], wu[UNR][CPL];
      int64_t row[UNR];
      bool ok[UNR][CPL];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        row[u] = row0 + (int64_t)(st + u) * rps;
        const bool rv = (st + u) < a.steps && row[u] < a.F;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = lir + lpr * c;
          ok[u][c] = rv && ch < a.cpr;
          if (ok[u][c]) {
            const size_t sbi = (size_t)(row[u] * nb + ch / L::CPS);
            wg[u][c] = L::load(Wg, a.F, nb, row[u], ch / L::CPS, ch % L::CPS);
            wu[u][c] = L::load(Wu, a.F, nb, row[u], ch / L::CPS, ch % L::CPS);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        double ag[TT], au[TT];
#pragma unroll
        for (int i = 0; i < TT; ++i) { ag[i] = 0.0; au[i] = 0.0; }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if (!ok[u][c]) continue;
          const int j = (lir + lpr * c) % L::CPS;
#pragma unroll
          for (int i = 0; i < TT; ++i) {
            if (tok[i] < 0) continue;
            int is[L::SPC];
            L::isums(wg[u][c], xw[i][c], bs[i][c], is);
            ag[i] += L::term(wg[u][c], j, is, bs[i][c], dx[i][c]);
            L::isums(wu[u][c], xw[i][c], bs[i][c], is);
            au[i] += L::term(wu[u][c], j, is, bs[i][c], dx[i][c]);
          }
        }
#pragma unroll
        for (int i = 0; i < TT; ++i) {
          const double g = group_sum_dpp(ag[i], lpr);
          const double uu = group_sum_dpp(au[i], lpr);
          if (lir == lpr - 1 && tok[i] >= 0 && (st + u) < a.steps && row[u] < a.F)
            a.hbuf[prow[i] * a.hstride + row[u]] = (float)(silu64(g) * uu);
        }
      }
    }
  }
}

// One token: gate/up (routing inline from the logits when NPER > 0).
template <int FMT, int CPL, int NPER>
__global__ __launch_bounds__(256) void k_gateup1(GateUpArgs a) {
  gateup1_body<FMT, CPL, NPER>(a, blockIdx.x, blockIdx.y);
}

// q8_K of one lane chunk of h (WPC fp32 values in registers), identical to
// the definition: the block amax is reduced over the GW = 256/WPC lanes of
// the block (aligned lane groups), then id = 127/amax (correctly rounded),
// q = rint(h*id) clamped, d = amax/127, per-16 sums.  Lanes whose chunk is
// absent pass have = false (their values do not enter any valid block).
// dbg (optional): q8_K row the chunk's bytes are also written to.
template <int FMT, int GW>
__device__ __forceinline__ void quant_h_regs(const float* hv, bool have, int ch, int* xw, int* bs, double& dx,
                                             uint8_t* dbg) {
  using L = Fmt<FMT>;
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < L::WPC; ++q) amax = fmaxf(amax, have ? fabsf(hv[q]) : 0.0f);
  amax = group_max_dpp<GW>(amax);
  const float id = amax == 0.0f ? 0.0f : __fdiv_rn(127.0f, amax);
  const bool zero = amax == 0.0f || __builtin_isinf(id);
#pragma unroll
  for (int q = 0; q < L::WPC / 4; ++q) {
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (!zero) {
      q0 = q8_code(hv[4 * q], id); q1 = q8_code(hv[4 * q + 1], id);
      q2 = q8_code(hv[4 * q + 2], id); q3 = q8_code(hv[4 * q + 3], id);
    }
    xw[q] = (int)((uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                  ((uint32_t)(q3 & 255) << 24));
    const int s4 = q0 + q1 + q2 + q3;
    if ((q & 3) == 0) bs[q >> 2] = s4; else bs[q >> 2] += s4;
  }
  dx = zero ? 0.0 : (double)__fdiv_rn(amax, 127.0f);
  if (dbg != nullptr && have) {
    const int j = ch % L::CPS;
    uint8_t* blk = dbg + (size_t)(ch / L::CPS) * kQ8KBytes;
#pragma unroll
    for (int q = 0; q < L::XDW; ++q) gst_u32(blk + 4 + L::xoff(j, q), (uint32_t)xw[q]);
#pragma unroll
    for (int t = 0; t < L::NBS; ++t) gst_i16(blk + 260 + 2 * L::bsidx(j, t), (int16_t)bs[t]);
    if (j == 0) gst_f32(blk, (float)dx);
  }
}

// q8_K of the chunk(s) this lane holds, loading the fp32 h row first (the
// chunk's elements in the order of its activation dwords).
template <int FMT, int CPL>
__device__ __forceinline__ void quant_h_chunks(const float* __restrict__ hrow, int lir, int lpr, int cpr,
                                               bool have, int xw[CPL][Fmt<FMT>::XDW],
                                               int bs[CPL][Fmt<FMT>::NBS], double dx[CPL],
                                               uint8_t* dbg) {
  using L = Fmt<FMT>;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = lir + lpr * c;
    const bool v = have && ch < cpr;
    float hv[L::WPC];
    const float* hb = hrow + (ch / L::CPS) * 256;
#pragma unroll
    for (int q = 0; q < L::WPC / 4; ++q) {
      float4 f = v ? gld_f4(hb + L::xoff(ch % L::CPS, q)) : make_float4(0.f, 0.f, 0.f, 0.f);
      hv[4 * q] = f.x; hv[4 * q + 1] = f.y; hv[4 * q + 2] = f.z; hv[4 * q + 3] = f.w;
    }
    quant_h_regs<FMT, 256 / L::WPC>(hv, v, ch, xw[c], bs[c], dx[c], dbg);
  }
}

template <int FMT, int TT, int CPL, int UNR>
__global__ __launch_bounds__(256) void k_down(DownArgs a) {
  using L = Fmt<FMT>;
  const Slot sl = decode_slot(blockIdx.y, a.mode, a.max_union, a.active, a.offsets, a.T, a.gemv_max);
  if (!sl.valid) return;
  // An expert is resident only if all three of its matrices are present.
  const uint8_t* Wd = sl.shared ? a.sh_down : (const uint8_t*)a.down[sl.e];
  if (!sl.shared && (a.gate[sl.e] == nullptr || a.up[sl.e] == nullptr)) Wd = nullptr;

  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int lpr = a.lpr, rps = kWave / lpr, rig = lane / lpr, lir = lane % lpr;
  const int64_t nb = a.F / 256;
  const int64_t row0 = (int64_t)blockIdx.x * a.rb + (int64_t)wave * a.steps * rps + rig;
  const bool dbg_writer = blockIdx.x == 0 && wave == 0 && rig == 0;

  for (int tile = 0; tile < sl.n; tile += TT) {
    int tok[TT];
    int64_t prow[TT];
    double wt[TT];
    int xw[TT][CPL][L::XDW], bs[TT][CPL][L::NBS];
    double dx[TT][CPL];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      tok[i] = -1; prow[i] = 0; wt[i] = 0.0;
      if (tile + i < sl.n) {
        slot_token(sl, tile + i, a.pairs, a.T, a.k, tok[i], prow[i]);
        wt[i] = sl.shared ? (a.shared_scale ? (double)a.shared_scale[tok[i]] : 1.0) : (double)a.topk_w[prow[i]];
      }
      if (Wd != nullptr) {
        const float* hrow = a.hbuf + (tok[i] >= 0 ? prow[i] : 0) * a.hstride;
        uint8_t* dbg = nullptr;
        uint8_t* hq_base = sl.shared ? a.hq_sh : a.hq;
        if (dbg_writer && tok[i] >= 0 && hq_base != nullptr)
          dbg = hq_base + (sl.shared ? (int64_t)tok[i] : prow[i]) * a.hq_stride;
        quant_h_chunks<FMT, CPL>(hrow, lir, lpr, a.cpr, tok[i] >= 0, xw[i], bs[i], dx[i], dbg);
      }
    }
    for (int st = 0; st < a.steps; st += UNR) {
      typename L::W wd[UNR][CPL];
      int64_t row[UNR];
      bool ok[UNR][CPL];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        row[u] = row0 + (int64_t)(st + u) * rps;
        const bool rv = (st + u) < a.steps && row[u] < a.H && Wd != nullptr;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = lir + lpr * c;
          ok[u][c] = rv && ch < a.cpr;
          if (ok[u][c])
            wd[u][c] = L::load(Wd, a.H, nb, row[u], ch / L::CPS, ch % L::CPS);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        double ay[TT];
#pragma unroll
        for (int i = 0; i < TT; ++i) ay[i] = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if (!ok[u][c]) continue;
          const int j = (lir + lpr * c) % L::CPS;
#pragma unroll
          for (int i = 0; i < TT; ++i) {
            if (tok[i] < 0) continue;
            int is[L::SPC];
            L::isums(wd[u][c], xw[i][c], bs[i][c], is);
            ay[i] += L::term(wd[u][c], j, is, bs[i][c], dx[i][c]);
          }
        }
#pragma unroll
        for (int i = 0; i < TT; ++i) {
          const double yv = group_sum_dpp(ay[i], lpr);
          if (lir == lpr - 1 && tok[i] >= 0 && (st + u) < a.steps && row[u] < a.H)
            a.yp[prow[i] * a.H + row[u]] = (float)(wt[i] * yv);
        }
      }
    }
  }

}

// One token, one chunk per lane: the down rows of one slot's row block, the
// same work and results as k_down<FMT, 1, 1, UNR>, ordered for latency.  The
// fp32 h chunk loads go out first, then the weight loads of up to kDownT1Steps
// wave steps (all issued: a step or row past the end reloads the block's first
// row, a chunk past the row the last chunk), so the q8_K(h) quantization waits
// for h only and the weights of every step are in flight together; the dot
// products then keep only the valid steps' results.
constexpr int kDownT1Steps = 8;
template <int FMT>
__global__ __launch_bounds__(256) void k_down_t1(DownArgs a) {
  using L = Fmt<FMT>;
  constexpr int U = kDownT1Steps;
  const Slot sl = decode_slot(blockIdx.y, a.mode, a.max_union, a.active, a.offsets, a.T, a.gemv_max);
  if (!sl.valid) return;
  // An expert is resident only if all three of its matrices are present.
  const uint8_t* Wd = sl.shared ? a.sh_down : (const uint8_t*)a.down[sl.e];
  if (!sl.shared && (a.gate[sl.e] == nullptr || a.up[sl.e] == nullptr)) Wd = nullptr;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int lpr = a.lpr, rps = kWave / lpr, rig = lane / lpr, lir = lane % lpr;
  const int64_t nb = a.F / 256;
  const int64_t row0 = (int64_t)blockIdx.x * a.rb + (int64_t)wave * a.steps * rps + rig;
  const int64_t row_dup = row0 < a.H ? row0 : a.H - 1;
  const bool dbg_writer = blockIdx.x == 0 && wave == 0 && rig == 0;

  int tok;
  int64_t prow;
  slot_token(sl, 0, a.pairs, a.T, a.k, tok, prow);
  const double wt = sl.shared ? (a.shared_scale ? (double)a.shared_scale[tok] : 1.0) : (double)a.topk_w[prow];
  if (Wd == nullptr) {                        // not resident: its pair adds nothing
    for (int st = 0; st < a.steps; ++st) {
      const int64_t row = row0 + (int64_t)st * rps;
      if (lir == lpr - 1 && row < a.H) a.yp[prow * a.H + row] = (float)(wt * 0.0);
    }
    return;
  }
  const int ch = lir, cl = ch < a.cpr ? ch : a.cpr - 1;
  const bool have = ch < a.cpr;
  // the lane's fp32 h chunk (elements in the order of its activation dwords)
  float hv[L::WPC];
  {
    const float* hb = a.hbuf + prow * a.hstride + (cl / L::CPS) * 256;
#pragma unroll
    for (int q = 0; q < L::WPC / 4; ++q) {
      const float4 f = gld_f4(hb + L::xoff(cl % L::CPS, q));
      hv[4 * q] = f.x; hv[4 * q + 1] = f.y; hv[4 * q + 2] = f.z; hv[4 * q + 3] = f.w;
    }
  }
  typename L::W wd[U];
  auto load_steps = [&](int st0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = row0 + (int64_t)(st0 + u) * rps;
      const int64_t rl = (st0 + u) < a.steps && row < a.H ? row : row_dup;
      wd[u] = L::load(Wd, a.H, nb, rl, cl / L::CPS, cl % L::CPS);
    }
  };
  int xw[L::XDW], bs[L::NBS];
  double dx;
  auto dot_steps = [&](int st0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = row0 + (int64_t)(st0 + u) * rps;
      const bool ok = have && (st0 + u) < a.steps && row < a.H;
      int is[L::SPC];
      L::isums(wd[u], xw, bs, is);
      const double t = L::term(wd[u], cl % L::CPS, is, bs, dx);
      const double yv = group_sum_dpp(ok ? t : 0.0, lpr);
      if (lir == lpr - 1 && (st0 + u) < a.steps && row < a.H) a.yp[prow * a.H + row] = (float)(wt * yv);
    }
  };
  load_steps(0);
  __builtin_amdgcn_sched_barrier(0);
  {
    uint8_t* dbg = nullptr;
    uint8_t* hq_base = sl.shared ? a.hq_sh : a.hq;
    if (dbg_writer && hq_base != nullptr) dbg = hq_base + (sl.shared ? (int64_t)tok : prow) * a.hq_stride;
    quant_h_regs<FMT, 256 / L::WPC>(hv, have, ch, xw, bs, dx, dbg);
  }
  dot_steps(0);
  for (int st0 = U; st0 < a.steps; st0 += U) {   // more than U wave steps (one row per wave step)
    load_steps(st0);
    dot_steps(st0);
  }
}

// y[t] (=|+=) fl32(sum_slot yp[t*k+slot] + yp[T*k+t]) summed in fp64, slots in
// rank order, then the shared expert: the weighted per-pair outputs were
// staged in fp32 by the down kernels (rounding each of the k+1 terms to fp32
// first moves y by about 1e-7 relative, far inside the y tolerance; the
// bit-exact q8_K(h) lies upstream of it).
// Four consecutive outputs per thread, a workgroup per (token, 1024 columns):
// the staged rows of up to kCombineRows slots are loaded before they are
// added (in slot order), so a thread waits for one round trip per that many
// slots.
constexpr int kCombineRows = 12;
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ yp, int64_t T, int64_t H, int k,
                                                 int has_shared, float* __restrict__ y, int accumulate,
                                                 int blocks_per_row) {
  const int64_t t = (int64_t)(blockIdx.x / (unsigned)blocks_per_row);
  const int64_t c = ((int64_t)(blockIdx.x % (unsigned)blocks_per_row) * 256 + threadIdx.x) * 4;
  if (t >= T || c >= H) return;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  const float* base = yp + t * k * H + c;
  for (int s = 0; s < k; s += kCombineRows) {
    float4 v[kCombineRows];
#pragma unroll
    for (int j = 0; j < kCombineRows; ++j)
      if (s + j < k) v[j] = gld_f4(base + (int64_t)(s + j) * H);
#pragma unroll
    for (int j = 0; j < kCombineRows; ++j) {
      if (s + j < k) {
        a0 += (double)v[j].x; a1 += (double)v[j].y; a2 += (double)v[j].z; a3 += (double)v[j].w;
      }
    }
  }
  if (has_shared) {
    const float4 v = gld_f4(yp + (T * k + t) * H + c);
    a0 += (double)v.x; a1 += (double)v.y; a2 += (double)v.z; a3 += (double)v.w;
  }
  float* out = y + t * H + c;
  const bool al = (reinterpret_cast<uintptr_t>(y) & 15) == 0;   // the caller's y may be only 4-byte aligned
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

// One token (decode): down rows and the weighted combine, slot table from
// the gate/up kernel.
template <int FMT, int CPL>
__global__ __launch_bounds__(256) void k_down_rows1(DownArgs a) {
  down1_body<FMT, CPL, kDown1Steps>(a, blockIdx.x);
}

// ------------------------------------------------------------ dispatch

#define MOEQ_GU(F, TT, C) \
  hipLaunchKernelGGL((k_gateup<F, TT, C, (TT == 1 ? 4 : 2)>), grid, dim3(256), 0, s, a)
#define MOEQ_DN(F, TT, C)                                                   \
  if (TT == 1 && C == 1) hipLaunchKernelGGL((k_down_t1<F>), grid, dim3(256), 0, s, a); \
  else hipLaunchKernelGGL((k_down<F, TT, C, 2>), grid, dim3(256), 0, s, a)

#define MOEQ_SWITCH_CPL(M, F, TT)            \
  switch (cpl) {                             \
    case 1: M(F, TT, 1); break;              \
    case 2: M(F, TT, 2); break;              \
    case 4: M(F, TT, 4); break;              \
    default: return -2;                      \
  }
#define MOEQ_SWITCH_TT(M, F)                                  \
  if (tt == 1) { MOEQ_SWITCH_CPL(M, F, 1) }                   \
  else if (tt == 4) { MOEQ_SWITCH_CPL(M, F, 4) }              \
  else return -2;
#define MOEQ_SWITCH_FMT(M)                                    \
  switch (fmt) {                                              \
    case FQ4K: { MOEQ_SWITCH_TT(M, FQ4K) } break;             \
    case FQ6K: { MOEQ_SWITCH_TT(M, FQ6K) } break;             \
    case FQ2K: { MOEQ_SWITCH_TT(M, FQ2K) } break;             \
    case FQ80: { MOEQ_SWITCH_TT(M, FQ80) } break;             \
    case FQ3K: { MOEQ_SWITCH_TT(M, FQ3K) } break;             \
    case FQ5K: { MOEQ_SWITCH_TT(M, FQ5K) } break;             \
    case FQ40: { MOEQ_SWITCH_TT(M, FQ40) } break;             \
    case FQ51: { MOEQ_SWITCH_TT(M, FQ51) } break;             \
    default: return -2;                                       \
  }

int launch_gateup(int fmt, int tt, int cpl, dim3 grid, const GateUpArgs& a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  MOEQ_SWITCH_FMT(MOEQ_GU)
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

#define MOEQ_G1(F, NP, C) hipLaunchKernelGGL((k_gateup1<F, C, NP>), grid, dim3(256), 0, s, a)
#define MOEQ_G1_CPL(F, NP)                    \
  switch (cpl) {                              \
    case 1: MOEQ_G1(F, NP, 1); break;         \
    case 2: MOEQ_G1(F, NP, 2); break;         \
    case 4: MOEQ_G1(F, NP, 4); break;         \
    default: return -2;                       \
  }
#define MOEQ_G1_NP(F)                                            \
  switch (nper) {                                                \
    case 0: { MOEQ_G1_CPL(F, 0) } break;                         \
    case 4: { MOEQ_G1_CPL(F, 4) } break;                         \
    case 8: { MOEQ_G1_CPL(F, 8) } break;                         \
    case 16: { MOEQ_G1_CPL(F, 16) } break;                       \
    case 64: { MOEQ_G1_CPL(F, 64) } break;                       \
    default: return -2;                                          \
  }

int launch_gateup1(int fmt, int nper, int cpl, dim3 grid, const GateUpArgs& a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  switch (fmt) {
    case FQ4K: { MOEQ_G1_NP(FQ4K) } break;
    case FQ6K: { MOEQ_G1_NP(FQ6K) } break;
    case FQ2K: { MOEQ_G1_NP(FQ2K) } break;
    case FQ80: { MOEQ_G1_NP(FQ80) } break;
    case FQ3K: { MOEQ_G1_NP(FQ3K) } break;
    case FQ5K: { MOEQ_G1_NP(FQ5K) } break;
    case FQ40: { MOEQ_G1_NP(FQ40) } break;
    case FQ51: { MOEQ_G1_NP(FQ51) } break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_down(int fmt, int tt, int cpl, dim3 grid, const DownArgs& a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return 0;
  MOEQ_SWITCH_FMT(MOEQ_DN)
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

#define MOEQ_R1(FM, TT, C) \
  hipLaunchKernelGGL((k_down_rows1<FM, C>), grid, dim3(256), (size_t)(a.k + a.has_shared) * (a.F / 256) * kLdsQ8, s, a)

int launch_down_rows1(int fmt, int cpl, dim3 grid, const DownArgs& a, hipStream_t s) {
  if (grid.x == 0) return 0;
  const int tt = 1;
  MOEQ_SWITCH_FMT(MOEQ_R1)
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_combine(const float* yp, int64_t T, int64_t H, int k, int has_shared, float* y, int accumulate,
                   hipStream_t s) {
  if (T * H == 0) return 0;
  if (H % 4 != 0) return -2;                      // (H is a multiple of 256)
  const int bpr = (int)((H / 4 + 255) / 256);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(T * bpr)), dim3(256), 0, s, yp, T, H, k, has_shared, y, accumulate,
                     bpr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moeq
