// One-token (decode) expert FFN bodies: gate/up rows of one slot with the
// routing taken inline, and down rows of every slot with the combine.
#pragma once
#include "formats.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace moeq {

// The routing outputs of one token, written by one wave that holds the
// winners in rank order (lane s < k: expert my_i, weight my_w): ids and
// weights, then the lists (pairs ordered by expert; for one token the pair of
// slot s is s) and the expert union.
__device__ void write_routing_t1(const GateUpArgs& a, int my_i, float my_w) {
  const int lane = lane_id(), k = a.k;
  int pos = 0;
  for (int j = 0; j < k; ++j) {
    const int idj = __builtin_amdgcn_readlane(my_i, j);
    pos += (lane < k && idj < my_i) ? 1 : 0;
  }
  if (lane < k) {
    a.ids_out[lane] = my_i;
    a.w_out[lane] = my_w;
    a.active_out[1 + pos] = my_i;
    a.pairs_out[pos] = lane;
  }
  if (lane == 0) a.active_out[0] = k;
  for (int64_t e0 = 0; e0 <= a.E; e0 += kWave) {
    const int64_t e = e0 + lane;
    int c = 0;
    for (int j = 0; j < k; ++j) c += __builtin_amdgcn_readlane(my_i, j) < e ? 1 : 0;
    if (e <= a.E) a.offsets_out[e] = c;
  }
}

// One token, gate/up rows of one workgroup (row block bx of slot `slot`).
// Slot u is the u-th ranked expert (u == k: the shared expert);
// with NPER > 0 the workgroup routes inline from the logits (every wave runs
// the same register top-k, so all workgroups agree), otherwise it reads
// topk_ids.  The token's activation chunks are loaded after the weight
// loads: during the routing only the logits and pointer tables are in flight.
template <int FMT, int CPL, int NPER>
__device__ __forceinline__ void gateup1_body(const GateUpArgs& a, int bx, int slot) {
  using L = Fmt<FMT>;
  constexpr int UNR = 2;   // the host gives at most 2 wave steps (2 / rows per step)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int lpr = a.lpr, rps = kWave / lpr, rig = lane / lpr, lir = lane % lpr;
  const int64_t nb = a.H / 256;
  const bool shared = a.mode == kModeShared || (a.mode == kModeBoth && slot == a.k);
  const uint8_t *Wg, *Wu;
  int64_t prow;
  const void* Wd;
  double wt;
  if (shared) {
    Wg = a.sh_gate; Wu = a.sh_up; prow = a.k;
    Wd = a.sh_down_rec;
    wt = a.shared_scale ? (double)a.shared_scale[0] : 1.0;
  } else {
    int e;
    if constexpr (NPER > 0) {
      // Every wave routes for itself (the same register top-k from the
      // logits in every wave and workgroup), so no wave waits for another.
      {
        uint64_t pg[NPER <= 8 ? NPER : 1], pu[NPER <= 8 ? NPER : 1], pd[NPER <= 8 ? NPER : 1];
        if constexpr (NPER <= 8) {
          // candidates' matrix pointers load with the logits; the winner's
          // owner lane hands them over (no dependent table load)
#pragma unroll
          for (int i = 0; i < NPER; ++i) {
            const int64_t ec = lane + (int64_t)kWave * i;
            pg[i] = ec < a.E ? (uint64_t)a.gate[ec] : 0;
            pu[i] = ec < a.E ? (uint64_t)a.up[ec] : 0;
            pd[i] = ec < a.E ? (uint64_t)a.down[ec] : 0;
          }
        }
        int my_i;
        float my_w;
        topk_wave_regs<NPER>(a.logits, a.E, a.k, a.gating, a.scale, my_i, my_w);
        if (bx == 0 && slot == 0 && wave == 0) write_routing_t1(a, my_i, my_w);
        e = __builtin_amdgcn_readlane(my_i, slot);
        const float wsel = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), slot));
        uint64_t g0, u0, d0;
        if constexpr (NPER <= 8) {
          const int owner = e & (kWave - 1), idx = e / kWave;
          g0 = pg[0]; u0 = pu[0]; d0 = pd[0];
#pragma unroll
          for (int i = 1; i < NPER; ++i) {
            g0 = idx == i ? pg[i] : g0;
            u0 = idx == i ? pu[i] : u0;
            d0 = idx == i ? pd[i] : d0;
          }
          auto bcast = [&](uint64_t v) {
            const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, owner);
            const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), owner);
            return (uint64_t)lo | ((uint64_t)hi << 32);
          };
          g0 = bcast(g0); u0 = bcast(u0); d0 = bcast(d0);
        } else {
          g0 = (uint64_t)a.gate[e]; u0 = (uint64_t)a.up[e]; d0 = (uint64_t)a.down[e];
        }
        Wg = (const uint8_t*)g0;
        Wu = (const uint8_t*)u0;
        Wd = (const void*)d0;
        wt = (double)wsel;
      }
    } else {
      e = a.topk_ids[slot];
      wt = (double)a.topk_w[slot];
      Wg = (const uint8_t*)a.gate[e];
      Wu = (const uint8_t*)a.up[e];
      Wd = a.down[e];
    }
    if (Wd == nullptr || Wu == nullptr) Wg = nullptr;
    prow = slot;
  }
  if (a.slots != nullptr && threadIdx.x < kSlotCopies) {
    // copy c of this slot's record comes from the workgroup of this grid row
    // whose flat index is c modulo 8; when the row has fewer than 8
    // workgroups, workgroup 0 also writes the copies no workgroup sits on
    const int gx = (int)gridDim.x, c = (int)threadIdx.x;
    const int r = (c - gx * (int)blockIdx.y) & (kSlotCopies - 1);
    if (r == bx || (bx == 0 && r >= gx)) {
      SlotRec* rec = a.slots + (int64_t)c * (a.k + 1) + (shared ? a.k : slot);
      rec->wd = (Wg == nullptr || Wu == nullptr) ? nullptr : Wd;
      rec->wt = wt;
    }
  }
  if (Wg == nullptr || Wu == nullptr) return;   // not resident: its pair adds nothing
  // At most UNR wave steps (the host's bound), so one pass covers the rows:
  // the weight loads go out first, then the token's activation chunks, which
  // the dot products need together with them.  Every load is issued (a step
  // or row past the end reloads the wave's first row, a chunk past the row
  // the last chunk; none of them is used): a conditional load would leave
  // the compiler register copies that wait for it before the next loads.
  const int64_t row0 = (int64_t)bx * (4 * a.steps * rps) + (int64_t)wave * a.steps * rps + rig;
  const int64_t row_dup = row0 < a.F ? row0 : a.F - 1;
  typename L::W wg[UNR][CPL], wu[UNR][CPL];
  int64_t row[UNR];
  bool ok[UNR][CPL];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    row[u] = row0 + (int64_t)u * rps;
    const bool rv = u < a.steps && row[u] < a.F;
    const int64_t rl = rv ? row[u] : row_dup;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lir + lpr * c, cl = ch < a.cpr ? ch : a.cpr - 1;
      ok[u][c] = rv && ch < a.cpr;
      wg[u][c] = L::load(Wg, a.F, nb, rl, cl / L::CPS, cl % L::CPS);
      wu[u][c] = L::load(Wu, a.F, nb, rl, cl / L::CPS, cl % L::CPS);
    }
  }
  int xw[CPL][L::XDW], bs[CPL][L::NBS];
  double dx[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = lir + lpr * c;
    load_x_chunk<FMT>(a.xq, ch < a.cpr ? ch : a.cpr - 1, xw[c], bs[c], dx[c]);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any arithmetic below
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    double ag = 0.0, au = 0.0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      // computed on every lane (on the reloaded data where not ok), kept
      // where ok: a branch here would let the compiler sink loads into it
      const int ch = lir + lpr * c, j = (ch < a.cpr ? ch : a.cpr - 1) % L::CPS;
      int is[L::SPC];
      L::isums(wg[u][c], xw[c], bs[c], is);
      const double tg = L::term(wg[u][c], j, is, bs[c], dx[c]);
      L::isums(wu[u][c], xw[c], bs[c], is);
      const double tu = L::term(wu[u][c], j, is, bs[c], dx[c]);
      ag += ok[u][c] ? tg : 0.0;
      au += ok[u][c] ? tu : 0.0;
    }
    const double g = group_sum_dpp(ag, lpr);
    const double uu = group_sum_dpp(au, lpr);
    if (lir == lpr - 1 && u < a.steps && row[u] < a.F)
      gst_f32(a.hbuf + prow * a.hstride + row[u], (float)(silu64(g) * uu));
  }
}


// LDS q8_K block of the down kernels: f32 d | 12 pad | i8 q[256] | i16 bsums[16]
constexpr int kLdsQ8 = 304;

template <int FMT>
__device__ __forceinline__ void load_x_chunk_lds(const uint8_t* xrow, int c, int* xw, int* bs, double& dx) {
  using L = Fmt<FMT>;
  const int j = c % L::CPS;
  const uint8_t* blk = xrow + (c / L::CPS) * kLdsQ8;
  dx = (double)*reinterpret_cast<const float*>(blk);
#pragma unroll
  for (int i = 0; i < L::XDW; i += 4) {   // dwords i .. i+3 are contiguous in every format
    const uint4 v = *reinterpret_cast<const uint4*>(blk + 16 + L::xoff(j, i));
    xw[i] = (int)v.x; xw[i + 1] = (int)v.y; xw[i + 2] = (int)v.z; xw[i + 3] = (int)v.w;
  }
#pragma unroll
  for (int t = 0; t < L::NBS; ++t) bs[t] = (int)(int16_t)ld_u16(blk + 272 + 2 * L::bsidx(j, t));
}

// One token, down rows of one workgroup (row block bx).  The workgroup owns
// ST wave steps of rps output rows for every selected expert and
// the shared one.  It turns the k+1 fp32 h rows into q8_K blocks in LDS once
// (a pure function of h, identical in every workgroup; workgroup 0 also
// stores them as the q8_K(h) view) while the weight loads of the first round
// of slots are in flight.  Waves then take slots round-robin, read their
// activation chunks from LDS, and leave w * (W_d h^) per (slot rank, row) in
// LDS; the sum over slots in rank order, then the shared expert, happens in
// the workgroup.
static_assert(kLdsQ8Blocks * kLdsQ8Blocks < 65536, "the 16-bit reciprocal quotient of down1_body needs b * nb < 2^16");

template <int FMT, int CPL, int ST>
__device__ __forceinline__ void down1_body(const DownArgs& a, int bx) {
  using L = Fmt<FMT>;
  constexpr int kMaxSlots = 33, kMaxRows = 64;
  constexpr int SG = CPL == 1 ? 3 : 1;      // slots whose loads are in flight together
  extern __shared__ __align__(16) uint8_t hq_lds[];   // [n_slots][nbF] q8_K blocks
  __shared__ double yps[kMaxSlots][kMaxRows];
  __shared__ const uint8_t* swd[kMaxSlots];
  __shared__ double swt[kMaxSlots];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int lpr = a.lpr, rps = kWave / lpr, rig = lane / lpr, lir = lane % lpr;
  const int64_t nb = a.F / 256;
  const int rows_wg = rps * ST;            // at most kMaxRows (checked by the host)
  const int64_t row_base = (int64_t)bx * rows_wg;
  const int n_routed = a.k;
  const int n_slots = n_routed + a.has_shared;
  const int nblk = n_slots * (int)nb;       // at most kLdsQ8Blocks (checked by the host)
  // block b of the h rows is block b - s*nb of slot s = b / nb; with
  // b < kLdsQ8Blocks, nb <= kLdsQ8Blocks the quotient is (b * inv_nb) >> 16
  const uint32_t inv_nb = (65536u + (uint32_t)nb - 1) / (uint32_t)nb;

  // The down weight loads wait for the slot table the gate/up kernel left
  // (each slot's down matrix and weight): read it first, from the copy of
  // this workgroup's XCD, before the h loads are in flight.
  __shared__ const uint8_t* sfb;            // first resident slot's down matrix, null if none
  // y (=|+=) result: the old y of this thread's output row is loaded now, with
  // the slot records, so the final sum does not wait for a round trip
  float y_old = 0.0f;
  if (a.accumulate && threadIdx.x < rows_wg && row_base + threadIdx.x < a.H) y_old = gld_f32(a.y + row_base + threadIdx.x);
  const uint8_t* my_wd = nullptr;
  if (threadIdx.x < n_slots) {
    const SlotRec* rec = a.slots + (int64_t)(bx & (kSlotCopies - 1)) * (a.k + 1) + threadIdx.x;
    my_wd = (const uint8_t*)rec->wd;
    swd[threadIdx.x] = my_wd;
    swt[threadIdx.x] = rec->wt;
  }
  if (wave == 0) {                           // n_slots <= kMaxSlots <= 64: all in wave 0
    const uint64_t res = __ballot(my_wd != nullptr);
    const uint64_t first = __shfl((uint64_t)my_wd, res ? __builtin_ctzll(res) : 0);
    if (lane == 0) sfb = res ? (const uint8_t*)first : nullptr;
  }
  // this wave's q8_K(h) blocks (wave, wave+4, ...): fp32 loads
  float4 hv[kQ8PerWave];
#pragma unroll
  for (int j = 0; j < kQ8PerWave; ++j) {
    const int b = wave + 4 * j;
    if (b < nblk) {
      const int s = (int)(((uint32_t)b * inv_nb) >> 16), bb = b - s * (int)nb;
      hv[j] = gld_f4(a.hbuf + (int64_t)s * a.hstride + bb * 256 + 4 * lane);
    }
  }
  __syncthreads();
  const uint8_t* const fb = sfb;
  if (fb == nullptr) {                       // no resident slot: every pair adds nothing
    if (threadIdx.x < rows_wg) {
      const int64_t rr = row_base + threadIdx.x;
      if (rr < a.H) gst_f32(a.y + rr, a.accumulate ? (float)((double)y_old + 0.0) : 0.0f);
    }
    return;
  }

  // weight loads of one round: SG slots of this wave, every wave step of the
  // workgroup's rows (all in flight together).  Every load is issued (a slot
  // past the list or not resident reads the first resident slot's rows, a
  // row or chunk past the end the last one; their products are discarded),
  // so the q8_K(h) work below waits for the h loads only, not for these.
  typename L::W w[ST][SG][CPL];
  bool okk[ST][SG][CPL];
  auto issue = [&](int s0) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int64_t row = row_base + (int64_t)st * rps + rig;
      const int64_t rl = row < a.H ? row : a.H - 1;
#pragma unroll
      for (int j = 0; j < SG; ++j) {
        const int s = s0 + 4 * j;
        const uint8_t* W = s < n_slots ? swd[s] : nullptr;
        const uint8_t* Wl = W != nullptr ? W : fb;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = lir + lpr * c, cl = ch < a.cpr ? ch : a.cpr - 1;
          okk[st][j][c] = W != nullptr && ch < a.cpr && row < a.H;
          w[st][j][c] = L::load(Wl, a.H, nb, rl, cl / L::CPS, cl % L::CPS);
        }
      }
    }
  };
  issue(wave);                               // first round in flight during the q8_K(h) work

  // q8_K(h) into LDS
#pragma unroll
  for (int j = 0; j < kQ8PerWave; ++j) {
    const int b = wave + 4 * j;
    if (b < nblk) {
      const int s = (int)(((uint32_t)b * inv_nb) >> 16), bb = b - s * (int)nb;
      uint8_t* o = hq_lds + b * kLdsQ8;
      float amax = fmaxf(fmaxf(fabsf(hv[j].x), fabsf(hv[j].y)), fmaxf(fabsf(hv[j].z), fabsf(hv[j].w)));
      amax = wave_max_f(amax);
      const float id = amax == 0.0f ? 0.0f : __fdiv_rn(127.0f, amax);
      const bool zero = amax == 0.0f || __builtin_isinf(id);
      int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
      if (!zero) {
        q0 = q8_code(hv[j].x, id); q1 = q8_code(hv[j].y, id);
        q2 = q8_code(hv[j].z, id); q3 = q8_code(hv[j].w, id);
      }
      const uint32_t qw = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                          ((uint32_t)(q3 & 255) << 24);
      int sum4 = q0 + q1 + q2 + q3;
      sum4 += dpp_all_i<kDppXor1>(sum4);
      sum4 += dpp_all_i<kDppXor2>(sum4);
      const float dq = zero ? 0.0f : __fdiv_rn(amax, 127.0f);
      *reinterpret_cast<uint32_t*>(o + 16 + 4 * lane) = qw;
      if ((lane & 3) == 0) *reinterpret_cast<int16_t*>(o + 272 + 2 * (lane >> 2)) = (int16_t)sum4;
      if (lane == 0) *reinterpret_cast<float*>(o) = dq;
    }
  }
  __syncthreads();
  // workgroup 0 stores the q8_K(h) view from LDS (here rather than in the
  // loop above, whose waits would otherwise cover weight loads behind these
  // stores)
  if (bx == 0) {
    for (int b = wave; b < nblk; b += 4) {
      const int s = (int)(((uint32_t)b * inv_nb) >> 16), bb = b - s * (int)nb;
      uint8_t* view = s >= n_routed ? a.hq_sh : a.hq;
      if (view == nullptr || swd[s] == nullptr) continue;
      const uint8_t* o = hq_lds + b * kLdsQ8;
      uint8_t* gq = view + (s >= n_routed ? 0 : (int64_t)s) * a.hq_stride + bb * kQ8KBytes;
      gst_u32(gq + 4 + 4 * lane, *reinterpret_cast<const uint32_t*>(o + 16 + 4 * lane));
      if (lane < 16) gst_i16(gq + 260 + 2 * lane, *reinterpret_cast<const int16_t*>(o + 272 + 2 * lane));
      if (lane == 0) gst_f32(gq, *reinterpret_cast<const float*>(o));
    }
  }

  for (int s0 = wave; s0 < n_slots; s0 += 4 * SG) {
    if (s0 != wave) issue(s0);
#pragma unroll
    for (int st = 0; st < ST; ++st) {
#pragma unroll
      for (int j = 0; j < SG; ++j) {
        const int s = s0 + 4 * j;
        double ay = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          // every lane computes (on the reloaded data where not okk) and
          // keeps the product where okk: no branch to sink the loads into
          const int ch = lir + lpr * c, cl = ch < a.cpr ? ch : a.cpr - 1;
          const int sl = s < n_slots ? s : 0;
          int xw[L::XDW], bs[L::NBS];
          double dx;
          load_x_chunk_lds<FMT>(hq_lds + (int64_t)sl * nb * kLdsQ8, cl, xw, bs, dx);
          int is[L::SPC];
          L::isums(w[st][j][c], xw, bs, is);
          const double t = L::term(w[st][j][c], cl % L::CPS, is, bs, dx);
          ay += okk[st][j][c] ? t : 0.0;
        }
        const double yv = group_sum_dpp(ay, lpr);
        if (s < n_slots && lir == lpr - 1) yps[s][st * rps + rig] = swt[s] * yv;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < rows_wg) {
    const int64_t rr = row_base + threadIdx.x;
    if (rr < a.H) {
      double acc = 0.0;
      for (int p = 0; p < n_routed; ++p) acc += yps[p][threadIdx.x];
      if (a.has_shared) acc += yps[n_routed][threadIdx.x];
      gst_f32(a.y + rr, a.accumulate ? (float)((double)y_old + acc) : (float)acc);
    }
  }
}

}  // namespace moeq
