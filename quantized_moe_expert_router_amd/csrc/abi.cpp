// C ABI of libmoeq: argument validation on the host, workspace layout, and
// kernel dispatch.  Every check runs before anything is enqueued.
#include <algorithm>
#include <cfloat>
#include <climits>

#include "../../include/moeq.h"
#include "formats.hpp"
#include "launch.hpp"
#include "mfma_plan.hpp"
#include "ceilings.hpp"
#include "route_small.hpp"

using namespace moeq;

namespace {

constexpr int64_t kMaxE = 4096;
static_assert(kMaxE <= kPlanMaxE, "the tile planner's LDS scratch holds kPlanMaxE + 1 entries");
constexpr int kMaxK = 32;
constexpr int64_t kMaxStack = 4096;   // layers per moeq_moe_stack call
constexpr int kRowBlock = 64;     // rows per expert-major down work item

bool fmt_ok(int f) {
  return f == MOEQ_Q4_K || f == MOEQ_Q6_K || f == MOEQ_Q2_K || f == MOEQ_Q8_0 || f == MOEQ_Q3_K || f == MOEQ_Q5_K ||
         f == MOEQ_Q4_0 || f == MOEQ_Q5_1;
}
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
int hip_status(int rc) { return rc == 0 ? MOEQ_OK : (rc == -2 ? MOEQ_E_UNSUPPORTED : MOEQ_E_HIP); }

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Lane geometry of a GEMV over matrices with `cols` columns in format fmt.
struct LaneGeo {
  int cpr, lpr, rps, cpl;
};
bool lane_geo(int fmt, int64_t cols, LaneGeo* g) {
  const int wpc = geo_of(fmt).wpc;
  const int64_t cpr = cols / wpc;
  if (cpr < 1 || cpr > 256) return false;
  g->cpr = (int)cpr;
  if (cpr <= 64) {
    g->lpr = next_pow2((int)cpr);
    g->cpl = 1;
  } else {
    g->lpr = 64;
    g->cpl = cpr <= 128 ? 2 : 4;
  }
  g->rps = 64 / g->lpr;
  return true;
}

// Rows per expert up to which the dot-product (GEMV) kernels run; experts with
// more rows (and the shared expert when T exceeds it) go to the int8 MFMA
// grouped GEMM.  AUTO: one token runs the one-token dot-product kernels; more
// tokens run every expert on matrix cores (8-row tiles for experts with at
// most 8 rows).  Measured on MI355X, the MFMA tiles beat the dot-product
// kernels from one row per expert up whenever T > 1 (verify, 16-token chunk,
// prefill), because the per-token dot products leave the vector ALUs.
int gemv_max_of(const moeq_ffn_desc* d) {
  if (d->path == MOEQ_PATH_GEMV) return INT32_MAX;
  if (d->path == MOEQ_PATH_MFMA) return 0;
  return d->T == 1 ? INT32_MAX : 0;
}

// Chunks of at most kAllThinT tokens put every routed expert in 8-row tiles
// (at most two per expert): no expert then needs a 32-row tile, and the two
// 32-row launches, which would find no tile, are left out.
constexpr int kThinT = kThinRows;    // rows of the MFMA tiles of experts with few rows
constexpr int kAllThinT = 2 * kThinT;
// The most rows an expert may have and still take 8-row tiles.
int thin_max_of(const moeq_ffn_desc* d) { return d->T <= kAllThinT ? kAllThinT : kThinT; }

// Upper bound on the 32-row MFMA tiles of the routed experts: sum over experts
// with more than thr rows of ceil(n_e / 32) <= (T*k + 31 * U) / 32, with U the
// number of such experts.
int64_t mfma_max_tiles(const moeq_ffn_desc* d, int thr) {
  const int64_t P = d->T * d->k;
  if (d->T <= thr || d->T <= kAllThinT) return 0;
  const int64_t U = std::min<int64_t>(d->E, P / (thr + 1));
  return (P + 31 * U) / 32 + 1;
}
// Upper bound on the 8-row MFMA tiles: one per expert with more than thr rows
// when only experts of at most 8 rows take them; otherwise (every expert,
// n_e <= T rows) sum ceil(n_e / 8) <= U + (T*k - U) / 8 (each tile past an
// expert's first takes 8 more rows) and <= U * ceil(T / 8).
int64_t mfma_max_thin(const moeq_ffn_desc* d, int thr) {
  const int64_t P = d->T * d->k;
  if (d->T <= thr) return 0;
  const int64_t U = std::min<int64_t>(d->E, P / (thr + 1));
  if (thin_max_of(d) == kThinT) return U;
  return std::min<int64_t>(U + (P - U) / kThinT, U * ((d->T + kThinT - 1) / kThinT));
}

struct FfnLayout {
  int64_t Fmax, nrows, max_tiles, max_thin;
  size_t off_h, off_yp, off_hq, off_hqs, off_slots, off_tiles, off_thin, off_count, total;
};
FfnLayout ffn_layout(const moeq_ffn_desc* d) {
  FfnLayout L{};
  const bool sh = d->sh_gate != nullptr;
  L.Fmax = sh ? std::max(d->F, d->F_shared) : d->F;
  L.nrows = d->T * d->k + d->T;
  L.max_tiles = mfma_max_tiles(d, gemv_max_of(d));
  L.max_thin = mfma_max_thin(d, gemv_max_of(d));
  size_t o = 0;
  L.off_h = o;   o += align256((size_t)L.nrows * L.Fmax * sizeof(float));
  L.off_yp = o;  o += align256((size_t)L.nrows * d->H * sizeof(float));
  L.off_hq = o;  o += align256((size_t)d->T * d->k * (d->F / 256) * kQ8KBytes);
  L.off_hqs = o; o += align256(sh ? (size_t)d->T * (d->F_shared / 256) * kQ8KBytes : 0);
  L.off_slots = o; o += align256((size_t)kSlotCopies * (d->k + 1) * sizeof(SlotRec));
  L.off_tiles = o; o += align256((size_t)L.max_tiles * sizeof(int4));
  L.off_thin = o;  o += align256((size_t)L.max_thin * sizeof(int4));
  L.off_count = o; o += 256;                     // [0]: 32-row tiles, [1]: 8-row tiles
  L.total = o;
  return L;
}

// The MFMA tile lists of the FFN workspace at wsb.
MfmaPlan ffn_plan(const moeq_ffn_desc* d, const FfnLayout& L, uint8_t* wsb) {
  int32_t* count = (int32_t*)(wsb + L.off_count);
  return MfmaPlan{gemv_max_of(d), (int)L.max_tiles, (int4*)(wsb + L.off_tiles), count,
                  (int4*)(wsb + L.off_thin), count + 1, thin_max_of(d)};
}

// The routed 8-row tiles take the fp32-h variant (see launch_mfma) when both
// of their launches can and the tiles are few (256-row gate/up workgroups
// would not fill the chip; with many tiles the q8_K(h) epilogue is faster).
bool routed_thin_hf(const moeq_ffn_desc* d) {
  return !fmt_sub_scaled(d->fmt_gate) && !fmt_sub_scaled(d->fmt_down) && d->H / 256 <= kHfMaxBlocks &&
         d->F / 256 <= kHfMaxBlocks && ffn_layout(d).max_thin * (d->F / 256) < kHfMaxWorkgroups;
}

// Chunks of 2..8 tokens with at most 64 pairs and at most 512 experts, every
// expert on the MFMA path in fp32-h 8-row tiles, route inline in their first
// gate/up launch (route_small.hpp) instead of in a selection launch.
bool small_route_ok(const moeq_ffn_desc* d) {
  if (d->T < 2 || d->T > kSmallRouteMaxT || d->T * d->k > kSmallPairs || d->E > kSmallRouteMaxE) return false;
  return gemv_max_of(d) == 0 && routed_thin_hf(d);
}

int check_ffn_desc(const moeq_ffn_desc* d) {
  if (!d) return MOEQ_E_INVALID;
  if (d->T < 0 || d->H <= 0 || d->F <= 0 || d->E < 1 || d->E > kMaxE) return MOEQ_E_INVALID;
  if (d->H % 256 || d->F % 256) return MOEQ_E_INVALID;
  if (d->k < 1 || d->k > kMaxK || d->k > d->E) return MOEQ_E_INVALID;
  if (d->T * d->k > INT32_MAX / 2) return MOEQ_E_INVALID;
  if (!fmt_ok(d->fmt_gate) || !fmt_ok(d->fmt_up) || !fmt_ok(d->fmt_down)) return MOEQ_E_UNSUPPORTED;
  if (d->fmt_gate != d->fmt_up) return MOEQ_E_UNSUPPORTED;
  if (!d->gate || !d->up || !d->down) return MOEQ_E_INVALID;
  const int nsh = (d->sh_gate != nullptr) + (d->sh_up != nullptr) + (d->sh_down != nullptr);
  if (nsh != 0 && nsh != 3) return MOEQ_E_INVALID;
  if (nsh == 3) {
    if (d->F_shared <= 0 || d->F_shared % 256) return MOEQ_E_INVALID;
    if (!fmt_ok(d->sh_fmt_gate) || !fmt_ok(d->sh_fmt_up) || !fmt_ok(d->sh_fmt_down)) return MOEQ_E_UNSUPPORTED;
    if (d->sh_fmt_gate != d->sh_fmt_up) return MOEQ_E_UNSUPPORTED;
  }
  if (d->path != MOEQ_PATH_AUTO && d->path != MOEQ_PATH_GEMV && d->path != MOEQ_PATH_MFMA)
    return MOEQ_E_INVALID;
  if (d->accumulate != 0 && d->accumulate != 1) return MOEQ_E_INVALID;
  const int naux = (d->aux_stream != nullptr) + (d->aux_fork != nullptr) + (d->aux_join != nullptr);
  if (naux != 0 && naux != 3) return MOEQ_E_INVALID;
  LaneGeo g;
  if (!lane_geo(d->fmt_gate, d->H, &g) || !lane_geo(d->fmt_down, d->F, &g)) return MOEQ_E_UNSUPPORTED;
  if (nsh == 3 && (!lane_geo(d->sh_fmt_gate, d->H, &g) || !lane_geo(d->sh_fmt_down, d->F_shared, &g)))
    return MOEQ_E_UNSUPPORTED;
  return MOEQ_OK;
}

}  // namespace

extern "C" {

const char* moeq_status_string(int status) {
  switch (status) {
    case MOEQ_OK: return "ok";
    case MOEQ_E_INVALID: return "invalid argument";
    case MOEQ_E_UNSUPPORTED: return "unsupported format, gating, path or shape";
    case MOEQ_E_WORKSPACE: return "workspace too small";
    case MOEQ_E_HIP: return "HIP launch failed";
    case MOEQ_E_STATIC_LIMIT: return "needs more workspace than the static 32 MiB of moeq_moe_layer_noalloc";
  }
  return "unknown status";
}

int moeq_quantize_q8K(const float* x, int64_t rows, int64_t cols, void* out, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 256) return MOEQ_E_INVALID;
  if (rows == 0) return MOEQ_OK;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 4)) return MOEQ_E_INVALID;
  return hip_status(launch_quantize_q8K(x, rows, cols, out, (hipStream_t)stream));
}

size_t moeq_route_workspace(const moeq_route_desc* d) {
  if (!d || d->T < 0 || d->E < 1) return 0;
  return route_ws_bytes(d->T, d->E, d->H);
}

int moeq_route(const moeq_route_desc* d, const float* x, const float* w_router, const float* bias,
               double* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* pairs,
               int32_t* active, void* x_q8K, void* ws, size_t ws_bytes, void* stream) {
  if (!d) return MOEQ_E_INVALID;
  if (d->T < 0 || d->H <= 0 || d->H % 4 || d->E < 1 || d->E > kMaxE) return MOEQ_E_INVALID;
  if (d->k < 1 || d->k > kMaxK || d->k > d->E) return MOEQ_E_INVALID;
  if (d->gating < MOEQ_SOFTMAX_TOPK || d->gating > MOEQ_SIGMOID_TOPK) return MOEQ_E_UNSUPPORTED;
  if (d->T * (int64_t)d->k > INT32_MAX / 2) return MOEQ_E_INVALID;
  if (!expert_offsets || !active) return MOEQ_E_INVALID;
  if (d->T > 0) {
    if (!x || !w_router || !topk_ids || !topk_w || !pairs) return MOEQ_E_INVALID;
    if (!aligned(x, 16) || !aligned(w_router, 16) || (bias && !aligned(bias, 4))) return MOEQ_E_INVALID;
    if (logits && !aligned(logits, 8)) return MOEQ_E_INVALID;
    if (x_q8K && (d->H % 256 || !aligned(x_q8K, 4))) return MOEQ_E_INVALID;
    if (!ws || !aligned(ws, 256)) return MOEQ_E_INVALID;
    if (ws_bytes < route_ws_bytes(d->T, d->E, d->H)) return MOEQ_E_WORKSPACE;
  }
  return hip_status(launch_route(d->T, d->H, d->E, d->k, d->gating, d->scale, x, w_router, bias, logits,
                                 topk_ids, topk_w, expert_offsets, pairs, active, x_q8K, ws,
                                 (hipStream_t)stream));
}

size_t moeq_packed_bytes(int32_t fmt, int64_t rows, int64_t cols) {
  if (!fmt_ok(fmt) || rows <= 0 || cols <= 0 || cols % 256) return 0;
  return packed_bytes_of(fmt, rows, cols);
}

int moeq_pack_experts(int32_t fmt, const void* aos, int64_t n_mats, int64_t rows, int64_t cols, void* packed,
                      void* stream) {
  if (!fmt_ok(fmt)) return MOEQ_E_UNSUPPORTED;
  if (n_mats < 0 || rows <= 0 || cols <= 0 || cols % 256) return MOEQ_E_INVALID;
  if (n_mats == 0) return MOEQ_OK;
  if (!aos || !packed || !aligned(packed, 256)) return MOEQ_E_INVALID;
  return hip_status(launch_pack(fmt, aos, n_mats, rows, cols, packed, (hipStream_t)stream));
}

size_t moeq_expert_ffn_workspace(const moeq_ffn_desc* d) {
  if (check_ffn_desc(d) != MOEQ_OK) return 0;
  return ffn_layout(d).total;
}

namespace {

// Routing the one-token gate/up kernel does itself from the logits (fused
// layer path); null when the routing comes from moeq_route.
struct InlineRoute {
  const double* logits;
  int gating;
  float scale;
  int32_t *ids, *offsets, *pairs, *active;
  float* w;
};

int nper_of(int64_t E) { return E <= 256 ? 4 : E <= 512 ? 8 : E <= 1024 ? 16 : 64; }

constexpr int64_t kSideMaxT = 256;

// The caller's auxiliary stream and events (moeq_ffn_desc::aux_*), or none.
bool has_aux(const moeq_ffn_desc* d) { return d->aux_stream != nullptr; }

// The stream the shared expert's launches go to: the caller's auxiliary
// stream, ordered after everything enqueued on s so far.
int fork_aux(const moeq_ffn_desc* d, hipStream_t s, hipStream_t* out) {
  hipEvent_t fork = (hipEvent_t)d->aux_fork;
  hipStream_t aux = (hipStream_t)d->aux_stream;
  if (hipEventRecord(fork, s) != hipSuccess || hipStreamWaitEvent(aux, fork, 0) != hipSuccess) return -1;
  *out = aux;
  return 0;
}

// s waits for everything enqueued on the auxiliary stream so far.
int join_aux(const moeq_ffn_desc* d, hipStream_t s) {
  hipEvent_t join = (hipEvent_t)d->aux_join;
  if (hipEventRecord(join, (hipStream_t)d->aux_stream) != hipSuccess || hipStreamWaitEvent(s, join, 0) != hipSuccess)
    return -1;
  return 0;
}

// The shared expert's tiles take the fp32-h variant when both of its
// launches can and its tiles are few (as routed_thin_hf).
bool shared_thin_hf(const moeq_ffn_desc* d) {
  const int64_t tiles = (d->T + kThinT - 1) / kThinT;
  return !fmt_sub_scaled(d->sh_fmt_gate) && !fmt_sub_scaled(d->sh_fmt_down) && d->H / 256 <= kHfMaxBlocks &&
         d->F_shared / 256 <= kHfMaxBlocks && tiles * (d->F_shared / 256) < kHfMaxWorkgroups;
}

// A chunk of 2 to 16 tokens on the MFMA path whose routed and shared tiles
// are all fp32-h 8-row tiles: both go into the same gate/up and down
// launches (launch_mfma_hf2, or launch_mfma_route_gateup2 when the chunk
// routes inline), with no auxiliary stream.
bool shared_in_routed_launches(const moeq_ffn_desc* d) {
  if (d->sh_gate == nullptr || d->T < 2 || d->T > kAllThinT || gemv_max_of(d) != 0) return false;
  return routed_thin_hf(d) && shared_thin_hf(d) && mfma_hf2_pair(d->fmt_gate, d->sh_fmt_gate) &&
         mfma_hf2_pair(d->fmt_down, d->sh_fmt_down);
}

// A shared expert that is not a slot of the routed launches (another shape
// or format, or the MFMA path) runs on the caller's auxiliary stream, up to
// kSideMaxT tokens, when one is given.
bool shared_apart(const moeq_ffn_desc* d) {
  const bool sh = d->sh_gate != nullptr;
  const bool same_shape = sh && d->sh_fmt_gate == d->fmt_gate && d->sh_fmt_down == d->fmt_down &&
                          d->F_shared == d->F;
  const bool mfma = d->T > gemv_max_of(d);
  return sh && (mfma || !same_shape) && d->T <= kSideMaxT && has_aux(d) && !shared_in_routed_launches(d);
}

// What ffn_enqueue enqueues: everything (the shared expert forked at its
// start when it runs apart), or, when the caller has recorded the fork event
// on s earlier (before the selection), the shared expert's launches on the
// auxiliary stream only, or everything else (joined before the combine).
enum FfnPart { kFfnAll, kFfnSharedApart, kFfnRoutedWithForked };

// Enqueue the expert FFN (everything after the routing) on `s`.
int ffn_enqueue(const moeq_ffn_desc* d, const void* x_q8K, const int32_t* topk_ids, const float* topk_w,
                const int32_t* expert_offsets, const int32_t* pairs, const int32_t* active,
                const float* shared_scale, float* y, uint8_t* wsb, const InlineRoute* ir, bool planned,
                hipStream_t s, FfnPart part = kFfnAll) {
  const FfnLayout L = ffn_layout(d);
  const bool sh = d->sh_gate != nullptr;
  const bool same_shape = sh && d->sh_fmt_gate == d->fmt_gate && d->sh_fmt_down == d->fmt_down &&
                          d->F_shared == d->F;
  const int thr = gemv_max_of(d);
  const bool one = d->T == 1 && thr >= 1;       // the one-token dot-product kernels
  const bool gemv = thr >= 1;                    // any expert on the dot-product path
  const bool mfma = d->T > thr;                  // any expert on the MFMA path
  const int tt = one ? 1 : 4;
  const int max_union = (int)std::min<int64_t>(d->E, d->T * d->k);
  const bool small_ir = ir != nullptr && !one;   // inline routing of a small chunk (small_route_ok)
  int rc;

  auto gu_args = [&](int mode, int64_t F, const LaneGeo& g) {
    GateUpArgs a{};
    a.gate = d->gate; a.up = d->up; a.down = d->down;
    a.sh_gate = (const uint8_t*)d->sh_gate; a.sh_up = (const uint8_t*)d->sh_up;
    a.mode = mode; a.T = d->T; a.H = d->H; a.F = F; a.k = d->k;
    a.xq = (const uint8_t*)x_q8K; a.offsets = expert_offsets; a.pairs = pairs; a.active = active;
    a.max_union = max_union;
    a.hbuf = (float*)(wsb + L.off_h); a.hstride = L.Fmax;
    a.lpr = g.lpr; a.cpr = g.cpr; a.steps = std::max(1, 2 / g.rps);
    a.gemv_max = thr;
    a.topk_ids = topk_ids; a.topk_w = topk_w; a.E = d->E;
    a.slots = (SlotRec*)(wsb + L.off_slots);
    a.shared_scale = shared_scale;
    a.sh_down_rec = d->sh_down;
    if (ir != nullptr) {
      a.logits = ir->logits; a.gating = ir->gating; a.scale = ir->scale;
      a.ids_out = ir->ids; a.w_out = ir->w; a.offsets_out = ir->offsets; a.pairs_out = ir->pairs;
      a.active_out = ir->active;
    }
    return a;
  };
  auto gateup = [&](int mode, int fmt, int64_t F, int n_slots, hipStream_t st) -> int {
    LaneGeo g;
    lane_geo(fmt, d->H, &g);
    GateUpArgs a = gu_args(mode, F, g);
    const int rows_per_wg = 4 * a.steps * g.rps;
    dim3 grid((unsigned)((F + rows_per_wg - 1) / rows_per_wg), (unsigned)n_slots);
    if (one) {
      const int nper = (ir != nullptr && mode != kModeShared) ? nper_of(d->E) : 0;
      return launch_gateup1(fmt, nper, g.cpl, grid, a, st);
    }
    return launch_gateup(fmt, tt, g.cpl, grid, a, st);
  };
  auto down_args = [&](int mode, int fmt, int64_t F, LaneGeo* g) {
    lane_geo(fmt, F, g);
    DownArgs a{};
    a.slots = (const SlotRec*)(wsb + L.off_slots);
    a.topk_ids = topk_ids;
    a.gate = d->gate; a.up = d->up; a.down = d->down; a.sh_down = (const uint8_t*)d->sh_down;
    a.mode = mode; a.T = d->T; a.H = d->H; a.F = F; a.k = d->k;
    a.topk_w = topk_w; a.shared_scale = shared_scale;
    a.offsets = expert_offsets; a.pairs = pairs; a.active = active; a.max_union = max_union;
    a.hbuf = (const float*)(wsb + L.off_h); a.hstride = L.Fmax;
    a.yp = (float*)(wsb + L.off_yp);
    a.hq = wsb + L.off_hq;
    a.hq_sh = sh ? wsb + L.off_hqs : nullptr;
    a.hq_stride = (F / 256) * kQ8KBytes;
    a.lpr = g->lpr; a.cpr = g->cpr; a.rb = kRowBlock; a.steps = kRowBlock / (4 * g->rps);
    a.gemv_max = thr;
    a.has_shared = sh ? 1 : 0;
    a.y = y; a.accumulate = d->accumulate;
    return a;
  };
  auto down = [&](int mode, int fmt, int64_t F, int n_slots, hipStream_t st) -> int {
    LaneGeo g;
    DownArgs a = down_args(mode, fmt, F, &g);
    dim3 grid((unsigned)(d->H / kRowBlock), (unsigned)n_slots);
    return launch_down(fmt, tt, g.cpl, grid, a, st);
  };
  // int8 MFMA tiles: mode 0 = gate/up (+ q8_K(h)), mode 1 = down
  int4* tiles = (int4*)(wsb + L.off_tiles);
  int4* thin_tiles = (int4*)(wsb + L.off_thin);
  int32_t* tcount = (int32_t*)(wsb + L.off_count);
  // fp32 h between gate/up and down for the 8-row tiles (see launch_mfma)
  // when both of their launches can take it and the tiles are few (256-row
  // gate/up workgroups would not fill the chip; with many tiles the q8_K(h)
  // epilogue is faster)
  auto hf_ok = [&](bool shared_exp) { return shared_exp ? shared_thin_hf(d) : routed_thin_hf(d); };
  // The arguments and grid of one MFMA launch (fmt, hf and the grid returned).
  auto mfma_prep = [&](int mode, bool shared_exp, bool thin, bool fold, int& fmt, bool& hf, unsigned& gx,
                       unsigned& gy) -> MfmaArgs {
    hf = thin && hf_ok(shared_exp);
    MfmaArgs a{};
    a.shared = shared_exp ? 1 : 0;
    a.tiles = thin ? thin_tiles : tiles;
    a.count = thin ? tcount + 1 : tcount;
    a.pairs = pairs; a.k = d->k; a.T = d->T;
    a.topk_w = topk_w; a.shared_scale = shared_scale;
    a.yp = (float*)(wsb + L.off_yp);
    a.y = fold ? y : nullptr;
    a.accumulate = d->accumulate;
    const int64_t Fx = shared_exp ? d->F_shared : d->F;
    const int64_t hq_stride = (Fx / 256) * kQ8KBytes;
    uint8_t* hq = shared_exp ? wsb + L.off_hqs : wsb + L.off_hq;
    a.hf = (float*)(wsb + L.off_h) + (shared_exp ? d->T * d->k * L.Fmax : 0);
    a.hf_stride = L.Fmax;
    const int tm = thin ? kThinT : 32;
    // routed 32-row tiles: a multiple of 8 workgroups at least as many as the
    // tiles (the kernels map workgroups to tiles XCD by XCD)
    gx = shared_exp ? (unsigned)((d->T + tm - 1) / tm) : (unsigned)(thin ? L.max_thin : (L.max_tiles + 7) / 8 * 8);
    a.gate = d->gate; a.up = d->up; a.down = d->down;
    if (mode == 0) {
      fmt = shared_exp ? d->sh_fmt_gate : d->fmt_gate;
      a.sh_w0 = (const uint8_t*)d->sh_gate; a.sh_w1 = (const uint8_t*)d->sh_up;
      a.N = Fx; a.K = d->H;
      a.src = (const uint8_t*)x_q8K; a.src_stride = (d->H / 256) * kQ8KBytes;
      a.hq = hq; a.hq_stride = hq_stride;
      gy = (unsigned)(Fx / (hf ? kHfRows : 256));
    } else {
      fmt = shared_exp ? d->sh_fmt_down : d->fmt_down;
      a.sh_w0 = (const uint8_t*)d->sh_down;
      a.N = d->H; a.K = Fx;
      a.src = hq; a.src_stride = hq_stride;
      a.hq = hq; a.hq_stride = hq_stride;   // fp32 h: the q8_K(h) view is written while staging
      gy = (unsigned)(d->H / 256);
    }
    // Row blocks per workgroup: enough workgroups to fill the chip several
    // times over, the rest of the rows looped inside (start-up and staging
    // paid once per workgroup).
    const int64_t nrb = gy;
    a.rb = std::max<int64_t>(1, std::min<int64_t>(nrb, (int64_t)gx * nrb / 2048));
    gy = (unsigned)((nrb + a.rb - 1) / a.rb);
    return a;
  };
  auto mfma_launch = [&](int mode, bool shared_exp, bool thin, hipStream_t st, bool fold = false) -> int {
    int fmt;
    bool hf;
    unsigned gx, gy;
    const MfmaArgs a = mfma_prep(mode, shared_exp, thin, fold, fmt, hf, gx, gy);
    if (mode == 0 && thin && !shared_exp && small_ir) {
      // a small chunk: these tiles route inline (and write the routing
      // outputs and the 8-row tile list the down launch reads)
      const SmallRoute sr{ir->logits, d->E, ir->gating, ir->scale, ir->ids, ir->w, ir->offsets, ir->pairs,
                          ir->active, ffn_plan(d, L, wsb)};
      return launch_mfma_route_gateup(fmt, dim3(gx, gy), a, sr, st);
    }
    return launch_mfma(fmt, mode, thin, hf, dim3(gx, gy), a, st);
  };

  if (mfma && !planned && part != kFfnSharedApart) {
    if ((rc = launch_mfma_plan(active, expert_offsets, ffn_plan(d, L, wsb), s))) return rc;
  }
  // A shared expert that is not a slot of the routed launches (another shape
  // or format, or the MFMA path) runs its gate/up and down on the caller's
  // auxiliary stream when one is given, forked after everything above and
  // joined before the combine: it reads only x, its own h rows and its own
  // staged output rows.  Up to kSideMaxT tokens the routed launches leave
  // most of the chip idle; past it they fill it and the shared expert stays
  // on s.
  const bool sh_apart = shared_apart(d);
  if (part != kFfnAll && !sh_apart) return -2;
  hipStream_t ss = s;
  // One token: the routed gate/up (a few hundred workgroups, the chip is not
  // full) is captured before the shared expert's launches, so that a
  // captured graph keeps it on the queue of the launch before it; the fork
  // event is recorded first, so the shared expert still waits for nothing
  // more than before.
  const bool routed_first = sh_apart && one && part == kFfnAll;
  if (routed_first) {
    if (hipEventRecord((hipEvent_t)d->aux_fork, s) != hipSuccess) return -1;
    ss = (hipStream_t)d->aux_stream;
  } else if (sh_apart && part == kFfnAll && (rc = fork_aux(d, s, &ss))) {
    return rc;
  }
  if (part != kFfnAll) ss = (hipStream_t)d->aux_stream;
  // Past kSideMaxT tokens the shared expert stays on s; the 8-row tiles of the
  // experts with few rows then run on the auxiliary stream beside the 32-row
  // tiles (they read the lists and write only their own pairs' rows), joined
  // before the shared expert's down tiles or the combine, which read every
  // staged row.
  const bool thin_apart = mfma && !sh_apart && d->T > kSideMaxT && has_aux(d);
  hipStream_t ts = s;
  if (thin_apart && (rc = fork_aux(d, s, &ts))) return rc;
  // gate/up: h[pair, f] = fl32(silu(g) u)  (dot-product path: fp32 h rows;
  // MFMA path: q8_K(h) rows straight away)
  const int n_routed_slots = one ? d->k : max_union;
  // the shared expert goes first when it has a stream of its own (it starts
  // at once), after the routed launches otherwise.  Beside the routed
  // launches, a shared expert of up to 16 tokens takes 8-row fp32-h tiles:
  // two of them give its gate/up and down several times the workgroups of one
  // 32-row tile (its weights are read once per tile), so it no longer trails
  // the routed launches, whose workgroups hold the CUs.
  const bool dual = shared_in_routed_launches(d);
  const bool sh_thin = d->T <= kThinT || ((ss != s || dual) && d->T <= 2 * kThinT && hf_ok(true));
  auto shared_gateup = [&]() -> int {
    if (!sh || (gemv && same_shape)) return 0;
    return mfma ? mfma_launch(0, true, sh_thin, ss) : gateup(kModeShared, d->sh_fmt_gate, d->F_shared, 1, ss);
  };
  // A shared expert on the MFMA path (32-row tiles) that runs after the
  // routed down launches on the same stream also does the combine (no
  // k_combine launch).
  const bool fold_combine = sh && mfma && !gemv && ss == s && !sh_thin;
  auto shared_down = [&]() -> int {
    if (!sh || (gemv && same_shape)) return 0;
    return mfma ? mfma_launch(1, true, sh_thin, ss, fold_combine)
                : down(kModeShared, d->sh_fmt_down, d->F_shared, 1, ss);
  };
  if (dual) {
    // the routed and the shared expert's 8-row tiles in one gate/up and one
    // down launch (the shared tiles first), then the combine
    for (int mode = 0; mode < 2; ++mode) {
      int fr, fs;
      bool hr, hs;
      unsigned gxr, gyr, gxs, gys;
      const MfmaArgs ar = mfma_prep(mode, false, true, false, fr, hr, gxr, gyr);
      const MfmaArgs as = mfma_prep(mode, true, true, false, fs, hs, gxs, gys);
      if (!hr || !hs) return -2;
      const dim3 grid(gxs + gxr, std::max(gyr, gys));
      if (mode == 0 && small_ir) {
        // the routed tiles route inline (as in mfma_launch)
        const SmallRoute sr{ir->logits, d->E, ir->gating, ir->scale, ir->ids, ir->w, ir->offsets, ir->pairs,
                            ir->active, ffn_plan(d, L, wsb)};
        if ((rc = launch_mfma_route_gateup2(fr, fs, grid, ar, as, sr, (int)gxs, s))) return rc;
      } else if ((rc = launch_mfma_hf2(mode, fr, fs, grid, ar, as, (int)gxs, s))) {
        return rc;
      }
    }
    return launch_combine((const float*)(wsb + L.off_yp), d->T, d->H, d->k, 1, y, d->accumulate, s);
  }
  if (part == kFfnSharedApart) {
    // the auxiliary stream waits for the fork point the caller recorded
    if (hipStreamWaitEvent(ss, (hipEvent_t)d->aux_fork, 0) != hipSuccess) return -1;
    if ((rc = shared_gateup())) return rc;
    return shared_down();
  }
  if (ss != s && part == kFfnAll && !routed_first && (rc = shared_gateup())) return rc;
  if (gemv) {
    if (same_shape) {
      if ((rc = gateup(kModeBoth, d->fmt_gate, d->F, n_routed_slots + 1, s))) return rc;
    } else {
      if ((rc = gateup(kModeRouted, d->fmt_gate, d->F, n_routed_slots, s))) return rc;
    }
  }
  if (routed_first) {
    if (hipStreamWaitEvent(ss, (hipEvent_t)d->aux_fork, 0) != hipSuccess) return -1;
    if ((rc = shared_gateup())) return rc;
  }
  if (mfma) {
    if (L.max_tiles > 0 && (rc = mfma_launch(0, false, false, s))) return rc;
    if ((rc = mfma_launch(0, false, true, ts))) return rc;
  }
  if (ss == s && (rc = shared_gateup())) return rc;
  // down and the weighted combine
  if (one && (!sh || same_shape) && (d->k + (sh ? 1 : 0)) * (d->F / 256) <= kLdsQ8Blocks) {
    LaneGeo g;
    DownArgs a = down_args(kModeBoth, d->fmt_down, d->F, &g);
    a.steps = kDown1Steps;
    const int rows_wg = g.rps * a.steps;
    dim3 grid((unsigned)((d->H + rows_wg - 1) / rows_wg));
    return launch_down_rows1(d->fmt_down, g.cpl, grid, a, s);
  }
  if (ss != s && part == kFfnAll && (rc = shared_down())) return rc;
  if (gemv) {
    if (same_shape) {
      if ((rc = down(kModeBoth, d->fmt_down, d->F, max_union + 1, s))) return rc;
    } else {
      if ((rc = down(kModeRouted, d->fmt_down, d->F, max_union, s))) return rc;
    }
  }
  if (mfma) {
    if (L.max_tiles > 0 && (rc = mfma_launch(1, false, false, s))) return rc;
    if ((rc = mfma_launch(1, false, true, ts))) return rc;
  }
  if (thin_apart && (rc = join_aux(d, s))) return rc;
  if (ss == s && (rc = shared_down())) return rc;
  if (ss != s && (rc = join_aux(d, s))) return rc;
  if (fold_combine) return 0;
  return launch_combine((const float*)(wsb + L.off_yp), d->T, d->H, d->k, sh ? 1 : 0, y, d->accumulate, s);
}

}  // namespace

int moeq_expert_ffn(const moeq_ffn_desc* d, const void* x_q8K, const int32_t* topk_ids, const float* topk_w,
                    const int32_t* expert_offsets, const int32_t* pairs, const int32_t* active,
                    const float* shared_scale, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_ffn_desc(d);
  if (rc != MOEQ_OK) return rc;
  if (d->T == 0) return MOEQ_OK;
  if (!x_q8K || !topk_ids || !topk_w || !expert_offsets || !pairs || !active || !y) return MOEQ_E_INVALID;
  if (!aligned(x_q8K, 4) || !aligned(y, 4) || !aligned(topk_w, 4)) return MOEQ_E_INVALID;
  if (!ws || !aligned(ws, 256)) return MOEQ_E_INVALID;
  if (ws_bytes < ffn_layout(d).total) return MOEQ_E_WORKSPACE;
  return hip_status(ffn_enqueue(d, x_q8K, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y,
                                (uint8_t*)ws, nullptr, false, (hipStream_t)stream));
}

namespace {
struct LayerLayout {
  size_t off_ffn, off_route, off_xq, total;
};
LayerLayout layer_layout(const moeq_route_desc* r, const moeq_ffn_desc* f) {
  LayerLayout L{};
  size_t o = 0;
  L.off_ffn = o;   o += align256(ffn_layout(f).total);
  L.off_route = o; o += align256(route_ws_bytes(r->T, r->E, r->H));
  L.off_xq = o;    o += align256((size_t)r->T * (r->H / 256) * kQ8KBytes);
  L.total = o;
  return L;
}
int check_layer(const moeq_route_desc* r, const moeq_ffn_desc* f) {
  if (!r || !f) return MOEQ_E_INVALID;
  int rc = check_ffn_desc(f);
  if (rc != MOEQ_OK) return rc;
  if (r->T != f->T || r->H != f->H || r->E != f->E || r->k != f->k) return MOEQ_E_INVALID;
  if (r->gating < MOEQ_SOFTMAX_TOPK || r->gating > MOEQ_SIGMOID_TOPK) return MOEQ_E_UNSUPPORTED;
  return MOEQ_OK;
}
}  // namespace

size_t moeq_moe_layer_workspace(const moeq_route_desc* r, const moeq_ffn_desc* f) {
  if (check_layer(r, f) != MOEQ_OK) return 0;
  return layer_layout(r, f).total;
}

namespace {
// RMS pre-norm of the layer's input (a stack of layers): gains g (null: all
// ones), eps; xn: room for the normalised rows [T, H] when they are written.
struct NormIn {
  const float* g;
  double eps;
  float* xn;
};

// Enqueue one whole layer (arguments already checked); with nrm, the layer's
// input is the RMS pre-norm of x (fused into the router launch for one token).
int layer_enqueue(const moeq_route_desc* r, const moeq_ffn_desc* f, const float* x, const float* w_router,
                  const float* bias, double* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                  int32_t* pairs, int32_t* active, const float* shared_scale, float* y, uint8_t* wsb,
                  hipStream_t s, const NormIn* nrm = nullptr) {
  int rc;
  const LayerLayout L = layer_layout(r, f);
  void* xq = wsb + L.off_xq;
  const bool one = r->T == 1 && gemv_max_of(f) >= 1;
  if (nrm != nullptr && !(one && r->H <= kNorm1MaxH)) {
    if ((rc = launch_rms_norm(x, r->T, r->H, nrm->g, nrm->eps, nrm->xn, s))) return hip_status(rc);
    x = nrm->xn;
    nrm = nullptr;
  }
  if (one) {
    // one token: logits + q8_K(x) in one launch, then gate/up routes inline
    double* lg = logits ? logits : (double*)(wsb + L.off_route);
    rc = nrm ? launch_logits_norm1(r->H, r->E, x, nrm->g, nrm->eps, w_router, bias, lg, xq, s)
             : launch_logits(1, r->H, r->E, x, w_router, bias, lg, xq, s, nullptr);
    if (rc) return hip_status(rc);
    InlineRoute ir{lg, r->gating, r->scale, topk_ids, expert_offsets, pairs, active, topk_w};
    return hip_status(ffn_enqueue(f, xq, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y, wsb, &ir,
                                  false, s));
  }
  if (small_route_ok(f)) {
    // a small chunk: logits + q8_K(x) in one launch, then the first gate/up
    // launch routes inline (no selection launch)
    double* lg = logits ? logits : (double*)(wsb + L.off_route);
    if ((rc = launch_logits(r->T, r->H, r->E, x, w_router, bias, lg, xq, s,
                                 wsb + L.off_route + route_part_off(r->T, r->E, r->H)))) return hip_status(rc);
    InlineRoute ir{lg, r->gating, r->scale, topk_ids, expert_offsets, pairs, active, topk_w};
    return hip_status(ffn_enqueue(f, xq, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y, wsb, &ir,
                                  true, s));
  }
  // the routing kernel also builds the MFMA tile lists of the FFN (one launch fewer)
  const FfnLayout FL = ffn_layout(f);
  const int thr = gemv_max_of(f);
  const bool mfma = f->T > thr;
  const MfmaPlan plan = ffn_plan(f, FL, wsb + L.off_ffn);
  if (shared_apart(f)) {
    // A shared expert that runs apart needs only q8_K(x): it forks after the
    // logits launch, not after the selection, so it starts earlier.  The
    // selection is enqueued before the shared expert's launches, so that a
    // captured graph keeps the routed chain on the queue of the launches
    // before it (a chain that changes queue waits about 10 us at each change).
    double* lg = logits ? logits : (double*)(wsb + L.off_route);
    if ((rc = launch_logits(r->T, r->H, r->E, x, w_router, bias, lg, xq, s,
                                 wsb + L.off_route + route_part_off(r->T, r->E, r->H)))) return hip_status(rc);
    if (hipEventRecord((hipEvent_t)f->aux_fork, s) != hipSuccess) return MOEQ_E_HIP;
    if ((rc = launch_route(r->T, r->H, r->E, r->k, r->gating, r->scale, x, w_router, bias, lg, topk_ids, topk_w,
                           expert_offsets, pairs, active, xq, wsb + L.off_route, s, mfma ? &plan : nullptr, true)))
      return hip_status(rc);
    if ((rc = ffn_enqueue(f, xq, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y, wsb, nullptr,
                          mfma, s, kFfnSharedApart)))
      return hip_status(rc);
    return hip_status(ffn_enqueue(f, xq, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y, wsb,
                                  nullptr, mfma, s, kFfnRoutedWithForked));
  }
  if ((rc = launch_route(r->T, r->H, r->E, r->k, r->gating, r->scale, x, w_router, bias, logits, topk_ids, topk_w,
                         expert_offsets, pairs, active, xq, wsb + L.off_route, s, mfma ? &plan : nullptr)))
    return hip_status(rc);
  return hip_status(ffn_enqueue(f, xq, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale, y, wsb,
                                nullptr, mfma, s));
}
}  // namespace

int moeq_moe_layer(const moeq_route_desc* r, const moeq_ffn_desc* f, const float* x, const float* w_router,
                   const float* bias, double* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                   int32_t* pairs, int32_t* active, const float* shared_scale, float* y, void* ws,
                   size_t ws_bytes, void* stream) {
  int rc = check_layer(r, f);
  if (rc != MOEQ_OK) return rc;
  if (r->T == 0) {
    if (!expert_offsets || !active) return MOEQ_E_INVALID;
    return hip_status(launch_route(0, r->H, r->E, r->k, r->gating, r->scale, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, expert_offsets, nullptr, active, nullptr, nullptr,
                                   (hipStream_t)stream));
  }
  if (!x || !w_router || !topk_ids || !topk_w || !expert_offsets || !pairs || !active || !y) return MOEQ_E_INVALID;
  if (!aligned(x, 16) || !aligned(w_router, 16) || (bias && !aligned(bias, 4)) || !aligned(y, 4))
    return MOEQ_E_INVALID;
  if (logits && !aligned(logits, 8)) return MOEQ_E_INVALID;
  if (!ws || !aligned(ws, 256)) return MOEQ_E_INVALID;
  if (ws_bytes < layer_layout(r, f).total) return MOEQ_E_WORKSPACE;
  return layer_enqueue(r, f, x, w_router, bias, logits, topk_ids, topk_w, expert_offsets, pairs, active, shared_scale,
                       y, (uint8_t*)ws, (hipStream_t)stream);
}

namespace {
// Workspace of a stack: the largest layer workspace (the layers run one after
// the other on one stream), then the normalised input rows [T, H].
struct StackLayout {
  size_t off_xn, total;
};
StackLayout stack_layout(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L) {
  size_t b = 0;
  for (int64_t l = 0; l < L; ++l) b = std::max(b, layer_layout(r, &f[l]).total);
  return StackLayout{b, b + align256((size_t)r->T * r->H * sizeof(float))};
}
int check_stack(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L) {
  if (!r || !f || L < 1 || L > kMaxStack) return MOEQ_E_INVALID;
  for (int64_t l = 0; l < L; ++l) {
    const int rc = check_layer(r, &f[l]);
    if (rc != MOEQ_OK) return rc;
    if (f[l].accumulate != 0) return MOEQ_E_INVALID;
  }
  return MOEQ_OK;
}
bool eps_ok(float eps) { return eps >= 0.0f && eps <= FLT_MAX; }   // finite, not negative (NaN fails)
}  // namespace

int moeq_rms_norm(const float* x, int64_t T, int64_t H, const float* gamma, float eps, float* out, void* stream) {
  if (T < 0 || H <= 0 || H % 256 != 0 || !eps_ok(eps)) return MOEQ_E_INVALID;
  if (T == 0) return MOEQ_OK;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16) || (gamma && !aligned(gamma, 16))) return MOEQ_E_INVALID;
  return hip_status(launch_rms_norm(x, T, H, gamma, (double)eps, out, (hipStream_t)stream));
}

size_t moeq_moe_stack_workspace(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L) {
  if (check_stack(r, f, L) != MOEQ_OK) return 0;
  return stack_layout(r, f, L).total;
}

int moeq_moe_stack(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L, const float* const* w_router,
                   const float* const* bias, const float* const* norm_w, float norm_eps, const float* x,
                   int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* pairs, int32_t* active,
                   const float* const* shared_scale, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_stack(r, f, L);
  if (rc != MOEQ_OK) return rc;
  if (!w_router || !expert_offsets || !active || !eps_ok(norm_eps)) return MOEQ_E_INVALID;
  const int64_t T = r->T, k = r->k, E = r->E;
  const int64_t n_pairs = std::max<int64_t>(1, T * k), n_active = 1 + std::min<int64_t>(E, T * k);
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    for (int64_t l = 0; l < L; ++l)
      if ((rc = hip_status(launch_route(0, r->H, E, r->k, r->gating, r->scale, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, expert_offsets + l * (E + 1), nullptr,
                                        active + l * n_active, nullptr, nullptr, s))))
        return rc;
    return MOEQ_OK;
  }
  if (!x || !topk_ids || !topk_w || !pairs || !y) return MOEQ_E_INVALID;
  if (!aligned(x, 16) || !aligned(y, 16)) return MOEQ_E_INVALID;
  for (int64_t l = 0; l < L; ++l) {
    if (!w_router[l] || !aligned(w_router[l], 16)) return MOEQ_E_INVALID;
    if (bias && bias[l] && !aligned(bias[l], 4)) return MOEQ_E_INVALID;
    if (norm_w && norm_w[l] && !aligned(norm_w[l], 16)) return MOEQ_E_INVALID;
  }
  if (!ws || !aligned(ws, 256)) return MOEQ_E_INVALID;
  const StackLayout SL = stack_layout(r, f, L);
  if (ws_bytes < SL.total) return MOEQ_E_WORKSPACE;
  // the residual stream: y = x, then every layer reads y and adds its output
  // to y (in place: a layer has consumed its input in its first launch, and
  // writes y only in its last)
  if (x != y && hipMemcpyAsync(y, x, (size_t)T * r->H * sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MOEQ_E_HIP;
  uint8_t* wsb = (uint8_t*)ws;
  for (int64_t l = 0; l < L; ++l) {
    moeq_ffn_desc fl = f[l];
    fl.accumulate = 1;
    const NormIn nrm{norm_w ? norm_w[l] : nullptr, (double)norm_eps, (float*)(wsb + SL.off_xn)};
    if ((rc = layer_enqueue(r, &fl, y, w_router[l], bias ? bias[l] : nullptr, nullptr, topk_ids + l * T * k,
                            topk_w + l * T * k, expert_offsets + l * (E + 1), pairs + l * n_pairs,
                            active + l * n_active, shared_scale ? shared_scale[l] : nullptr, y, wsb, s, &nrm)))
      return rc;
  }
  return MOEQ_OK;
}

int moeq_ffn_h_view(const moeq_ffn_desc* d, void* ws, size_t ws_bytes, void** hq_routed, void** hq_shared) {
  int rc = check_ffn_desc(d);
  if (rc != MOEQ_OK) return rc;
  if (!ws || !hq_routed || !hq_shared) return MOEQ_E_INVALID;
  const FfnLayout L = ffn_layout(d);
  if (ws_bytes < L.total) return MOEQ_E_WORKSPACE;
  *hq_routed = (uint8_t*)ws + L.off_hq;
  *hq_shared = d->sh_gate ? (uint8_t*)ws + L.off_hqs : nullptr;
  return MOEQ_OK;
}

int moeq_debug_subdots(int32_t fmt, const void* packed_w, int64_t rows, int64_t cols, const void* x_q8K,
                       int64_t n_x, int32_t* out, void* stream) {
  if (!fmt_ok(fmt)) return MOEQ_E_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % 256 || n_x < 0) return MOEQ_E_INVALID;
  if (n_x == 0) return MOEQ_OK;
  if (!packed_w || !x_q8K || !out || !aligned(packed_w, 256) || !aligned(x_q8K, 4) || !aligned(out, 4))
    return MOEQ_E_INVALID;
  return hip_status(launch_subdots(fmt, packed_w, rows, cols, x_q8K, n_x, out, (hipStream_t)stream));
}

int moeq_debug_mfma_sums(int32_t fmt, const void* packed_w, int64_t rows, int64_t cols, const void* x_q8K,
                         int64_t n_x, int32_t* out, void* stream) {
  if (!fmt_ok(fmt)) return MOEQ_E_UNSUPPORTED;
  if (rows <= 0 || rows % 256 || cols <= 0 || cols % 256 || n_x < 0) return MOEQ_E_INVALID;
  if (n_x == 0) return MOEQ_OK;
  if (!packed_w || !x_q8K || !out || !aligned(packed_w, 256) || !aligned(x_q8K, 4) || !aligned(out, 16))
    return MOEQ_E_INVALID;
  if ((n_x + 31) / 32 > INT32_MAX || rows / 256 > 65535) return MOEQ_E_UNSUPPORTED;
  return hip_status(launch_mfma_ints(fmt, packed_w, rows, cols, x_q8K, n_x, out, (hipStream_t)stream));
}

int moeq_ceiling_read(const void* buf, int64_t bytes, int32_t n_blocks, uint64_t* out, void* stream) {
  if (!buf || !out || !aligned(buf, 16) || !aligned(out, 8)) return MOEQ_E_INVALID;
  if (bytes <= 0 || bytes % 16 || n_blocks < 1 || n_blocks > kCeilMaxBlocks) return MOEQ_E_INVALID;
  return hip_status(launch_ceiling_read(buf, bytes, n_blocks, out, (hipStream_t)stream));
}

int moeq_ceiling_mfma_i8(int64_t iters, int32_t n_blocks, int32_t* out, void* stream) {
  if (!out || !aligned(out, 4)) return MOEQ_E_INVALID;
  if (iters < 1 || n_blocks < 1 || n_blocks > kCeilMaxBlocks) return MOEQ_E_INVALID;
  return hip_status(launch_ceiling_mfma_i8(iters, n_blocks, out, (hipStream_t)stream));
}

}  // extern "C"
