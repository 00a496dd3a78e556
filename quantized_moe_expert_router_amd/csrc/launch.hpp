// Host-side launchers of libmoeq's kernels (internal; the public surface is moeq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

// Which slots a FFN launch covers: the routed union, the shared expert, or both
// (the shared expert as one more slot when it has the routed shape and format).
constexpr int kModeRouted = 0, kModeShared = 1, kModeBoth = 2;

// One-token down kernel: q8_K(h) blocks of the k+1 slots staged in LDS (at most
// 4 waves x kQ8PerWave blocks), output rows per workgroup.
constexpr int kQ8PerWave = 9;
constexpr int kLdsQ8Blocks = 4 * kQ8PerWave;
constexpr int kDown1Steps = 1;

// One token: what the down kernel needs per slot (slot k = shared expert),
// written by the gate/up kernel.  The table holds kSlotCopies copies of the
// k+1 records, copy c written by a gate/up workgroup whose flat index is c
// modulo 8 and read by the down workgroups with that index modulo 8: workgroups
// are dealt to the 8 XCDs in turn, so the reader usually finds the record in
// its own XCD's L2.  Every copy is complete whatever the placement.
constexpr int kSlotCopies = 8;
struct SlotRec {
  const void* wd;   // packed down matrix, null when the expert is not resident
  double wt;        // gate weight (shared: shared_scale or 1)
};

struct GateUpArgs {
  const void* const* gate;
  const void* const* up;
  const void* const* down;      // only checked for residency
  const uint8_t* sh_gate;
  const uint8_t* sh_up;
  int mode;
  int64_t T, H, F;              // F: rows of this launch's gate/up matrices
  int k;
  const uint8_t* xq;            // q8_K(x) [T, H/256]
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  int max_union;
  float* hbuf;                  // fp32 [T*k + T, hstride]
  int64_t hstride;
  int lpr, cpr, steps;
  int gemv_max;                 // experts with more rows than this go to the MFMA path
  // one token (k_gateup1)
  const int32_t* topk_ids;      // rank-ordered experts (when not routing inline)
  const double* logits;         // [E] logits to route inline from, or null
  int64_t E;
  int gating;
  float scale;
  int32_t* ids_out;             // routing outputs written when routing inline
  float* w_out;
  int32_t* offsets_out;
  int32_t* pairs_out;
  int32_t* active_out;
  SlotRec* slots;               // per-slot records for the one-token down kernel
  const float* shared_scale;
  const float* topk_w;
  const void* sh_down_rec;      // shared down matrix, recorded in the slot table
};

struct DownArgs {
  const SlotRec* slots;
  const int32_t* topk_ids;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const uint8_t* sh_down;
  int mode;
  int64_t T, H, F;              // F: inner size of this launch's down matrices
  int k;
  const float* topk_w;
  const float* shared_scale;
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  int max_union;
  const float* hbuf;
  int64_t hstride;
  float* yp;                    // fp32 [T*k + T, H] weighted per-pair outputs
  uint8_t* hq;                  // q8_K(h) rows of routed pairs [T*k], or null
  uint8_t* hq_sh;               // q8_K(h) rows of the shared expert [T], or null
  int64_t hq_stride;            // bytes per row for this launch's F
  int lpr, cpr, steps, rb;      // rb = rows per work item = 4 * steps * (64 / lpr)
  int gemv_max;                 // experts with more rows than this go to the MFMA path
  int has_shared;
  float* y;
  int accumulate;
};

// int8 MFMA grouped GEMM (experts with more than gemv_max rows).  Tiles of 32
// activation rows come from the plan (routed experts) or cover all T tokens
// (shared expert).
// Where and how the MFMA tile lists are built: experts with more than thr
// rows; those with at most thin_max rows take ceil(rows / 8) 8-row tiles,
// the others 32-row tiles (at most max_tiles of them).
struct MfmaPlan {
  int thr, max_tiles;
  int4* tiles;
  int32_t* count;
  int4* thin;
  int32_t* thin_count;
  int thin_max;
};

struct MfmaArgs {
  int shared;
  const int4* tiles;            // routed: (expert, first row, rows, list offset)
  const int32_t* count;         // routed: number of tiles
  const void* const* gate;      // routed expert tables (an expert is resident only if
  const void* const* up;        // all three of its matrices are present)
  const void* const* down;
  const uint8_t* sh_w0;         // shared: gate (mode 0) or down (mode 1)
  const uint8_t* sh_w1;         // shared: up (mode 0)
  const int32_t* pairs;
  int k;
  int64_t T;
  int64_t N, K;                 // weight rows and columns of this launch's matrices
  int64_t rb;                   // 256-row blocks per workgroup (grid.y = ceil(N/256 / rb))
  const uint8_t* src;           // q8_K rows: x by token (mode 0), h by pair row (mode 1)
  int64_t src_stride;
  uint8_t* hq;                  // q8_K(h) rows: mode 0 writes them; with fp32 h, mode 1
  int64_t hq_stride;            //   writes them (the quantised view of its staged rows)
  float* hf;                    // fp32 h rows (fp32-h launches only): mode 0 writes them,
  int64_t hf_stride;            //   mode 1 quantises them to q8_K while staging
  const float* topk_w;
  const float* shared_scale;
  float* yp;                    // mode 1: fp32 [T*k + T, H]
  float* y;                     // shared mode 1 only: not null = the tiles also do the combine
  int accumulate;               //   into y (y = or += the token's summed rows)
};

int launch_quantize_q8K(const float* x, int64_t rows, int64_t cols, void* out, hipStream_t s);
// RMS pre-norm of token rows (g null: all ones) into out (fp32, 16-byte aligned rows).
int launch_rms_norm(const float* x, int64_t rows, int64_t cols, const float* g, double eps, float* out,
                    hipStream_t s);
int launch_pack(int fmt, const void* aos, int64_t n_mats, int64_t rows, int64_t cols, void* packed,
                hipStream_t s);
// Exact integer parts of the super-block terms by the MFMA tile code (test hook).
int launch_mfma_ints(int fmt, const void* W, int64_t N, int64_t K, const void* xq, int64_t n_x, int32_t* out,
                     hipStream_t s);
int launch_subdots(int fmt, const void* w, int64_t rows, int64_t cols, const void* xq, int64_t n_x,
                   int32_t* out, hipStream_t s);
size_t route_ws_bytes(int64_t T, int64_t E, int64_t H);
// part: scratch of the split-K logits (route workspace at route_part_off), or null
int launch_logits(int64_t T, int64_t H, int64_t E, const float* x, const float* W, const float* bias,
                  double* logits, void* xq, hipStream_t s, void* part);
size_t route_part_off(int64_t T, int64_t E, int64_t H);
// One token: RMS pre-norm fused into the router logits and q8_K (H <= kNorm1MaxH).
constexpr int64_t kNorm1MaxH = 4096;
int launch_logits_norm1(int64_t H, int64_t E, const float* x, const float* g, double eps, const float* W,
                        const float* bias, double* logits, void* xq, hipStream_t s);
// have_logits (at most 256 tokens, logits given): the logits and q8_K(x)
// are already enqueued; only the selection and lists are.
int launch_route(int64_t T, int64_t H, int64_t E, int k, int gating, float scale, const float* x,
                 const float* W, const float* bias, double* logits, int32_t* ids, float* w,
                 int32_t* offsets, int32_t* pairs, int32_t* active, void* xq, void* ws, hipStream_t s,
                 const MfmaPlan* plan = nullptr, bool have_logits = false);
int launch_gateup(int fmt, int tt, int cpl, dim3 grid, const GateUpArgs& a, hipStream_t s);
int launch_gateup1(int fmt, int nper, int cpl, dim3 grid, const GateUpArgs& a, hipStream_t s);
int launch_down(int fmt, int tt, int cpl, dim3 grid, const DownArgs& a, hipStream_t s);
int launch_down_rows1(int fmt, int cpl, dim3 grid, const DownArgs& a, hipStream_t s);
int launch_mfma_plan(const int32_t* active, const int32_t* offsets, const MfmaPlan& p, hipStream_t s);
// hf: the fp32-h variant (8-row resident tiles of formats other than Q6_K;
// mode 0 workgroups then cover kHfRows weight rows instead of 256).
constexpr int kHfRows = 64;
constexpr int kHfMaxBlocks = 16;   // K (256-blocks) up to which 8-row tiles keep their activations in LDS
constexpr int64_t kHfMaxWorkgroups = 1024;   // fp32 h only while 256-row gate/up tiles x row blocks stay below this
int launch_mfma(int fmt, int mode, bool thin, bool hf, dim3 grid, const MfmaArgs& a, hipStream_t s);
// The routed 8-row fp32-h tiles (a) and the shared expert's (sa, nsh tiles)
// in one launch (mode 0 gate/up, 1 down); grid.x = nsh + routed tiles.  -2
// when the format pair has no such kernel (mfma_hf2_pair).
bool mfma_hf2_pair(int fmt_r, int fmt_s);
int launch_mfma_hf2(int mode, int fmt_r, int fmt_s, dim3 grid, const MfmaArgs& a, const MfmaArgs& sa, int nsh,
                    hipStream_t s);
// Formats whose MFMA tiles scale each sub-block's result in int32 (no fp32-h tiles).
inline bool fmt_sub_scaled(int fmt) { return fmt == FQ6K || fmt == FQ3K; }
int launch_combine(const float* yp, int64_t T, int64_t H, int k, int has_shared, float* y, int accumulate,
                   hipStream_t s);

}  // namespace moeq
