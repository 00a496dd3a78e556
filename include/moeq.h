/*
 * moeq.h -- C ABI of libmoeq.so: the routed-expert FFN of one MoE layer on an
 * AMD MI355X (gfx950), over quantised expert weights resident in HBM.
 *
 * The path (router -> top-k gating -> q8_K activations -> dequant-dot gate/up
 * -> SwiGLU -> q8_K(h) -> dequant-dot down -> gate-weighted sum with a shared
 * expert) is the per-layer MoE step of the SSD/RAM-tiered engines on the
 * pages; here every expert of the layer sits in device memory, so the
 * streaming tiers are not part of it.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory unless marked (host).  `stream` is a
 *     hipStream_t (NULL = the null stream).  Work is enqueued asynchronously
 *     on `stream`; nothing synchronises, allocates device memory, creates a
 *     stream or event, or reads the environment or any state of its own:
 *     the library holds no mutable global state apart from the static
 *     workspace of moeq_moe_layer_noalloc (the MoE kernels never
 *     consult global state and every launch gets explicit per-expert
 *     pointers: Pulsar README, 'How the streaming works'; session state is
 *     preallocated by the caller: Strata summary, execution paragraph).
 *     Calls that take a workspace use only that workspace for scratch;
 *     concurrent calls must not share one.
 *   - moeq_expert_ffn and moeq_moe_layer run a shared expert that is not a
 *     slot of the routed launches (another shape or format, or the MFMA
 *     path, up to 256 tokens) on the caller's auxiliary stream when the FFN
 *     descriptor names one (aux_stream with two events, all caller-owned),
 *     otherwise on `stream`.  The auxiliary stream is ordered after `stream`
 *     (in moeq_moe_layer, when a selection launch runs, after the router
 *     logits launch, so the shared expert runs beside the selection) and
 *     joined back into `stream` by the two events before the call's last
 *     launch, so every effect of the call is still ordered on `stream`, in
 *     graph capture too.  Calls that may run concurrently need their own
 *     auxiliary stream and events.
 *   - The caller owns every buffer, stream and event; nothing is retained
 *     after the call.
 *   - Return value: MOEQ_OK (0) or a negative moeq_status.  All argument
 *     checks (sizes, NULLs, alignment, workspace size, supported formats)
 *     happen on the host before anything is enqueued; a failed check leaves
 *     the outputs untouched.  MOEQ_E_HIP means a launch failed.
 *   - Integer outputs (q8_K bytes, ids, lists, sub-block dots) are
 *     deterministic.  Floating outputs are deterministic for a given input
 *     and launch shape.
 *   - Inputs must be finite.
 *
 * Block formats.  The pages name the formats (Pulsar README, 'Get a model':
 * the routed-expert formats it reads, q2_K, q3_K, q4_0, q4_K, q5_K, q5_1 and
 * q6_K among them, dense tensors requantised to q8_0; 'Fidelity notes': activations
 * quantised to q8_K with integer dots) but print no byte layout, so the
 * exchange layout is this library's own (little-endian):
 *   q8_K  292 B / 256 : f32 d | i8 q[256] | i16 bsums[16]          x ~ d*q
 *   Q4_K  144 B / 256 : f16 d | f16 dmin | 12 B six-bit scales then mins
 *                       (bit stream) | 128 B quants (byte 32g+i = element
 *                       64g+i low nibble, 64g+32+i high nibble)
 *                                                      w = d*sc_j*q - dmin*m_j
 *   Q2_K   84 B / 256 : f16 d | f16 dmin | 16 B (sc_j | m_j << 4) | 64 B quants
 *                       (byte 32h+i bits 2s..2s+1 = element 128h+32s+i)
 *                                                      w = d*sc_j*q - dmin*m_j
 *   Q6_K  210 B / 256 : f16 d | i8 sc[16] | 128 B low nibbles (byte 64h+i =
 *                       element 128h+i low, 128h+64+i high) | 64 B high pairs
 *                       (byte 32h+i bits 2s..2s+1 = element 128h+32s+i)
 *                                                      w = d*sc_j*(q-32)
 *   Q8_0   34 B /  32 : f16 d | i8 q[32]                w = d*q
 *   Q3_K  110 B / 256 : f16 d | 12 B six-bit scales (bit stream, stored
 *                       sc_j + 32) | 64 B low pairs (byte 32h+i bits 2s..2s+1
 *                       = element 128h+32s+i) | 32 B high bits (byte i bit b =
 *                       element 32b+i); q = low + 4*high, sub-blocks of 16
 *                                                      w = d*sc_j*(q-4)
 *   Q5_K  176 B / 256 : Q4_K's 144 bytes (the low nibbles as its quants) | 32 B
 *                       high bits (byte i bit b = element 32b+i); q = low +
 *                       16*high, sub-blocks of 32      w = d*sc_j*q - dmin*m_j
 *   Q4_0   18 B /  32 : f16 d | 16 B (byte i = element i low nibble, element
 *                       16+i high nibble)              w = d*(q-8)
 *   Q5_1   24 B /  32 : f16 d | f16 m | 4 B (bit i = bit 4 of element i) |
 *                       16 B nibbles as Q4_0           w = d*q + m
 * A matrix [rows, cols] is rows of blocks back to back.  Kernels read a
 * repacked ("packed") form made once by moeq_pack_experts.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOEQ_OK = 0,
    MOEQ_E_INVALID = -1,      /* bad size, NULL pointer, misalignment */
    MOEQ_E_UNSUPPORTED = -2,  /* format / gating / path / shape not supported */
    MOEQ_E_WORKSPACE = -3,    /* workspace smaller than the query returns */
    MOEQ_E_HIP = -4,          /* a HIP launch or API call failed */
    MOEQ_E_STATIC_LIMIT = -5  /* moeq_moe_layer_noalloc: the call needs more than
                                 MOEQ_NOALLOC_MAX_BYTES of workspace */
} moeq_status;

typedef enum {
    MOEQ_Q4_K = 1, MOEQ_Q6_K = 2, MOEQ_Q2_K = 3, MOEQ_Q8_0 = 4, MOEQ_Q3_K = 5, MOEQ_Q5_K = 6,
    MOEQ_Q4_0 = 7, MOEQ_Q5_1 = 8
} moeq_wfmt;

typedef enum {
    MOEQ_SOFTMAX_TOPK = 0,   /* softmax over the k selected logits */
    MOEQ_SOFTMAX_ALL = 1,    /* softmax over all E logits, not renormalised */
    MOEQ_SIGMOID_TOPK = 2    /* sigmoid of the k selected, divided by their sum */
} moeq_gating;

/*
 * Which kernels compute the expert dot products.  GEMV: per-row integer dot
 * products on the vector ALUs (the pages' decode path, Pulsar README,
 * 'Fidelity notes').  MFMA: int8 matrix-core tiles (the pages' quantized
 * tensor-core prefill, Pulsar README, 'What it does today', prefill
 * paragraphs; Strata article, long-prompt section).  AUTO:
 * GEMV for one token, MFMA for more.  Every path gives the same ids, lists and
 * q8_K(h) bytes; y differs only by floating summation order.
 */
typedef enum { MOEQ_PATH_AUTO = 0, MOEQ_PATH_GEMV = 1, MOEQ_PATH_MFMA = 2 } moeq_path;

/* Human-readable name of a status code (host, static string). */
const char* moeq_status_string(int status);

/*
 * q8_K quantisation of activation rows (Pulsar README, 'Fidelity notes':
 * activations go to q8_K before integer dots).  x: fp32 [rows, cols],
 * row-major, 16-byte aligned; cols % 256 == 0.  out: rows * cols/256 blocks of
 * 292 B, 4-byte aligned.  Per 256-block, in fp32 with round-half-even:
 * amax = max|x|; if amax == 0 or 127/amax overflows the block is all zero;
 * else id = 127/amax, q = clamp(rint(x*id), -127, 127), d = amax/127,
 * bsums[j] = sum of q[16j..16j+15].  rows == 0 is a no-op.
 */
int moeq_quantize_q8K(const float* x, int64_t rows, int64_t cols, void* out, void* stream);

/* Router descriptor.  1 <= k <= min(E, 32); E <= 4096; H % 4 == 0. */
typedef struct {
    int64_t T, H, E;
    int32_t k;
    int32_t gating;   /* moeq_gating */
    float scale;      /* multiplies every gate weight (1.0 for plain gating) */
} moeq_route_desc;

/* Workspace bytes moeq_route needs for this descriptor (host). */
size_t moeq_route_workspace(const moeq_route_desc* d);

/*
 * Router, top-k gating and token x expert lists for T tokens (the router runs
 * per layer on device: Pulsar README, 'How the streaming works'; one expert
 * union per chunk-layer: Pulsar README, DeepSeek-V4-Flash paragraph; the
 * softmax router of Qwen3 MoE models and the sigmoid router with a shared
 * expert: Pulsar README, 'What it does today', RRLab digest of Pulsar,
 * section 2).
 *   x        fp32 [T, H]        w_router fp32 [E, H]      bias fp32 [E] or NULL
 *   logits   fp64 [T, E] or NULL: l = sum_i w_router[e,i]*x[t,i] (+ bias[e]),
 *            accumulated in fp64
 *   topk_ids int32 [T, k]: the k experts first under (l desc, index asc), in
 *            that order (ties go to the lower index)
 *   topk_w   fp32 [T, k]: gate weights (computed in fp64, times scale)
 *   expert_offsets int32 [E+1], pairs int32 [T*k]: pairs[offsets[e] ..
 *            offsets[e+1]) holds t*k+slot for every pair routed to e, t rising
 *   active   int32 [1 + min(E, T*k)]: active[0] = n experts with a pair,
 *            active[1..n] = those experts, ascending (the expert union)
 *   x_q8K    q8_K rows of x [T, H/256 blocks] or NULL: when given (H % 256 == 0),
 *            the router launch also quantises x exactly as moeq_quantize_q8K
 * T == 0 writes offsets = 0 and active[0] = 0.  ws: moeq_route_workspace bytes,
 * 256-byte aligned.
 * Without a logits output (logits NULL), more than 256 tokens, H % 256 == 0,
 * E <= 1024 and top-k gating (softmax or sigmoid over the k selected), the
 * logits run as an approximate bf16 contraction whose error is bounded per
 * logit, and only the experts that can still be among the k get exact fp64
 * logits, from which the selection and the gate weights are made.  The pages
 * run one router per chunk-layer (Pulsar README, DeepSeek-V4-Flash
 * paragraph) and give no precision for it; this library keeps the selection
 * that of fp64 logits either way, so the outputs are the same as with a
 * logits output.
 */
int moeq_route(const moeq_route_desc* d, const float* x, const float* w_router, const float* bias,
               double* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
               int32_t* pairs, int32_t* active, void* x_q8K, void* ws, size_t ws_bytes, void* stream);

/*
 * Bytes of one packed [rows, cols] matrix of format fmt (0 if unsupported or
 * cols % 256 != 0).  Host arithmetic only.  The packed form is what an
 * expert slab becomes once it is resident on the device (expert slabs are
 * uploaded to the GPU as they arrive and the kernels get plain device
 * pointers: Pulsar README, 'How the streaming works'; the K-quant expert
 * formats: Pulsar README, 'Get a model').
 */
size_t moeq_packed_bytes(int32_t fmt, int64_t rows, int64_t cols);

/*
 * One-time repack of n_mats exchange-format matrices [rows, cols] (stored
 * back to back in `aos`, device memory, any alignment) into the kernels'
 * packed form (n_mats * moeq_packed_bytes, back to back, 256-byte aligned,
 * caller-owned).  cols % 256 == 0.  Done once when an expert slab becomes
 * resident (Pulsar README, 'How the streaming works').  The packed bytes
 * hold the same codes and scales, reordered so that each super-block loads
 * as contiguous runs.  A fused gate_up tensor (Pulsar README, 'Get a
 * model': fused gate_up tensors) of an expert, [2F, H] with the gate rows
 * first, is two [F, H] matrices back to back: packed with n_mats = 2 per
 * expert, the first packed matrix is its gate and the second its up.
 * n_mats == 0 is a no-op; errors: MOEQ_E_UNSUPPORTED for an unknown format,
 * MOEQ_E_INVALID for bad sizes, NULLs or packed not 256-byte aligned.
 */
int moeq_pack_experts(int32_t fmt, const void* aos, int64_t n_mats, int64_t rows, int64_t cols,
                      void* packed, void* stream);

/*
 * FFN descriptor.  gate/up: [F, H] per expert, down: [H, F]; H, F % 256 == 0.
 * gate, up, down: device arrays of E pointers to packed matrices; a NULL entry
 * means the expert is not resident in this call, so its pairs add nothing
 * (each launch gets explicit per-expert pointers and a NULL slot means "not
 * mine": Pulsar README, 'How the streaming works').  fmt_gate must equal
 * fmt_up.  sh_*: packed shared-expert matrices ([F_shared, H] / [H, F_shared])
 * or all NULL for no shared expert (top-k plus an always-on shared expert:
 * Pulsar README model table).
 */
typedef struct {
    int64_t T, H, F, E;
    int32_t k;
    int32_t fmt_gate, fmt_up, fmt_down;
    const void* const* gate;
    const void* const* up;
    const void* const* down;
    int64_t F_shared;
    int32_t sh_fmt_gate, sh_fmt_up, sh_fmt_down;
    const void* sh_gate;
    const void* sh_up;
    const void* sh_down;
    int32_t path;        /* moeq_path */
    int32_t accumulate;  /* 0: y = result, 1: y += result */
    /* Optional caller-owned auxiliary stream (hipStream_t) and two events
     * (hipEvent_t, made with hipEventDisableTiming) on the same device, for
     * a shared expert that runs apart from the routed launches: all three
     * NULL (everything on `stream`) or all three set (else MOEQ_E_INVALID). */
    void* aux_stream;
    void* aux_fork;
    void* aux_join;
} moeq_ffn_desc;

/* Workspace bytes moeq_expert_ffn needs for this descriptor (host). */
size_t moeq_expert_ffn_workspace(const moeq_ffn_desc* d);

/*
 * Routed-expert FFN over the token x expert lists from moeq_route.
 *   x_q8K   q8_K rows of x [T, H/256 blocks]
 *   topk_ids, topk_w  int32 / fp32 [T, k]; expert_offsets, pairs, active: all
 *           as moeq_route writes them (the FFN trusts their consistency)
 *   shared_scale fp32 [T] or NULL (= 1.0 per token)
 *   y       fp32 [T, H]:  y[t] (=|+=) sum_slot topk_w[t,slot] * down_e(q8K(h))
 *                                    + shared_scale[t] * down_sh(q8K(h_sh))
 *           with h = fl32(silu(g) * u), g = gate_e . xhat, u = up_e . xhat;
 *           per-super-block integer dots combined in fp64, sums in fp64.
 *           One token: y is rounded to fp32 once.  More tokens: each
 *           weighted pair term is rounded to fp32 when staged, then the k+1
 *           terms of a token are summed in fp64 and rounded (about 1e-7
 *           relative on y).
 * ws: moeq_expert_ffn_workspace bytes, 256-byte aligned; contents on entry
 * are ignored.
 */
int moeq_expert_ffn(const moeq_ffn_desc* d, const void* x_q8K, const int32_t* topk_ids, const float* topk_w,
                    const int32_t* expert_offsets, const int32_t* pairs, const int32_t* active,
                    const float* shared_scale, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole hot path of one MoE layer in one call: moeq_route (with q8_K(x)
 * into the workspace) followed by moeq_expert_ffn, with the same outputs and
 * the same conventions.  r and f must agree on T, H, E and k.  For one token
 * it enqueues three kernels: router logits with q8_K(x); gate/up, where every
 * workgroup takes the top-k from the logits itself and one workgroup writes
 * the routing outputs; down with the weighted combine.  Each launch boundary
 * is the only synchronisation (per-layer launches are the floor of a decode
 * step: Strata summary, execution paragraph).  A chunk of 2..8 tokens with at
 * most 64 (token, slot) pairs and at most 512 experts, every expert on the
 * int8 matrix-core path in its fp32-h 8-row tiles (the MTP verify rows: one
 * router readback and one expert union per chunk-layer, Pulsar README,
 * DeepSeek-V4-Flash paragraph), routes the same way: router logits with
 * q8_K(x), then gate/up tiles that each select the chunk's experts from the
 * logits and form its union themselves (one workgroup writes the routing
 * outputs), down, the combine.  Other shapes run the two calls back to back.
 * Outputs are the same on every route.  logits may be NULL; the FFN's q8_K(h)
 * view (moeq_ffn_h_view with f and this ws) stays valid after the call.
 */
size_t moeq_moe_layer_workspace(const moeq_route_desc* r, const moeq_ffn_desc* f);
int moeq_moe_layer(const moeq_route_desc* r, const moeq_ffn_desc* f, const float* x, const float* w_router,
                   const float* bias, double* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                   int32_t* pairs, int32_t* active, const float* shared_scale, float* y, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * RMS pre-norm of T token rows: out[t, i] = fl32((x[t, i] * r_t) * gamma[i]),
 * r_t = 1 / sqrt(mean_i(x[t, i]^2) + eps), everything before the final
 * rounding in fp64 (the squares are exact; only the order of the sum's
 * additions is the kernel's).  This is the input normalisation of the
 * pre-norm decoder blocks of the MoE models the engines run (Pulsar README
 * and Strata summary: whole Qwen and DeepSeek-style models); the pages give
 * the models, not this step, so its precision is this library's choice.  It
 * is the glue between the MoE layers of moeq_moe_stack, exported so a caller
 * can form the same layer input.
 *   x, out  fp32 [T, H], 16-byte aligned; out may equal x (in place)
 *   gamma   fp32 [H], 16-byte aligned, or NULL (all ones)
 *   eps     finite, >= 0
 * H a positive multiple of 256; T == 0 is a no-op.  Errors: MOEQ_E_INVALID.
 */
int moeq_rms_norm(const float* x, int64_t T, int64_t H, const float* gamma, float eps, float* out, void* stream);

/*
 * A stack of L MoE layers over the same T tokens on a pre-norm residual
 * stream: y = x, then for l = 0 .. L-1, y += MoE_l(RMSNorm_l(y)).  These are
 * the MoE blocks of a decode step run one after the other; the attention
 * blocks between them belong to the model around this path, and per-layer
 * launches are captured as one graph (Strata summary, execution paragraph).
 * Layer l is exactly moeq_rms_norm(y, T, H, norm_w[l], norm_eps, xn) then
 * moeq_moe_layer(r, f[l] with accumulate = 1, xn, w_router[l], bias[l], NULL
 * logits, ..., y), with its routing outputs at offset l of each output array,
 * and its results are bit-identical to those two calls.  For one token (H <=
 * 4096, decode GEMV path) the norm is fused into the router launch: no
 * normalised copy is written and the layer stays three kernels.  Without the
 * norm, a chain of SwiGLU experts (quadratic in their input's scale) grows
 * without bound.
 *   f            host array [L] of FFN descriptors; every one agrees with r
 *                on T, H, E, k and has accumulate == 0 (the stack accumulates)
 *   w_router     host array [L] of device pointers fp32 [E, H] (16-byte aligned)
 *   bias         host array [L] of device pointers fp32 [E] (entries may be NULL) or NULL
 *   norm_w       host array [L] of device pointers fp32 [H] (16-byte aligned;
 *                entries may be NULL = all ones) or NULL
 *   norm_eps     finite, >= 0
 *   shared_scale host array [L] of device pointers fp32 [T] (entries may be NULL) or NULL
 *   x, y         fp32 [T, H], 16-byte aligned; y may equal x (in place)
 *   topk_ids, topk_w [L, T, k]; expert_offsets [L, E+1];
 *   pairs [L, max(1, T*k)]; active [L, 1 + min(E, T*k)]
 * ws: moeq_moe_stack_workspace bytes (the largest layer workspace and room
 * for the normalised rows), 256-byte aligned.  1 <= L <= 4096.  Errors as
 * moeq_moe_layer.
 */
size_t moeq_moe_stack_workspace(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L);
int moeq_moe_stack(const moeq_route_desc* r, const moeq_ffn_desc* f, int64_t L, const float* const* w_router,
                   const float* const* bias, const float* const* norm_w, float norm_eps, const float* x,
                   int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* pairs, int32_t* active,
                   const float* const* shared_scale, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moeq_moe_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * moeq_moe_layer, whose kernels it runs; the workspace is instead a static
 * device array of MOEQ_NOALLOC_MAX_BYTES (32 MiB) inside the library, one
 * per GPU, held from the library's load until the process ends.  The call
 * allocates nothing; on its first call on a device (the current device) it
 * looks up that device's array once.  Every call on a GPU shares that GPU's
 * array, so calls whose work may overlap on one GPU race: order them (one
 * stream, or events).  `stream` must belong to the current device (NULL =
 * its null stream).  Errors: as moeq_moe_layer; MOEQ_E_STATIC_LIMIT when
 * moeq_moe_layer_workspace(r, f) exceeds MOEQ_NOALLOC_MAX_BYTES (the request
 * is rejected before anything is enqueued).  moeq_ffn_h_view does not apply.
 */
#define MOEQ_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int moeq_moe_layer_noalloc(const moeq_route_desc* r, const moeq_ffn_desc* f, const float* x,
                           const float* w_router, const float* bias, double* logits, int32_t* topk_ids,
                           float* topk_w, int32_t* expert_offsets, int32_t* pairs, int32_t* active,
                           const float* shared_scale, float* y, void* stream);

/*
 * Test hook (GPU kernel selftests against CPU references and a bit-exact
 * gate: Pulsar README, 'Tests'): where a finished moeq_expert_ffn call left
 * q8_K(h) inside `ws` (host arithmetic only, nothing is enqueued).
 * *hq_routed: [T*k] rows of F/256 blocks, row p = pair t*k+slot (rows of
 * absent experts are unspecified); *hq_shared: [T] rows of F_shared/256
 * blocks, or NULL without a shared expert.  The pointers point into the
 * caller's ws.  Errors: as the descriptor checks of moeq_expert_ffn, plus
 * MOEQ_E_WORKSPACE when ws_bytes is below moeq_expert_ffn_workspace.
 */
int moeq_ffn_h_view(const moeq_ffn_desc* d, void* ws, size_t ws_bytes, void** hq_routed,
                    void** hq_shared);

/*
 * Test hook (GPU kernel selftests against CPU references: Pulsar README,
 * 'Tests'; exact integer dots of K-quant weights with q8_K activations:
 * Pulsar README, 'Fidelity notes'): the exact int32 sub-block dots of a
 * packed matrix with q8_K rows, computed by the same device dot routines the
 * dot-product (GEMV) kernels use.  Enqueued on `stream`; n_x == 0 is a no-op.
 *   packed_w [rows, cols] packed fmt; x_q8K [n_x, cols/256 blocks]
 *   out int32 [n_x, rows, cols/sub]: sum over sub-block j of code * q_x, where
 *   sub = 32 (Q4_K, Q5_K, Q8_0, Q4_0, Q5_1) or 16 (Q2_K, Q3_K, Q6_K) and
 *   code = q (Q4_K, Q5_K, Q2_K, Q5_1), q-32 (Q6_K), q-4 (Q3_K), q-8 (Q4_0),
 *   signed q (Q8_0).
 */
int moeq_debug_subdots(int32_t fmt, const void* packed_w, int64_t rows, int64_t cols,
                       const void* x_q8K, int64_t n_x, int32_t* out, void* stream);

/*
 * Test hook (a one-row GPU-versus-CPU integer arbiter: Pulsar README, 'What
 * it does today', CPU-lane paragraph; GPU kernel selftests against CPU
 * references: Pulsar README, 'Tests'): the exact integer parts of every
 * super-block term, computed by the int8 MFMA tile code of the MFMA path (the
 * same MFMA and unpack routines, the same LDS staging of q8_K rows).
 *   packed_w [rows, cols] packed fmt, rows % 256 == 0; x_q8K [n_x, cols/256
 *   blocks]; out int32 [n_x, rows, cols/256, 8], 16-byte aligned:
 *     Q4_K, Q5_K, Q2_K: (S1, S2, 0...) with S1 = sum_j sc_j isum_j,
 *                 S2 = sum_j m_j bsum_j (bsum over the sub-block's 32 / 16
 *                 activations)
 *     Q6_K, Q3_K: (S1, S2, 0...) with S1 = sum_j sc_j isum_j over the codes
 *                 q - 32 (Q6_K) or q - 4 (Q3_K) and S2 = sum_j sc_j bsum_j
 *     Q8_0, Q4_0, Q5_1: isum_b of the eight 32-blocks of the super-block
 *                 (over q - 8 for Q4_0, over q for Q5_1, whose min term
 *                 m_b bsum_b is not part of it)
 * Enqueued on `stream`; n_x == 0 is a no-op.  Errors: MOEQ_E_UNSUPPORTED for
 * an unknown format, MOEQ_E_INVALID for bad sizes, NULLs or misalignment.
 */
int moeq_debug_mfma_sums(int32_t fmt, const void* packed_w, int64_t rows, int64_t cols,
                         const void* x_q8K, int64_t n_x, int32_t* out, void* stream);

/*
 * Measurement helpers: the ceilings that the kernels' rooflines are read
 * against beside the nominal peaks (the pages judge their own multi-row
 * kernels by profiler utilisation of the memory units and of DRAM: Pulsar
 * README, ThinkingCap paragraph).  Neither touches any other state.
 *
 * moeq_ceiling_read: reads every 16-byte word of buf (device, 16-byte
 *   aligned; bytes a positive multiple of 16) once, with n_blocks workgroups
 *   of 256 threads in a grid-stride loop of plain 16-byte global loads, four
 *   in flight per thread.  Workgroup b writes the wrapping 64-bit sum of the
 *   32-bit words it read to out[b] (device, n_blocks uint64 entries, 8-byte
 *   aligned), so the sum of out modulo 2^64 is the sum of all 32-bit words of
 *   buf.  The achieved bandwidth is bytes over the launch's duration.
 * moeq_ceiling_mfma_i8: n_blocks workgroups of 4 waves; each wave runs iters
 *   steps of four independent v_mfma_i32_32x32x32_i8 on registers holding
 *   bytes of 1 (4 * 65536 integer operations per step, no memory traffic)
 *   and writes 128 * iters modulo 2^32 to out[4 b + w] (device, 4 * n_blocks
 *   int32 entries, 4-byte aligned) for wave w of workgroup b.
 * Both enqueue on `stream`.  Errors: MOEQ_E_INVALID for a NULL or misaligned
 * pointer, bytes <= 0 or not a multiple of 16, n_blocks outside 1..2^22, or
 * iters < 1; MOEQ_E_HIP when the launch fails.
 */
int moeq_ceiling_read(const void* buf, int64_t bytes, int32_t n_blocks, uint64_t* out, void* stream);
int moeq_ceiling_mfma_i8(int64_t iters, int32_t n_blocks, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEQ_H */
