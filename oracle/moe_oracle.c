/*
 * moe_oracle.c -- plain, slow CPU oracle of the routed-expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library and never calls it.
 *
 * What it computes (one MoE layer, per token t):
 *   (stack)        x = RMSNorm(y) of the residual stream y, then y += MoE(x)
 *   router logits  l[t,e] = sum_i Wr[e,i] * x[t,i] (+ b[e])         fp64
 *       (the router runs per layer on the resident input: Pulsar README,
 *        'How the streaming works'; the router stays in VRAM: Strata summary,
 *        three-tier offload paragraph)
 *   top-k          the k experts first under the order (l desc, index asc)
 *   gating         softmax over the selected k (Qwen-style softmax router,
 *                  Pulsar README 'What it does today'), softmax over all E
 *                  (variant), or sigmoid over the selected k renormalised
 *                  (sigmoid-gated router with a shared expert, RRLab digest of
 *                  Pulsar, section 2, Ornith-397B entry)
 *   q8_K(x)        int8 per 256-block, fp32 scale, per-16 sums (activations
 *                  quantised to q8_K before integer dots: Pulsar README,
 *                  'Fidelity notes')
 *   gate/up        g = Wg[e] xhat, u = Wu[e] xhat with the dequantised weights
 *   SwiGLU         h = fl32(silu(g) * u)
 *   down           y_p = Wd[e] q8_K(h)^
 *   combine        y[t] = fl32(sum_slot w_slot y_p + s_t y_shared)
 *                  (top-k of E plus an always-on shared expert: Pulsar README,
 *                  model table)
 *
 * Floating point: everything after the integer codes is fp64 with sequential
 * sums, except the three fp32 rounding points the method fixes: q8_K
 * arithmetic, h and y.  Build with -O2 -fno-fast-math -ffp-contract=off.
 *
 * Block formats (exchange layout; the pages name the formats but print no
 * byte layout, so this layout is the repository's own, little-endian):
 *   q8_K  292 B : f32 d | i8 qs[256] | i16 bsums[16]
 *   Q4_K  144 B : f16 d | f16 dmin | u8 sm[12] | u8 qs[128]
 *                 sm = bit stream: 8 six-bit scales (bits 0..47) then 8 six-bit
 *                 mins (bits 48..95); qs: byte 32g+i holds element 64g+i (low
 *                 nibble) and 64g+32+i (high nibble); sub-blocks of 32
 *                 w = d*sc_j*q - dmin*m_j
 *   Q2_K   84 B : f16 d | f16 dmin | u8 sm[16] (low nibble sc_j, high m_j) |
 *                 u8 qs[64]: byte 32h+i holds element 128h+32s+i in bits 2s..2s+1;
 *                 sub-blocks of 16;  w = d*sc_j*q - dmin*m_j
 *   Q6_K  210 B : f16 d | i8 sc[16] | u8 ql[128] | u8 qh[64]
 *                 ql byte 64h+i: low 4 bits of element 128h+i (low nibble) and
 *                 128h+64+i (high nibble); qh byte 32h+i: high 2 bits of element
 *                 128h+32s+i in bits 2s..2s+1; sub-blocks of 16; w = d*sc_j*(q-32)
 *   Q8_0   34 B : f16 d | i8 qs[32];  w = d*q
 *   Q3_K  110 B : f16 d | u8 sc[12] (bit stream: 16 six-bit values, stored
 *                 sc_j + 32) | u8 ql[64] (as Q2_K's qs: low 2 bits) | u8 qh[32]
 *                 (byte i bit b: high bit of element 32b+i); q = low + 4*high;
 *                 sub-blocks of 16; w = d*sc_j*(q-4)
 *   Q5_K  176 B : the 144 bytes of Q4_K (its quants are the low nibbles) |
 *                 u8 qh[32] (byte i bit b: bit 4 of element 32b+i); sub-blocks
 *                 of 32; w = d*sc_j*q - dmin*m_j
 *   Q4_0   18 B : f16 d | u8 qs[16] (byte i: element i low nibble, element
 *                 16+i high nibble);  w = d*(q-8)
 *   Q5_1   24 B : f16 d | f16 m | u8 qh[4] (bit i of the little-endian word:
 *                 bit 4 of element i) | u8 qs[16] as Q4_0;  w = d*q + m
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { F_Q4_K = 1, F_Q6_K = 2, F_Q2_K = 3, F_Q8_0 = 4, F_Q3_K = 5, F_Q5_K = 6, F_Q4_0 = 7, F_Q5_1 = 8 };
enum { G_SOFTMAX_TOPK = 0, G_SOFTMAX_ALL = 1, G_SIGMOID_TOPK = 2 };

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 to double, exact. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ----------------------------------------------------------- block codes */

int orc_block_bytes(int fmt)
{
    switch (fmt) {
    case F_Q4_K: return 144;
    case F_Q6_K: return 210;
    case F_Q2_K: return 84;
    case F_Q8_0: return 34;
    case F_Q3_K: return 110;
    case F_Q5_K: return 176;
    case F_Q4_0: return 18;
    case F_Q5_1: return 24;
    }
    return 0;
}

int orc_block_weights(int fmt) { return (fmt == F_Q8_0 || fmt == F_Q4_0 || fmt == F_Q5_1) ? 32 : 256; }

/* Elements per sub-block: the unit that carries one scale (and min). */
int orc_subblock(int fmt)
{
    switch (fmt) {
    case F_Q4_K: return 32;
    case F_Q6_K: return 16;
    case F_Q2_K: return 16;
    case F_Q8_0: return 32;
    case F_Q3_K: return 16;
    case F_Q5_K: return 32;
    case F_Q4_0: return 32;
    case F_Q5_1: return 32;
    }
    return 0;
}

/* The offset subtracted from the stored code: w = d*sc*(q - offset) (Q6_K, Q3_K, Q4_0). */
static int code_offset(int fmt) { return fmt == F_Q6_K ? 32 : fmt == F_Q3_K ? 4 : fmt == F_Q4_0 ? 8 : 0; }

/* Bits [pos, pos + n) of a little-endian byte stream. */
static int stream_bits(const uint8_t* p, int pos, int n)
{
    int v = 0, bit;
    for (bit = 0; bit < n; bit++)
        v |= ((p[(pos + bit) >> 3] >> ((pos + bit) & 7)) & 1) << bit;
    return v;
}

/*
 * Decode one block into integer codes.  q[] gets the quant code of every
 * element (Q6_K: 0..63 before the -32 offset; Q3_K: 0..7 before the -4
 * offset; Q4_0: 0..15 before the -8 offset; Q8_0: signed), sc[]/m[] the
 * per-sub-block scale and min codes (m = 0 where the format has none),
 * d/dmin the fp16 super-scales as doubles.
 */
int orc_block_codes(int fmt, const uint8_t* b, double* d, double* dmin, int* sc, int* m, int* q)
{
    int i, j, g, h, s;
    switch (fmt) {
    case F_Q4_K: {
        const uint8_t* sm = b + 4;
        const uint8_t* qs = b + 16;
        *d = orc_half_to_double(rd16(b));
        *dmin = orc_half_to_double(rd16(b + 2));
        for (j = 0; j < 8; j++) {
            int vs = 0, vm = 0, bit;
            for (bit = 0; bit < 6; bit++) {
                int ns = 6 * j + bit, nm = 48 + 6 * j + bit;
                vs |= ((sm[ns >> 3] >> (ns & 7)) & 1) << bit;
                vm |= ((sm[nm >> 3] >> (nm & 7)) & 1) << bit;
            }
            sc[j] = vs;
            m[j] = vm;
        }
        for (g = 0; g < 4; g++)
            for (i = 0; i < 32; i++) {
                q[64 * g + i] = qs[32 * g + i] & 15;
                q[64 * g + 32 + i] = qs[32 * g + i] >> 4;
            }
        return 0;
    }
    case F_Q2_K: {
        const uint8_t* sm = b + 4;
        const uint8_t* qs = b + 20;
        *d = orc_half_to_double(rd16(b));
        *dmin = orc_half_to_double(rd16(b + 2));
        for (j = 0; j < 16; j++) {
            sc[j] = sm[j] & 15;
            m[j] = sm[j] >> 4;
        }
        for (h = 0; h < 2; h++)
            for (s = 0; s < 4; s++)
                for (i = 0; i < 32; i++)
                    q[128 * h + 32 * s + i] = (qs[32 * h + i] >> (2 * s)) & 3;
        return 0;
    }
    case F_Q6_K: {
        const uint8_t* scb = b + 2;
        const uint8_t* ql = b + 18;
        const uint8_t* qh = b + 146;
        *d = orc_half_to_double(rd16(b));
        *dmin = 0.0;
        for (j = 0; j < 16; j++) {
            sc[j] = (int)(int8_t)scb[j];
            m[j] = 0;
        }
        for (h = 0; h < 2; h++)
            for (i = 0; i < 64; i++) {
                q[128 * h + i] = ql[64 * h + i] & 15;
                q[128 * h + 64 + i] = ql[64 * h + i] >> 4;
            }
        for (h = 0; h < 2; h++)
            for (s = 0; s < 4; s++)
                for (i = 0; i < 32; i++)
                    q[128 * h + 32 * s + i] |= ((qh[32 * h + i] >> (2 * s)) & 3) << 4;
        return 0;
    }
    case F_Q3_K: {
        const uint8_t* ql = b + 14;
        const uint8_t* qh = b + 78;
        *d = orc_half_to_double(rd16(b));
        *dmin = 0.0;
        for (j = 0; j < 16; j++) {
            sc[j] = stream_bits(b + 2, 6 * j, 6) - 32;
            m[j] = 0;
        }
        for (h = 0; h < 2; h++)
            for (s = 0; s < 4; s++)
                for (i = 0; i < 32; i++)
                    q[128 * h + 32 * s + i] = (ql[32 * h + i] >> (2 * s)) & 3;
        for (s = 0; s < 8; s++)
            for (i = 0; i < 32; i++)
                q[32 * s + i] += 4 * ((qh[i] >> s) & 1);
        return 0;
    }
    case F_Q5_K: {
        const uint8_t* qh = b + 144;
        if (orc_block_codes(F_Q4_K, b, d, dmin, sc, m, q))
            return -1;
        for (s = 0; s < 8; s++)
            for (i = 0; i < 32; i++)
                q[32 * s + i] += 16 * ((qh[i] >> s) & 1);
        return 0;
    }
    case F_Q4_0:
    case F_Q5_1: {
        const uint8_t* qs = b + (fmt == F_Q4_0 ? 2 : 8);
        *d = orc_half_to_double(rd16(b));
        *dmin = fmt == F_Q5_1 ? orc_half_to_double(rd16(b + 2)) : 0.0;   /* Q5_1: the min m */
        sc[0] = 1;
        m[0] = 0;
        for (i = 0; i < 16; i++) {
            q[i] = qs[i] & 15;
            q[16 + i] = qs[i] >> 4;
        }
        if (fmt == F_Q5_1)
            for (i = 0; i < 32; i++)
                q[i] += 16 * ((b[4 + i / 8] >> (i % 8)) & 1);
        return 0;
    }
    case F_Q8_0: {
        *d = orc_half_to_double(rd16(b));
        *dmin = 0.0;
        sc[0] = 1;
        m[0] = 0;
        for (i = 0; i < 32; i++)
            q[i] = (int)(int8_t)b[2 + i];
        return 0;
    }
    }
    return -1;
}

/* Dequantise one block to fp64 with the format's closed form. */
static int dequant_block(int fmt, const uint8_t* b, double* out)
{
    double d, dmin;
    int sc[16], m[16], q[256], i;
    int nw = orc_block_weights(fmt), sb = orc_subblock(fmt);
    if (orc_block_codes(fmt, b, &d, &dmin, sc, m, q))
        return -1;
    for (i = 0; i < nw; i++) {
        int j = i / sb;
        switch (fmt) {
        case F_Q4_K:
        case F_Q5_K:
        case F_Q2_K: out[i] = d * (double)sc[j] * (double)q[i] - dmin * (double)m[j]; break;
        case F_Q6_K:
        case F_Q3_K:
        case F_Q4_0: out[i] = d * (double)sc[j] * (double)(q[i] - code_offset(fmt)); break;
        case F_Q5_1: out[i] = d * (double)q[i] + dmin; break;
        case F_Q8_0: out[i] = d * (double)q[i]; break;
        }
    }
    return 0;
}

/* Dequantise a row of `cols` weights (cols / block_weights blocks back to back). */
int orc_dequant_row(int fmt, const uint8_t* row, int64_t cols, double* out)
{
    int bw = orc_block_weights(fmt), bb = orc_block_bytes(fmt);
    int64_t b;
    if (!bw || cols % bw)
        return -1;
    for (b = 0; b < cols / bw; b++)
        if (dequant_block(fmt, row + b * bb, out + b * bw))
            return -1;
    return 0;
}

/* ------------------------------------------------------------------ pre-norm */

/*
 * RMS pre-norm of each row (the input of a pre-norm decoder's MoE block in a
 * stack of layers; the pages run whole models of such blocks but do not
 * spell this step out, so the precision is a reading):
 *   r = 1 / sqrt(mean_i x_i^2 + eps), sequential fp64 sum of the squares;
 *   out_i = fl32((x_i * r) * g_i), both products in fp64 (g NULL: g_i = 1).
 */
void orc_rms_norm(const float* x, int64_t rows, int64_t cols, const float* g, double eps, float* out)
{
    int64_t t, i;
    for (t = 0; t < rows; t++) {
        const float* xr = x + t * cols;
        double ss = 0.0, r;
        for (i = 0; i < cols; i++)
            ss += (double)xr[i] * (double)xr[i];
        r = 1.0 / sqrt(ss / (double)cols + eps);
        for (i = 0; i < cols; i++)
            out[t * cols + i] = (float)(((double)xr[i] * r) * (g ? (double)g[i] : 1.0));
    }
}

/* ------------------------------------------------------------------ q8_K */

/*
 * q8_K of one row (cols % 256 == 0), fp32 arithmetic, round half to even:
 *   amax = max |x|; a block is all-zero if amax == 0 or 127/amax overflows;
 *   otherwise id = fl32(127/amax), q = clamp(rint(fl32(x*id)), -127, 127),
 *   d = fl32(amax/127), bsums[j] = sum of q over elements 16j..16j+15.
 */
void orc_quantize_q8K_row(const float* x, int64_t cols, uint8_t* out)
{
    int64_t b;
    int i, j;
    for (b = 0; b < cols / 256; b++) {
        const float* xb = x + b * 256;
        uint8_t* o = out + b * 292;
        float amax = 0.0f, id, d;
        int8_t qs[256];
        int16_t bs[16];
        for (i = 0; i < 256; i++) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        id = (amax == 0.0f) ? 0.0f : 127.0f / amax;
        if (amax == 0.0f || isinf(id)) {
            memset(o, 0, 292);
            continue;
        }
        d = amax / 127.0f;
        for (i = 0; i < 256; i++) {
            float v = rintf(xb[i] * id);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            qs[i] = (int8_t)v;
        }
        for (j = 0; j < 16; j++) {
            int s = 0;
            for (i = 0; i < 16; i++)
                s += qs[16 * j + i];
            bs[j] = (int16_t)s;
        }
        memcpy(o, &d, 4);
        memcpy(o + 4, qs, 256);
        memcpy(o + 260, bs, 32);
    }
}

void orc_quantize_q8K(const float* x, int64_t rows, int64_t cols, uint8_t* out)
{
    int64_t r;
    for (r = 0; r < rows; r++)
        orc_quantize_q8K_row(x + r * cols, cols, out + r * (cols / 256) * 292);
}

/* xhat = d * q per element, fp64. */
void orc_dequant_q8K_row(const uint8_t* q8, int64_t cols, double* out)
{
    int64_t b;
    int i;
    for (b = 0; b < cols / 256; b++) {
        float d;
        memcpy(&d, q8 + b * 292, 4);
        for (i = 0; i < 256; i++)
            out[b * 256 + i] = (double)d * (double)(int8_t)q8[b * 292 + 4 + i];
    }
}

/* ---------------------------------------------------------------- router */

/* One expert's sort key: the order is (logit desc, index asc). */
typedef struct {
    double l;
    int32_t e;
} rank_item;

static int cmp_rank(const void* a, const void* b)
{
    const rank_item* x = (const rank_item*)a;
    const rank_item* y = (const rank_item*)b;
    if (x->l > y->l) return -1;
    if (x->l < y->l) return 1;
    return x->e < y->e ? -1 : (x->e > y->e);
}

/* Router of one token: logits, ids and weights as orc_route describes. */
static int route_one(int64_t H, int64_t E, int k, int gating, double scale, const float* x,
                     const float* Wr, const float* bias, double* logits, int32_t* ids, float* w,
                     rank_item* order, double* l)
{
    int64_t e, i;
    int s;
    for (e = 0; e < E; e++) {
        double acc = 0.0;
        for (i = 0; i < H; i++)
            acc += (double)Wr[e * H + i] * (double)x[i];
        if (bias)
            acc += (double)bias[e];
        l[e] = acc;
        order[e].l = acc;
        order[e].e = (int32_t)e;
        if (logits)
            logits[e] = acc;
    }
    qsort(order, (size_t)E, sizeof(rank_item), cmp_rank);
    for (s = 0; s < k; s++)
        ids[s] = order[s].e;
    if (gating == G_SOFTMAX_TOPK) {
        double mx = order[0].l, z = 0.0;
        for (s = 0; s < k; s++)
            z += exp(order[s].l - mx);
        for (s = 0; s < k; s++)
            w[s] = (float)(exp(order[s].l - mx) / z * scale);
    } else if (gating == G_SOFTMAX_ALL) {
        double mx = order[0].l, z = 0.0;
        for (e = 0; e < E; e++)
            z += exp(l[e] - mx);
        for (s = 0; s < k; s++)
            w[s] = (float)(exp(order[s].l - mx) / z * scale);
    } else if (gating == G_SIGMOID_TOPK) {
        double z = 0.0;
        for (s = 0; s < k; s++)
            z += 1.0 / (1.0 + exp(-order[s].l));
        for (s = 0; s < k; s++)
            w[s] = (float)(1.0 / (1.0 + exp(-order[s].l)) / z * scale);
    } else {
        return -1;
    }
    return 0;
}

/*
 * Router for T tokens: logits (fp64, sequential sum, bias added last), the
 * top-k ids in rank order and fp32 gate weights (computed in fp64, times
 * `scale`, rounded once).  logits may be NULL.  Tokens are independent and
 * run in parallel (OpenMP); each keeps its own sort keys.
 */
int orc_route(int64_t T, int64_t H, int64_t E, int k, int gating, double scale,
              const float* x, const float* Wr, const float* bias,
              double* logits, int32_t* ids, float* w)
{
    int64_t t;
    int bad = 0;
    if (k < 1 || k > E)
        return -1;
    if (gating != G_SOFTMAX_TOPK && gating != G_SOFTMAX_ALL && gating != G_SIGMOID_TOPK)
        return -1;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (t = 0; t < T; t++) {
        rank_item* order = (rank_item*)malloc(sizeof(rank_item) * E);
        double* l = (double*)malloc(sizeof(double) * E);
        bad |= route_one(H, E, k, gating, scale, x + t * H, Wr, bias, logits ? logits + t * E : NULL,
                         ids + t * k, w + t * k, order, l);
        free(order);
        free(l);
    }
    return bad ? -1 : 0;
}

/*
 * Token x expert lists: offsets[e]..offsets[e+1] index `pairs`, which holds
 * t*k+slot for every pair routed to e, in increasing t.  active[0] = number
 * of experts with at least one pair, active[1..] = those experts ascending.
 */
void orc_lists(int64_t T, int k, int64_t E, const int32_t* ids,
               int32_t* offsets, int32_t* pairs, int32_t* active)
{
    int64_t e, t, pos = 0, na = 0;
    int s;
    for (e = 0; e < E; e++) {
        offsets[e] = (int32_t)pos;
        for (t = 0; t < T; t++)
            for (s = 0; s < k; s++)
                if (ids[t * k + s] == e)
                    pairs[pos++] = (int32_t)(t * k + s);
        if (pos > offsets[e])
            active[1 + na++] = (int32_t)e;
    }
    offsets[E] = (int32_t)pos;
    active[0] = (int32_t)na;
}

/* ------------------------------------------------------------- integers */

/*
 * Exact int32 dot of each sub-block of each weight row with each q8_K row:
 * out[n][r][j] = sum over sub-block j of (weight code) * q_x, where the weight
 * code is q (Q4_K, Q5_K, Q2_K, Q5_1), q-32 (Q6_K), q-4 (Q3_K), q-8 (Q4_0) or
 * the signed q (Q8_0).
 */
int orc_subdots(int fmt, const uint8_t* w, int64_t rows, int64_t cols,
                const uint8_t* xq, int64_t n_x, int32_t* out)
{
    int bw = orc_block_weights(fmt), bb = orc_block_bytes(fmt), sbw = orc_subblock(fmt);
    int64_t nsub = cols / sbw, nblk = cols / bw, n, r, b;
    if (!bw || cols % 256)
        return -1;
#pragma omp parallel for collapse(2) private(b) schedule(static)
    for (n = 0; n < n_x; n++)
        for (r = 0; r < rows; r++)
            for (b = 0; b < nblk; b++) {
                double d, dmin;
                int sc[16], m[16], q[256], i;
                const uint8_t* blk = w + (r * nblk + b) * bb;
                orc_block_codes(fmt, blk, &d, &dmin, sc, m, q);
                for (i = 0; i < bw / sbw; i++) {
                    int32_t acc = 0;
                    int e;
                    for (e = 0; e < sbw; e++) {
                        int64_t col = b * bw + i * sbw + e;
                        int code = q[i * sbw + e] - code_offset(fmt);
                        int qx = (int8_t)xq[n * (cols / 256) * 292 + (col / 256) * 292 + 4 + col % 256];
                        acc += code * qx;
                    }
                    out[(n * rows + r) * nsub + b * (bw / sbw) + i] = acc;
                }
            }
    return 0;
}

/*
 * The sub-block scales and mins of every block of a [rows, cols] matrix, as
 * orc_block_codes decodes them: sc[((r * nblk) + b) * 16 + j] and m likewise
 * for sub-block j of block b of row r (nblk = cols / block width; Q8_0 blocks
 * have one sub-block with sc = 1, m = 0; unused entries are 0).
 */
int orc_scales_matrix(int fmt, const uint8_t* w, int64_t rows, int64_t cols, int32_t* sc, int32_t* m)
{
    int bw = orc_block_weights(fmt), bb = orc_block_bytes(fmt);
    int64_t nblk, r, b;
    if (!bw || cols % bw)
        return -1;
    nblk = cols / bw;
    for (r = 0; r < rows; r++)
        for (b = 0; b < nblk; b++) {
            double d, dmin;
            int s16[16] = {0}, m16[16] = {0}, q[256], j;
            if (orc_block_codes(fmt, w + (r * nblk + b) * bb, &d, &dmin, s16, m16, q))
                return -1;
            for (j = 0; j < 16; j++) {
                sc[(r * nblk + b) * 16 + j] = j < bw / orc_subblock(fmt) ? s16[j] : 0;
                m[(r * nblk + b) * 16 + j] = j < bw / orc_subblock(fmt) ? m16[j] : 0;
            }
        }
    return 0;
}

/*
 * The integer formulation of one row dot, summed per 256 super-block in fp64:
 *   Q4_K/Q5_K/Q2_K: d_x * (d * sum_j sc_j isum_j - dmin * sum_j m_j bsum_j)
 *   Q6_K/Q3_K:      d_x * d * sum_j sc_j isum_j (isum over the codes q - offset)
 *   Q8_0/Q4_0/Q5_1: d_x * sum_b (d_b isum_b + m_b bsum_b), isum over q - offset,
 *                   m_b the Q5_1 min (0 otherwise)
 * Used only to check that it equals the fp64 dequantised dot.
 */
double orc_dot_intform(int fmt, const uint8_t* wrow, int64_t cols, const uint8_t* xq)
{
    int64_t sb;
    double total = 0.0;
    for (sb = 0; sb < cols / 256; sb++) {
        float dxf;
        const uint8_t* xb = xq + sb * 292;
        const int8_t* qx = (const int8_t*)(xb + 4);
        int16_t bsums[16];
        double dx;
        memcpy(&dxf, xb, 4);
        memcpy(bsums, xb + 260, 32);
        dx = (double)dxf;
        if (orc_block_weights(fmt) == 32) {
            double acc = 0.0;
            int b;
            for (b = 0; b < 8; b++) {
                double d, dmin;
                int sc[1], m[1], q[32], e;
                int32_t is = 0, bs = bsums[2 * b] + bsums[2 * b + 1];
                orc_block_codes(fmt, wrow + (sb * 8 + b) * orc_block_bytes(fmt), &d, &dmin, sc, m, q);
                for (e = 0; e < 32; e++)
                    is += (q[e] - code_offset(fmt)) * qx[b * 32 + e];
                acc += d * (double)is + dmin * (double)bs;   /* dmin: Q5_1's min, else 0 */
            }
            total += dx * acc;
        } else {
            double d, dmin;
            int sc[16], m[16], q[256], j, e;
            int sbw = orc_subblock(fmt);
            int64_t S1 = 0, S2 = 0;
            orc_block_codes(fmt, wrow + sb * orc_block_bytes(fmt), &d, &dmin, sc, m, q);
            for (j = 0; j < 256 / sbw; j++) {
                int32_t is = 0, bs = 0;
                for (e = 0; e < sbw; e++) {
                    int code = q[j * sbw + e] - code_offset(fmt);
                    is += code * qx[j * sbw + e];
                }
                for (e = 0; e < sbw / 16; e++)
                    bs += bsums[j * sbw / 16 + e];
                S1 += (int64_t)sc[j] * is;
                S2 += (int64_t)m[j] * bs;
            }
            total += dx * (d * (double)S1 - dmin * (double)S2);
        }
    }
    return total;
}

/* ------------------------------------------------------------------- FFN */

/* sum_c a[c] * b[c], fp64, sequential in c. */
static double dot_seq(const double* a, const double* b, int64_t n)
{
    double acc = 0.0;
    int64_t c;
    for (c = 0; c < n; c++)
        acc += a[c] * b[c];
    return acc;
}

/* out[r] = sum_c W[r,c] * v[c], fp64, sequential; W dequantised row by row. */
int orc_matvec(int fmt, const uint8_t* W, int64_t rows, int64_t cols, const double* v, double* out)
{
    int64_t r, rb = cols / orc_block_weights(fmt) * orc_block_bytes(fmt);
    double* rowbuf;
    if (!orc_block_weights(fmt) || cols % orc_block_weights(fmt))
        return -1;
    rowbuf = (double*)malloc(sizeof(double) * cols);
    for (r = 0; r < rows; r++) {
        orc_dequant_row(fmt, W + r * rb, cols, rowbuf);
        out[r] = dot_seq(rowbuf, v, cols);
    }
    free(rowbuf);
    return 0;
}

/* The dequantised [rows, cols] matrix in fp64 (rows in parallel). */
static double* dequant_matrix(int fmt, const uint8_t* W, int64_t rows, int64_t cols)
{
    int64_t r, rb = cols / orc_block_weights(fmt) * orc_block_bytes(fmt);
    double* out = (double*)malloc(sizeof(double) * rows * cols);
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; r++)
        orc_dequant_row(fmt, W + r * rb, cols, out + r * cols);
    return out;
}

static double silu64(double z) { return z / (1.0 + exp(-z)); }

/* A dequantised expert: gate/up [F, H], down [H, F]. */
typedef struct {
    int64_t F;
    double *g, *u, *d;
} expert64;

/*
 * One expert on one token.  xhat: dequantised q8_K(x) [H].  Writes
 * hq (q8_K(h), F/256 blocks), yp [H], and optionally g, u, h [F].
 *   g = Wg xhat, u = Wu xhat (fp64), h = fl32(silu(g) u), hhat = q8_K(h)^,
 *   yp = Wd hhat (fp64)
 */
static void expert_one(int64_t H, const expert64* X, const double* xhat, uint8_t* hq, double* yp,
                       double* g_out, double* u_out, float* h_out)
{
    const int64_t F = X->F;
    double* g = (double*)malloc(sizeof(double) * F);
    double* u = (double*)malloc(sizeof(double) * F);
    float* h = (float*)malloc(sizeof(float) * F);
    double* hhat = (double*)malloc(sizeof(double) * F);
    int64_t f, r;
    for (f = 0; f < F; f++)
        g[f] = dot_seq(X->g + f * H, xhat, H);
    for (f = 0; f < F; f++)
        u[f] = dot_seq(X->u + f * H, xhat, H);
    for (f = 0; f < F; f++)
        h[f] = (float)(silu64(g[f]) * u[f]);
    orc_quantize_q8K_row(h, F, hq);
    orc_dequant_q8K_row(hq, F, hhat);
    for (r = 0; r < H; r++)
        yp[r] = dot_seq(X->d + r * F, hhat, F);
    if (g_out) memcpy(g_out, g, sizeof(double) * F);
    if (u_out) memcpy(u_out, u, sizeof(double) * F);
    if (h_out) memcpy(h_out, h, sizeof(float) * F);
    free(g); free(u); free(h); free(hhat);
}

/*
 * Expert FFN for the tokens listed in sel[0..n_sel).  Per selected token:
 *   y[n,:]    fp32 [H]
 *   hq[n, s]  q8_K(h) of slot s (s = k is the shared expert), F_s/256 blocks,
 *             laid out with a stride of (Fmax/256)*292 bytes per slot; zero
 *             for a slot whose expert is absent
 *   g,u,h     (optional, may be NULL) [n, k+1, Fmax] diagnostics
 * gate/up/down: host arrays [E] of AoS matrices; NULL = not resident (its
 * pairs contribute nothing).  sh_*: shared expert or NULL.  shared_scale:
 * [T] or NULL (= 1).  ids / w: the router's output [T, k].
 *
 * Each pair (token, slot) is computed on its own (expert_one); the experts are
 * visited one at a time, each dequantised once for all of its pairs, and then
 * every token sums its slots in slot order, the shared expert last:
 *   y[t] = fl32( sum_s w[t,s] * yp[t,s] + shared_scale[t] * yp[t,shared] )
 */
int orc_expert_ffn(int64_t T, int64_t H, int64_t F, int64_t E, int k,
                   int fg, int fu, int fd,
                   const uint8_t* const* gate, const uint8_t* const* up, const uint8_t* const* down,
                   int64_t Fs, int sfg, int sfu, int sfd,
                   const uint8_t* sh_gate, const uint8_t* sh_up, const uint8_t* sh_down,
                   const float* x, const int32_t* ids, const float* w, const float* shared_scale,
                   const int64_t* sel, int64_t n_sel,
                   float* y, uint8_t* hq, double* g_diag, double* u_diag, float* h_diag)
{
    const int64_t Fmax = (sh_gate && Fs > F) ? Fs : F;
    const int64_t hq_stride = Fmax / 256 * 292;
    const int64_t n_slots = n_sel * (k + 1);
    int64_t n, e, i;
    double *xhat, *yp;
    char* done;
    int64_t *count, *start, *fill, *list;
    if (H % 256 || F % 256 || (sh_gate && Fs % 256))
        return -1;
    for (n = 0; n < n_sel; n++) {
        int s;
        if (sel[n] < 0 || sel[n] >= T)
            return -1;
        for (s = 0; s < k; s++)
            if (ids[sel[n] * k + s] < 0 || ids[sel[n] * k + s] >= E)
                return -1;
    }
    if (hq)
        memset(hq, 0, (size_t)(n_slots * hq_stride));

    /* q8_K(x) of each selected token, dequantised */
    xhat = (double*)malloc(sizeof(double) * n_sel * H);
#pragma omp parallel for schedule(static)
    for (n = 0; n < n_sel; n++) {
        uint8_t* xq = (uint8_t*)malloc((size_t)(H / 256 * 292));
        orc_quantize_q8K_row(x + sel[n] * H, H, xq);
        orc_dequant_q8K_row(xq, H, xhat + n * H);
        free(xq);
    }

    /* the (token, slot) pairs of each expert; index E is the shared expert */
    count = (int64_t*)calloc((size_t)(E + 2), sizeof(int64_t));
    start = (int64_t*)calloc((size_t)(E + 2), sizeof(int64_t));
    fill = (int64_t*)calloc((size_t)(E + 2), sizeof(int64_t));
    list = (int64_t*)malloc(sizeof(int64_t) * (n_slots > 0 ? n_slots : 1));
    for (n = 0; n < n_sel; n++) {
        int s;
        for (s = 0; s < k; s++)
            count[ids[sel[n] * k + s]]++;
        count[E]++;
    }
    for (e = 0; e <= E; e++)
        start[e + 1] = start[e] + count[e];
    for (n = 0; n < n_sel; n++) {
        int s;
        for (s = 0; s < k; s++) {
            e = ids[sel[n] * k + s];
            list[start[e] + fill[e]++] = n * (k + 1) + s;
        }
        list[start[E] + fill[E]++] = n * (k + 1) + k;
    }

    yp = (double*)calloc((size_t)(n_slots * H), sizeof(double));
    done = (char*)calloc((size_t)(n_slots > 0 ? n_slots : 1), 1);
    for (e = 0; e <= E; e++) {
        expert64 X;
        int64_t j;
        int fmt_g, fmt_u, fmt_d;
        const uint8_t *Wg, *Wu, *Wd;
        if (count[e] == 0)
            continue;
        if (e < E) {
            Wg = gate[e]; Wu = up[e]; Wd = down[e];
            X.F = F; fmt_g = fg; fmt_u = fu; fmt_d = fd;
        } else {
            Wg = sh_gate; Wu = sh_up; Wd = sh_down;
            X.F = Fs; fmt_g = sfg; fmt_u = sfu; fmt_d = sfd;
        }
        if (!Wg || !Wu || !Wd)
            continue;                       /* not resident: its pairs add nothing */
        X.g = dequant_matrix(fmt_g, Wg, X.F, H);
        X.u = dequant_matrix(fmt_u, Wu, X.F, H);
        X.d = dequant_matrix(fmt_d, Wd, H, X.F);
#pragma omp parallel for schedule(dynamic, 1)
        for (j = start[e]; j < start[e + 1]; j++) {
            const int64_t p = list[j], pn = p / (k + 1);
            expert_one(H, &X, xhat + pn * H, hq ? hq + p * hq_stride : NULL, yp + p * H,
                       g_diag ? g_diag + p * Fmax : NULL, u_diag ? u_diag + p * Fmax : NULL,
                       h_diag ? h_diag + p * Fmax : NULL);
            done[p] = 1;
        }
        free(X.g); free(X.u); free(X.d);
    }

    /* the weighted sum of each token, slot order, shared expert last */
#pragma omp parallel for schedule(static)
    for (n = 0; n < n_sel; n++) {
        const int64_t t = sel[n];
        double* acc = (double*)calloc((size_t)H, sizeof(double));
        int s;
        for (s = 0; s <= k; s++) {
            const int64_t p = n * (k + 1) + s;
            double wt;
            if (!done[p])
                continue;
            wt = s < k ? (double)w[t * k + s] : (shared_scale ? (double)shared_scale[t] : 1.0);
            for (i = 0; i < H; i++)
                acc[i] += wt * yp[p * H + i];
        }
        for (i = 0; i < H; i++)
            y[n * H + i] = (float)acc[i];
        free(acc);
    }
    free(xhat); free(yp); free(done); free(count); free(start); free(fill); free(list);
    return 0;
}
