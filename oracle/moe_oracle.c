/*
 * moe_oracle.c -- CPU oracle for the A8W4 fused mixture-of-experts layer
 * (and its A16W4 variant, further down).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, FP64 statement of
 * what the layer computes.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the HIP library; the product path never calls it.
 *
 * The layer follows aiter PR 5609, "Add DeepSeek V4.1 Flash TP4 gfx950 MoE
 * tuning", section Configuration: activations are 8-bit floats and expert
 * weights 4-bit MX values, each run of 32 along the reduction sharing one
 * power-of-two scale; the gate and up projections sit in alternate rows of
 * one matrix; the gate goes through SiLU; the routing probability scales
 * each route only after the down projection; the result is bfloat16.  The
 * span of one call follows aiter PR 5904, "Add tuned a8w4 fused-MoE configs
 * for DeepSeek V4.1-Flash (TP4 + EP, gfx950)", section "Fused-MoE kernel,
 * expert-parallel benchmark": it groups routes by expert, runs both GEMMs
 * and re-quantises the values passed between them.
 *
 * Number formats are the ones those names denote:
 *   E2M1 (MXFP4 element), E8M0 (MX block scale): OCP Microscaling Formats
 *   (MX) v1.0, element and scale tables.
 *   E4M3 "FN" (FP8 activations): OCP 8-bit Floating Point v1.0, E4M3 row.
 *
 * Readings taken where the pages are silent (each one is listed in the
 * design notes of the repository):
 *   - FP8 is E4M3FN (bias 7, largest finite 448, no infinities).
 *   - Block scale: E = floor(log2(amax)) - 8 (8 is the largest exponent of
 *     E4M3), clamped to [-127, 127]; amax = 0 gives E = -127.  Elements are
 *     v * 2^-E rounded to the nearest finite E4M3 value, ties to the even
 *     code, which saturates magnitudes above 448.  Zero keeps its sign.
 *   - The requantised intermediate is SiLU(g)*u computed exactly (FP64 here),
 *     with no BF16 rounding before the requantisation.
 *   - w13 row 2j is gate j and row 2j+1 is up j; element 2i of a row sits in
 *     the low nibble of byte i and element 2i+1 in the high nibble.
 *   - Sorted ids are (k << 24) | t; padding holds the sentinel value M.
 *     Routes of one expert keep ascending flat index t*topk + k; experts
 *     are visited in ascending local id; experts with no route get no block.
 *   - Expert ids outside [expert_offset, expert_offset + E) are skipped.
 *   - The routing weight multiplies the stage-two result; the top-k sum runs
 *     in ascending k in FP64 and is rounded once to BF16 (nearest, even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent field 0 is subnormal: m * 0.5.  OCP MX v1.0, FP4 E2M1. */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0: 2^(u - 127); code 255 is NaN.  OCP MX v1.0, scale format. */
double oracle_e8m0_value(int code)
{
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

/* E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities.
 * OCP 8-bit Floating Point v1.0, E4M3. */
double oracle_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* BF16 bits -> value (the top half of an IEEE binary32). */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Nearest BF16 to x, ties to even, overflow to infinity (IEEE default
 * rounding applied once to the exact FP64 value). */
uint16_t oracle_bf16_rne(double x)
{
    if (isnan(x)) return 0x7FC0;
    double ax = fabs(x);
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (ax == 0.0) return sign;
    int e;
    frexp(ax, &e);                 /* ax = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;                /* floor(log2 ax) */
    if (ex < -126) ex = -126;      /* subnormal range keeps the 2^-133 step */
    double quantum = ldexp(1.0, ex - 7);
    double r = nearbyint(ax / quantum) * quantum;  /* ties to even multiple */
    /* Overflow: anything that rounds beyond the largest finite value. */
    if (r > bf16_max) return sign | 0x7F80;
    float rf = (float)r;           /* exact: r is a BF16 value */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return sign | (uint16_t)(u >> 16);
}

/* Decode tables filled from the decoders above, so that the dot products
 * below read a value per code instead of recomputing it.  g_e4m3_pos holds the
 * 127 non-negative finite E4M3 values; entry c is the value of code c, and the
 * values increase with the code. */
static double g_e4m3_pos[127];
static double g_e4m3_all[256];
static double g_e2m1_all[16];
static double g_e8m0_all[256];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void)
{
    if (g_e4m3_ready) return;
    for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = oracle_e4m3_value(c);
    for (int c = 0; c < 256; ++c) g_e4m3_all[c] = oracle_e4m3_value(c);
    for (int c = 0; c < 256; ++c) g_e8m0_all[c] = oracle_e8m0_value(c);
    for (int c = 0; c < 16; ++c) g_e2m1_all[c] = oracle_e2m1_value(c);
    g_e4m3_ready = 1;
}

/* Encode one value: the nearest finite E4M3 value, ties to the even code
 * (the even mantissa), magnitudes beyond 448 saturating to 448.  The sign is
 * kept, so -0 and negatives that round to zero give 0x80. */
int oracle_e4m3_encode(double x)
{
    e4m3_table_init();
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    int code;
    if (a >= g_e4m3_pos[126]) {
        code = 126;
    } else {
        /* largest lo with table[lo] <= a */
        int lo = 0, hi = 126;
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (g_e4m3_pos[mid] <= a) lo = mid; else hi = mid;
        }
        double dlo = a - g_e4m3_pos[lo], dhi = g_e4m3_pos[hi] - a;
        if (dlo < dhi) code = lo;
        else if (dhi < dlo) code = hi;
        else code = (lo % 2 == 0) ? lo : hi;
    }
    return neg ? (code | 0x80) : code;
}

/* Exponent of the per-1x32 scale for a block whose largest magnitude is
 * amax: floor(log2 amax) - 8, clamped to [-127, 127]; -127 for amax = 0. */
int oracle_block_exponent(double amax)
{
    if (!(amax > 0.0)) return -127;
    int e;
    frexp(amax, &e);
    int E = (e - 1) - 8;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* Quantise one block of n values (n = 32 on the path) to E4M3 codes plus one
 * E8M0 scale code.  OCP MX v1.0 conversion with E4M3 elements. */
void oracle_quant_block(const double* v, int n, uint8_t* q, uint8_t* scale_code)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int E = oracle_block_exponent(amax);
    *scale_code = (uint8_t)(E + 127);
    for (int i = 0; i < n; ++i) q[i] = (uint8_t)oracle_e4m3_encode(ldexp(v[i], -E));
}

/* --------------------------------------------------- activation quantiser */

/* hidden BF16 [M, H] -> codes [M, H] and scales [M, H/32], one E8M0 scale
 * per run of 32 consecutive values along H (the per-1x32 activation scaling
 * of the Configuration section of aiter PR 5609). */
void oracle_quant_act(int64_t M, int64_t H, const uint16_t* x, uint8_t* q, uint8_t* s)
{
    e4m3_table_init();
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        double blk[32];
        for (int64_t b = 0; b < H / 32; ++b) {
            for (int i = 0; i < 32; ++i) blk[i] = oracle_bf16_value(x[t * H + b * 32 + i]);
            oracle_quant_block(blk, 32, q + t * H + b * 32, s + t * (H / 32) + b);
        }
    }
}

/* ------------------------------------------------------------------- sort */

/* Group the local routes by expert into blocks of bm rows.
 * Writes sorted_ids[0 .. num_padded) and block_expert[0 .. num_padded/bm);
 * returns num_padded, or -1 if it would exceed capacity. */
int64_t oracle_sort(int64_t M, int topk, int E, int expert_offset, int bm,
                    const int32_t* topk_ids, int32_t* sorted_ids,
                    int32_t* block_expert, int64_t capacity)
{
    int64_t R = M * topk;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        int64_t start = pos;
        for (int64_t f = 0; f < R; ++f) {
            int64_t le = (int64_t)topk_ids[f] - expert_offset;
            if (le != e) continue;
            if (pos >= capacity) return -1;
            int64_t t = f / topk, k = f % topk;
            sorted_ids[pos++] = (int32_t)((k << 24) | t);
        }
        int64_t cnt = pos - start;
        if (cnt == 0) continue;
        int64_t padded = (cnt + bm - 1) / bm * bm;
        while (pos < start + padded) {
            if (pos >= capacity) return -1;
            sorted_ids[pos++] = (int32_t)M;
        }
        for (int64_t b = start / bm; b < (start + padded) / bm; ++b) block_expert[b] = e;
    }
    return pos;
}

/* ------------------------------------------------------- one routed token */

/* Value of element kk of row `row` of an MXFP4 matrix stored as
 * codes [rows, K/2] (two per byte, low nibble first) and scales [rows, K/32]. */
static inline double mxfp4_elem(const uint8_t* codes, const uint8_t* scales,
                                int64_t K, int64_t row, int64_t kk)
{
    uint8_t byte = codes[row * (K / 2) + kk / 2];
    int c = (kk & 1) ? (byte >> 4) : (byte & 15);
    return g_e2m1_all[c] * g_e8m0_all[scales[row * (K / 32) + kk / 32]];
}

/* Stage one and the intermediate requantisation for one route of a token to
 * local expert e.
 *   a_q/a_s : the token's quantised activation row (H codes, H/32 scales)
 *   w13/_s  : expert e's gate/up matrix [2I, H/2] and scales [2I, H/32]
 *   gu      : out, 2I values: gate_j at 2j, up_j at 2j+1, in FP64 (may be NULL)
 *   gu_abs  : out, 2I values: the sums of |a_k w_k| of the same dot products,
 *             the scale an accumulation error of each is measured against
 *             (may be NULL)
 *   h       : out, I values of SiLU(gate) * up in FP64 (may be NULL)
 *   iq, is  : out, the requantised intermediate (I codes, I/32 scales)
 */
void oracle_stage1(int64_t H, int64_t I,
                   const uint8_t* a_q, const uint8_t* a_s,
                   const uint8_t* w13, const uint8_t* w13_s,
                   double* gu, double* gu_abs, double* h, uint8_t* iq, uint8_t* is)
{
    e4m3_table_init();
    double* a = (double*)malloc(sizeof(double) * H);
    double* hv = (double*)malloc(sizeof(double) * I);
    for (int64_t kk = 0; kk < H; ++kk)
        a[kk] = g_e4m3_all[a_q[kk]] * g_e8m0_all[a_s[kk / 32]];

    /* g_j from row 2j, u_j from row 2j+1; SiLU(g) * u */
    for (int64_t j = 0; j < I; ++j) {
        double g = 0.0, u = 0.0, ga = 0.0, ua = 0.0;
        for (int64_t kk = 0; kk < H; ++kk) {
            double pg = a[kk] * mxfp4_elem(w13, w13_s, H, 2 * j, kk);
            double pu = a[kk] * mxfp4_elem(w13, w13_s, H, 2 * j + 1, kk);
            g += pg;
            u += pu;
            ga += fabs(pg);
            ua += fabs(pu);
        }
        if (gu) {
            gu[2 * j] = g;
            gu[2 * j + 1] = u;
        }
        if (gu_abs) {
            gu_abs[2 * j] = ga;
            gu_abs[2 * j + 1] = ua;
        }
        hv[j] = g / (1.0 + exp(-g)) * u;
    }
    if (h) memcpy(h, hv, sizeof(double) * I);

    /* intermediate quantisation, per 1x32 along j */
    for (int64_t c = 0; c < I / 32; ++c) oracle_quant_block(hv + 32 * c, 32, iq + 32 * c, is + c);
    free(a);
    free(hv);
}

/* Stage two for one route: y_h = sum_j inter_j * w2[e][h, j] in FP64, with
 * inter the dequantised intermediate (I codes, I/32 scales); y_abs (may be
 * NULL) receives sum_j |inter_j * w2[e][h, j]|. */
void oracle_stage2(int64_t H, int64_t I, const uint8_t* iq, const uint8_t* is,
                   const uint8_t* w2, const uint8_t* w2_s, double* y, double* y_abs)
{
    e4m3_table_init();
    double* iv = (double*)malloc(sizeof(double) * I);
    for (int64_t j = 0; j < I; ++j)
        iv[j] = g_e4m3_all[iq[j]] * g_e8m0_all[is[j / 32]];
    for (int64_t hh = 0; hh < H; ++hh) {
        double acc = 0.0, aa = 0.0;
        for (int64_t j = 0; j < I; ++j) {
            double p = iv[j] * mxfp4_elem(w2, w2_s, I, hh, j);
            acc += p;
            aa += fabs(p);
        }
        y[hh] = acc;
        if (y_abs) y_abs[hh] = aa;
    }
    free(iv);
}

/* Both stages for one route (y may be NULL to stop after the requantisation). */
void oracle_route(int64_t H, int64_t I,
                  const uint8_t* a_q, const uint8_t* a_s,
                  const uint8_t* w13, const uint8_t* w13_s,
                  const uint8_t* w2, const uint8_t* w2_s,
                  double* h, uint8_t* iq, uint8_t* is, double* y)
{
    oracle_stage1(H, I, a_q, a_s, w13, w13_s, NULL, NULL, h, iq, is);
    if (y) oracle_stage2(H, I, iq, is, w2, w2_s, y, NULL);
}

/* Combine: o[t] = sum over local slots k, ascending, of w[t,k] * y[t,k] in
 * FP64 (the routing weight is applied here, after stage two), then BF16.
 * y holds [ntok, topk, H]; non-local slots are skipped. */
static void combine(int64_t H, int E, int expert_offset, int topk,
                    const int32_t* topk_ids, const float* topk_weights,
                    const int64_t* tokens, int64_t ntok, const double* y,
                    double* out_f64, uint16_t* out_bf16)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int64_t hh = 0; hh < H; ++hh) {
            double o = 0.0;
            for (int k = 0; k < topk; ++k) {
                int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
                if (le < 0 || le >= E) continue;
                o += (double)topk_weights[t * topk + k] * y[(i * topk + k) * H + hh];
            }
            if (out_f64) out_f64[i * H + hh] = o;
            out_bf16[i * H + hh] = oracle_bf16_rne(o);
        }
    }
}

/* ------------------------------------------------------------ whole layer */

/* The layer's output for a list of tokens.
 *   hidden      BF16 [M, H]; topk_ids i32 [M, topk]; topk_weights f32 [M, topk]
 *   w13 [E, 2I, H/2], w13_s [E, 2I, H/32], w2 [E, H, I/2], w2_s [E, H, I/32]
 *   tokens      the ntok token indices to evaluate (NULL = all M in order)
 *   out_f64     [ntok, H] the FP64 combine before rounding (may be NULL)
 *   out_bf16    [ntok, H] the BF16 output
 * A token with no local route gives a row of +0. */
void oracle_forward(int64_t M, int64_t H, int64_t I, int E, int expert_offset, int topk,
                    const uint16_t* hidden, const int32_t* topk_ids, const float* topk_weights,
                    const uint8_t* w13, const uint8_t* w13_s,
                    const uint8_t* w2, const uint8_t* w2_s,
                    const int64_t* tokens, int64_t ntok,
                    double* out_f64, uint16_t* out_bf16)
{
    e4m3_table_init();
    if (!tokens) ntok = M;
    int64_t nroute = ntok * topk;
    /* y for every (listed token, slot); computed in parallel over routes */
    double* y = (double*)calloc((size_t)(nroute > 0 ? nroute : 1) * H, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nroute; ++r) {
        int64_t i = r / topk, k = r % topk;
        int64_t t = tokens ? tokens[i] : i;
        int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
        if (le < 0 || le >= E) continue;
        uint8_t* aq = (uint8_t*)malloc(H);
        uint8_t* as = (uint8_t*)malloc(H / 32);
        uint8_t* iq = (uint8_t*)malloc(I);
        uint8_t* is = (uint8_t*)malloc(I / 32);
        double blk[32];
        for (int64_t b = 0; b < H / 32; ++b) {
            for (int q = 0; q < 32; ++q) blk[q] = oracle_bf16_value(hidden[t * H + b * 32 + q]);
            oracle_quant_block(blk, 32, aq + b * 32, as + b);
        }
        oracle_route(H, I, aq, as,
                     w13 + le * (2 * I) * (H / 2), w13_s + le * (2 * I) * (H / 32),
                     w2 + le * H * (I / 2), w2_s + le * H * (I / 32),
                     NULL, iq, is, y + r * H);
        free(aq); free(as); free(iq); free(is);
    }
    combine(H, E, expert_offset, topk, topk_ids, topk_weights, tokens, ntok, y, out_f64, out_bf16);
    free(y);
}

/* Stage two and the combine of oracle_forward, applied to a given
 * requantised intermediate instead of the one stage one would produce:
 *   inter_q [ntok, topk, I], inter_s [ntok, topk, I/32] for the listed tokens'
 *   slots (rows of non-local slots are ignored).
 * Used to check the output given another implementation's intermediate. */
void oracle_forward_given_intermediate(int64_t M, int64_t H, int64_t I, int E, int expert_offset,
                                       int topk, const int32_t* topk_ids, const float* topk_weights,
                                       const uint8_t* w2, const uint8_t* w2_s,
                                       const int64_t* tokens, int64_t ntok,
                                       const uint8_t* inter_q, const uint8_t* inter_s,
                                       double* out_f64, uint16_t* out_bf16, double* out_abs)
{
    e4m3_table_init();
    if (!tokens) ntok = M;
    int64_t nroute = ntok * topk;
    double* y = (double*)calloc((size_t)(nroute > 0 ? nroute : 1) * H, sizeof(double));
    double* ya = out_abs ? (double*)calloc((size_t)(nroute > 0 ? nroute : 1) * H, sizeof(double)) : NULL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nroute; ++r) {
        int64_t i = r / topk, k = r % topk;
        int64_t t = tokens ? tokens[i] : i;
        int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
        if (le < 0 || le >= E) continue;
        oracle_stage2(H, I, inter_q + r * I, inter_s + r * (I / 32),
                      w2 + le * H * (I / 2), w2_s + le * H * (I / 32), y + r * H, ya ? ya + r * H : NULL);
    }
    combine(H, E, expert_offset, topk, topk_ids, topk_weights, tokens, ntok, y, out_f64, out_bf16);
    if (out_abs) {
        /* sum over local slots of |w[t,k]| * sum_j |inter_j w2[h, j]|: the
         * scale the accumulation errors of stage two are measured against */
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < ntok; ++i) {
            int64_t t = tokens ? tokens[i] : i;
            for (int64_t hh = 0; hh < H; ++hh) {
                double o = 0.0;
                for (int k = 0; k < topk; ++k) {
                    int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
                    if (le < 0 || le >= E) continue;
                    o += fabs((double)topk_weights[t * topk + k]) * ya[(i * topk + k) * H + hh];
                }
                out_abs[i * H + hh] = o;
            }
        }
        free(ya);
    }
    free(y);
}

/* ------------------------------------------------- A16W4 variant (one route) */

/* The A16W4 variant of the layer (aiter PR 6286, "Retune gfx942 a16w4
 * DSv4.1 tiles for Triton 3.8": moe_gemm_a16w4 with w1 under apply_swiglu,
 * w2 separate, BF16 activations, MXFP4 weights).  Readings taken where that
 * page is silent: the activations enter unquantised (their exact BF16
 * values); w13/w2 layout, interleave, nibble order and the SwiGLU are those
 * of the A8W4 layer above (SiLU(g) * u, no clamp); the intermediate between
 * the two GEMMs is BF16 (nearest, ties to even) -- the 16-bit activation
 * type of the second GEMM; the routing weight multiplies the stage-two
 * result and the top-k sum is the A8W4 combine.
 *
 * Stage one for one route: h_j = BF16(SiLU(g_j) * u_j) with g_j, u_j the FP64
 * dot products of the token's BF16 row with rows 2j and 2j+1 of w13[e].
 *   x    the token's BF16 row (H values)
 *   gu   out, 2I values: g_j at 2j, u_j at 2j+1 (may be NULL)
 *   h64  out, I values of SiLU(g) * u before the rounding (may be NULL)
 *   hb   out, I BF16 values of the intermediate */
void oracle_a16_stage1(int64_t H, int64_t I, const uint16_t* x,
                       const uint8_t* w13, const uint8_t* w13_s, double* gu, double* h64, uint16_t* hb)
{
    e4m3_table_init();
    double* a = (double*)malloc(sizeof(double) * H);
    for (int64_t kk = 0; kk < H; ++kk) a[kk] = oracle_bf16_value(x[kk]);
    for (int64_t j = 0; j < I; ++j) {
        double g = 0.0, u = 0.0;
        for (int64_t kk = 0; kk < H; ++kk) {
            g += a[kk] * mxfp4_elem(w13, w13_s, H, 2 * j, kk);
            u += a[kk] * mxfp4_elem(w13, w13_s, H, 2 * j + 1, kk);
        }
        double h = g / (1.0 + exp(-g)) * u;
        if (gu) {
            gu[2 * j] = g;
            gu[2 * j + 1] = u;
        }
        if (h64) h64[j] = h;
        hb[j] = oracle_bf16_rne(h);
    }
    free(a);
}

/* Stage two for one route of the A16W4 variant: y_h = sum_j h_j * w2[e][h, j]
 * in FP64 over the BF16 intermediate h. */
void oracle_a16_stage2(int64_t H, int64_t I, const uint16_t* hb,
                       const uint8_t* w2, const uint8_t* w2_s, double* y)
{
    e4m3_table_init();
    double* hv = (double*)malloc(sizeof(double) * I);
    for (int64_t j = 0; j < I; ++j) hv[j] = oracle_bf16_value(hb[j]);
    for (int64_t hh = 0; hh < H; ++hh) {
        double acc = 0.0;
        for (int64_t j = 0; j < I; ++j) acc += hv[j] * mxfp4_elem(w2, w2_s, I, hh, j);
        y[hh] = acc;
    }
    free(hv);
}

/* The A16W4 layer's output for a list of tokens (arguments as
 * oracle_forward); inter_bf16, if not NULL, receives the BF16 intermediate
 * [ntok, topk, I] of the listed tokens' local slots (others left as given). */
void oracle_a16_forward(int64_t M, int64_t H, int64_t I, int E, int expert_offset, int topk,
                        const uint16_t* hidden, const int32_t* topk_ids, const float* topk_weights,
                        const uint8_t* w13, const uint8_t* w13_s,
                        const uint8_t* w2, const uint8_t* w2_s,
                        const int64_t* tokens, int64_t ntok,
                        uint16_t* inter_bf16, double* out_f64, uint16_t* out_bf16)
{
    e4m3_table_init();
    if (!tokens) ntok = M;
    int64_t nroute = ntok * topk;
    double* y = (double*)calloc((size_t)(nroute > 0 ? nroute : 1) * H, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nroute; ++r) {
        int64_t i = r / topk, k = r % topk;
        int64_t t = tokens ? tokens[i] : i;
        int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
        if (le < 0 || le >= E) continue;
        uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * I);
        oracle_a16_stage1(H, I, hidden + t * H, w13 + le * (2 * I) * (H / 2),
                          w13_s + le * (2 * I) * (H / 32), NULL, NULL, hb);
        if (inter_bf16) memcpy(inter_bf16 + r * I, hb, sizeof(uint16_t) * I);
        oracle_a16_stage2(H, I, hb, w2 + le * H * (I / 2), w2_s + le * H * (I / 32), y + r * H);
        free(hb);
    }
    combine(H, E, expert_offset, topk, topk_ids, topk_weights, tokens, ntok, y, out_f64, out_bf16);
    free(y);
}

/* The A16W4 intermediate of a list of routes (flat index f = t*topk+k): the
 * BF16 values hb [nr, I], and optionally SiLU(g) * u before the rounding
 * h_f64 [nr, I] and the gate/up sums gu_f64 [nr, 2I] (g_j at 2j, u_j at
 * 2j + 1).  Non-local routes give all-zero rows. */
void oracle_a16_intermediate(int64_t M, int64_t H, int64_t I, int E, int expert_offset, int topk,
                             const uint16_t* hidden, const int32_t* topk_ids,
                             const uint8_t* w13, const uint8_t* w13_s,
                             const int64_t* routes, int64_t nr,
                             double* gu_f64, double* h_f64, uint16_t* hb)
{
    e4m3_table_init();
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        int64_t f = routes[r], t = f / topk;
        int64_t le = (int64_t)topk_ids[f] - expert_offset;
        memset(hb + r * I, 0, sizeof(uint16_t) * I);
        if (h_f64) memset(h_f64 + r * I, 0, sizeof(double) * I);
        if (gu_f64) memset(gu_f64 + r * 2 * I, 0, sizeof(double) * 2 * I);
        if (le < 0 || le >= E) continue;
        oracle_a16_stage1(H, I, hidden + t * H, w13 + le * (2 * I) * (H / 2),
                          w13_s + le * (2 * I) * (H / 32), gu_f64 ? gu_f64 + r * 2 * I : NULL,
                          h_f64 ? h_f64 + r * I : NULL, hb + r * I);
    }
}

/* Stage two and the combine of oracle_a16_forward applied to a given BF16
 * intermediate inter [ntok, topk, I] of the listed tokens' slots (rows of
 * non-local slots are ignored): to check the output given another
 * implementation's intermediate. */
void oracle_a16_forward_given_intermediate(int64_t M, int64_t H, int64_t I, int E, int expert_offset,
                                           int topk, const int32_t* topk_ids, const float* topk_weights,
                                           const uint8_t* w2, const uint8_t* w2_s,
                                           const int64_t* tokens, int64_t ntok, const uint16_t* inter,
                                           double* out_f64, uint16_t* out_bf16)
{
    e4m3_table_init();
    if (!tokens) ntok = M;
    int64_t nroute = ntok * topk;
    double* y = (double*)calloc((size_t)(nroute > 0 ? nroute : 1) * H, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nroute; ++r) {
        int64_t i = r / topk, k = r % topk;
        int64_t t = tokens ? tokens[i] : i;
        int64_t le = (int64_t)topk_ids[t * topk + k] - expert_offset;
        if (le < 0 || le >= E) continue;
        oracle_a16_stage2(H, I, inter + r * I, w2 + le * H * (I / 2), w2_s + le * H * (I / 32), y + r * H);
    }
    combine(H, E, expert_offset, topk, topk_ids, topk_weights, tokens, ntok, y, out_f64, out_bf16);
    free(y);
}

/* The requantised intermediate of a list of routes (flat index f = t*topk+k),
 * for comparison with the stage-one output.  Routes that are not local give
 * all-zero rows.  h_f64 [nr, I] (SiLU(gate) * up), gu_f64 [nr, 2I] (gate
 * and up, interleaved as the rows of w13) and gu_abs_f64 [nr, 2I] (the sums
 * of |a_k w_k| of those dot products) may be NULL. */
void oracle_intermediate(int64_t M, int64_t H, int64_t I, int E, int expert_offset, int topk,
                         const uint16_t* hidden, const int32_t* topk_ids,
                         const uint8_t* w13, const uint8_t* w13_s,
                         const int64_t* routes, int64_t nr,
                         double* gu_f64, double* gu_abs_f64, double* h_f64, uint8_t* iq, uint8_t* is)
{
    e4m3_table_init();
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        int64_t f = routes[r], t = f / topk;
        int64_t le = (int64_t)topk_ids[f] - expert_offset;
        memset(iq + r * I, 0, I);
        memset(is + r * (I / 32), 0, I / 32);
        if (h_f64) memset(h_f64 + r * I, 0, sizeof(double) * I);
        if (gu_f64) memset(gu_f64 + r * 2 * I, 0, sizeof(double) * 2 * I);
        if (gu_abs_f64) memset(gu_abs_f64 + r * 2 * I, 0, sizeof(double) * 2 * I);
        if (le < 0 || le >= E) continue;
        uint8_t* aq = (uint8_t*)malloc(H);
        uint8_t* as = (uint8_t*)malloc(H / 32);
        double blk[32];
        for (int64_t b = 0; b < H / 32; ++b) {
            for (int q = 0; q < 32; ++q) blk[q] = oracle_bf16_value(hidden[t * H + b * 32 + q]);
            oracle_quant_block(blk, 32, aq + b * 32, as + b);
        }
        oracle_stage1(H, I, aq, as,
                      w13 + le * (2 * I) * (H / 2), w13_s + le * (2 * I) * (H / 32),
                      gu_f64 ? gu_f64 + r * 2 * I : NULL, gu_abs_f64 ? gu_abs_f64 + r * 2 * I : NULL,
                      h_f64 ? h_f64 + r * I : NULL, iq + r * I, is + r * (I / 32));
        free(aq); free(as);
    }
}

/* Router of the backbone configurations: for each token, its k_routed
 * largest logits among E_routed (equal values: the lower expert id first),
 * in descending order, and as weights the softmax of the chosen logits --
 * the softmax over all E_routed logits renormalised over the chosen ones,
 * which is the same in exact arithmetic -- in FP64.  With a shared expert
 * (shared_id >= 0), slot k_routed holds it with weight 1 (the "fused shared
 * expert" of the prefill configuration).  logits [M, E_routed] float32;
 * ids [M, k] int32 and weights [M, k] double, k = k_routed + (shared >= 0). */
void oracle_softmax_topk(int64_t M, int Er, int kr, int shared_id, const float* logits,
                         int32_t* ids, double* weights)
{
    const int k = kr + (shared_id >= 0 ? 1 : 0);
    unsigned char* used = (unsigned char*)malloc((size_t)Er);
    for (int64_t t = 0; t < M; ++t) {
        const float* l = logits + t * Er;
        int32_t* id = ids + t * k;
        double* wt = weights + t * k;
        memset(used, 0, (size_t)Er);
        for (int s = 0; s < kr; ++s) {
            int best = -1;
            for (int e = 0; e < Er; ++e)
                if (!used[e] && (best < 0 || l[e] > l[best])) best = e;
            used[best] = 1;
            id[s] = best;
        }
        const double top = (double)l[id[0]];
        double sum = 0.0;
        for (int s = 0; s < kr; ++s) {
            wt[s] = exp((double)l[id[s]] - top);
            sum += wt[s];
        }
        for (int s = 0; s < kr; ++s) wt[s] /= sum;
        if (shared_id >= 0) {
            id[kr] = shared_id;
            wt[kr] = 1.0;
        }
    }
    free(used);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
