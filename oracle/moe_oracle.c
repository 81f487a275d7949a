/*
 * moe_oracle.c -- CPU oracle for the Mixture-of-Experts FFN forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is built into oracle/liboracle.so and is
 * loaded by the test-suite, by the smoke check and by the benchmark's CPU
 * baseline, never by the library it checks.  It shares no code, header, table
 * or constant with the HIP implementation.
 *
 * Plain, slow, obviously correct: every value is computed in double precision
 * (fp64) straight from its definition, one token (or one row) at a time, with no
 * blocking or reordering.  The only exception is the re-quantisation of the
 * SwiGLU output to fp8 on the W4A8 path, whose integer codes are decided in
 * float32 (the precision the kernel takes that decision in).
 *
 * Sources (web pages; section named, no line numbers):
 *  [FI6343]  FlashInfer PR #6343 "[SM90] Add W4A8 MegaMoE support" -- the fused
 *            kernel description (dispatch, both FFN GEMMs with NVFP4 weights and
 *            FP8 activations, SwiGLU, top-k combine; NVFP4 -> FP8 dequant) and
 *            its Usage section (-1 masks a route; FP32 routing weights; FP32
 *            input scales per 128 channels; E4M3 weight scale per 16 values
 *            for NVFP4 weights, E8M0 per 32 values for MXFP4 weights).
 *  [FI6517]  its follow-up #6517, point 4 (weight preparation: low-nibble-first
 *            packing, NVFP4 scales bounded by 6*scale <= 448, MXFP4 scales kept
 *            within 2^-5..2^6 for groups with nonzero codes, per-expert global
 *            scales) and the split family's note that the second GEMM's
 *            activation scales are per 128 like the first's.
 *  [MG3971]  Megatron-LM PR #3971 "Support GEMM + Swiglu fused MLP" -- the
 *            moe_mlp_glu_interleave_size option (gate/up interleave).
 *  [MG5984]  Megatron-LM PR #5984, commit log: the fused fc1 weight is laid out
 *            [gate | up]; "Add ClampedSwiGLU to MoE mlp_op_fuser".
 *  [MG4089]  Megatron-LM PR #4089 "add permute fusion into hybrid ep" --
 *            permute before the experts, unpermute inside the combine.
 *
 * Readings of the pages where they are silent (also listed with the design
 * notes of the repository):
 *  - routing: softmax over all E experts, then the k most probable experts,
 *    then their k probabilities renormalised to sum to one.  The selection
 *    compares the fp32 logits (softmax is strictly increasing, so the order is
 *    the same, and no tie can come from rounding or underflow of a
 *    probability); equal logits go to the lower expert id; slots are ordered by
 *    descending probability.  A dropped slot gets expert -1 and keeps its
 *    weight; the combine skips it and does not renormalise again.
 *  - permutation: rows grouped by expert id ascending, and within one expert by
 *    ascending slot id s = t*k + j (a stable counting sort).
 *  - SwiGLU: h = silu(g) * u with silu(g) = g / (1 + exp(-g)); with a clamp c>0
 *    both g and u are first clamped to [-c, c].
 *  - interleave il>0: stored W1 row il*2*q + r is gate row q*il + r (r < il)
 *    and up row q*il + r - il (r >= il).
 *  - fp8 is OCP E4M3FN (bias 7, max 448, no infinities, subnormals kept);
 *    conversions round to nearest even and saturate to +-448.
 *  - NVFP4 -> FP8 dequant: the weight code's e2m1 value times its block scale's
 *    e4m3 value, rounded to e4m3; the per-expert global scale multiplies the
 *    GEMM result.
 *  - W4A8 SwiGLU output: re-quantised per (row, 128 columns) with
 *    s = amax/448 (s = 1 if that is 0), q = e4m3(h / s), in float32.
 *  - MXFP4 weights (precision 2): the weight's value is its e2m1 value times
 *    2^(E8M0 code - 127) (the OCP MX scale format: a power of two, bias 127,
 *    code 255 NaN), exactly, with no rounding to FP8; the per-expert global
 *    scale multiplies the GEMM result, and activations, SwiGLU, h re-quantised
 *    to FP8 and the second GEMM are as for NVFP4.  The pages' kernel decodes
 *    MXFP4 to FP8 first, which is exact for the scales they require
 *    (2^-5..2^6 for groups with nonzero codes [FI6517]), so on those inputs
 *    both readings give the same value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* number formats                                                             */
/* ------------------------------------------------------------------------- */

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity. */
double orc_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP E2M1 (FP4): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent 0 is subnormal (m * 0.5). */
double orc_e2m1_value(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* OCP E8M0 (the MX scale): 2^(c - 127); code 255 is NaN. */
double orc_e8m0_value(uint8_t c)
{
    return c == 255 ? NAN : ldexp(1.0, (int)c - 127);
}

/* Nearest E4M3FN code to v, ties to the even code, saturating at +-448; a NaN
 * gives the NaN code with its sign (0x7F or 0xFF).  The 127 non-negative finite codes 0x00..0x7E have increasing magnitude, so
 * the nearest one is found by a binary search over their values. */
static double e4m3_mag[127]; /* magnitudes of the non-negative finite codes 0x00..0x7E */

__attribute__((constructor)) static void init_e4m3_mag(void)
{
    for (int i = 0; i < 127; i++)
        e4m3_mag[i] = orc_e4m3_value((uint8_t)i);
}

uint8_t orc_e4m3_encode(double v)
{
    const double *mag = e4m3_mag;
    uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
    double a = fabs(v);
    int lo, hi, c;
    if (isnan(v))
        return (signbit(v) ? 0x80 : 0) | 0x7F;
    if (a >= mag[126])
        return sign | 126;
    lo = 0;
    hi = 126; /* invariant: mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    if (a - mag[lo] < mag[hi] - a)
        c = lo;
    else if (a - mag[lo] > mag[hi] - a)
        c = hi;
    else
        c = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)c;
}

/* NVFP4 -> FP8 dequant of one weight: e2m1(code) * e4m3(block scale), rounded to
 * E4M3 [FI6343, nvfp4_dequant: NVFP4 -> FP8].  The product is exact in fp64.  The
 * pages define finite block scales only; a NaN scale (0x7F, 0xFF) gives the NaN
 * code whose sign is that of the product: sign(code) xor sign(scale). */
uint8_t orc_fp4_to_fp8(uint8_t code4, uint8_t scale8)
{
    if ((scale8 & 0x7F) == 0x7F)
        return (uint8_t)(0x7F | ((((code4 >> 3) ^ (scale8 >> 7)) & 1) << 7));
    return orc_e4m3_encode(orc_e2m1_value(code4 & 15) * orc_e4m3_value(scale8));
}

/* ------------------------------------------------------------------------- */
/* routing  [FI6343 Usage: expert ids with -1 masking a route, FP32 weights]  */
/* ------------------------------------------------------------------------- */

static void route_token(int E, int k, const float *l, const uint8_t *drop, int32_t *idx, double *w)
{
    double p[256], lmax = -INFINITY, z = 0.0, zk = 0.0;
    unsigned char taken[256];
    /* softmax over all E experts */
    for (int e = 0; e < E; e++)
        if ((double)l[e] > lmax)
            lmax = (double)l[e];
    for (int e = 0; e < E; e++) {
        p[e] = exp((double)l[e] - lmax);
        z += p[e];
    }
    for (int e = 0; e < E; e++) {
        p[e] /= z;
        taken[e] = 0;
    }
    /* top-k: k rounds of "largest remaining, lower id on ties" */
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || l[e] > l[best]))
                best = e;
        taken[best] = 1;
        idx[j] = best;
    }
    /* renormalise over the k selected */
    for (int j = 0; j < k; j++)
        zk += p[idx[j]];
    for (int j = 0; j < k; j++)
        w[j] = p[idx[j]] / zk;
    if (drop)
        for (int j = 0; j < k; j++)
            if (drop[j])
                idx[j] = -1;
}

void orc_route(int T, int E, int k, const float *logits, const uint8_t *slot_drop, int32_t *topk_idx,
               double *topk_w)
{
    for (int t = 0; t < T; t++)
        route_token(E, k, logits + (size_t)t * E, slot_drop ? slot_drop + (size_t)t * k : NULL,
                    topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

/* ------------------------------------------------------------------------- */
/* permutation tables: stable counting sort of slots by expert [MG4089]       */
/* ------------------------------------------------------------------------- */

void orc_tables(int T, int k, int E, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                int32_t *row_src, int32_t *slot_row)
{
    long S = (long)T * k, r = 0;
    for (long s = 0; s < S; s++) {
        slot_row[s] = -1;
        row_src[s] = -1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++) {
        counts[e] = 0;
        for (long s = 0; s < S; s++)
            if (topk_idx[s] == e) {
                row_src[r] = (int32_t)s;
                slot_row[s] = (int32_t)r;
                r++;
                counts[e]++;
            }
        offsets[e + 1] = (int32_t)r;
    }
}

/* x_perm[r] = x[row_src[r] / k] for the R live rows (a pure copy). */
void orc_permute_rows(long R, int k, int H, const int32_t *row_src, const uint16_t *x, uint16_t *x_perm)
{
    for (long r = 0; r < R; r++)
        memcpy(x_perm + (size_t)r * H, x + (size_t)(row_src[r] / k) * H, (size_t)H * sizeof(uint16_t));
}

/* out[t] = sum over valid slots j (ascending) of w[t][j] * y_perm[slot_row[t*k+j]] */
void orc_combine_bf16(int T, int k, int H, const uint16_t *y_perm, const int32_t *slot_row, const float *topk_w,
                      double *out)
{
    for (int t = 0; t < T; t++) {
        double *o = out + (size_t)t * H;
        for (int c = 0; c < H; c++)
            o[c] = 0.0;
        for (int j = 0; j < k; j++) {
            int32_t r = slot_row[(size_t)t * k + j];
            if (r < 0)
                continue;
            for (int c = 0; c < H; c++)
                o[c] += (double)topk_w[(size_t)t * k + j] * bf16_value(y_perm[(size_t)r * H + c]);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* one expert's SwiGLU FFN on one row                                         */
/* ------------------------------------------------------------------------- */

/* stored W1 row holding gate (up=0) or up (up=1) column n of the SwiGLU input */
static long w1_row(int I, int il, int n, int up)
{
    if (il == 0)
        return up ? (long)I + n : n;
    return (long)(n / il) * 2 * il + (up ? il : 0) + n % il;
}

static double swiglu(double g, double u, double clamp)
{
    if (clamp > 0) {
        g = g < -clamp ? -clamp : (g > clamp ? clamp : g);
        u = u < -clamp ? -clamp : (u > clamp ? clamp : u);
    }
    return g / (1.0 + exp(-g)) * u;
}

/* bf16 expert [MG3971, MG5984]: y = (silu(x W_gate^T) * (x W_up^T)) W2^T, all fp64 */
static void ffn_bf16(int H, int I, int il, double clamp, const uint16_t *xrow, const uint16_t *w1e,
                     const uint16_t *w2e, double *h, double *y)
{
    for (int n = 0; n < I; n++) {
        const uint16_t *wg = w1e + w1_row(I, il, n, 0) * H, *wu = w1e + w1_row(I, il, n, 1) * H;
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; c++) {
            double xv = bf16_value(xrow[c]);
            g += xv * bf16_value(wg[c]);
            u += xv * bf16_value(wu[c]);
        }
        h[n] = swiglu(g, u, clamp);
    }
    for (int c = 0; c < H; c++) {
        const uint16_t *w = w2e + (size_t)c * I;
        double acc = 0.0;
        for (int n = 0; n < I; n++)
            acc += h[n] * bf16_value(w[n]);
        y[c] = acc;
    }
}

/* weight at (row, col) of a packed [N][K] matrix, before its global scale.  NVFP4 (mx = 0):
 * the FP8 dequant of e2m1 * e4m3 block scale (one per 16 along K), through lut.  MXFP4
 * (mx = 1): e2m1 * 2^(e8m0 block scale - 127) (one per 32 along K), exactly. */
static double w4_value(const uint8_t *packed, const uint8_t *bscale, int K, long row, int col,
                       const double *lut, int mx)
{
    uint8_t byte = packed[row * (K / 2) + col / 2];
    uint8_t code = (col % 2 == 0) ? (byte & 15) : (byte >> 4); /* low nibble = even element [FI6517] */
    if (mx)
        return orc_e2m1_value(code) * orc_e8m0_value(bscale[row * (K / 32) + col / 32]);
    return lut[code * 256 + bscale[row * (K / 16) + col / 16]];
}

/* W4A8 expert [FI6343]: FP8 activations with per-128 scales x NVFP4 weights
 * dequantised to FP8 (or MXFP4 weights, mx = 1), clamped SwiGLU, h re-quantised to
 * FP8 per 128, second GEMM. */
static void ffn_w4a8(int H, int I, int il, double clamp, const uint8_t *x8, const float *xs, const uint8_t *w1e,
                     const uint8_t *w1b, double w1g, const uint8_t *w2e, const uint8_t *w2b, double w2g,
                     const double *lut, int mx, double *xd, double *h, double *y)
{
    float hf[128];
    for (int c = 0; c < H; c++)
        xd[c] = orc_e4m3_value(x8[c]) * (double)xs[c / 128];
    for (int n = 0; n < I; n++) {
        long rg = w1_row(I, il, n, 0), ru = w1_row(I, il, n, 1);
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; c++) {
            g += xd[c] * w4_value(w1e, w1b, H, rg, c, lut, mx);
            u += xd[c] * w4_value(w1e, w1b, H, ru, c, lut, mx);
        }
        h[n] = swiglu(g * w1g, u * w1g, clamp);
    }
    /* re-quantise h per 128 columns; the codes are decided in float32 */
    for (int b = 0; b < I / 128; b++) {
        float amax = 0.0f, s;
        for (int i = 0; i < 128; i++) {
            hf[i] = (float)h[b * 128 + i];
            if (fabsf(hf[i]) > amax)
                amax = fabsf(hf[i]);
        }
        s = amax / 448.0f;
        if (s == 0.0f)
            s = 1.0f;
        for (int i = 0; i < 128; i++) {
            float q = hf[i] / s;
            h[b * 128 + i] = orc_e4m3_value(orc_e4m3_encode((double)q)) * (double)s;
        }
    }
    for (int c = 0; c < H; c++) {
        double acc = 0.0;
        for (int n = 0; n < I; n++)
            acc += h[n] * w4_value(w2e, w2b, I, c, n, lut, mx);
        y[c] = acc * w2g;
    }
}

/* value of every (e2m1 code, e4m3 block scale) pair after the FP8 dequant */
static double *fp4_fp8_lut(void)
{
    double *lut = (double *)malloc(sizeof(double) * 16 * 256);
    for (int c = 0; c < 16; c++)
        for (int s = 0; s < 256; s++)
            lut[c * 256 + s] = orc_e4m3_value(orc_fp4_to_fp8((uint8_t)c, (uint8_t)s));
    return lut;
}

/* ------------------------------------------------------------------------- */
/* per-row expert FFN: y[i] = FFN_{expert[i]}(x[token[i]])                    */
/* ------------------------------------------------------------------------- */

void orc_ffn_rows_bf16(long n, const int32_t *token, const int32_t *expert, int H, int I, int il, double clamp,
                       const uint16_t *x, const uint16_t *w1, const uint16_t *w2, double *y)
{
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * I);
#pragma omp for schedule(dynamic, 1)
        for (long i = 0; i < n; i++) {
            size_t e = (size_t)expert[i];
            ffn_bf16(H, I, il, clamp, x + (size_t)token[i] * H, w1 + e * 2 * I * H, w2 + e * H * I, h,
                     y + (size_t)i * H);
        }
        free(h);
    }
}

/* mx = 0: NVFP4 weights (block scales [E][N][K/16]); mx = 1: MXFP4 ([E][N][K/32]) */
void orc_ffn_rows_w4a8(long n, const int32_t *token, const int32_t *expert, int H, int I, int il, double clamp,
                       const uint8_t *x8, const float *xs, const uint8_t *w1, const uint8_t *w1b,
                       const float *w1g, const uint8_t *w2, const uint8_t *w2b, const float *w2g, int mx, double *y)
{
    double *lut = fp4_fp8_lut();
    const int bk = mx ? 32 : 16; /* K values per block scale */
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * I), *xd = (double *)malloc(sizeof(double) * H);
#pragma omp for schedule(dynamic, 1)
        for (long i = 0; i < n; i++) {
            size_t e = (size_t)expert[i], t = (size_t)token[i];
            ffn_w4a8(H, I, il, clamp, x8 + t * H, xs + t * (H / 128), w1 + e * 2 * I * (H / 2),
                     w1b + e * 2 * I * (H / bk), w1g[e], w2 + e * H * (I / 2), w2b + e * H * (I / bk), w2g[e], lut,
                     mx, xd, h, y + (size_t)i * H);
        }
        free(h);
        free(xd);
    }
    free(lut);
}

/* ------------------------------------------------------------------------- */
/* the whole forward for a list of tokens                                     */
/* out[i] = sum_{valid j} w_j * FFN_{e_j}(x[t_i]),  route -> experts -> combine */
/* ------------------------------------------------------------------------- */

void orc_moe_forward(int n_tok, const int32_t *tokens, int T, int H, int I, int E, int k, int prec, int il,
                     double clamp, const float *logits, const uint8_t *slot_drop, const void *x, const float *x_scale,
                     const void *w1, const void *w1_bscale, const float *w1_gscale, const void *w2,
                     const void *w2_bscale, const float *w2_gscale, double *out)
{
    double *lut = prec != 0 ? fp4_fp8_lut() : NULL;
    const int mx = prec == 2, bk = mx ? 32 : 16; /* K values per weight block scale */
    (void)T;
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * I), *xd = (double *)malloc(sizeof(double) * H);
        double *y = (double *)malloc(sizeof(double) * H);
        int32_t idx[256];
        double w[256];
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n_tok; i++) {
            size_t t = (size_t)tokens[i];
            double *o = out + (size_t)i * H;
            route_token(E, k, logits + t * E, slot_drop ? slot_drop + t * k : NULL, idx, w);
            for (int c = 0; c < H; c++)
                o[c] = 0.0;
            for (int j = 0; j < k; j++) {
                size_t e;
                if (idx[j] < 0)
                    continue;
                e = (size_t)idx[j];
                if (prec == 0)
                    ffn_bf16(H, I, il, clamp, (const uint16_t *)x + t * H, (const uint16_t *)w1 + e * 2 * I * H,
                             (const uint16_t *)w2 + e * H * I, h, y);
                else
                    ffn_w4a8(H, I, il, clamp, (const uint8_t *)x + t * H, x_scale + t * (H / 128),
                             (const uint8_t *)w1 + e * 2 * I * (H / 2), (const uint8_t *)w1_bscale + e * 2 * I * (H / bk),
                             w1_gscale[e], (const uint8_t *)w2 + e * H * (I / 2),
                             (const uint8_t *)w2_bscale + e * H * (I / bk), w2_gscale[e], lut, mx, xd, h, y);
                for (int c = 0; c < H; c++)
                    o[c] += w[j] * y[c];
            }
        }
        free(h);
        free(xd);
        free(y);
    }
    free(lut);
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
