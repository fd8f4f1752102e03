/*
 * moe_oracle.c -- plain CPU oracle of the prefill routed-expert product.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): never linked into the library.
 *
 * Written for clarity, not speed: plain loops, fp32 arithmetic in the order
 * the method states, no blocking or reordering.  Build flags:
 *   gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ plan --
 * "Strata" PR #3752, commit list and Approach: the token rows are scattered
 * into expert-sorted rows so that each expert's rows are contiguous; the
 * CTAs take 64-row chunks of the experts, largest expert first; each expert
 * runs its own row count (no padding to a group maximum). */
int orc_plan(const int32_t *ids, int T, int K, int E, int C,
             int32_t *counts, int32_t *offsets, int32_t *perm,
             int32_t *chunks, int max_chunks)
{
    const int R = T * K;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int i = 0; i < R; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return -1;
        counts[ids[i]] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    /* stable: flattened index i = t*K+k in ascending order inside a bucket */
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int i = 0; i < R; ++i) perm[fill[ids[i]]++] = i;
    free(fill);

    /* experts by descending count, ties by ascending id (selection of the
     * next largest; O(E^2) is fine for an oracle) */
    char *taken = (char *)calloc((size_t)(E > 0 ? E : 1), 1);
    int n = 0;
    for (int step = 0; step < E; ++step) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || counts[e] > counts[best]) best = e;
        }
        taken[best] = 1;
        for (int r0 = 0; r0 < counts[best]; r0 += C) {
            if (n >= max_chunks) { free(taken); return -1; }
            int nr = counts[best] - r0;
            if (nr > C) nr = C;
            chunks[4 * n + 0] = best;
            chunks[4 * n + 1] = offsets[best] + r0;
            chunks[4 * n + 2] = nr;
            chunks[4 * n + 3] = 0;
            ++n;
        }
    }
    free(taken);
    return n;
}

/* ------------------------------------------------------------------ q8_1 --
 * q8_1 (the activation format of the int8 path; "Strata" PR #3752 quantizes
 * both the scattered token rows and H to it): 32 values, one scale
 * d = max|x| / 127, int8 values, and the block's integer sum. */
void orc_q8_1_block(const float *x, float *d_out, int32_t *s_out, int8_t *q)
{
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    const float d = amax / 127.0f;
    int32_t s = 0;
    for (int j = 0; j < 32; ++j) {
        int v = 0;
        if (d != 0.0f) {
            float y = roundf(x[j] / d);          /* halves away from zero */
            if (y > 127.0f) y = 127.0f;          /* only reachable when d is subnormal */
            if (y < -127.0f) y = -127.0f;
            v = (int)y;
        }
        q[j] = (int8_t)v;
        s += v;
    }
    *d_out = d;
    *s_out = s;
}

void orc_q8_1_row(const float *x, int cols, uint8_t *row)
{
    const int nb = cols / 32;
    int8_t *q = (int8_t *)row;
    float *d = (float *)(row + cols);
    int32_t *s = (int32_t *)(row + cols + 4 * nb);
    for (int b = 0; b < nb; ++b) {
        float db;
        int32_t sb;
        orc_q8_1_block(x + 32 * b, &db, &sb, q + 32 * b);
        memcpy(d + b, &db, 4);
        memcpy(s + b, &sb, 4);
    }
}

void orc_quantize_scatter(const float *X, int T, int H, int K,
                          const int32_t *perm, int R,
                          const int32_t *rows, int n_rows, uint8_t *out)
{
    (void)T;
    const size_t rb = (size_t)H + (size_t)H / 32 * 8;
    const int n = rows ? n_rows : R;
    for (int i = 0; i < n; ++i) {
        const int r = rows ? rows[i] : i;
        const int token = perm[r] / K;
        orc_q8_1_row(X + (size_t)token * H, H, out + (size_t)i * rb);
    }
}

/* --------------------------------------------------------------- weights --
 * Q2_0 ("Strata" PR #2145 description): 64-value blocks, 2-bit codes, one
 * binary16 scale per block shared by the block's two 32-value halves;
 * weight = d * (code - 2).  Byte layout (ours): per expert a codes plane of
 * rows*cols/64 16-byte blocks (row-major by row, block), value 16*j+b of a
 * block in byte b, bits 2j..2j+1; then a scales plane of rows*cols/64
 * binary16 values in the same order.
 * NL4 (the 4-bit non-linear down format; PR #3752 names IQ4_NL, whose table
 * is not printed): 32-value blocks, 4-bit codes into a 16-entry int8
 * codebook, one binary16 scale; weight = d * codebook[code].  Value b in the
 * low nibble of byte b, value 16+b in the high nibble; codes plane then
 * scales plane as for Q2_0. */
static float half_to_float(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int mant = h & 0x3ff;
    float v;
    if (expo == 0)
        v = ldexpf((float)mant, -24);                 /* zero / subnormal */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexpf((float)(mant | 0x400), expo - 25);
    return sign ? -v : v;
}

void orc_decode_row(int wtype, const uint8_t *expert, int wrows, int cols,
                    int n, const int8_t *codebook, int8_t *vals, float *dw)
{
    if (wtype == ORC_Q2_0) {
        const int nb = cols / 64;
        const uint8_t *codes = expert + (size_t)n * nb * 16;
        const uint8_t *scales = expert + (size_t)wrows * nb * 16 + (size_t)n * nb * 2;
        for (int beta = 0; beta < nb; ++beta) {
            const uint8_t *blk = codes + 16 * beta;
            for (int v = 0; v < 64; ++v) {
                const int j = v / 16, b = v % 16;
                const int code = (blk[b] >> (2 * j)) & 3;
                vals[64 * beta + v] = (int8_t)(code - 2);
            }
            uint16_t h;
            memcpy(&h, scales + 2 * beta, 2);
            const float d = half_to_float(h);
            dw[2 * beta] = d;
            dw[2 * beta + 1] = d;
        }
    } else {
        const int nb = cols / 32;
        const uint8_t *codes = expert + (size_t)n * nb * 16;
        const uint8_t *scales = expert + (size_t)wrows * nb * 16 + (size_t)n * nb * 2;
        for (int b = 0; b < nb; ++b) {
            const uint8_t *blk = codes + 16 * b;
            for (int v = 0; v < 32; ++v) {
                const int code = v < 16 ? (blk[v] & 0xf) : (blk[v - 16] >> 4);
                vals[32 * b + v] = codebook[code];
            }
            uint16_t h;
            memcpy(&h, scales + 2 * b, 2);
            dw[b] = half_to_float(h);
        }
    }
}

/* -------------------------------------------------------------- products --
 * "Strata" PR #3752: every product keeps the int8 values, the scales and the
 * per-32-value epilogue in K order; the integer dot of a 32-value block is
 * exact.  Epilogue (our reading of the per-32 form, one rounding per block):
 *   acc <- fmaf(dx_b, dw_b * (float)dot_b, acc),  b ascending, acc0 = 0.
 * For Q2_0, |dot| <= 32*127*2 and dw has 11 significant bits, so
 * dw_b*(float)dot_b is exact and each step is one correctly rounded
 * acc + dx*dw*dot. */
static int expert_product_impl(int wtype, const uint8_t *w_base, const uint64_t *w_off,
                               int n_expert, int wrows, int cols, const int8_t *codebook,
                               const uint8_t *act, const int32_t *act_expert, int n_act,
                               float *out, int32_t *dots)
{
    const int nb = cols / 32;
    const size_t rb = (size_t)cols + (size_t)nb * 8;
    int8_t *vals = (int8_t *)malloc((size_t)wrows * cols);
    float *dw = (float *)malloc(sizeof(float) * (size_t)wrows * nb);
    int status = 0;
    for (int e = 0; e < n_expert && status == 0; ++e) {
        int used = 0;
        for (int i = 0; i < n_act; ++i) used |= (act_expert[i] == e);
        if (!used) continue;
        const uint8_t *w = w_base + w_off[e];
        for (int n = 0; n < wrows; ++n)
            orc_decode_row(wtype, w, wrows, cols, n, codebook,
                           vals + (size_t)n * cols, dw + (size_t)n * nb);
        for (int i = 0; i < n_act; ++i) {
            if (act_expert[i] != e) continue;
            const uint8_t *row = act + (size_t)i * rb;
            const int8_t *q = (const int8_t *)row;
            const float *dx = (const float *)(row + cols);
            for (int n = 0; n < wrows; ++n) {
                const int8_t *wv = vals + (size_t)n * cols;
                const float *wd = dw + (size_t)n * nb;
                float acc = 0.0f;
                for (int b = 0; b < nb; ++b) {
                    int32_t dot = 0;
                    for (int j = 0; j < 32; ++j)
                        dot += (int32_t)q[32 * b + j] * (int32_t)wv[32 * b + j];
                    if (dots)
                        dots[((size_t)i * wrows + n) * nb + b] = dot;
                    float dxb;
                    memcpy(&dxb, dx + b, 4);
                    acc = fmaf(dxb, wd[b] * (float)dot, acc);
                }
                if (out) out[(size_t)i * wrows + n] = acc;
            }
        }
    }
    for (int i = 0; i < n_act; ++i)
        if (act_expert[i] < 0 || act_expert[i] >= n_expert) status = -1;
    free(vals);
    free(dw);
    return status;
}

int orc_expert_product(int wtype, const uint8_t *w_base, const uint64_t *w_off,
                       int n_expert, int wrows, int cols, const int8_t *codebook,
                       const uint8_t *act, const int32_t *act_expert, int n_act,
                       float *out)
{
    return expert_product_impl(wtype, w_base, w_off, n_expert, wrows, cols, codebook,
                               act, act_expert, n_act, out, NULL);
}

int orc_block_dots(int wtype, const uint8_t *w_base, const uint64_t *w_off,
                   int n_expert, int wrows, int cols, const int8_t *codebook,
                   const uint8_t *act, const int32_t *act_expert, int n_act,
                   int32_t *dots)
{
    return expert_product_impl(wtype, w_base, w_off, n_expert, wrows, cols, codebook,
                               act, act_expert, n_act, NULL, dots);
}

/* ---------------------------------------------------------------- swiglu --
 * "Strata" PR #3752, swiglu_quant commit: swiglu of the gate/up row, then
 * q8_1 of each 32-value block of the result, in one pass, H never stored.
 * The expression is not printed; our reading is silu(g) * u with
 * silu(g) = g / (1 + e^-g) in fp32, where e^-g is the binary32 value
 * nearest to the exact exponential, computed in binary64 and rounded once
 * (a double rounding could only differ where e^-g lies within about 2^-29 of
 * a binary32 rounding boundary; for every binary32 g this C library's result
 * rounds as an 80-bit exponential does, which the host tests check). */
float orc_swiglu(float g, float u)
{
    const float e = (float)exp(-(double)g);
    const float silu = g / (1.0f + e);
    return silu * u;
}

void orc_swiglu_rows(const float *gu, int rows, int F, int interleaved, float *h)
{
    for (int r = 0; r < rows; ++r) {
        const float *row = gu + (size_t)r * 2 * F;
        for (int j = 0; j < F; ++j) {
            const float g = interleaved ? row[2 * j] : row[j];
            const float u = interleaved ? row[2 * j + 1] : row[F + j];
            h[(size_t)r * F + j] = orc_swiglu(g, u);
        }
    }
}

void orc_swiglu_q8(const float *gu, int rows, int F, int interleaved, uint8_t *hq)
{
    const size_t rb = (size_t)F + (size_t)F / 32 * 8;
    float *h = (float *)malloc(sizeof(float) * (size_t)F);
    for (int r = 0; r < rows; ++r) {
        orc_swiglu_rows(gu + (size_t)r * 2 * F, 1, F, interleaved, h);
        orc_q8_1_row(h, F, hq + (size_t)r * rb);
    }
    free(h);
}

/* --------------------------------------------------------------- combine --
 * The step after the down product ("Strata" PR #3752 names the MoE combine
 * among the prompt-path fusions its port leaves out; no formula is printed).
 * Our reading is the usual weighted sum of a token's expert outputs,
 * out[t][n] = sum over k of w[t][k] * dm[t*K + k][n], evaluated in fp32 as
 * one fused multiply-add per term, k ascending, from 0. */
void orc_combine(const float *dm, const float *w, int T, int K, int H, float *out)
{
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k)
                acc = fmaf(w[(size_t)t * K + k], dm[((size_t)t * K + k) * H + n], acc);
            out[(size_t)t * H + n] = acc;
        }
}
