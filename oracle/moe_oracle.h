/*
 * moe_oracle.h -- plain CPU oracle of the prefill routed-expert product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library or its Python binding may
 * include, link, load or call this code; only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg use it.  It shares no source with the
 * GPU path.
 *
 * Every routine is a direct, slow restatement of what the pages define:
 *   - "Strata" PR #3752 (GP100 weight-stationary experts), commit list and
 *     Approach section: tokens quantized to q8_1 and scattered into
 *     expert-sorted rows, one gate/up product over all experts, one fused
 *     swiglu + q8_1 pass, one down product into one row per (token, expert),
 *     64-row chunks of the experts taken largest expert first, every product
 *     keeping int8 values, scales and a per-32-value float epilogue in K order;
 *     the integer sum of one 32-value block is exact, so only the order of the
 *     float epilogue decides the bits.
 *   - "Strata" PR #2145 (fused int8 prompt experts on Turing), description:
 *     Q2_0 weights in 64-value blocks whose two 32-value halves share the
 *     block's scale d; int32 sums exact in any order.
 * Byte layouts of q8_1, Q2_0 and NL4 are this project's own (the pages never
 * print them); they are documented where each routine reads them.
 *
 * Precision: the pages fix fp32 for the quantizer's scale and for the
 * epilogue (PR #2145 names the FP32 epilogue as what bounds its kernel), so the oracle computes in fp32,
 * built with -ffp-contract=off; every fused multiply-add is an explicit fmaf.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_Q2_0 1
#define ORC_NL4 2

/* Plan: stable counting sort of the (token, slot) pairs by expert.
 * ids[T*K]: expert of slot k of token t at t*K+k.  Outputs:
 *   counts[E], offsets[E+1] (exclusive prefix sum), perm[R] (sorted row ->
 *   t*K+k, ascending t*K+k inside each expert), chunks[4*n] = (expert,
 *   first sorted row, row count <= C, 0), experts in descending row count,
 *   ties by ascending expert id, each expert's chunks in row order.
 * Returns the number of chunks, or -1 if an id is out of range or
 * max_chunks is too small. */
int orc_plan(const int32_t *ids, int T, int K, int E, int C,
             int32_t *counts, int32_t *offsets, int32_t *perm,
             int32_t *chunks, int max_chunks);

/* q8_1 of one 32-value block: d = amax/127 (fp32), q = round-half-away(x/d)
 * clamped to [-127,127], s = sum q; a block whose d is 0 quantizes to zeros. */
void orc_q8_1_block(const float *x, float *d, int32_t *s, int8_t *q);

/* One q8_1 row of `cols` values (cols % 32 == 0), row layout:
 * q[cols] int8, then d[cols/32] fp32, then s[cols/32] int32. */
void orc_q8_1_row(const float *x, int cols, uint8_t *row);

/* Quantize-and-scatter: sorted row r holds q8_1 of token perm[r]/K.
 * rows[n_rows] selects which sorted rows to produce (NULL: all R rows, in
 * order); out receives n_rows q8_1 rows of H values. */
void orc_quantize_scatter(const float *X, int T, int H, int K,
                          const int32_t *perm, int R,
                          const int32_t *rows, int n_rows, uint8_t *out);

/* Decode weight row n of one expert: vals[cols] the signed integer weights
 * (Q2_0: code-2; NL4: codebook[code]) and dw[cols/32] the block scale that
 * applies to each 32-value block (Q2_0: both halves of a 64-block share it). */
void orc_decode_row(int wtype, const uint8_t *expert, int wrows, int cols,
                    int n, const int8_t *codebook, int8_t *vals, float *dw);

/* Expert product.  For each activation row i (a q8_1 row of `cols` values)
 * with expert act_expert[i], out[i*wrows + n] for every weight row n:
 *   acc = 0; for each 32-block b in K order:
 *     dot = sum_j q[b][j] * w[n][b*32+j]          (int32, exact)
 *     acc = fmaf(dx[b], dw[n][b] * (float)dot, acc)
 * The weights of expert e start at w_base + w_off[e]. */
int orc_expert_product(int wtype, const uint8_t *w_base, const uint64_t *w_off,
                       int n_expert, int wrows, int cols, const int8_t *codebook,
                       const uint8_t *act, const int32_t *act_expert, int n_act,
                       float *out);

/* The int32 block dots of the same product: dots[(i*wrows + n)*(cols/32) + b]. */
int orc_block_dots(int wtype, const uint8_t *w_base, const uint64_t *w_off,
                   int n_expert, int wrows, int cols, const int8_t *codebook,
                   const uint8_t *act, const int32_t *act_expert, int n_act,
                   int32_t *dots);

/* SwiGLU of one value pair: silu(g) * u with silu(g) = g / (1 + E) in fp32,
 * E = e^-g rounded to the nearest binary32 (via binary64). */
float orc_swiglu(float g, float u);

/* swiglu + q8_1 of `rows` gate/up rows: gu row = [gate F | up F] (split
 * layout) or [g0 u0 g1 u1 ...] (interleaved != 0); h_j = swiglu(g_j, u_j);
 * hq row = q8_1 of h (F values). */
void orc_swiglu_q8(const float *gu, int rows, int F, int interleaved, uint8_t *hq);

/* Unfused swiglu: h[rows][F] floats (for the composition check). */
void orc_swiglu_rows(const float *gu, int rows, int F, int interleaved, float *h);

/* MoE combine: out[T*H], out[t][n] = fmaf chain over k ascending of
 * w[t*K+k] * dm[(t*K+k)*H + n], starting from 0.0f.  dm[T*K*H] holds one
 * row per (token, slot), w[T*K] the routing weights. */
void orc_combine(const float *dm, const float *w, int T, int K, int H, float *out);

#ifdef __cplusplus
}
#endif
#endif
