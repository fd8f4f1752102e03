/*
 * abi_chain.c -- the prefill routed-expert product driven from plain C
 * through include/moe_prefill.h, checked against the C oracle.
 *
 * Test code: it links the library and the oracle (oracle/moe_oracle.h), and
 * uses the HIP runtime only to allocate device memory and copy bytes; no
 * Python and no torch.  Every launch goes to the default stream (NULL).
 *
 * Layer: 64 tokens, hidden 256, n_ff 128, 8 experts, top-2 (the smallest
 * layer of the parity suite), seeded synthetic inputs from a 64-bit LCG:
 * X ~ N(0,1) by Box-Muller; each token's two experts distinct and uniform;
 * Q2_0 codes uniform bytes (four uniform 2-bit codes each); binary16 block
 * scales with exponent uniform in {2^-7, 2^-6, 2^-5} and a uniform 10-bit
 * mantissa (values in [0.0078, 0.0625)).
 *
 * Checks (the parity suite's rule): the q8_1 bytes of X and of H equal the
 * oracle's; the gate/up and down outputs equal it bit for bit; the fused
 * gate/up + swiglu launch writes the same H bytes as the two-step form.
 * Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe_prefill.h"
#include "../../oracle/moe_oracle.h"

enum { T = 64, H = 256, F = 128, E = 8, K = 2, R = T * K, CHUNK = 64 };

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static uint32_t lcg32(void) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 32);
}
static double unif(void) { return (lcg32() + 0.5) / 4294967296.0; }

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,              \
                    hipGetErrorString(e_));                                        \
            exit(2);                                                               \
        }                                                                          \
    } while (0)
#define MOE_OK_(x)                                                                 \
    do {                                                                           \
        int s_ = (x);                                                              \
        if (s_ != MOE_OK) {                                                        \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,              \
                    moe_status_string(s_));                                        \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

/* One product's weights for all experts, row-major planes, Q2_0. */
static uint8_t *make_q2_weights(int rows, int cols, size_t *bytes, uint64_t *off) {
    const size_t per = moe_weight_bytes(MOE_W_Q2_0, rows, cols);
    const size_t nb = (size_t)rows * (size_t)(cols / 64);
    uint8_t *w = (uint8_t *)malloc(per * E);
    for (int e = 0; e < E; ++e) {
        uint8_t *x = w + per * e;
        off[e] = per * e;
        for (size_t i = 0; i < nb * 16; ++i) x[i] = (uint8_t)lcg32();
        uint16_t *sc = (uint16_t *)(x + nb * 16);
        for (size_t i = 0; i < nb; ++i) {
            const uint32_t ex = 8 + lcg32() % 3;          /* 2^-7 .. 2^-5 */
            sc[i] = (uint16_t)((ex << 10) | (lcg32() & 0x3FFu));
        }
    }
    *bytes = per * E;
    return w;
}

static void *dev_copy(const void *h, size_t n) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n));
    if (h) HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

int main(void) {
    /* inputs */
    float *x = (float *)malloc(sizeof(float) * T * H);
    for (int i = 0; i < T * H; i += 2) {
        const double r = sqrt(-2.0 * log(unif())), a = 6.283185307179586 * unif();
        x[i] = (float)(r * cos(a));
        x[i + 1] = (float)(r * sin(a));
    }
    int32_t ids[R];
    for (int t = 0; t < T; ++t) {
        int pool[E];
        for (int e = 0; e < E; ++e) pool[e] = e;
        for (int k = 0; k < K; ++k) {
            const int j = k + (int)(lcg32() % (uint32_t)(E - k));
            const int tmp = pool[k]; pool[k] = pool[j]; pool[j] = tmp;
            ids[t * K + k] = pool[k];
        }
    }
    size_t gu_bytes, dn_bytes;
    uint64_t gu_off[E], dn_off[E];
    uint8_t *w_gu = make_q2_weights(2 * F, H, &gu_bytes, gu_off);
    uint8_t *w_dn = make_q2_weights(H, F, &dn_bytes, dn_off);

    /* device: raw and packed weights, plan workspace, activations */
    void *d_x = dev_copy(x, sizeof(float) * T * H);
    void *d_gu_raw = dev_copy(w_gu, gu_bytes), *d_gu = dev_copy(NULL, gu_bytes);
    void *d_dn_raw = dev_copy(w_dn, dn_bytes), *d_dn = dev_copy(NULL, dn_bytes);
    const size_t ws_bytes = moe_plan_device_bytes(T, K, E, CHUNK);
    void *d_ws = dev_copy(NULL, ws_bytes);
    const size_t xq_bytes = moe_q8_1_bytes(R, H), hq_bytes = moe_q8_1_bytes(R, F);
    void *d_xq = dev_copy(NULL, xq_bytes), *d_hq = dev_copy(NULL, hq_bytes);
    void *d_hq2 = dev_copy(NULL, hq_bytes);
    void *d_g = dev_copy(NULL, sizeof(float) * R * 2 * F);
    void *d_dm = dev_copy(NULL, sizeof(float) * R * H);

    moe_weights raw_gu = {MOE_W_Q2_0, 2 * F, H, E, d_gu_raw, gu_bytes, gu_off, NULL};
    moe_weights raw_dn = {MOE_W_Q2_0, H, F, E, d_dn_raw, dn_bytes, dn_off, NULL};
    MOE_OK_(moe_weights_pack(&raw_gu, d_gu, gu_bytes, NULL));
    MOE_OK_(moe_weights_pack(&raw_dn, d_dn, dn_bytes, NULL));
    moe_weights p_gu = {MOE_W_Q2_0 | MOE_W_TILED, 2 * F, H, E, d_gu, gu_bytes, gu_off, NULL};
    moe_weights p_dn = {MOE_W_Q2_0 | MOE_W_TILED, H, F, E, d_dn, dn_bytes, dn_off, NULL};
    moe_plan *plan = NULL;
    MOE_OK_(moe_prefill_plan(ids, T, K, E, CHUNK, &p_gu, &p_dn, d_ws, ws_bytes, NULL, &plan));

    /* the path: four launches, then the fused gate/up + swiglu into a second H */
    MOE_OK_(quantize_scatter(plan, (const float *)d_x, d_xq, NULL));
    MOE_OK_(expert_gate_up(plan, d_xq, (float *)d_g, NULL));
    MOE_OK_(swiglu_q8(plan, (const float *)d_g, d_hq, NULL));
    MOE_OK_(expert_down(plan, d_hq, (float *)d_dm, NULL));
    MOE_OK_(expert_gate_up_swiglu_q8(plan, d_xq, d_hq2, NULL));
    HIP_OK(hipDeviceSynchronize());

    uint8_t *xq = (uint8_t *)malloc(xq_bytes), *hq = (uint8_t *)malloc(hq_bytes);
    uint8_t *hq2 = (uint8_t *)malloc(hq_bytes);
    float *g = (float *)malloc(sizeof(float) * R * 2 * F), *dm = (float *)malloc(sizeof(float) * R * H);
    HIP_OK(hipMemcpy(xq, d_xq, xq_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hq, d_hq, hq_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hq2, d_hq2, hq_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g, d_g, sizeof(float) * R * 2 * F, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dm, d_dm, sizeof(float) * R * H, hipMemcpyDeviceToHost));

    /* the oracle on the same inputs */
    int32_t counts[E], offsets[E + 1], perm[R], chunks[4 * (R + E)];
    if (orc_plan(ids, T, K, E, CHUNK, counts, offsets, perm, chunks, R + E) < 0) return 3;
    int32_t row_e[R];
    for (int e = 0; e < E; ++e)
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) row_e[r] = e;
    uint8_t *xq_ref = (uint8_t *)malloc(xq_bytes), *hq_ref = (uint8_t *)malloc(hq_bytes);
    float *g_ref = (float *)malloc(sizeof(float) * R * 2 * F);
    float *dms = (float *)malloc(sizeof(float) * R * H);
    orc_quantize_scatter(x, T, H, K, perm, R, NULL, R, xq_ref);
    if (orc_expert_product(ORC_Q2_0, w_gu, gu_off, E, 2 * F, H, NULL, xq_ref, row_e, R, g_ref)) return 3;
    orc_swiglu_q8(g_ref, R, F, 0, hq_ref);
    if (orc_expert_product(ORC_Q2_0, w_dn, dn_off, E, H, F, NULL, hq_ref, row_e, R, dms)) return 3;

    int fail = 0;
    if (memcmp(xq, xq_ref, xq_bytes)) { fprintf(stderr, "q8_1 bytes of X differ\n"); fail = 1; }
    if (memcmp(g, g_ref, sizeof(float) * R * 2 * F)) { fprintf(stderr, "gate/up bits differ\n"); fail = 1; }
    if (memcmp(hq, hq2, hq_bytes)) { fprintf(stderr, "fused and two-step H bytes differ\n"); fail = 1; }
    const size_t hrb = hq_bytes / R;
    int h_rows = 0, dm_rows = 0;
    for (int r = 0; r < R; ++r) {
        h_rows += memcmp(hq + hrb * r, hq_ref + hrb * r, hrb) != 0;
        dm_rows += memcmp(dm + (size_t)perm[r] * H, dms + (size_t)r * H, sizeof(float) * H) != 0;
    }
    printf("rows %d, rows whose H bytes differ %d, rows whose down outputs differ %d\n", R, h_rows, dm_rows);
    if (h_rows) { fprintf(stderr, "H bytes differ\n"); fail = 1; }
    if (dm_rows) { fprintf(stderr, "down product bits differ\n"); fail = 1; }

    moe_plan_destroy(plan);
    printf(fail ? "FAIL\n" : "OK\n");
    return fail;
}
