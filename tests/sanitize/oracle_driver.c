/*
 * Drives every oracle function on small, ragged inputs so that an
 * address/undefined-behaviour sanitizer build can check the oracle's memory
 * accesses and integer arithmetic.  Inputs come from a fixed linear
 * congruential sequence (test scaffolding, not part of any operator).
 * Exit status 0 when every call returns; the sanitizers abort otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "h3oracle.h"

static uint32_t lcg = 12345u;
static float next_f(void) {
    lcg = lcg * 1664525u + 1013904223u;
    return (float)((int32_t)(lcg >> 8) - (1 << 23)) / (float)(1 << 23);
}
static void fill_f32(float* p, int64_t n) {
    for (int64_t i = 0; i < n; ++i) p[i] = next_f();
}
static void fill_bf16(uint16_t* p, int64_t n) {
    for (int64_t i = 0; i < n; ++i) p[i] = oracle_f32_to_bf16(next_f());
}

int main(void) {
    oracle_set_num_threads(2);
    const int64_t rows = 37, D = 24, G = 3, rpg = 13;  /* ragged groups */
    float* x = malloc(rows * D * 4);
    float* y = malloc(rows * D * 4);
    float* h = malloc(rows * D * 4);
    float* mod = malloc(3 * G * D * 4);
    uint16_t* xb = malloc(rows * D * 2);
    uint16_t* yb = malloc(rows * D * 2);
    uint16_t* hb = malloc(rows * D * 2);
    uint16_t* modb = malloc(3 * G * D * 2);
    fill_f32(x, rows * D); fill_f32(h, rows * D); fill_f32(mod, 3 * G * D);
    fill_bf16(xb, rows * D); fill_bf16(hb, rows * D); fill_bf16(modb, 3 * G * D);
    int64_t grp[37];
    for (int i = 0; i < 37; ++i) grp[i] = (i * 7) % G;

    int32_t* pos = malloc(rows * 3 * 4);
    oracle_positions(pos, rows, 1000003, 2, 3, 5, 4);

    oracle_adaln_modulate(y, ORACLE_F32, x, ORACLE_F32, mod, mod + G * D, ORACLE_F32, NULL, rpg,
                          rows, D, 1e-6f);
    oracle_adaln_modulate(yb, ORACLE_BF16, x, ORACLE_F32, mod, mod + G * D, ORACLE_F32, grp, 1,
                          rows, D, 1e-6f);
    oracle_adaln_modulate(yb, ORACLE_BF16, xb, ORACLE_BF16, modb, modb + G * D, ORACLE_BF16, NULL,
                          rpg, rows, D, 1e-6f);
    oracle_adaln_affine_modulate(y, ORACLE_F32, x, ORACLE_F32, mod + 2 * G * D, mod + 2 * G * D,
                                 mod, mod + G * D, ORACLE_F32, NULL, rpg, rows, D, 1e-6f);
    oracle_adaln_affine_modulate(yb, ORACLE_BF16, xb, ORACLE_BF16, modb + 2 * G * D, modb,
                                 modb, modb + G * D, ORACLE_BF16, grp, 1, rows, D, 1e-6f);
    oracle_gated_residual(x, ORACLE_F32, hb, ORACLE_BF16, mod, NULL, rpg, rows, D);
    oracle_gated_residual(xb, ORACLE_BF16, hb, ORACLE_BF16, modb, grp, 1, rows, D);
    oracle_gated_residual_adaln(x, ORACLE_F32, h, ORACLE_F32, mod, yb, ORACLE_BF16,
                                mod + G * D, mod + 2 * G * D, NULL, rpg, rows, D, 1e-6f);

    float* gu = malloc(rows * 2 * D * 4);
    fill_f32(gu, rows * 2 * D);
    oracle_swiglu(y, gu, ORACLE_F32, rows, D);

    const int32_t heads = 3, Dh = 32;
    float* inv = malloc(Dh / 2 * 4);
    oracle_rope_inv_freq(inv, 8, 8, 16, 10000.0);
    float* q = malloc(rows * heads * Dh * 4);
    float* k = malloc(rows * heads * Dh * 4);
    float* qo = malloc(rows * heads * Dh * 4);
    float* ko = malloc(rows * heads * Dh * 4);
    float w[32];
    fill_f32(q, rows * heads * Dh); fill_f32(k, rows * heads * Dh); fill_f32(w, 32);
    for (int mode = 0; mode < 2; ++mode)
        oracle_qk_rmsnorm_rope3d(qo, ko, q, k, w, w, ORACLE_F32, rows, heads, Dh, 1e-6f, pos, 8, 8,
                                 16, 10000.0, mode, ORACLE_PAIR_INTERLEAVED);
    oracle_qk_rmsnorm_rope3d(qo, ko, q, k, w, w, ORACLE_F32, rows, heads, Dh, 1e-6f, pos, 16, 0,
                             16, 10000.0, 0, ORACLE_PAIR_HALF_SPLIT);

    double l1[2];
    oracle_residual_l1(l1, x, h, ORACLE_F32, rows, D);
    oracle_residual_l1(l1, xb, hb, ORACLE_BF16, rows, D);

    /* router: 37 rows in blocks of 8 (a short last block) */
    const int32_t block = 8;
    const int64_t nb = (rows + block - 1) / block;
    double* pq = malloc(heads * nb * Dh * 8);
    double* pk = malloc(heads * nb * Dh * 8);
    double* sc = malloc(heads * nb * nb * 8);
    oracle_subblock_pool(pq, q, ORACLE_F32, rows, heads, Dh, block);
    oracle_subblock_pool(pk, k, ORACLE_F32, rows, heads, Dh, block);
    oracle_subblock_scores(sc, pq, pk, heads, nb, nb, Dh);
    const int64_t keep = oracle_subblock_keep(nb, 0.75, 10, 10);
    int32_t* kv = malloc(heads * nb * keep * 4);
    oracle_subblock_select(kv, sc, heads, nb, nb, keep);
    for (int64_t i = 0; i < heads * nb * keep; ++i)
        if (kv[i] < 0 || kv[i] >= nb) return 2;

    free(x); free(y); free(h); free(mod); free(xb); free(yb); free(hb); free(modb); free(pos);
    free(gu); free(inv); free(q); free(k); free(qo); free(ko); free(pq); free(pk); free(sc);
    free(kv);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
