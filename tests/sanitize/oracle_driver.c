/*
 * oracle_driver.c -- runs every function of the CPU reference on small
 * ragged inputs (and on bad arguments) under AddressSanitizer and
 * UndefinedBehaviorSanitizer; built and run by tests/test_sanitize.py.
 * Exit status 0 when every call returned what it should.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "nosa_oracle.h"

static uint32_t rng = 12345u;
static double uniform(void)
{
    rng = rng * 1664525u + 1013904223u;
    return ((rng >> 8) + 0.5) / 16777216.0;
}

static int fail(const char* what)
{
    fprintf(stderr, "oracle driver: %s\n", what);
    return 1;
}

int main(void)
{
    nosa_ref_params p = {4, 2, 128, 64, 32, 16, 2, 128, 0.0, 0.0};
    const int B = 3;
    const int32_t Lk[3] = {300, 90, 31};
    const int32_t Lq[3] = {70, 1, 31};
    int32_t cu_k[4] = {0}, cu_q[4] = {0};
    for (int s = 0; s < B; ++s) {
        cu_k[s + 1] = cu_k[s] + Lk[s];
        cu_q[s + 1] = cu_q[s] + Lq[s];
    }
    const int d = p.head_dim, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
    const int total_k = cu_k[B], total_q = cu_q[B];
    uint16_t* k = malloc(sizeof(uint16_t) * total_k * Hkv * d);
    uint16_t* v = malloc(sizeof(uint16_t) * total_k * Hkv * d);
    uint16_t* q = malloc(sizeof(uint16_t) * total_q * Hq * d);
    for (int i = 0; i < total_k * Hkv * d; ++i) {
        k[i] = nosa_ref_bf16_round(2.0 * uniform() - 1.0);
        v[i] = nosa_ref_bf16_round(2.0 * uniform() - 1.0);
    }
    for (int i = 0; i < total_q * Hq * d; ++i) q[i] = nosa_ref_bf16_round(2.0 * uniform() - 1.0);
    const int max_nc = nosa_ref_num_keys(300, p.kernel, p.stride);
    const int max_qblk = 2, max_nb = 5, max_sel = p.topk + p.window / p.block_size;
    uint16_t* kc = calloc((size_t)B * Hkv * max_nc * d, sizeof(uint16_t));
    uint16_t* kc2 = calloc((size_t)B * Hkv * max_nc * d, sizeof(uint16_t));
    double* scores = malloc(sizeof(double) * B * max_qblk * Hkv * max_nb);
    int32_t* sel = malloc(sizeof(int32_t) * B * max_qblk * Hkv * max_sel);
    int32_t* cnt = malloc(sizeof(int32_t) * B * max_qblk * Hkv);
    double* out = malloc(sizeof(double) * total_q * Hq * d);
    double* lse = malloc(sizeof(double) * total_q * Hq);
    nosa_ref_set_num_threads(2);

    if (nosa_ref_check_params(&p) != 0) return fail("valid parameters rejected");
    if (nosa_ref_forward(&p, q, cu_q, k, v, cu_k, B, max_nc, max_qblk, max_nb, max_sel, kc, scores, sel,
                         cnt, out, lse) != 0)
        return fail("forward");
    for (int i = 0; i < total_q * Hq * d; ++i)
        if (!isfinite(out[i])) return fail("non-finite output");
    /* pooled keys appended token by token equal the full build */
    int32_t valid[3] = {0, 0, 0};
    for (int t = 1; t <= 300; ++t) {
        int32_t cu[4] = {0};
        for (int s = 0; s < B; ++s) cu[s + 1] = cu[s] + (t < Lk[s] ? t : Lk[s]);
        /* the tokens of each sequence stay where the full layout has them */
        uint16_t* kk = malloc(sizeof(uint16_t) * (cu[B] > 0 ? cu[B] : 1) * Hkv * d);
        for (int s = 0; s < B; ++s)
            for (int x = 0; x < cu[s + 1] - cu[s]; ++x)
                for (int e = 0; e < Hkv * d; ++e)
                    kk[((size_t)cu[s] + x) * Hkv * d + e] = k[((size_t)cu_k[s] + x) * Hkv * d + e];
        if (nosa_ref_append_keys(&p, kk, cu, valid, B, max_nc, kc2) != 0) return fail("append");
        for (int s = 0; s < B; ++s) valid[s] = cu[s + 1] - cu[s];
        free(kk);
    }
    for (size_t i = 0; i < (size_t)B * Hkv * max_nc * d; ++i)
        if (kc[i] != kc2[i]) return fail("appended keys differ from the full build");
    /* front end */
    const int hidden = 64;
    uint16_t* x = malloc(sizeof(uint16_t) * B * hidden);
    uint16_t* w = malloc(sizeof(uint16_t) * (Hq + 2 * Hkv) * d * hidden);
    for (int i = 0; i < B * hidden; ++i) x[i] = nosa_ref_bf16_round(uniform() - 0.5);
    for (int i = 0; i < (Hq + 2 * Hkv) * d * hidden; ++i) w[i] = nosa_ref_bf16_round(uniform() - 0.5);
    const int32_t pos[3] = {5, 0, 70000};
    uint16_t* qf = malloc(sizeof(uint16_t) * B * Hq * d);
    uint16_t* kf = malloc(sizeof(uint16_t) * B * Hkv * d);
    uint16_t* vf = malloc(sizeof(uint16_t) * B * Hkv * d);
    if (nosa_ref_qkv_rope(&p, hidden, 10000.0, NULL, x, w, pos, B, qf, kf, vf) != 0) return fail("qkv_rope");
    /* bad arguments are rejected, never dereferenced */
    nosa_ref_params bad = p;
    bad.num_kv_heads = 3;
    if (nosa_ref_check_params(&bad) == 0) return fail("Hkv not dividing Hq accepted");
    if (nosa_ref_forward(&bad, q, cu_q, k, v, cu_k, B, max_nc, max_qblk, max_nb, max_sel, kc, scores, sel, cnt,
                         out, lse) == 0)
        return fail("forward with bad parameters accepted");
    if (nosa_ref_compress_keys(&p, NULL, cu_k, B, max_nc, kc) == 0) return fail("NULL keys accepted");
    if (nosa_ref_block_scores(&p, q, cu_q, kc, max_nc, cu_k, B, 1, max_nb, scores) == 0)
        return fail("too few query blocks accepted");
    free(k); free(v); free(q); free(kc); free(kc2); free(scores); free(sel); free(cnt); free(out); free(lse);
    free(x); free(w); free(qf); free(kf); free(vf);
    printf("oracle driver: ok\n");
    return 0;
}
