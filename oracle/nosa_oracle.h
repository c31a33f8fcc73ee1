/*
 * nosa_oracle.h -- declarations of the plain CPU reference (test infrastructure
 * only; the HIP library neither includes nor links this).  Layouts and
 * semantics are described at the top of nosa_oracle.c.  Every function returns
 * 0 on success and a negative code on a bad argument.
 */
#ifndef NOSA_ORACLE_H
#define NOSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nosa_ref_params {
    int num_q_heads;   /* Hq                                              */
    int num_kv_heads;  /* Hkv, divides Hq; group size G = Hq / Hkv        */
    int head_dim;      /* d                                               */
    int block_size;    /* tokens per KV block (and queries per q-block)   */
    int kernel;        /* pooling window, tokens                          */
    int stride;        /* pooling stride, tokens                          */
    int topk;          /* blocks chosen in addition to the local window   */
    int window;        /* local window, tokens, multiple of block_size    */
    double scale;      /* <= 0 selects 1/sqrt(head_dim)                   */
    double locality;   /* gamma_0 in [0, 1]: share of topk kept for the   */
                       /* candidate blocks nearest the window             */
} nosa_ref_params;

int nosa_ref_check_params(const nosa_ref_params* p);
int nosa_ref_num_keys(int L, int kernel, int stride);
uint16_t nosa_ref_bf16_round(double x);
double nosa_ref_bf16_to_double(uint16_t bits);
int nosa_ref_num_threads(void);

int nosa_ref_compress_keys(const nosa_ref_params* p, const uint16_t* k, const int32_t* cu_k,
                           int B, int max_nc, uint16_t* kc);
int nosa_ref_append_keys(const nosa_ref_params* p, const uint16_t* k, const int32_t* cu_k,
                         const int32_t* valid_len, int B, int max_nc, uint16_t* kc);
void nosa_ref_set_num_threads(int n);
int nosa_ref_block_scores(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                          const uint16_t* kc, int max_nc, const int32_t* cu_k, int B,
                          int max_qblk, int max_nb, double* scores);
int nosa_ref_select_blocks(const nosa_ref_params* p, const double* scores, const int32_t* cu_q,
                           const int32_t* cu_k, int B, int max_qblk, int max_nb, int max_sel,
                           int32_t* sel, int32_t* count);
int nosa_ref_sparse_attend(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                           const uint16_t* k, const uint16_t* v, const int32_t* cu_k, int B,
                           const int32_t* sel, const int32_t* count, int max_qblk, int max_sel,
                           double* out, double* lse);
int nosa_ref_qkv_rope(const nosa_ref_params* p, int hidden, double theta, const double* inv_freq,
                      const uint16_t* x, const uint16_t* w, const int32_t* pos, int B,
                      uint16_t* q, uint16_t* k, uint16_t* v);
int nosa_ref_forward(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                     const uint16_t* k, const uint16_t* v, const int32_t* cu_k, int B,
                     int max_nc, int max_qblk, int max_nb, int max_sel, uint16_t* kc,
                     double* scores, int32_t* sel, int32_t* count, double* out, double* lse);

#ifdef __cplusplus
}
#endif
#endif
