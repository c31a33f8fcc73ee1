/*
 * nosa_oracle.c -- plain, slow CPU reference of the NOSA sparse-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP
 * library; the two meet only through the seeded input generator.
 *
 * What it computes (sources are the web pages on NOSA; each function names the
 * passage it follows):
 *   1. compressed keys: mean of K over windows of `kernel` tokens taken every
 *      `stride` tokens, stored as bf16;
 *   2. compressed attention of every query head against those keys (softmax per
 *      head), summed over the heads that share a KV head (GQA group);
 *   3. CIS pooling: mean of those scores over the compressed keys whose window
 *      overlaps a `block_size`-token block -> one importance per block;
 *   4. the local window (the last window/block_size blocks) is always kept, and
 *      the `topk` most important of the remaining blocks are added (ties go to the
 *      lower block index);
 *   5. exact causal softmax attention over the tokens of the kept blocks only.
 *
 * Arithmetic: every dot product, exponential and sum is done in double.  The
 * compressed keys are the bf16 round-to-nearest-even of the exact window mean
 * (the sum of `kernel` bf16 numbers is exact in double for any inputs whose
 * exponents span less than ~45 binades).  Inputs are bf16 bit patterns
 * (uint16_t); everything else is plain row-major C arrays.
 *
 * Layouts (all row-major, all host memory owned by the caller):
 *   q   [total_q][Hq][d]      bf16 bits, rows of sequence s at cu_q[s]..cu_q[s+1]
 *                             (cu_q == NULL: one query per sequence, row s)
 *   k,v [total_k][Hkv][d]     bf16 bits, tokens of sequence s at cu_k[s]..cu_k[s+1]
 *   kc  [B][Hkv][max_nc][d]   bf16 bits
 *   scores [B][max_qblk][Hkv][max_nb]  double, -INFINITY where undefined
 *   sel    [B][max_qblk][Hkv][max_sel] int32 block ids ascending, -1 padding
 *   count  [B][max_qblk][Hkv]          int32
 *   out    [total_q][Hq][d]   double;  lse [total_q][Hq] double (natural log)
 *
 * The queries of a sequence are the last Lq positions of its context
 * ([L-Lq, L)); they are grouped into query blocks of block_size consecutive
 * queries counted from the first one.  A decode step is the case Lq = 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "nosa_oracle.h"

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, written from the
 * definition: bf16 keeps 8 significant bits for normal numbers (exponent of
 * the leading bit >= -126) and a fixed quantum of 2^-133 below that.  The
 * rounding itself is nearbyint() in the default (nearest-even) mode on an
 * exactly scaled copy, so there is exactly one rounding. */
uint16_t nosa_ref_bf16_round(double x)
{
    if (isnan(x)) return 0x7fc0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    if (isinf(x)) return signbit(x) ? 0xff80 : 0x7f80;
    int e;
    frexp(x, &e);                 /* |x| = m * 2^e, 0.5 <= m < 1: leading bit 2^(e-1) */
    int qexp = e - 8;             /* quantum of an 8-significant-bit number          */
    if (qexp < -133) qexp = -133; /* bf16 subnormal quantum                          */
    double r = ldexp(nearbyint(ldexp(x, -qexp)), qexp);
    float f = (float)r;           /* exact: r is a bf16 value (or overflows to inf)  */
    if (fabs(r) >= 0x1p128) f = signbit(r) ? -INFINITY : INFINITY;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

double nosa_ref_bf16_to_double(uint16_t bits) { return bf16_value(bits); }

/* ------------------------------------------------------------- helpers --- */

/* Number of complete pooling windows in the first L tokens: window j covers
 * tokens [j*stride, j*stride + kernel). */
int nosa_ref_num_keys(int L, int kernel, int stride)
{
    if (L < kernel) return 0;
    return (L - kernel) / stride + 1;
}

static int seq_len(const int32_t* cu, int s) { return cu[s + 1] - cu[s]; }

static int q_len(const int32_t* cu_q, int s) { return cu_q ? cu_q[s + 1] - cu_q[s] : 1; }

static int q_row0(const int32_t* cu_q, int s) { return cu_q ? cu_q[s] : s; }

static double eff_scale(const nosa_ref_params* p)
{
    return p->scale > 0.0 ? p->scale : 1.0 / sqrt((double)p->head_dim);
}

int nosa_ref_check_params(const nosa_ref_params* p)
{
    if (!p) return -1;
    if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0) return -2;
    if (p->num_q_heads % p->num_kv_heads != 0) return -3;
    if (p->block_size <= 0 || p->kernel <= 0 || p->stride <= 0) return -4;
    if (p->topk < 0 || p->window < 0) return -5;
    if (p->window % p->block_size != 0) return -6;
    if (!(p->locality >= 0.0 && p->locality <= 1.0)) return -7;
    return 0;
}

/* ---------------------------------------------------- 1. compressed keys --- */

/* Pooled keys (page "NOSA-1B 性能基准全解析", section 三.3 两阶段注意力, and the
 * config table of section 四: pooling with kernel 32, stride 16; page
 * "从论文到代码", section 2: the pooling is applied to k per sequence through
 * cu_seqlens).  Key j of KV head g is the mean of K[t][g][:] over
 * t in [j*stride, j*stride + kernel), rounded once to bf16. */
int nosa_ref_compress_keys(const nosa_ref_params* p, const uint16_t* k, const int32_t* cu_k,
                           int B, int max_nc, uint16_t* kc)
{
    if (B < 0 || (B > 0 && (!k || !cu_k || !kc))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hkv = p->num_kv_heads, d = p->head_dim;
    for (int s = 0; s < B; ++s)
        if (nosa_ref_num_keys(seq_len(cu_k, s), p->kernel, p->stride) > max_nc) return -2;
    memset(kc, 0, sizeof(uint16_t) * (size_t)B * Hkv * max_nc * d);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s)
        for (int g = 0; g < Hkv; ++g) {
            const int L = seq_len(cu_k, s);
            const int nc = nosa_ref_num_keys(L, p->kernel, p->stride);
            for (int j = 0; j < nc; ++j)
                for (int c = 0; c < d; ++c) {
                    double sum = 0.0;
                    for (int t = j * p->stride; t < j * p->stride + p->kernel; ++t)
                        sum += bf16_value(k[((size_t)(cu_k[s] + t) * Hkv + g) * d + c]);
                    kc[(((size_t)s * Hkv + g) * max_nc + j) * d + c] =
                        nosa_ref_bf16_round(sum / p->kernel);
                }
        }
    return 0;
}

/* The same keys for a cache that grows (a decode step appends tokens): for
 * each sequence, only keys j in [n_c(valid_len[s]), n_c(L_s)) are computed,
 * the keys of the first valid_len[s] tokens being already in kc; nothing
 * else in kc is touched.  Each key is the same exact window mean as above, so
 * appending token by token gives the full build's keys. */
int nosa_ref_append_keys(const nosa_ref_params* p, const uint16_t* k, const int32_t* cu_k,
                         const int32_t* valid_len, int B, int max_nc, uint16_t* kc)
{
    if (B < 0 || (B > 0 && (!k || !cu_k || !valid_len || !kc))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hkv = p->num_kv_heads, d = p->head_dim;
    for (int s = 0; s < B; ++s) {
        if (nosa_ref_num_keys(seq_len(cu_k, s), p->kernel, p->stride) > max_nc) return -2;
        if (valid_len[s] < 0 || valid_len[s] > seq_len(cu_k, s)) return -3;
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s)
        for (int g = 0; g < Hkv; ++g) {
            const int L = seq_len(cu_k, s);
            const int j0 = nosa_ref_num_keys(valid_len[s], p->kernel, p->stride);
            const int nc = nosa_ref_num_keys(L, p->kernel, p->stride);
            for (int j = j0; j < nc; ++j)
                for (int c = 0; c < d; ++c) {
                    double sum = 0.0;
                    for (int t = j * p->stride; t < j * p->stride + p->kernel; ++t)
                        sum += bf16_value(k[((size_t)(cu_k[s] + t) * Hkv + g) * d + c]);
                    kc[(((size_t)s * Hkv + g) * max_nc + j) * d + c] =
                        nosa_ref_bf16_round(sum / p->kernel);
                }
        }
    return 0;
}

/* --------------------------------------------- 2+3. block importance ------ */

/* Importance of every KV block for every query block.
 *
 * Compressed attention (page "NOSA-1B 性能基准全解析", section 三.3: coarse scores
 * from attention over the pooled keys; page "NOSA-1B 模型家族全景", the core
 * principle: compressed attention filters history first): for each query at
 * position p and each head h of KV group g, the softmax over the pooled keys
 * the query can see (window end j*stride+kernel <= p+1) of scale * q_h . Kc_j.
 * These probabilities are summed over the group's heads and over the query
 * block's queries.
 *
 * CIS pooling (page "NOSA-1B 模型家族全景", the note on cis_pooling.py: a mean
 * pooling of the scores): the importance of block b is the mean of the summed
 * probabilities over the pooled keys whose token window overlaps block b,
 * i.e. j*stride < (b+1)*block_size and j*stride + kernel > b*block_size, among
 * the keys visible to the block's last query.  No such key -> -INFINITY. */
int nosa_ref_block_scores(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                          const uint16_t* kc, int max_nc, const int32_t* cu_k, int B,
                          int max_qblk, int max_nb, double* scores)
{
    /* required pointers (cu_q may be NULL: one query per sequence) */
    if (B < 0 || (B > 0 && (!q || !kc || !cu_k || !scores))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hq = p->num_q_heads, Hkv = p->num_kv_heads, G = Hq / Hkv, d = p->head_dim;
    const int bs = p->block_size;
    const double scale = eff_scale(p);
    for (int s = 0; s < B; ++s) {
        const int L = seq_len(cu_k, s), Lq = q_len(cu_q, s);
        if (Lq > L || Lq < 0) return -2;
        if ((Lq + bs - 1) / bs > max_qblk) return -3;
        if ((L + bs - 1) / bs > max_nb) return -4;
        if (nosa_ref_num_keys(L, p->kernel, p->stride) > max_nc) return -5;
    }
    for (size_t i = 0; i < (size_t)B * max_qblk * Hkv * max_nb; ++i) scores[i] = -INFINITY;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s)
        for (int g = 0; g < Hkv; ++g) {
            const int L = seq_len(cu_k, s), Lq = q_len(cu_q, s);
            const int nqb = (Lq + bs - 1) / bs;
            const int nc_all = nosa_ref_num_keys(L, p->kernel, p->stride);
            double* sigma = (double*)calloc(nc_all > 0 ? nc_all : 1, sizeof(double));
            double* z = (double*)malloc(sizeof(double) * (nc_all > 0 ? nc_all : 1));
            for (int r = 0; r < nqb; ++r) {
                const int i0 = r * bs, i1 = (r + 1) * bs < Lq ? (r + 1) * bs : Lq;
                const int p_last = L - Lq + i1 - 1;
                const int nc_blk = nosa_ref_num_keys(p_last + 1, p->kernel, p->stride);
                for (int j = 0; j < nc_blk; ++j) sigma[j] = 0.0;
                for (int i = i0; i < i1; ++i) {
                    const int pos = L - Lq + i;
                    const int nc = nosa_ref_num_keys(pos + 1, p->kernel, p->stride);
                    if (nc == 0) continue;
                    for (int h = g * G; h < (g + 1) * G; ++h) {
                        const uint16_t* qh = q + ((size_t)(q_row0(cu_q, s) + i) * Hq + h) * d;
                        double zmax = -INFINITY;
                        for (int j = 0; j < nc; ++j) {
                            const uint16_t* kj = kc + (((size_t)s * Hkv + g) * max_nc + j) * d;
                            double dot = 0.0;
                            for (int c = 0; c < d; ++c) dot += bf16_value(qh[c]) * bf16_value(kj[c]);
                            z[j] = scale * dot;
                            if (z[j] > zmax) zmax = z[j];
                        }
                        double den = 0.0;
                        for (int j = 0; j < nc; ++j) den += exp(z[j] - zmax);
                        for (int j = 0; j < nc; ++j) sigma[j] += exp(z[j] - zmax) / den;
                    }
                }
                double* out = scores + (((size_t)s * max_qblk + r) * Hkv + g) * max_nb;
                const int nb = p_last / bs + 1;
                for (int b = 0; b < nb; ++b) {
                    double sum = 0.0;
                    int cnt = 0;
                    for (int j = 0; j < nc_blk; ++j) {
                        const int w0 = j * p->stride, w1 = j * p->stride + p->kernel;
                        if (w0 < (b + 1) * bs && w1 > b * bs) {
                            sum += sigma[j];
                            ++cnt;
                        }
                    }
                    out[b] = cnt ? sum / cnt : -INFINITY;
                }
            }
            free(z);
            free(sigma);
        }
    return 0;
}

/* ------------------------------------------------------------ 4. select --- */

typedef struct {
    double score;
    int block;
} cand_t;

/* Order: higher score first, then lower block index. */
static int cand_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->block > y->block) - (x->block < y->block);
}

/* Block selection (page "NOSA-1B 性能基准全解析", section 三.2 显式局部性约束:
 * a 1024-token window of 64-token blocks, i.e. about 16 nearby blocks, is
 * always attended and TopK picks 64 high-scoring blocks; section 三.3: TopK over
 * the coarse scores; page "NOSA-1B 模型家族全景", core principle: explicit local
 * window of 1024 tokens).  Window = the last window/block_size blocks up to and
 * including the block of the query block's last query; the topk best of the
 * earlier blocks are added.  Output ascending, padded with -1.
 *
 * Locality constraint (page "NOSA技术架构解析", section 1.2: a minimum
 * locality gamma_0 -- the share of local blocks that must be kept -- and a
 * query-aware share kq/k of the budget; in every setting the page prints,
 * 1.2 and 4.1, the two add up to one): of the topk budget,
 * k_loc = round(gamma_0 * topk) goes to the candidates nearest the window
 * (kept whatever the query), the other topk - k_loc to the best of the
 * remaining candidates by score. */
int nosa_ref_select_blocks(const nosa_ref_params* p, const double* scores, const int32_t* cu_q,
                           const int32_t* cu_k, int B, int max_qblk, int max_nb, int max_sel,
                           int32_t* sel, int32_t* count)
{
    /* required pointers (cu_q may be NULL: one query per sequence) */
    if (B < 0 || (B > 0 && (!scores || !cu_k || !sel || !count))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hkv = p->num_kv_heads, bs = p->block_size, w = p->window / p->block_size;
    if (max_sel < p->topk + w) return -2;
    for (size_t i = 0; i < (size_t)B * max_qblk * Hkv * max_sel; ++i) sel[i] = -1;
    for (size_t i = 0; i < (size_t)B * max_qblk * Hkv; ++i) count[i] = 0;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s)
        for (int g = 0; g < Hkv; ++g) {
            const int L = seq_len(cu_k, s), Lq = q_len(cu_q, s);
            const int nqb = (Lq + bs - 1) / bs;
            for (int r = 0; r < nqb; ++r) {
                const int i1 = (r + 1) * bs < Lq ? (r + 1) * bs : Lq;
                const int p_last = L - Lq + i1 - 1;
                const int nb = p_last / bs + 1;
                if (nb > max_nb) {
#pragma omp atomic write
                    err = -3;
                    continue;
                }
                const int first_win = nb - w > 0 ? nb - w : 0;
                const double* sc = scores + (((size_t)s * max_qblk + r) * Hkv + g) * max_nb;
                char* keep = (char*)calloc(nb, 1);
                for (int b = first_win; b < nb; ++b) keep[b] = 1;
                /* the local share: the k_loc candidates right before the window */
                const int k_loc = (int)floor(p->locality * p->topk + 0.5);
                const int n_loc = k_loc < first_win ? k_loc : first_win;
                for (int b = first_win - n_loc; b < first_win; ++b) keep[b] = 1;
                /* the query-aware share among the candidates before those */
                const int ncand = first_win - n_loc;
                const int k_q = p->topk - k_loc;
                if (ncand > 0 && k_q > 0) {
                    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * ncand);
                    for (int b = 0; b < ncand; ++b) {
                        c[b].score = sc[b];
                        c[b].block = b;
                    }
                    qsort(c, ncand, sizeof(cand_t), cand_cmp);
                    const int take = k_q < ncand ? k_q : ncand;
                    for (int i = 0; i < take; ++i) keep[c[i].block] = 1;
                    free(c);
                }
                int32_t* out = sel + (((size_t)s * max_qblk + r) * Hkv + g) * max_sel;
                int n = 0;
                for (int b = 0; b < nb; ++b)
                    if (keep[b]) out[n++] = b;
                count[((size_t)s * max_qblk + r) * Hkv + g] = n;
                free(keep);
            }
        }
    return err;
}

/* ------------------------------------------------------------ 5. attend --- */

/* Exact attention on the kept blocks (page "NOSA-1B 性能基准全解析", sections
 * 三.2-三.3: exact attention over the TopK blocks; the rest of the history is
 * only seen through the pooled keys).  For the query at position p and head h:
 * softmax over t <= p with block(t) kept of scale * q_h . K[t], applied to V.
 * lse = log of the softmax denominator (natural log, unshifted logits). */
int nosa_ref_sparse_attend(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                           const uint16_t* k, const uint16_t* v, const int32_t* cu_k, int B,
                           const int32_t* sel, const int32_t* count, int max_qblk, int max_sel,
                           double* out, double* lse)
{
    /* required pointers (cu_q may be NULL: one query per sequence) */
    if (B < 0 || (B > 0 && (!q || !k || !v || !cu_k || !sel || !count || !out || !lse))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hq = p->num_q_heads, Hkv = p->num_kv_heads, G = Hq / Hkv, d = p->head_dim;
    const int bs = p->block_size;
    const double scale = eff_scale(p);
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s)
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;
            const int L = seq_len(cu_k, s), Lq = q_len(cu_q, s);
            const int nb_max = (L + bs - 1) / bs;
            char* keep = (char*)malloc(nb_max > 0 ? nb_max : 1);
            double* logit = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
            for (int i = 0; i < Lq; ++i) {
                const int r = i / bs;
                const int pos = L - Lq + i;
                const size_t row = (size_t)(q_row0(cu_q, s) + i) * Hq + h;
                const int32_t* sl = sel + (((size_t)s * max_qblk + r) * Hkv + g) * max_sel;
                const int n = count[((size_t)s * max_qblk + r) * Hkv + g];
                memset(keep, 0, nb_max > 0 ? nb_max : 1);
                for (int x = 0; x < n; ++x) {
                    if (sl[x] < 0 || sl[x] >= nb_max) {
#pragma omp atomic write
                        err = -2;
                        continue;
                    }
                    keep[sl[x]] = 1;
                }
                double m = -INFINITY;
                for (int t = 0; t <= pos; ++t) {
                    if (!keep[t / bs]) continue;
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c)
                        dot += bf16_value(q[row * d + c]) *
                               bf16_value(k[((size_t)(cu_k[s] + t) * Hkv + g) * d + c]);
                    logit[t] = scale * dot;
                    if (logit[t] > m) m = logit[t];
                }
                double den = 0.0;
                for (int t = 0; t <= pos; ++t)
                    if (keep[t / bs]) den += exp(logit[t] - m);
                double* o = out + row * d;
                for (int c = 0; c < d; ++c) o[c] = 0.0;
                if (den > 0.0) {
                    for (int t = 0; t <= pos; ++t) {
                        if (!keep[t / bs]) continue;
                        const double w = exp(logit[t] - m) / den;
                        for (int c = 0; c < d; ++c)
                            o[c] += w * bf16_value(v[((size_t)(cu_k[s] + t) * Hkv + g) * d + c]);
                    }
                    lse[row] = m + log(den);
                } else {
                    lse[row] = -INFINITY;
                }
            }
            free(logit);
            free(keep);
        }
    return err;
}

/* -------------------------------------------------------- whole step ----- */

/* The whole step in the pages' order: pool the keys, score, pool the scores
 * into block importance, select, attend. */
int nosa_ref_forward(const nosa_ref_params* p, const uint16_t* q, const int32_t* cu_q,
                     const uint16_t* k, const uint16_t* v, const int32_t* cu_k, int B,
                     int max_nc, int max_qblk, int max_nb, int max_sel, uint16_t* kc,
                     double* scores, int32_t* sel, int32_t* count, double* out, double* lse)
{
    int rc = nosa_ref_compress_keys(p, k, cu_k, B, max_nc, kc);
    if (rc) return rc - 10;
    rc = nosa_ref_block_scores(p, q, cu_q, kc, max_nc, cu_k, B, max_qblk, max_nb, scores);
    if (rc) return rc - 20;
    rc = nosa_ref_select_blocks(p, scores, cu_q, cu_k, B, max_qblk, max_nb, max_sel, sel, count);
    if (rc) return rc - 30;
    rc = nosa_ref_sparse_attend(p, q, cu_q, k, v, cu_k, B, sel, count, max_qblk, max_sel, out, lse);
    if (rc) return rc - 40;
    return 0;
}

/* ------------------------------------------ 0. projections and rotary ---- */

/* The attention front end of one decode token per sequence (page "NOSA技术架构
 * 解析", section 2.1: the QKV projection, the rotary position encoding and the
 * importance scoring make up one step of the decode path).  Token b has the
 * hidden state x[b][0 .. hidden) and position pos[b].  The projection is
 * y[o] = sum_c w[o][c] x[b][c] over the rows o of w: Hq heads of q, then Hkv
 * heads of k, then Hkv heads of v, head_dim rows each.  Within each q and k
 * head, channel i and channel i + head_dim/2 (i < head_dim/2) are rotated as
 * one pair by the angle pos[b] * inv_freq[i]: with c = cos, s = sin,
 *   (y[i], y[i + d/2]) -> (y[i] c - y[i + d/2] s, y[i + d/2] c + y[i] s);
 * v is not rotated.  Every result is rounded once to bf16.  inv_freq NULL
 * means theta^(-2i/d).  Layouts: x [B][hidden], w [(Hq + 2 Hkv) d][hidden]
 * (bf16 bits), q [B][Hq][d], k and v [B][Hkv][d] (bf16 bits). */
int nosa_ref_qkv_rope(const nosa_ref_params* p, int hidden, double theta, const double* inv_freq,
                      const uint16_t* x, const uint16_t* w, const int32_t* pos, int B,
                      uint16_t* q, uint16_t* k, uint16_t* v)
{
    if (B < 0 || (B > 0 && (!x || !w || !pos || !q || !k || !v))) return -9;
    if (nosa_ref_check_params(p)) return -1;
    const int Hq = p->num_q_heads, Hkv = p->num_kv_heads, d = p->head_dim, half = d / 2;
    if (hidden <= 0 || B < 0 || d % 2) return -2;
    if (!inv_freq && !(theta > 0.0)) return -3;
    const int heads = Hq + 2 * Hkv;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < heads; ++h) {
            double y[1024];
            if (d > 1024) return -4;
            for (int o = 0; o < d; ++o) {
                double acc = 0.0;
                const uint16_t* wr = w + ((size_t)h * d + o) * hidden;
                for (int c = 0; c < hidden; ++c)
                    acc += bf16_value(wr[c]) * bf16_value(x[(size_t)b * hidden + c]);
                y[o] = acc;
            }
            if (h < Hq + Hkv) {  /* q and k heads: the rotary encoding */
                for (int i = 0; i < half; ++i) {
                    const double f = inv_freq ? inv_freq[i] : pow(theta, -2.0 * i / d);
                    const double a = (double)pos[b] * f;
                    const double cs = cos(a), sn = sin(a);
                    const double lo = y[i], hi = y[i + half];
                    y[i] = lo * cs - hi * sn;
                    y[i + half] = hi * cs + lo * sn;
                }
            }
            uint16_t* dst = h < Hq ? q + ((size_t)b * Hq + h) * d
                          : h < Hq + Hkv ? k + ((size_t)b * Hkv + (h - Hq)) * d
                                         : v + ((size_t)b * Hkv + (h - Hq - Hkv)) * d;
            for (int o = 0; o < d; ++o) dst[o] = nosa_ref_bf16_round(y[o]);
        }
    return 0;
}

int nosa_ref_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (n >= 1). */
void nosa_ref_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
