// nosa_api.cpp -- the C ABI declared in include/nosa.h: argument validation,
// workspace planning and the order of kernel launches.  Validation runs on the
// host before anything is enqueued, so every error path is reachable without a
// GPU.  No allocation, no synchronisation, no global state.
#include <math.h>
#include <string.h>

#include "nosa_internal.h"

namespace nosa {
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Parameter checks shared by every entry point.
nosa_status check_params(const nosa_params* p)
{
    if (!p) return NOSA_ERR_NULL;
    if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 || p->block_size <= 0 ||
        p->kernel <= 0 || p->stride <= 0 || p->topk < 0 || p->window < 0)
        return NOSA_ERR_INVALID;
    if (p->num_q_heads % p->num_kv_heads != 0) return NOSA_ERR_INVALID;
    if (p->window % p->block_size != 0) return NOSA_ERR_INVALID;
    if (p->block_size % p->stride != 0) return NOSA_ERR_INVALID;
    if (!(p->scale == p->scale)) return NOSA_ERR_INVALID;  // NaN
    if (p->topk > (1 << 24) || p->window / p->block_size > (1 << 20)) return NOSA_ERR_INVALID;
    if (p->head_dim != kHeadDim || p->block_size != kBlock || p->kernel != kPoolK ||
        p->stride != kPoolS)
        return NOSA_ERR_UNSUPPORTED;
    if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return NOSA_ERR_UNSUPPORTED;
    return NOSA_OK;
}

nosa_status check_kv(const nosa_paged_kv* kv, int max_seqlen_k, bool need_kc_only)
{
    if (!kv) return NOSA_ERR_NULL;
    if (!kv->kc_pool || !kv->block_table || !kv->k_pool) return NOSA_ERR_NULL;
    if (!need_kc_only && !kv->v_pool) return NOSA_ERR_NULL;
    if (kv->max_blocks_per_seq <= 0 || kv->num_pages <= 0) return NOSA_ERR_INVALID;
    if ((long long)kv->max_blocks_per_seq * kBlock < (long long)max_seqlen_k)
        return NOSA_ERR_INVALID;
    return NOSA_OK;
}

nosa_status check_sizes(int batch, int max_seqlen_q, int max_seqlen_k)
{
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return NOSA_ERR_INVALID;
    if (batch > 0 && (max_seqlen_k < 1 || max_seqlen_q < 1)) return NOSA_ERR_INVALID;
    if (max_seqlen_q > max_seqlen_k && batch > 0) return NOSA_ERR_INVALID;
    if ((long long)ceil_div(max_seqlen_k, kBlock) > kMaxBlocks) return NOSA_ERR_UNSUPPORTED;
    return NOSA_OK;
}

int pick_score_tiles(long long tiles)
{
    // aim at ~2048 waves in flight; at most 8 tiles (128 keys) per wave
    long long t = tiles / 2048;
    if (t >= 8) return 8;
    if (t >= 4) return 4;
    if (t >= 2) return 2;
    return 1;
}

int pick_attn_rounds(long long blocks)
{
    // aim at ~1024 workgroups of 4 waves; at most 4 blocks per wave
    long long r = blocks / 4 / 1024;
    if (r < 1) r = 1;
    if (r > 4) r = 4;
    return (int)r;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

nosa_status make_plan(const nosa_params* p, int batch, int max_seqlen_k, Plan* pl)
{
    nosa_status st = check_params(p);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k);
    if (st != NOSA_OK) return st;
    Plan P;
    P.B = batch;
    P.Hq = p->num_q_heads;
    P.Hkv = p->num_kv_heads;
    P.G = P.Hq / P.Hkv;
    P.topk = p->topk;
    P.wblocks = p->window / p->block_size;
    P.max_sel = P.topk + P.wblocks;
    P.max_seqlen_k = max_seqlen_k;
    P.Lmax = max_seqlen_k;
    P.max_nc = num_keys(max_seqlen_k);
    P.max_nb = ceil_div(max_seqlen_k, kBlock);
    P.sel_span = P.max_sel < P.max_nb ? P.max_sel : P.max_nb;
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->head_dim);
    P.scale_log2 = (float)(scale * 1.4426950408889634);

    const int nc1 = P.max_nc > 0 ? P.max_nc : 1;
    P.score_tiles = pick_score_tiles((long long)batch * P.Hkv * ceil_div(nc1, 16));
    P.score_groups = ceil_div(nc1, 64 * P.score_tiles);
    P.nchunk = P.score_groups * 4;
    P.zstride = P.nchunk * 16 * P.score_tiles;

    const int span = P.sel_span > 0 ? P.sel_span : 1;
    P.attn_rounds = pick_attn_rounds((long long)batch * P.Hkv * span);
    P.nsplit = ceil_div(span, 4 * P.attn_rounds);

    const size_t B = (size_t)batch;
    size_t off = 0;
    P.off_z = off;      off += align256(B * P.Hq * (size_t)P.zstride * sizeof(float));
    P.off_zpart = off;  off += align256(B * P.Hq * (size_t)P.nchunk * sizeof(float2));
    P.off_scores = off; off += align256(B * P.Hkv * (size_t)P.max_nb * sizeof(float));
    P.off_sel = off;    off += align256(B * P.Hkv * (size_t)P.max_sel * sizeof(int32_t));
    P.off_cnt = off;    off += align256(B * P.Hkv * sizeof(int32_t));
    P.off_po = off;     off += align256(B * P.Hq * (size_t)P.nsplit * kHeadDim * sizeof(float));
    P.off_pml = off;    off += align256(B * P.Hq * (size_t)P.nsplit * sizeof(float2));
    P.bytes = off > 256 ? off : 256;
    *pl = P;
    return NOSA_OK;
}

}  // namespace nosa

using namespace nosa;

namespace {

template <class T>
T* ws_at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

nosa_status hip_status(hipError_t e) { return e == hipSuccess ? NOSA_OK : NOSA_ERR_HIP; }

// Common checks of the query-side arguments (decode only in this build).
nosa_status check_queries(const int32_t* cu_seqlens_q, int max_seqlen_q)
{
    if (cu_seqlens_q != nullptr || max_seqlen_q > 1) return NOSA_ERR_UNSUPPORTED;
    return NOSA_OK;
}

}  // namespace

extern "C" {

int nosa_abi_version(void) { return NOSA_ABI_VERSION; }

const char* nosa_status_string(nosa_status s)
{
    switch (s) {
        case NOSA_OK: return "ok";
        case NOSA_ERR_NULL: return "a required pointer is NULL";
        case NOSA_ERR_INVALID: return "invalid or inconsistent arguments";
        case NOSA_ERR_UNSUPPORTED: return "no GPU kernel for this shape";
        case NOSA_ERR_WORKSPACE: return "workspace missing or too small";
        case NOSA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

nosa_status nosa_workspace_size(const nosa_params* params, int32_t batch, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, size_t* bytes)
{
    if (!params || !bytes) return NOSA_ERR_NULL;
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, max_seqlen_q, max_seqlen_k);
    if (st != NOSA_OK) return st;
    if (max_seqlen_q > 1) return NOSA_ERR_UNSUPPORTED;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    *bytes = pl.bytes;
    return NOSA_OK;
}

nosa_status nosa_compress_keys(const nosa_params* params, const nosa_paged_kv* kv,
                               const int32_t* cu_seqlens_k, const int32_t* kc_valid_len,
                               int32_t batch, int32_t max_seqlen_k, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    // no token anywhere (max_seqlen_k == 0) is a valid, empty request
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k > 0 ? max_seqlen_k : 1);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen_k, true);
    if (st != NOSA_OK) return st;
    if (!cu_seqlens_k) return NOSA_ERR_NULL;
    if (batch == 0 || max_seqlen_k == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    int gx = ceil_div(pl.max_nc > 0 ? pl.max_nc : 1, 16);
    if (kc_valid_len && gx > 64) gx = 64;  // grid-stride over whatever is left to pool
    return hip_status(launch_kc_build(pl, *kv, cu_seqlens_k, kc_valid_len, false, gx,
                                      as_stream(stream)));
}

nosa_status nosa_block_scores(const nosa_params* params, const nosa_paged_kv* kv,
                              const nosa_bf16* q, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, float* block_scores, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, max_seqlen_q, max_seqlen_k);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen_k, true);
    if (st != NOSA_OK) return st;
    if (!q || !cu_seqlens_k || !block_scores) return NOSA_ERR_NULL;
    st = check_queries(cu_seqlens_q, max_seqlen_q);
    if (st != NOSA_OK) return st;
    if (batch == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    float* z = ws_at<float>(workspace, pl.off_z);
    float2* zpart = ws_at<float2>(workspace, pl.off_zpart);
    st = hip_status(launch_scores(pl, *kv, q, cu_seqlens_k, z, zpart, s));
    if (st != NOSA_OK) return st;
    return hip_status(launch_select(pl, cu_seqlens_k, z, zpart, nullptr, block_scores, nullptr,
                                    nullptr, s));
}

nosa_status nosa_select_blocks(const nosa_params* params, const float* block_scores,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t* sel_idx, int32_t* sel_count, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, max_seqlen_q, max_seqlen_k);
    if (st != NOSA_OK) return st;
    if (!block_scores || !cu_seqlens_k || !sel_idx || !sel_count) return NOSA_ERR_NULL;
    st = check_queries(cu_seqlens_q, max_seqlen_q);
    if (st != NOSA_OK) return st;
    if (batch == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    return hip_status(launch_select(pl, cu_seqlens_k, nullptr, nullptr, block_scores, nullptr,
                                    sel_idx, sel_count, as_stream(stream)));
}

nosa_status nosa_sparse_attend(const nosa_params* params, const nosa_paged_kv* kv,
                               const nosa_bf16* q, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const int32_t* sel_idx,
                               const int32_t* sel_count, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, max_seqlen_q, max_seqlen_k);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen_k, false);
    if (st != NOSA_OK) return st;
    if (!q || !cu_seqlens_k || !sel_idx || !sel_count || !out) return NOSA_ERR_NULL;
    st = check_queries(cu_seqlens_q, max_seqlen_q);
    if (st != NOSA_OK) return st;
    if (batch == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    float* po = ws_at<float>(workspace, pl.off_po);
    float2* pml = ws_at<float2>(workspace, pl.off_pml);
    st = hip_status(launch_attend(pl, *kv, q, cu_seqlens_k, sel_idx, sel_count, po, pml, s));
    if (st != NOSA_OK) return st;
    return hip_status(launch_merge(pl, po, pml, out, lse, s));
}

nosa_status nosa_decode_step(const nosa_params* params, const nosa_paged_kv* kv,
                             const nosa_bf16* q, const int32_t* cu_seqlens_k, int32_t batch,
                             int32_t max_seqlen_k, float* out, float* lse, int32_t* sel_idx,
                             int32_t* sel_count, float* block_scores, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen_k, false);
    if (st != NOSA_OK) return st;
    if (!q || !cu_seqlens_k || !out) return NOSA_ERR_NULL;
    if ((sel_idx == nullptr) != (sel_count == nullptr)) return NOSA_ERR_NULL;
    if (batch == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    float* z = ws_at<float>(workspace, pl.off_z);
    float2* zpart = ws_at<float2>(workspace, pl.off_zpart);
    int32_t* sel = sel_idx ? sel_idx : ws_at<int32_t>(workspace, pl.off_sel);
    int32_t* cnt = sel_count ? sel_count : ws_at<int32_t>(workspace, pl.off_cnt);
    float* po = ws_at<float>(workspace, pl.off_po);
    float2* pml = ws_at<float2>(workspace, pl.off_pml);
    // the current token completes at most one pooled key per sequence
    st = hip_status(launch_kc_build(pl, *kv, cu_seqlens_k, nullptr, true, 1, s));
    if (st != NOSA_OK) return st;
    st = hip_status(launch_scores(pl, *kv, q, cu_seqlens_k, z, zpart, s));
    if (st != NOSA_OK) return st;
    st = hip_status(launch_select(pl, cu_seqlens_k, z, zpart, nullptr, block_scores, sel, cnt, s));
    if (st != NOSA_OK) return st;
    st = hip_status(launch_attend(pl, *kv, q, cu_seqlens_k, sel, cnt, po, pml, s));
    if (st != NOSA_OK) return st;
    return hip_status(launch_merge(pl, po, pml, out, lse, s));
}

}  // extern "C"
