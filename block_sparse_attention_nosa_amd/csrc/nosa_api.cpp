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

// Blocks of the topk budget given to the candidates nearest the window.
int local_blocks(const nosa_params* p)
{
    return (int)floor((double)p->locality * p->topk + 0.5);
}

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
    if (!(p->locality >= 0.f && p->locality <= 1.f)) return NOSA_ERR_INVALID;  // incl. NaN
    if (p->topk > (1 << 24) || p->window / p->block_size > (1 << 20)) return NOSA_ERR_INVALID;
    if (p->head_dim != kHeadDim || p->block_size != kBlock || p->kernel != kPoolK ||
        p->stride != kPoolS)
        return NOSA_ERR_UNSUPPORTED;
    if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return NOSA_ERR_UNSUPPORTED;
    if (p->window / p->block_size + local_blocks(p) > kMaxWindowBlocks) return NOSA_ERR_UNSUPPORTED;
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

// Tiles of 16 pooled keys per wave of a scoring workgroup (one of the
// compiled 1, 2, 4, 8; a chunk is 64 T keys): the smallest T that keeps the
// launch within about 1024 workgroups (four per CU) and a pair within
// kMaxChunks chunks.  Small T spreads a short context over many CUs: one CU
// streams only about 100 GB/s.
int pick_score_tiles(int nc, long long pairs)
{
    const int tiles = ceil_div(nc > 0 ? nc : 1, 16);
    for (int t : {1, 2, 4})
        if (ceil_div(tiles, 4 * t) <= kMaxChunks && pairs * ceil_div(tiles, 4 * t) <= 1024) return t;
    return 8;
}

// Blocks per wave (rounds, one of the compiled 1, 2, 3, 4, 6, 8) and
// workgroups per pair for `span` list entries per pair: about 512
// workgroups of kStep2Waves (4) waves in total -- two per CU, one dispatch
// round -- and at most `max_groups` partials per head.
void pick_split(int span, long long pairs, int max_groups, int* groups, int* rounds)
{
    static const int kRounds[] = {1, 2, 3, 4, 6, 8};
    constexpr int W = kStep2Waves;
    if (span <= 0) {
        *groups = 1;
        *rounds = 1;
        return;
    }
    const long long total_blocks = (long long)span * pairs;
    int pick = 5;
    for (int i = 0; i < 6; ++i)
        if (total_blocks <= (long long)W * 512 * kRounds[i]) {
            pick = i;
            break;
        }
    while (pick < 5 && ceil_div(span, W * kRounds[pick]) > max_groups) ++pick;
    *rounds = kRounds[pick];
    *groups = ceil_div(span, W * kRounds[pick]);
}

// Split of the stand-alone attention: each pair's `span` list entries are
// dealt round-robin to `groups` workgroups of four waves, `rounds` entries
// per wave.  A CU streams only so many bytes at a time, so the launch time is
// that of the busiest CU: the launch gets at most one workgroup per CU (of
// kCusTarget), or two when one would need more than 8 entries per wave, and
// every workgroup of a pair the same number of pages, give or take one.  (Two
// per CU with one page per wave measured slower at 16K batch 8: twice the
// partials for the merge.)  Batches too large for that fall back to
// pick_split.
void pick_attend_split(int span, long long pairs, int* groups, int* rounds)
{
    constexpr int kCusTarget = 256;
    static const int kRounds[] = {1, 2, 3, 4, 6, 8};
    if (span <= 0 || pairs <= 0) {
        *groups = 1;
        *rounds = 1;
        return;
    }
    for (int per_cu = 1; per_cu <= 2; ++per_cu) {
        const long long g = (long long)kCusTarget * per_cu / pairs;
        if (g < 1) break;
        int gmax = ceil_div(span, kStep2Waves);  // one page per wave at most
        gmax = gmax < kMaxSplit ? gmax : kMaxSplit;
        const int gr = (int)(g < gmax ? g : gmax);
        const int need = ceil_div(ceil_div(span, gr), kStep2Waves);
        for (int r : kRounds)
            if (r >= need) {
                *groups = gr;
                *rounds = r;
                return;
            }
    }
    pick_split(span, pairs, kMaxSplit, groups, rounds);
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
    // the locality share is exactly a longer forced window and a smaller top-k
    const int k_loc = local_blocks(p);
    P.topk = p->topk - k_loc;
    P.wblocks = p->window / p->block_size + k_loc;
    P.max_sel = P.topk + P.wblocks;
    P.max_seqlen_k = max_seqlen_k;
    P.Lmax = max_seqlen_k;
    P.max_nc = num_keys(max_seqlen_k);
    P.max_nb = ceil_div(max_seqlen_k, kBlock);
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->head_dim);
    P.scale_log2 = (float)(scale * 1.4426950408889634);

    const long long npairs = (long long)batch * P.Hkv;
    P.score_tiles = pick_score_tiles(P.max_nc, npairs);
    P.chunk_keys = 64 * P.score_tiles;
    P.nchunks = ceil_div(P.max_nc > 0 ? P.max_nc : 1, P.chunk_keys);
    P.nbk = P.nchunks * 16 * P.score_tiles;
    P.gp = ceil_div(P.G, 4) * 4;

    const int ncand = P.max_nb > P.wblocks ? P.max_nb - P.wblocks : 0;
    P.top_span = P.topk < ncand ? P.topk : ncand;
    P.wslots = P.wblocks < P.max_nb ? P.wblocks : P.max_nb;
    pick_split(P.top_span, npairs, kMaxSplit, &P.top_groups, &P.top_rounds);
    P.nsplit = P.top_groups + P.wslots;
    const int aspan = P.max_sel < P.max_nb ? P.max_sel : P.max_nb;
    pick_attend_split(aspan, (long long)batch * P.Hkv, &P.attend_groups, &P.attend_rounds);
    const int nparts = P.nsplit > P.attend_groups ? P.nsplit : P.attend_groups;

    const size_t B = (size_t)batch, pairs = B * P.Hkv;
    size_t off = 0;
    P.off_cml = off;      off += align256(pairs * P.nchunks * (size_t)P.G * sizeof(float2));
    P.off_spill = off;    off += align256(pairs * P.nchunks * (size_t)P.G * sizeof(float));
    P.off_bpart = off;    off += align256(pairs * P.nbk * (size_t)P.gp * sizeof(float));
    P.off_po = off;       off += align256(B * P.Hq * (size_t)nparts * kHeadDim * sizeof(float));
    P.off_pml = off;      off += align256(B * P.Hq * (size_t)nparts * sizeof(float2));
    P.bytes = off > 256 ? off : 256;
    *pl = P;
    return NOSA_OK;
}

void make_pf_plan(const Plan& pl, int max_seqlen_q, PfPlan* pf)
{
    PfPlan F;
    F.max_seqlen_q = max_seqlen_q;
    F.max_qblk = ceil_div(max_seqlen_q > 0 ? max_seqlen_q : 1, 64);
    F.npairs = pl.B * F.max_qblk * pl.Hkv;
    F.rows = 64 * pl.G;
    F.rtw = pl.G <= 1 ? 1 : pl.G <= 2 ? 2 : pl.G <= 4 ? 4 : 8;
    F.row_groups = ceil_div(4 * pl.G, 4 * F.rtw);
    // scoring workgroups: the pooled keys of a row group in chunks of
    // kPfChunk, spans of whole chunks (at most kPfMaxSpanChunks) sized for
    // about kPfScoreWorkgroups workgroups over the launch
    const int chunks = ceil_div(pl.max_nc > 0 ? pl.max_nc : 1, kPfChunk);
    const long long row_sets = (long long)F.npairs * F.row_groups;
    const long long want = row_sets > 0 ? (kPfScoreWorkgroups + row_sets - 1) / row_sets : 1;
    const int spans = (int)(want < chunks ? want : chunks);
    int per_span = ceil_div(chunks, spans > 0 ? spans : 1);
    per_span = per_span < kPfMaxSpanChunks ? per_span : kPfMaxSpanChunks;
    F.span = kPfChunk * per_span;
    F.key_splits = ceil_div(chunks, per_span);
    F.attn_groups = ceil_div(4 * pl.G, 8);
    const size_t np = (size_t)F.npairs;
    size_t off = 0;
    F.off_part = off;   off += align256(np * F.rows * (size_t)F.key_splits * sizeof(float2));
    F.off_colsum = off; off += align256(np * F.row_groups * (size_t)F.key_splits * F.span * sizeof(float));
    F.off_rlse = off;   off += align256(np * F.rows * sizeof(float));
    F.bytes = off > 256 ? off : 256;
    *pf = F;
}

Workspace carve(const Plan& pl, void* ws)
{
    char* base = static_cast<char*>(ws);
    Workspace w;
    w.cml = reinterpret_cast<float2*>(base + pl.off_cml);
    w.spill = reinterpret_cast<float*>(base + pl.off_spill);
    w.bpart = reinterpret_cast<float*>(base + pl.off_bpart);
    w.po = reinterpret_cast<float*>(base + pl.off_po);
    w.pml = reinterpret_cast<float2*>(base + pl.off_pml);
    return w;
}

}  // namespace nosa

using namespace nosa;

namespace {

nosa_status hip_status(hipError_t e) { return e == hipSuccess ? NOSA_OK : NOSA_ERR_HIP; }

// Arguments of the front end; fills the plan of the decode batch.
nosa_status front_check(const nosa_params* p, const nosa_front_params* f, const nosa_paged_kv* kv,
                        const nosa_bf16* x, const nosa_bf16* w, const int32_t* cu_k, int batch,
                        int max_seqlen_k, const nosa_bf16* q_out, Plan* pl)
{
    nosa_status st = check_params(p);
    if (st != NOSA_OK) return st;
    if (!f) return NOSA_ERR_NULL;
    if (f->hidden <= 0 || f->hidden % 256 != 0) return NOSA_ERR_INVALID;
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen_k, false);
    if (st != NOSA_OK) return st;
    if (!x || !w || !cu_k || !q_out) return NOSA_ERR_NULL;
    if (batch == 0) return NOSA_OK;
    return make_plan(p, batch, max_seqlen_k, pl);
}

float front_theta(const nosa_front_params* f) { return f->rope_theta > 0.f ? f->rope_theta : 10000.f; }

// Block cache of the offloaded KV: at least the query-aware share of the
// budget (every pick needs a slot), at most one slot per thread of a
// workgroup.  The window must hold a block, so that every pick is a complete
// block that no later step changes.
nosa_status check_cache(const Plan& pl, int cache_blocks)
{
    if (cache_blocks < pl.topk || cache_blocks <= 0) return NOSA_ERR_INVALID;
    if (cache_blocks > kMaxCacheSlots || pl.wblocks < 1) return NOSA_ERR_UNSUPPORTED;
    return NOSA_OK;
}

size_t offload_bytes(const Plan& pl, int cache_blocks)
{
    return pl.bytes + align256(2 * (size_t)pl.B * pl.Hkv * cache_blocks * sizeof(int32_t));
}

// The address at which the device reads pinned host memory p, or null when p
// is not memory the device can read.
const nosa_bf16* device_view(const nosa_bf16* p)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of the query
        return nullptr;
    }
    if (at.type != hipMemoryTypeHost || !at.devicePointer) return nullptr;
    const char* dev = static_cast<const char*>(at.devicePointer);
    if (at.hostPointer)
        dev += reinterpret_cast<const char*>(p) - static_cast<const char*>(at.hostPointer);
    return reinterpret_cast<const nosa_bf16*>(dev);
}

// Workspace of the whole-prompt prefill: the prefill scratch of one chunk,
// then the chunk's bookkeeping, importance and selection.
struct PromptLayout {
    int C = 0, mq = 0;  // chunk (queries), query blocks per chunk
    size_t off_cuk = 0, off_cuq = 0, off_valid = 0, off_qbase = 0, off_scores = 0, off_sel = 0,
           off_cnt = 0, bytes = 0;
};

PromptLayout prompt_layout(const Plan& pl, const PfPlan& pf, int B, int C)
{
    PromptLayout Y;
    Y.C = C;
    Y.mq = C / kBlock;
    const size_t b = (size_t)B, qb = b * Y.mq * pl.Hkv;
    size_t off = pf.bytes;
    Y.off_cuk = off;    off += align256((b + 1) * sizeof(int32_t));
    Y.off_cuq = off;    off += align256((b + 1) * sizeof(int32_t));
    Y.off_valid = off;  off += align256(b * sizeof(int32_t));
    Y.off_qbase = off;  off += align256(b * sizeof(int32_t));
    Y.off_scores = off; off += align256(qb * (size_t)pl.max_nb * sizeof(float));
    Y.off_sel = off;    off += align256(qb * (size_t)pl.max_sel * sizeof(int32_t));
    Y.off_cnt = off;    off += align256(qb * sizeof(int32_t));
    Y.bytes = off;
    return Y;
}

// Chunk length actually used: the requested one, capped by the longest
// prompt rounded up to whole blocks.
nosa_status prompt_plan(const nosa_params* p, int batch, int max_seqlen, int chunk, Plan* pl,
                        PfPlan* pf, PromptLayout* Y)
{
    nosa_status st = check_params(p);
    if (st != NOSA_OK) return st;
    if (chunk <= 0 || chunk % kBlock != 0) return NOSA_ERR_INVALID;
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen);
    if (st != NOSA_OK) return st;
    st = make_plan(p, batch, max_seqlen, pl);
    if (st != NOSA_OK) return st;
    const int cap = ceil_div(max_seqlen > 0 ? max_seqlen : 1, kBlock) * kBlock;
    const int C = chunk < cap ? chunk : cap;
    make_pf_plan(*pl, C, pf);
    *Y = prompt_layout(*pl, *pf, batch, C);
    return NOSA_OK;
}

// Query-side arguments: decode (cu_seqlens_q NULL, one query per sequence)
// or a chunk per sequence (cu_seqlens_q given, at most max_seqlen_q queries).
nosa_status check_queries(const int32_t* cu_seqlens_q, int max_seqlen_q)
{
    if (cu_seqlens_q == nullptr && max_seqlen_q > 1) return NOSA_ERR_INVALID;
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
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    PfPlan pf;
    make_pf_plan(pl, max_seqlen_q, &pf);
    *bytes = pl.bytes > pf.bytes ? pl.bytes : pf.bytes;
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
    // an incremental build pools an unknown share of each sequence: a bounded
    // grid whose waves stride over whatever is left
    const int pages = kc_valid_len && pl.max_nb > 256 ? 256 : pl.max_nb;
    return hip_status(launch_kc_build(pl, *kv, cu_seqlens_k, kc_valid_len, pages, as_stream(stream)));
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
    if (cu_seqlens_q) {
        PfPlan pf;
        make_pf_plan(pl, max_seqlen_q, &pf);
        if (!workspace || workspace_bytes < pf.bytes) return NOSA_ERR_WORKSPACE;
        return hip_status(launch_pf_scores(pl, pf, *kv, q, cu_seqlens_q, cu_seqlens_k, workspace,
                                           block_scores, as_stream(stream)));
    }
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    return hip_status(launch_scores_only(pl, *kv, q, cu_seqlens_k, carve(pl, workspace),
                                         block_scores, as_stream(stream)));
}

nosa_status nosa_check_inputs(const nosa_params* params, const nosa_paged_kv* kv,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t* flags, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, max_seqlen_q, max_seqlen_k);
    if (st != NOSA_OK) return st;
    if (!kv || !kv->block_table || !cu_seqlens_k || !flags) return NOSA_ERR_NULL;
    if (kv->max_blocks_per_seq <= 0 || kv->num_pages <= 0) return NOSA_ERR_INVALID;
    if ((long long)kv->max_blocks_per_seq * kBlock < (long long)max_seqlen_k) return NOSA_ERR_INVALID;
    st = check_queries(cu_seqlens_q, max_seqlen_q);
    if (st != NOSA_OK) return st;
    return hip_status(launch_check_inputs(cu_seqlens_k, cu_seqlens_q, kv->block_table,
                                          kv->max_blocks_per_seq, kv->num_pages, max_seqlen_k,
                                          max_seqlen_q, batch, flags, as_stream(stream)));
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
    return hip_status(launch_select(pl, cu_seqlens_k, cu_seqlens_q, max_seqlen_q, block_scores,
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
    if (cu_seqlens_q) {  // chunk attention: no workspace used
        PfPlan pf;
        make_pf_plan(pl, max_seqlen_q, &pf);
        return hip_status(launch_pf_attend(pl, pf, *kv, q, cu_seqlens_q, cu_seqlens_k, sel_idx,
                                           sel_count, out, lse, as_stream(stream)));
    }
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    return hip_status(launch_attend(pl, *kv, q, cu_seqlens_k, sel_idx, sel_count,
                                    carve(pl, workspace), out, lse, as_stream(stream)));
}

nosa_status nosa_prefill_sparse_workspace_size(const nosa_params* params, int32_t batch, int32_t max_seqlen,
                                        int32_t chunk, size_t* bytes)
{
    if (!params || !bytes) return NOSA_ERR_NULL;
    Plan pl;
    PfPlan pf;
    PromptLayout Y;
    const nosa_status st = prompt_plan(params, batch, max_seqlen, chunk, &pl, &pf, &Y);
    if (st != NOSA_OK) return st;
    *bytes = Y.bytes;
    return NOSA_OK;
}

nosa_status nosa_prefill_sparse(const nosa_params* params, const nosa_paged_kv* kv, const nosa_bf16* q,
                                const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                int32_t chunk, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    Plan pl;
    PfPlan pf;
    PromptLayout Y;
    nosa_status st = prompt_plan(params, batch, max_seqlen, chunk, &pl, &pf, &Y);
    if (st != NOSA_OK) return st;
    st = check_kv(kv, max_seqlen, false);
    if (st != NOSA_OK) return st;
    if (!q || !cu_seqlens || !out) return NOSA_ERR_NULL;
    if (batch == 0) return NOSA_OK;
    if (!workspace || workspace_bytes < Y.bytes) return NOSA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    int32_t* cu_k_c = reinterpret_cast<int32_t*>(ws + Y.off_cuk);
    int32_t* cu_q_c = reinterpret_cast<int32_t*>(ws + Y.off_cuq);
    int32_t* valid_c = reinterpret_cast<int32_t*>(ws + Y.off_valid);
    int32_t* qbase_c = reinterpret_cast<int32_t*>(ws + Y.off_qbase);
    float* scores = reinterpret_cast<float*>(ws + Y.off_scores);
    int32_t* sel = reinterpret_cast<int32_t*>(ws + Y.off_sel);
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + Y.off_cnt);
    const hipStream_t sm = as_stream(stream);
    const int C = Y.C, nch = ceil_div(max_seqlen, C);
    const int gx = C / kBlock + 1;  // pages holding the first token of a key one chunk completes
    for (int c = 0; c < nch; ++c) {
        hipError_t e = launch_chunk_setup(cu_seqlens, batch, pl.Lmax, c, C, cu_k_c, cu_q_c, valid_c,
                                          qbase_c, sm);
        if (e == hipSuccess) e = launch_kc_build(pl, *kv, cu_k_c, valid_c, gx, sm);
        if (e == hipSuccess)
            e = launch_pf_scores(pl, pf, *kv, q, cu_q_c, cu_k_c, workspace, scores, sm, qbase_c);
        if (e == hipSuccess) e = launch_select(pl, cu_k_c, cu_q_c, C, scores, sel, cnt, sm);
        if (e == hipSuccess)
            e = launch_pf_attend(pl, pf, *kv, q, cu_q_c, cu_k_c, sel, cnt, out, lse, sm, qbase_c);
        if (e != hipSuccess) return NOSA_ERR_HIP;
    }
    return NOSA_OK;
}

nosa_status nosa_offload_workspace_size(const nosa_params* params, int32_t batch,
                                        int32_t max_seqlen_k, int32_t cache_blocks, size_t* bytes)
{
    if (!params || !bytes) return NOSA_ERR_NULL;
    nosa_status st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k);
    if (st != NOSA_OK) return st;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    st = check_cache(pl, cache_blocks);
    if (st != NOSA_OK) return st;
    *bytes = offload_bytes(pl, cache_blocks);
    return NOSA_OK;
}

nosa_status nosa_offload_decode_step(const nosa_params* params, const nosa_offload_kv* kv,
                                     const nosa_bf16* q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t max_seqlen_k, float* out, float* lse,
                                     int32_t* sel_idx, int32_t* sel_count, int32_t* fetch_count,
                                     void* workspace, size_t workspace_bytes, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    st = check_sizes(batch, batch > 0 ? 1 : 0, max_seqlen_k);
    if (st != NOSA_OK) return st;
    if (!kv) return NOSA_ERR_NULL;
    if (!kv->k_host || !kv->v_host || !kv->kc_pool || !kv->block_table || !kv->k_recent ||
        !kv->v_recent || !kv->cache_k || !kv->cache_v || !kv->cache_map || !kv->cache_used)
        return NOSA_ERR_NULL;
    if (kv->max_blocks_per_seq <= 0 || kv->num_pages <= 0) return NOSA_ERR_INVALID;
    if ((long long)kv->max_blocks_per_seq * kBlock < (long long)max_seqlen_k) return NOSA_ERR_INVALID;
    if (!q || !cu_seqlens_k || !out) return NOSA_ERR_NULL;
    if ((sel_idx == nullptr) != (sel_count == nullptr)) return NOSA_ERR_NULL;
    if (batch == 0) return NOSA_OK;
    Plan pl;
    st = make_plan(params, batch, max_seqlen_k, &pl);
    if (st != NOSA_OK) return st;
    st = check_cache(pl, kv->cache_blocks);
    if (st != NOSA_OK) return st;
    const int need = pl.wblocks > 2 ? pl.wblocks : 2;
    if (kv->recent_blocks < need) return NOSA_ERR_INVALID;
    if (!workspace || workspace_bytes < offload_bytes(pl, kv->cache_blocks)) return NOSA_ERR_WORKSPACE;
    Offload off;
    off.k_host = device_view(kv->k_host);
    off.v_host = device_view(kv->v_host);
    if (!off.k_host || !off.v_host) return NOSA_ERR_INVALID;
    off.k_recent = kv->k_recent;
    off.v_recent = kv->v_recent;
    off.recent = kv->recent_blocks;
    off.cache_k = kv->cache_k;
    off.cache_v = kv->cache_v;
    off.cache_map = kv->cache_map;
    off.cache_used = kv->cache_used;
    off.cap = kv->cache_blocks;
    off.map_next = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + pl.bytes);
    off.used_next = off.map_next + (size_t)pl.B * pl.Hkv * kv->cache_blocks;
    off.fetch_out = fetch_count;
    nosa_paged_kv pk;
    pk.k_pool = off.k_host;
    pk.v_pool = off.v_host;
    pk.kc_pool = kv->kc_pool;
    pk.block_table = kv->block_table;
    pk.max_blocks_per_seq = kv->max_blocks_per_seq;
    pk.num_pages = kv->num_pages;
    return hip_status(launch_decode(pl, pk, q, cu_seqlens_k, carve(pl, workspace), out, lse,
                                    sel_idx, sel_count, nullptr, as_stream(stream), &off));
}

nosa_status nosa_pack_qkv_weights(const nosa_params* params, int32_t hidden, const nosa_bf16* w,
                                  nosa_bf16* packed, void* stream)
{
    nosa_status st = check_params(params);
    if (st != NOSA_OK) return st;
    if (!w || !packed) return NOSA_ERR_NULL;
    if (hidden <= 0 || hidden % 256 != 0) return NOSA_ERR_INVALID;
    return hip_status(launch_pack_qkv(params->num_q_heads, params->num_kv_heads, hidden, w, packed,
                                      as_stream(stream)));
}

nosa_status nosa_qkv_rope_append(const nosa_params* params, const nosa_front_params* front,
                                 const nosa_paged_kv* kv, const nosa_bf16* x,
                                 const nosa_bf16* w_packed, const int32_t* cu_seqlens_k,
                                 int32_t batch, int32_t max_seqlen_k, nosa_bf16* q_out,
                                 void* stream)
{
    Plan pl;
    nosa_status st = front_check(params, front, kv, x, w_packed, cu_seqlens_k, batch, max_seqlen_k,
                                 q_out, &pl);
    if (st != NOSA_OK || batch == 0) return st;
    return hip_status(launch_front(pl, *kv, x, w_packed, front->hidden, front_theta(front),
                                   front->inv_freq, cu_seqlens_k, q_out, as_stream(stream)));
}

nosa_status nosa_layer_decode_step(const nosa_params* params, const nosa_front_params* front,
                                   const nosa_paged_kv* kv, const nosa_bf16* x,
                                   const nosa_bf16* w_packed, const int32_t* cu_seqlens_k,
                                   int32_t batch, int32_t max_seqlen_k, nosa_bf16* q_out,
                                   float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    Plan pl;
    nosa_status st = front_check(params, front, kv, x, w_packed, cu_seqlens_k, batch, max_seqlen_k,
                                 q_out, &pl);
    if (st != NOSA_OK) return st;
    if (!out) return NOSA_ERR_NULL;
    if ((sel_idx == nullptr) != (sel_count == nullptr)) return NOSA_ERR_NULL;
    if (batch == 0) return NOSA_OK;
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    const hipStream_t sm = as_stream(stream);
    hipError_t e = launch_front(pl, *kv, x, w_packed, front->hidden, front_theta(front),
                                front->inv_freq, cu_seqlens_k, q_out, sm);
    if (e != hipSuccess) return NOSA_ERR_HIP;
    return hip_status(launch_decode(pl, *kv, q_out, cu_seqlens_k, carve(pl, workspace), out, lse,
                                    sel_idx, sel_count, nullptr, sm));
}

// Arguments of a decode step (all but the workspace); fills its plan.
static nosa_status decode_check(const nosa_params* params, const nosa_paged_kv* kv,
                                const nosa_bf16* q, const int32_t* cu_seqlens_k, int32_t batch,
                                int32_t max_seqlen_k, const float* out, const int32_t* sel_idx,
                                const int32_t* sel_count, Plan* pl)
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
    return make_plan(params, batch, max_seqlen_k, pl);
}

nosa_status nosa_decode_step(const nosa_params* params, const nosa_paged_kv* kv,
                             const nosa_bf16* q, const int32_t* cu_seqlens_k, int32_t batch,
                             int32_t max_seqlen_k, float* out, float* lse, int32_t* sel_idx,
                             int32_t* sel_count, float* block_scores, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    Plan pl;
    const nosa_status st = decode_check(params, kv, q, cu_seqlens_k, batch, max_seqlen_k, out,
                                        sel_idx, sel_count, &pl);
    if (st != NOSA_OK || batch == 0) return st;
    if (!workspace || workspace_bytes < pl.bytes) return NOSA_ERR_WORKSPACE;
    return hip_status(launch_decode(pl, *kv, q, cu_seqlens_k, carve(pl, workspace), out, lse,
                                    sel_idx, sel_count, block_scores, as_stream(stream)));
}

nosa_status nosa_decode_step_static(const nosa_params* params, const nosa_paged_kv* kv,
                                    const nosa_bf16* q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_k, float* out, float* lse,
                                    int32_t* sel_idx, int32_t* sel_count, float* block_scores,
                                    void* stream)
{
    Plan pl;
    const nosa_status st = decode_check(params, kv, q, cu_seqlens_k, batch, max_seqlen_k, out,
                                        sel_idx, sel_count, &pl);
    if (st != NOSA_OK || batch == 0) return st;
    if (pl.bytes > kStaticScratchBytes) return NOSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (static_scratch(&ws) != hipSuccess) return NOSA_ERR_HIP;
    return hip_status(launch_decode(pl, *kv, q, cu_seqlens_k, carve(pl, ws), out, lse, sel_idx,
                                    sel_count, block_scores, as_stream(stream)));
}

}  // extern "C"
