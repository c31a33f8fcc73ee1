/*
 * nosa.h -- C ABI of the MI355X (gfx950) NOSA sparse-attention library.
 *
 * The operation is the decode step of NOSA ("Native and Offloadable Sparse
 * Attention") as the pages on it describe it:
 *   - keys are mean-pooled into compressed keys (kernel 32, stride 16)
 *     [page "NOSA-1B 性能基准全解析", section 三.3 两阶段注意力 and the config table
 *     of section 四; page "从论文到代码", section 2: pooling of k with cu_seqlens];
 *   - each query head scores the compressed keys (compressed attention), the
 *     scores of the heads sharing a KV head are summed and mean-pooled into one
 *     importance per 64-token block (CIS score pooling)
 *     [page "NOSA-1B 模型家族全景", core principle and the cis_pooling.py note];
 *   - the top-k blocks plus the forced local window (1024 tokens = 16 blocks)
 *     are kept [page "NOSA-1B 性能基准全解析", section 三.2 显式局部性约束];
 *   - exact softmax attention runs over the kept blocks only [same page, 三.3].
 *
 * Conventions shared by every entry point
 *   - bf16 values are passed as their 16-bit patterns (nosa_bf16).
 *   - Every pointer except the two struct pointers and `workspace_bytes`-style
 *     host outputs is DEVICE memory owned by the caller; the library never
 *     allocates, frees or keeps a pointer after a call returns.  Buffers must
 *     stay alive until the work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work; none synchronises the host.
 *   - `max_seqlen_*` are host-side upper bounds of the device lengths, used to
 *     size grids without a device-to-host copy.  A device length above its
 *     bound, a non-monotone cu_seqlens or a block_table entry outside
 *     [0, num_pages) for a block the sequence holds is a contract violation
 *     that the other entry points do not detect (nosa_check_inputs does,
 *     on the device, when asked).  Entries past a sequence's last
 *     block may hold anything (the row is read ahead of the length, and such
 *     entries are clamped into the pool and never used).
 *   - Host-checkable arguments are validated before anything is enqueued: a
 *     NULL required pointer gives NOSA_ERR_NULL, inconsistent sizes
 *     NOSA_ERR_INVALID, a shape the library has no kernel for
 *     NOSA_ERR_UNSUPPORTED, a short workspace NOSA_ERR_WORKSPACE, and a failed
 *     HIP launch NOSA_ERR_HIP.  Nothing aborts.
 *   - Global state: a per-device cache of two device attributes (LDS per
 *     workgroup, compute units), read once and thread-safe, and the static
 *     scratch array of nosa_decode_step_static.  Calls of the other entry
 *     points on different streams may run concurrently as long as they do not
 *     share output or workspace buffers.
 *   - Workspace: device scratch memory of nosa_workspace_size() bytes, with
 *     no initial contents required and none kept between calls; reused
 *     across calls without clearing.  Calls sharing a workspace must be
 *     ordered (same stream): overlapping calls on one workspace race.
 *   - Queries: cu_seqlens_q NULL is decode (one query per sequence, row s of
 *     q, at position L_s - 1).  Otherwise cu_seqlens_q (device [batch+1])
 *     packs Lq_s <= L_s queries per sequence, the last Lq_s positions
 *     L_s - Lq_s .. L_s - 1 of its context (a prefill chunk), and the chunk
 *     is cut into query blocks of 64 consecutive queries from its start;
 *     query block r ends at position p_r = L_s - Lq_s + min(64r + 64, Lq_s) - 1
 *     and sees the blocks nb_r = p_r / block_size + 1 that hold tokens
 *     <= p_r.  [Page "NOSA技术架构解析", sections 1.1 and 1.3: besides full
 *     prefill with sparse decode, a mode runs prefill sparse as well; the
 *     64-query block is this library's unit for it, the decode step being
 *     the one-query case.]  max_qblk = ceil(max_seqlen_q / 64) (1 for
 *     decode).
 *
 * Supported shapes on the GPU: head_dim 128, block_size 64, kernel 32,
 * stride 16, window a multiple of 64 of at most 8192 tokens,
 * num_q_heads / num_kv_heads in [1, 16],
 * at most 8192 blocks (512K tokens) per sequence.
 *
 * Terms: L_s = cu_seqlens_k[s+1] - cu_seqlens_k[s] is the KV length of
 * sequence s, including the token being decoded.  n_c(L) = (L-32)/16 + 1 for
 * L >= 32 (else 0) compressed keys; key j pools tokens [16j, 16j+32).
 * nb(L) = ceil(L/64) blocks.  G = num_q_heads / num_kv_heads.
 */
#ifndef NOSA_H
#define NOSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NOSA_ABI_VERSION 5

typedef uint16_t nosa_bf16; /* bf16 bit pattern */

typedef enum nosa_status {
    NOSA_OK = 0,
    NOSA_ERR_NULL = 1,        /* a required pointer is NULL                 */
    NOSA_ERR_INVALID = 2,     /* sizes or parameters are inconsistent       */
    NOSA_ERR_UNSUPPORTED = 3, /* valid, but no GPU kernel for this shape    */
    NOSA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required    */
    NOSA_ERR_HIP = 5          /* a HIP call or kernel launch failed         */
} nosa_status;

/* Method parameters [page "NOSA-1B 性能基准全解析", config table of section 四:
 * TopK 64, window 1024, block 64, kernel 32 / stride 16; 16 query / 2 KV heads]. */
typedef struct nosa_params {
    int32_t num_q_heads;  /* Hq                                                   */
    int32_t num_kv_heads; /* Hkv; must divide Hq                                  */
    int32_t head_dim;     /* d (GPU: 128)                                         */
    int32_t block_size;   /* tokens per KV block = per page (GPU: 64)             */
    int32_t kernel;       /* pooling window in tokens (GPU: 32)                   */
    int32_t stride;       /* pooling stride in tokens (GPU: 16)                   */
    int32_t topk;         /* blocks chosen besides the window, >= 0               */
    int32_t window;       /* local window in tokens, a multiple of block_size     */
    float scale;          /* logit scale; <= 0 selects 1/sqrt(head_dim)          */
    float locality;       /* gamma_0 in [0, 1]; 0 = plain top-k (see below)      */
} nosa_params;

/* Locality constraint [page "NOSA技术架构解析", section 1.2: a minimum locality
 * gamma_0, the share of local KV blocks that must be kept, and a query-aware
 * share kq/k of the budget; every setting the page prints (sections 1.2 and
 * 4.1) has kq/k = 1 - gamma_0].  Of the topk budget, k_loc =
 * floor(locality * topk + 0.5) blocks are the candidates nearest the window
 * (kept whatever the query), the other topk - k_loc the best of the earlier
 * candidates by importance.  Equivalently: window + k_loc * block_size tokens
 * are forced and topk - k_loc blocks are selected, so window / block_size +
 * k_loc must stay within the supported window (128 blocks). */

/* Paged KV cache [page "NOSA技术架构解析", section 2.1: a PagedAttention-style
 * memory pool].  One page holds one block of block_size tokens for every KV
 * head.  Logical block b of sequence s lives in page block_table[s][b].
 *   k_pool  [num_pages][Hkv][block_size * d]
 *   v_pool  [num_pages][Hkv][block_size * d]
 *   kc_pool [num_pages][Hkv][block_size / stride * d]: compressed key j of
 *           sequence s is slot j % (block_size/stride) of page
 *           block_table[s][j / (block_size/stride)], so it needs no table of
 *           its own.
 *   block_table [batch][max_blocks_per_seq] int32.
 * Inside a page (of one KV head) elements are stored in matrix-core operand
 * order, in runs of 8 consecutive elements (16 bytes); with token x,
 * channel c, slot j and e = the element's index inside its run:
 *   k : offset (((4t + st) * 4 + kq) * 16 + m) * 8 + e holds token
 *       x = 32(t/2) + 8(m/4) + 4(t%2) + m%4, channel c = 32 st + 8 kq + e;
 *   v : offset (((8u + nt) * 4 + kq) * 16 + r) * 8 + e holds token
 *       x = 32u + 8kq + e, channel c = 16 nt + r;
 *   kc: offset (c8 * 4 + j) * 8 + e holds channel 8 c8 + e of slot j.
 * with t, st, kq in [0, 4), u in [0, 2), nt in [0, 8), m, r, c8 in [0, 16)
 * and j in [0, block_size / stride).  Each 1 KB run
 * of 64 x 16 bytes is what one wave's 16-byte-per-lane load fetches for one
 * matrix-core step.  The library writes kc_pool; the caller writes K and V. */
typedef struct nosa_paged_kv {
    const nosa_bf16* k_pool;
    const nosa_bf16* v_pool;
    nosa_bf16* kc_pool;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    int32_t num_pages;
} nosa_paged_kv;

/* Offloaded KV cache [page "NOSA-1B 性能基准全解析", section 三.1: most of the
 * KV cache lives outside GPU memory, which holds only what is in use; page
 * "NOSA技术架构解析", section 2.2: the host side is read directly, without
 * staging copies, and only blocks that changed are transferred].  K and V
 * pages of every block are in host memory; device memory holds the pooled
 * keys of every block, the pages of the recent blocks, and a cache of the
 * blocks picked by recent steps.
 *   k_host, v_host  pinned host memory (hipHostMalloc, or a pinned torch
 *                   tensor), [num_pages][Hkv][block_size * d] in the page
 *                   layout above; page block_table[s][b] holds block b of
 *                   sequence s.  Read by the GPU directly.
 *   kc_pool, block_table, max_blocks_per_seq, num_pages: as in nosa_paged_kv
 *                   (device).
 *   k_recent, v_recent  device [batch][recent_blocks][Hkv][block_size * d]:
 *                   block b of sequence s in slot b % recent_blocks.  Must
 *                   hold the last max(2, W) blocks of each sequence, W =
 *                   window / block_size + the locality share (the forced
 *                   blocks, and the tokens of the key the step appends), the
 *                   current token included; recent_blocks >= max(2, W).
 *   cache_k, cache_v  device [batch][Hkv][cache_blocks][block_size * d]: the
 *                   block cache of each (sequence, KV head), written by the
 *                   library.
 *   cache_map       device int32 [batch][Hkv][cache_blocks]: the block held
 *                   by each cache slot, -1 for none.  The caller sets every
 *                   entry to -1 before a sequence's first step (and whenever
 *                   the sequence in that batch row changes); the library keeps
 *                   it up to date afterwards.  cache_blocks must be at least
 *                   the query-aware share of topk (topk minus the locality
 *                   share) and at most 256.
 *   cache_used      device int32 [batch][Hkv][cache_blocks]: the sequence
 *                   length at the step that last picked each slot's block
 *                   (written by the library; no initial contents needed).
 *                   A miss takes the free slot (block not picked) that was
 *                   picked least recently, empty slots first.
 * Blocks before the recent ones must not change while they may be cached. */
typedef struct nosa_offload_kv {
    const nosa_bf16* k_host;
    const nosa_bf16* v_host;
    nosa_bf16* kc_pool;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    int32_t num_pages;
    const nosa_bf16* k_recent;
    const nosa_bf16* v_recent;
    int32_t recent_blocks;
    int32_t cache_blocks;
    nosa_bf16* cache_k;
    nosa_bf16* cache_v;
    int32_t* cache_map;
    int32_t* cache_used;
} nosa_offload_kv;

/* ABI version of the loaded library (NOSA_ABI_VERSION at its build). */
int nosa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* nosa_status_string(nosa_status status);

/* Workspace bytes needed by nosa_block_scores, nosa_sparse_attend and
 * nosa_decode_step for any batch of at most `batch` sequences whose lengths
 * are bounded by max_seqlen_q (queries; 1 for decode) and max_seqlen_k.
 * Host only; enqueues nothing.  Errors: NOSA_ERR_NULL (params or bytes NULL),
 * NOSA_ERR_INVALID, NOSA_ERR_UNSUPPORTED. */
nosa_status nosa_workspace_size(const nosa_params* params, int32_t batch, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, size_t* bytes);

/* Compressed-key builder [page "NOSA-1B 性能基准全解析", sections 三.3-三.4: mean
 * pooling with kernel 32 / stride 16].  For every sequence s and KV head,
 * writes keys j in [n_c(kc_valid_len[s]), n_c(L_s)) into kc_pool: key j is
 * the bf16 round-to-nearest-even of the exact mean of K over tokens
 * [16j, 16j+32).  The sums are formed in fp64, which is exact (so the order
 * of the additions does not matter) while the window's nonzero values of a
 * channel span at most 2^40 in magnitude; wider spans are rounded in fp64
 * first.  kc_valid_len (device, [batch] int32) is the number
 * of tokens whose keys are already pooled; NULL rebuilds every key.  Keys
 * outside that range are not touched.  cu_seqlens_k: device [batch+1]. */
nosa_status nosa_compress_keys(const nosa_params* params, const nosa_paged_kv* kv,
                               const int32_t* cu_seqlens_k, const int32_t* kc_valid_len,
                               int32_t batch, int32_t max_seqlen_k, void* stream);

/* Block importance [pages "NOSA-1B 性能基准全解析" 三.3 and "NOSA-1B 模型家族全景"
 * core principle].  For each row (sequence s, query block r, KV head g), with
 * the query block's queries i (one for decode) and the G heads h of g:
 *   z_ih[j] = scale * q_ih . Kc_j for every key j < n_c(p_r + 1);
 *   sigma[j] = sum_i sum_h softmax_ih(z_ih)[j];
 *   block_scores[s][r][g][b] = mean of sigma over the keys overlapping block b
 *   (keys 4b-1 .. 4b+3 that exist), -inf if none, for b < nb_r; -inf padding
 *   up to max_nb = ceil(max_seqlen_k / block_size); rows of absent query
 *   blocks are all -inf.
 * q: device [total queries][Hq][d] bf16 (decode: [batch][Hq][d]).
 * block_scores: device fp32 [batch][max_qblk][Hkv][max_nb].  Kc must be
 * valid for L_s tokens.  Needs a `workspace` of nosa_workspace_size bytes. */
nosa_status nosa_block_scores(const nosa_params* params, const nosa_paged_kv* kv,
                              const nosa_bf16* q, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, float* block_scores, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Block selection [page "NOSA-1B 性能基准全解析", section 三.2: a 1024-token window
 * of 64-token blocks is always attended and TopK adds the 64 best blocks].
 * For each row (sequence s, query block r, KV head g) with nb = nb_r blocks:
 * the window is the last min(nb, window/block_size) blocks; among the
 * earlier blocks the min(topk, count) with the largest block_scores are
 * added, ties going to the lower block index.  sel_idx receives the kept
 * block ids in ascending order, padded with -1 to
 * max_sel = topk + window/block_size; sel_count the number kept
 * (= min(nb, topk + window/block_size); 0 for absent query blocks).
 * block_scores: device fp32 [batch][max_qblk][Hkv][max_nb] as produced by
 * nosa_block_scores.  sel_idx: device int32 [batch][max_qblk][Hkv][max_sel];
 * sel_count: device int32 [batch][max_qblk][Hkv]. */
nosa_status nosa_select_blocks(const nosa_params* params, const float* block_scores,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t* sel_idx, int32_t* sel_count, void* stream);

/* Exact attention over the kept blocks [page "NOSA-1B 性能基准全解析", 三.2-三.3].
 * For query i of query block r of sequence s (at position p) and query head
 * h (KV head g = h / G): softmax over the tokens t <= p of the blocks listed
 * in sel_idx[s][r][g][0 .. sel_count) of scale * q_ih . K[t], applied to V
 * (decode: p = L_s - 1, r = 0).  out: device fp32 [total queries][Hq][d];
 * lse: device fp32 [total queries][Hq] (natural log of the softmax
 * denominator, -inf for a query that sees no token) or NULL.  Block ids must
 * be distinct and < nb_r.  Needs a `workspace` (see above) in decode; with
 * cu_seqlens_q none is used (workspace may be NULL). */
nosa_status nosa_sparse_attend(const nosa_params* params, const nosa_paged_kv* kv,
                               const nosa_bf16* q, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const int32_t* sel_idx,
                               const int32_t* sel_count, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* One whole decode step, all of the above in order:
 *   1. append the compressed keys completed by the current token (keys
 *      [n_c(L_s - 1), n_c(L_s)); Kc must already hold every key of the first
 *      L_s - 1 tokens);
 *   2. score, pool, select (as nosa_block_scores + nosa_select_blocks);
 *   3. attend (as nosa_sparse_attend).
 * q: device [batch][Hq][d] bf16, the query of each sequence at position
 * L_s - 1 (its K/V must already be in the pages).  out / lse as in
 * nosa_sparse_attend (lse may be NULL).  sel_idx / sel_count / block_scores
 * are optional outputs (NULL = not written) with the layouts above
 * (max_qblk = 1).  Needs a `workspace` (see above). */
nosa_status nosa_decode_step(const nosa_params* params, const nosa_paged_kv* kv,
                             const nosa_bf16* q, const int32_t* cu_seqlens_k, int32_t batch,
                             int32_t max_seqlen_k, float* out, float* lse, int32_t* sel_idx,
                             int32_t* sel_count, float* block_scores, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the static scratch array of nosa_decode_step_static. */
#define NOSA_STATIC_SCRATCH_BYTES (32u << 20)

/* nosa_decode_step for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture that must not allocate, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (without
 * the workspace), computation and results as nosa_decode_step, bit for bit
 * (the same kernels and launch plan); the step's partials go to a scratch
 * array the library holds in device memory, NOSA_STATIC_SCRATCH_BYTES per
 * device, from module load until the process ends.  Allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  The first call on a
 * device looks the array's device address up (once per device, thread-safe).
 * The array needs no initial contents and keeps whatever the last call left.
 * Every call on one device shares that device's array, so calls that may
 * overlap on one device (different streams, or host threads) race: order them
 * on one stream.  Errors: those of nosa_decode_step, with NOSA_ERR_WORKSPACE
 * when the step needs more than NOSA_STATIC_SCRATCH_BYTES (the size
 * nosa_workspace_size(params, batch, 1, max_seqlen_k) reports), checked on
 * the host before anything is enqueued. */
nosa_status nosa_decode_step_static(const nosa_params* params, const nosa_paged_kv* kv,
                                    const nosa_bf16* q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_k, float* out, float* lse,
                                    int32_t* sel_idx, int32_t* sel_count, float* block_scores,
                                    void* stream);

/* Workspace bytes needed by nosa_prefill_sparse for at most `batch` prompts
 * of at most max_seqlen tokens processed `chunk` queries at a time (chunk a
 * positive multiple of block_size).  Host only; enqueues nothing.  Errors as
 * nosa_workspace_size, plus NOSA_ERR_INVALID for a bad chunk. */
nosa_status nosa_prefill_sparse_workspace_size(const nosa_params* params, int32_t batch,
                                               int32_t max_seqlen, int32_t chunk, size_t* bytes);

/* Sparse prefill of whole prompts [page "NOSA技术架构解析", section 1.3: the
 * mode that is sparse from the first token on, beside the mode with a dense
 * prefill and sparse decoding].  Every query of every prompt attends as in
 * nosa_sparse_attend to the blocks selected for its query block (64 queries
 * from position 0 on) by nosa_block_scores + nosa_select_blocks, with the
 * keys of the prompt itself: the result equals those three calls with
 * cu_seqlens_q = cu_seqlens_k = cu_seqlens.  The prompt is processed in
 * chunks of `chunk` positions (the same for every sequence, a multiple of
 * block_size); chunk c pools the compressed keys its tokens complete, then
 * scores, selects and attends for its queries, so the workspace scales with
 * the chunk and not with the prompt.  The chunk does not change the
 * selection; the outputs may differ in the rounding of the attention weights
 * (bf16, relative to a running maximum), since an attention launch of few
 * workgroups splits each one's pages over two and merges the two partials.
 * K and V of every prompt token must already be in the pages; kc_pool is
 * written for every key of the prompts (as nosa_compress_keys with
 * kc_valid_len NULL).  q: device [total tokens][Hq][d] bf16 in cu_seqlens
 * order; cu_seqlens: device [batch+1], lengths <= max_seqlen.
 * out: device fp32 [total tokens][Hq][d]; lse: device fp32 [total tokens][Hq]
 * or NULL.  workspace: device, at least nosa_prefill_sparse_workspace_size
 * bytes for the same (params, batch, max_seqlen, chunk), owned by the
 * caller, contents irrelevant on entry.  Enqueued on `stream`; returns after
 * enqueueing.  Errors: NOSA_ERR_NULL, NOSA_ERR_INVALID (bad sizes, chunk or
 * table), NOSA_ERR_WORKSPACE, NOSA_ERR_UNSUPPORTED, NOSA_ERR_HIP. */
nosa_status nosa_prefill_sparse(const nosa_params* params, const nosa_paged_kv* kv,
                                const nosa_bf16* q, const int32_t* cu_seqlens, int32_t batch,
                                int32_t max_seqlen, int32_t chunk, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by nosa_offload_decode_step for at most `batch`
 * sequences of at most max_seqlen_k tokens and `cache_blocks` cache slots
 * per (sequence, KV head).  Host only.  Errors as nosa_workspace_size, plus
 * NOSA_ERR_INVALID / NOSA_ERR_UNSUPPORTED for a cache size outside
 * [topk - locality share, 256]. */
nosa_status nosa_offload_workspace_size(const nosa_params* params, int32_t batch,
                                        int32_t max_seqlen_k, int32_t cache_blocks, size_t* bytes);

/* One decode step over an offloaded KV cache (see nosa_offload_kv): the same
 * computation and results as nosa_decode_step over pools holding the same
 * pages, bit for bit.  The window (and locality) pages are read from the
 * recent ring, the top-k picks from the block cache; picks not in the cache
 * are read from host memory by the attention itself and written into cache
 * slots whose blocks were not picked, so a step transfers only the blocks its
 * selection adds.  fetch_count (optional, device int32 [batch][Hkv]) receives
 * the number of blocks read from host memory per (sequence, KV head).  Other
 * arguments and outputs as nosa_decode_step.  Errors: those of
 * nosa_decode_step; NOSA_ERR_INVALID when a host pool is not pinned memory the
 * device can read, or the ring or cache is too small; NOSA_ERR_UNSUPPORTED for
 * a window of no block or a cache of more than 256 slots. */
nosa_status nosa_offload_decode_step(const nosa_params* params, const nosa_offload_kv* kv,
                                     const nosa_bf16* q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t max_seqlen_k, float* out, float* lse,
                                     int32_t* sel_idx, int32_t* sel_count, int32_t* fetch_count,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Attention front end [page "NOSA技术架构解析", section 2.1: the QKV projection,
 * the rotary position encoding and the importance scoring are fused to cut
 * the launches of a decode step].  For the current token of each sequence
 * (position p = L_s - 1) with hidden state x[s][0 .. hidden):
 *   y = W x over the (Hq + 2 Hkv) * head_dim rows of W: the Hq query heads,
 *       then the Hkv key heads, then the Hkv value heads;
 *   q and k heads: channel i and channel i + head_dim/2 (i < head_dim/2)
 *       are turned as one pair by the angle p * inv_freq[i]:
 *       (y_i, y_(i+d/2)) -> (y_i cos - y_(i+d/2) sin, y_(i+d/2) cos + y_i sin);
 *   every value rounded to bf16 (fp32 accumulation, angles in fp64).
 * The queries go to q_out; k and v are written into the token's slot of page
 * block_table[s][p / block_size] of k_pool / v_pool (so the const of those
 * two members is cast away: this call writes them). */
typedef struct nosa_front_params {
    int32_t hidden;         /* width of x: a positive multiple of 256            */
    float rope_theta;       /* base of the angles; <= 0 selects 10000            */
    const float* inv_freq;  /* device [head_dim / 2] angle per position of each  */
                            /* pair, or NULL for rope_theta^(-2i / head_dim)     */
} nosa_front_params;

/* Packs row-major weights w [(Hq + 2 Hkv) * head_dim][hidden] (device bf16)
 * into the order the front end reads (device, the same number of elements;
 * owned by the caller, written here).  In the packed order, 16-row tile
 * T = 8 h + j holds rows 8j .. 8j+7 and 64+8j .. 64+8j+7 of head h; for run
 * kb of 256 hidden channels and k-step t, 64 lanes of 8 elements follow each
 * other, lane 16 grp + m holding row m of the tile (rows 8j + m, then
 * 64 + 8j + m - 8) at channels 256 kb + 32 t + 8 grp .. +7:
 *   packed[(((T * hidden/256 + kb) * 8 + t) * 64 + lane) * 8 + e].
 * Done once per weight matrix; enqueued on `stream`.  Errors: NOSA_ERR_NULL,
 * NOSA_ERR_INVALID (hidden not a positive multiple of 256),
 * NOSA_ERR_UNSUPPORTED (head_dim != 128), NOSA_ERR_HIP. */
nosa_status nosa_pack_qkv_weights(const nosa_params* params, int32_t hidden, const nosa_bf16* w,
                                  nosa_bf16* packed, void* stream);

/* The front end alone (one launch): q_out device [batch][Hq][head_dim] bf16;
 * x device [batch][hidden] bf16; w_packed from nosa_pack_qkv_weights;
 * cu_seqlens_k as in nosa_decode_step, the current token's page must exist.
 * Errors: NOSA_ERR_NULL, NOSA_ERR_INVALID, NOSA_ERR_UNSUPPORTED,
 * NOSA_ERR_HIP. */
nosa_status nosa_qkv_rope_append(const nosa_params* params, const nosa_front_params* front,
                                 const nosa_paged_kv* kv, const nosa_bf16* x,
                                 const nosa_bf16* w_packed, const int32_t* cu_seqlens_k,
                                 int32_t batch, int32_t max_seqlen_k, nosa_bf16* q_out,
                                 void* stream);

/* One decode step of an attention layer from its hidden states: the front end
 * (nosa_qkv_rope_append), then nosa_decode_step on the queries it made (four
 * launches).  Arguments as in those two calls; q_out receives the queries.
 * Needs a nosa_workspace_size workspace. */
nosa_status nosa_layer_decode_step(const nosa_params* params, const nosa_front_params* front,
                                   const nosa_paged_kv* kv, const nosa_bf16* x,
                                   const nosa_bf16* w_packed, const int32_t* cu_seqlens_k,
                                   int32_t batch, int32_t max_seqlen_k, nosa_bf16* q_out,
                                   float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Checks, on the device, the inputs the other entry points take on trust (the
 * contract stated at the top of this header; no page defines it): for every
 * sequence s, in one launch of a workgroup per sequence,
 *   bit 0 (NOSA_CHECK_CU_K):  cu_seqlens_k[0] != 0 or cu_seqlens_k[s+1] <
 *                             cu_seqlens_k[s];
 *   bit 1 (NOSA_CHECK_LEN_K): L_s outside [1, max_seqlen_k];
 *   bit 2 (NOSA_CHECK_TABLE): block_table[s][b] outside [0, num_pages) for a
 *                             block b < nb(min(max(L_s, 0), max_seqlen_k));
 *   bit 3 (NOSA_CHECK_CU_Q):  with cu_seqlens_q: cu_seqlens_q[0] != 0, a
 *                             decreasing entry, or Lq_s outside
 *                             [0, min(max_seqlen_q, L_s)].
 * flags: device int32, set to the OR of the bits found (0: every check
 * passed) when the work queued on `stream` is done; the caller reads it
 * after synchronising.  Only the length arrays and the table entries of the
 * blocks checked are read; no page is.  kv: only block_table,
 * max_blocks_per_seq and num_pages are used (the pools may be NULL).
 * cu_seqlens_q NULL checks a decode batch.  Errors: NOSA_ERR_NULL,
 * NOSA_ERR_INVALID (sizes as in the other calls), NOSA_ERR_UNSUPPORTED,
 * NOSA_ERR_HIP. */
#define NOSA_CHECK_CU_K 1
#define NOSA_CHECK_LEN_K 2
#define NOSA_CHECK_TABLE 4
#define NOSA_CHECK_CU_Q 8
nosa_status nosa_check_inputs(const nosa_params* params, const nosa_paged_kv* kv,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NOSA_H */
