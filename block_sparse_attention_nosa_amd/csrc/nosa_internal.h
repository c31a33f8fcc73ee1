// nosa_internal.h -- host-side plan, workspace carving and kernel launchers
// shared by the C ABI layer (nosa_api.cpp) and the kernels
// (nosa_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nosa.h"

namespace nosa {

// Shapes the library has kernels for.
constexpr int kHeadDim = 128;
constexpr int kBlock = 64;   // tokens per KV block = per page
constexpr int kPoolK = 32;   // pooling window
constexpr int kPoolS = 16;   // pooling stride
constexpr int kSlots = kBlock / kPoolS;  // compressed keys stored per page
constexpr int kMaxGroup = 16;            // query heads per KV head (MFMA N = 16)
constexpr int kMaxBlocks = 8192;         // blocks per sequence (LDS of the selector)
constexpr int kMaxSplit = 64;            // attention workgroups per pair (partials per head)
constexpr int kMaxWindowBlocks = 128;    // window blocks (one page per wave)
constexpr int kScoreWaves = 4;           // waves of a scoring workgroup
constexpr int kStep2Waves = 4;           // waves of an attention workgroup
constexpr int kMaxChunks = 64;           // scoring chunks per pair (one lane each when combined)
constexpr int kMaxCacheSlots = 256;      // block-cache slots per pair (offloaded KV): one per thread
constexpr size_t kStaticScratchBytes = NOSA_STATIC_SCRATCH_BYTES;  // nosa_decode_step_static

inline int num_keys(int L) { return L >= kPoolK ? (L - kPoolK) / kPoolS + 1 : 0; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Everything the launchers need, derived on the host from the arguments.
struct Plan {
    int B = 0, Hq = 0, Hkv = 0, G = 0;
    int topk = 0, wblocks = 0, max_sel = 0;
    int max_seqlen_k = 0, max_nc = 0, max_nb = 0;
    int Lmax = 0;  // device lengths are clamped to this (<= max_seqlen_k, table reach)
    float scale_log2 = 0.f;  // logit scale * log2(e)
    // scoring: chunks of 64 T pooled keys (T tiles of 16 keys per wave of a
    // four-wave workgroup), nchunks per pair, 16 T blocks per chunk
    int score_tiles = 1, chunk_keys = 64, nchunks = 1;
    int nbk = 16;           // blocks with a pooled-importance partial per pair = nchunks * 16 T
    int gp = 4;             // G rounded up to a multiple of 4 (stride of the partial rows)
    // attention: one 64-token block per wave, four-wave workgroups
    int top_span = 0;       // top-k entries per pair = min(topk, max_nb - window blocks)
    int top_groups = 0;     // top-k workgroups per pair of a decode step, >= 1
    int top_rounds = 1;     // top-k blocks per wave
    int wslots = 0;         // window pages per pair = min(window blocks, max_nb), a workgroup each
    int nsplit = 0;         // partials per head in a decode step = top_groups + wslots
    int attend_groups = 0;  // workgroups per pair of the stand-alone attention
    int attend_rounds = 1;  // blocks per wave of the stand-alone attention
    // workspace layout (bytes from the start of the workspace)
    size_t off_cml = 0, off_spill = 0, off_bpart = 0, off_po = 0, off_pml = 0, bytes = 0;
};

// Device pointers carved out of the caller's workspace.
struct Workspace {
    float2* cml;         // [pairs][G][nchunks] per head and chunk: (max z, sum 2^(z - max))
    float* spill;        // [pairs][G][nchunks] 2^(z - max) of the chunk's last key
    float* bpart;        // [pairs][nbk][gp] per block and head: sum of 2^(z - chunk max)
    float* po;           // [B][Hq][nsplit'][D] partial outputs
    float2* pml;         // [B][Hq][nsplit'] partial (max, sum)
};

// Chunked prefill (queries at the end of each sequence, blocks of 64 queries).
struct PfPlan {
    int max_seqlen_q = 0, max_qblk = 0, npairs = 0;  // pairs = (sequence, q-block, KV head)
    int rows = 0;         // 64 * G rows (query, head) per pair
    int rtw = 1;          // row tiles of 16 per wave in the scoring passes
    int row_groups = 0;   // scoring workgroups over the rows of a pair
    int key_splits = 0;   // scoring workgroups over the pooled keys of a pair
    int span = 0;         // pooled keys per such workgroup (a multiple of 128)
    int attn_groups = 0;  // attention workgroups (128 rows each) per pair
    size_t off_part = 0, off_colsum = 0, off_rlse = 0, bytes = 0;
};
constexpr int kPfScoreWorkgroups = 512;  // scoring workgroups a launch aims for
constexpr int kPfChunk = 128;           // pooled keys the scoring passes stage in LDS at a time
constexpr int kPfMaxSpanChunks = 16;    // chunks per scoring workgroup at most
constexpr int kPfSplitGroups = 256;  // one workgroup per CU or fewer: split each row group's pages
constexpr size_t kPfLdsBytes = 160 * 1024;  // LDS a gfx950 workgroup may use

// Offloaded KV (device pointers; the host pools as the device sees them).
struct Offload {
    const nosa_bf16* k_host;
    const nosa_bf16* v_host;
    const nosa_bf16* k_recent;  // [batch][recent][Hkv][page]: block b in slot b % recent
    const nosa_bf16* v_recent;
    int recent = 0;
    nosa_bf16* cache_k;         // [batch][Hkv][cap][page]
    nosa_bf16* cache_v;
    int32_t* cache_map;         // [batch][Hkv][cap]
    int32_t* cache_used;        // [batch][Hkv][cap]: length at the last pick
    int cap = 0;
    int32_t* map_next;          // workspace, as cache_map
    int32_t* used_next;         // workspace, as cache_used
    int32_t* fetch_out;         // [batch][Hkv] or null
};

// Builds the plan for a decode batch; returns NOSA_OK or an error.
nosa_status make_plan(const nosa_params* p, int batch, int max_seqlen_k, Plan* plan);
Workspace carve(const Plan& pl, void* ws);
void make_pf_plan(const Plan& pl, int max_seqlen_q, PfPlan* pf);

// ---- launchers (nosa_kernels.hip); all enqueue on `stream` and return the
// ---- hipGetLastError() of the launches.
hipError_t launch_kc_build(const Plan& pl, const nosa_paged_kv& kv, const int32_t* cu_k,
                           const int32_t* valid_len, int max_pages, hipStream_t stream);
hipError_t launch_scores_only(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                              const int32_t* cu_k, const Workspace& w, float* scores_out,
                              hipStream_t stream);
// cu_q == nullptr: one decode query per sequence; else q-blocks of a chunk.
hipError_t launch_select(const Plan& pl, const int32_t* cu_k, const int32_t* cu_q, int max_seqlen_q,
                         const float* scores_in, int32_t* sel, int32_t* cnt, hipStream_t stream);
hipError_t launch_attend(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const int32_t* sel, const int32_t* cnt,
                         const Workspace& w, float* out, float* lse, hipStream_t stream);
// Device address of this device's static scratch array (kStaticScratchBytes),
// looked up on the first call on each device.
hipError_t static_scratch(void** ptr);

// off: offloaded KV (kv then holds the host pools' device view, kc_pool and
// the block table).
hipError_t launch_decode(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const Workspace& w, float* out, float* lse,
                         int32_t* sel_out, int32_t* cnt_out, float* scores_out,
                         hipStream_t stream, const Offload* off = nullptr);

// qbase (optional, device [B]): first q / out row of each sequence in place
// of cu_q (the rows of a chunk inside a whole prompt).
hipError_t launch_pf_scores(const Plan& pl, const PfPlan& pf, const nosa_paged_kv& kv,
                            const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k,
                            void* ws, float* scores, hipStream_t stream,
                            const int32_t* qbase = nullptr);
// Needs no workspace.
hipError_t launch_pf_attend(const Plan& pl, const PfPlan& pf, const nosa_paged_kv& kv,
                            const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k,
                            const int32_t* sel, const int32_t* cnt, float* out, float* lse,
                            hipStream_t stream, const int32_t* qbase = nullptr);

// The device-side input checks of nosa_check_inputs: flags cleared, then one
// workgroup per sequence ORs in the bits it finds.
hipError_t launch_check_inputs(const int32_t* cu_k, const int32_t* cu_q, const int32_t* table,
                               int max_blocks, int num_pages, int Lmax, int Lqmax, int batch,
                               int32_t* flags, hipStream_t stream);

// Whole-prompt prefill, chunk by chunk (nosa_prefill.hip).
hipError_t launch_chunk_setup(const int32_t* cu, int B, int Lmax, int c, int C, int32_t* cu_k_c,
                              int32_t* cu_q_c, int32_t* valid_c, int32_t* qbase_c,
                              hipStream_t stream);

// Front end (nosa_front.hip).
hipError_t launch_pack_qkv(int Hq, int Hkv, int hidden, const nosa_bf16* w, nosa_bf16* packed,
                           hipStream_t stream);
hipError_t launch_front(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* x,
                        const nosa_bf16* w, int hidden, float theta, const float* inv_freq,
                        const int32_t* cu_k, nosa_bf16* q_out, hipStream_t stream);

}  // namespace nosa
