// nosa_internal.h -- host-side plan and kernel launchers shared by the C ABI
// layer (nosa_api.cpp) and the kernels (nosa_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nosa.h"

namespace nosa {

// Shapes with a kernel in this build.
constexpr int kHeadDim = 128;
constexpr int kBlock = 64;   // tokens per KV block = per page
constexpr int kPoolK = 32;   // pooling window
constexpr int kPoolS = 16;   // pooling stride
constexpr int kSlots = kBlock / kPoolS;  // compressed keys stored per page
constexpr int kMaxGroup = 16;            // query heads per KV head (MFMA N = 16)
constexpr int kMaxBlocks = 8192;         // blocks per sequence (LDS of the selector)

inline int num_keys(int L) { return L >= kPoolK ? (L - kPoolK) / kPoolS + 1 : 0; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Everything the launchers need, derived on the host from the arguments.
struct Plan {
    int B = 0, Hq = 0, Hkv = 0, G = 0;
    int topk = 0, wblocks = 0, max_sel = 0, sel_span = 0;  // sel_span = min(max_sel, max_nb)
    int max_seqlen_k = 0, max_nc = 0, max_nb = 0;
    int Lmax = 0;  // device lengths are clamped to this (<= max_seqlen_k, table reach)
    float scale_log2 = 0.f;  // logit scale * log2(e)
    // scoring: T tiles of 16 keys per wave, 4 waves per workgroup
    int score_tiles = 1, score_groups = 0, nchunk = 0, zstride = 0;
    // attention: R blocks per wave, 4 waves per workgroup
    int attn_rounds = 1, nsplit = 0;
    // workspace layout (bytes from the start of the workspace)
    size_t off_z = 0, off_zpart = 0, off_scores = 0, off_sel = 0, off_cnt = 0, off_po = 0,
           off_pml = 0, bytes = 0;
};

// Builds the plan for a decode batch; returns NOSA_OK or an error.
nosa_status make_plan(const nosa_params* p, int batch, int max_seqlen_k, Plan* plan);

// ---- launchers (nosa_kernels.hip); all enqueue on `stream` and return the
// ---- hipGetLastError() of the launch.
hipError_t launch_kc_build(const Plan& pl, const nosa_paged_kv& kv, const int32_t* cu_k,
                           const int32_t* valid_len, bool append_current, int grid_x,
                           hipStream_t stream);
hipError_t launch_scores(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, float* z, float2* zpart, hipStream_t stream);
// mode: pool from z (z != nullptr) or read scores_in; select if sel != nullptr.
hipError_t launch_select(const Plan& pl, const int32_t* cu_k, const float* z,
                         const float2* zpart, const float* scores_in, float* scores_out,
                         int32_t* sel, int32_t* cnt, hipStream_t stream);
hipError_t launch_attend(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const int32_t* sel, const int32_t* cnt,
                         float* po, float2* pml, hipStream_t stream);
hipError_t launch_merge(const Plan& pl, const float* po, const float2* pml, float* out,
                        float* lse, hipStream_t stream);

}  // namespace nosa
