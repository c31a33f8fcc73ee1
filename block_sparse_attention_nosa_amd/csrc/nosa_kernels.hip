// nosa_kernels.hip -- CDNA4 (gfx950) kernels of the NOSA sparse decode step.
//
// A decode step is two launches:
//   step1 : per (sequence, KV head) pair, "score" workgroups compute
//           z_h[j] = scale*log2(e) * q_h . Kc_j on MFMA with per-wave
//           (max, sum exp2) partials -- the wave owning the key completed by the
//           current token pools it from K first (fp64, one bf16 rounding) and
//           stores it -- while "window" workgroups attend the local-window
//           blocks, which need no selection.  The last score workgroup of a
//           pair (atomic counter) turns the partials into per-head log-sum-exp,
//           pools block importance, radix-selects the top-k candidates and
//           writes their (block, page) list.
//   step2 : workgroups attend the selected blocks (one block per wave, every
//           K/V load of the block in flight at once); the last workgroup of a
//           pair merges the window and top-k partials into out / lse.
// Stand-alone entry points reuse the same pieces: kc_build (pooled keys),
// step1 in scores mode (importance only), select (from given importance) and
// step2 in attend mode (given block ids).
//
// Sources: page "NOSA-1B 性能基准全解析" (sections 三.2 local window and TopK
// blocks, 三.3 two-stage attention with kernel 32 / stride 16 pooling, 三.4 the
// mean-pool kernel), page "NOSA-1B 模型家族全景" (core principle: compressed
// attention filters KV blocks, CIS score mean pooling), page "NOSA技术架构解析"
// (section 2.1: paged KV pool; section 5.1: importance scores kept in fp32).
//
// Shared device helpers (MFMA operand layout, one-page attention, the
// selector) are in nosa_device.h.
//
// Cross-workgroup hand-off ("last one done"): data that another workgroup of
// the same launch reads (logits, per-wave partials, attention partials) is
// written and read with agent-scope relaxed atomic accesses, which this chip
// performs coherently across its L2s (sc1) without whole-cache write-back or
// invalidation.  Each workgroup waits for its stores to complete, then bumps
// the pair's counter; the workgroup that sees count-1 resets the counter to
// zero for the next call and finishes the pair.  Counters therefore start and
// end every call at zero.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nosa_device.h"

namespace nosa {

// ------------------------------------------------------- pooled keys ---

// Round a double to bf16, nearest-even, in one step from its bit pattern.
__device__ __forceinline__ uint32_t bf16_from_f64(double x)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t mag = u & 0x7fffffffffffffffull;
    if (mag > 0x7ff0000000000000ull) return 0x7fc0u;            // NaN
    const int e = (int)(mag >> 52) - 1023;                        // unbiased exponent
    if (e > 127) return sign | 0x7f80u;                           // beyond bf16 range
    if (e >= -126) {                                              // normal in bf16
        const uint64_t r = mag + ((1ull << 44) - 1) + ((mag >> 45) & 1);  // RNE at bit 45
        const uint64_t t = r >> 45;                               // 11-bit exp | 7-bit mant
        const int e2 = (int)(t >> 7) - 1023 + 127;
        if (e2 >= 255) return sign | 0x7f80u;
        return sign | ((uint32_t)e2 << 7) | (uint32_t)(t & 0x7f);
    }
    // bf16 subnormal range: fixed quantum 2^-133; rint rounds half to even
    const double m = rint(fabs(x) * 0x1p133);
    return sign | (uint32_t)m;
}

__device__ __forceinline__ void acc8(double (&acc)[8], uint4 w)
{
    acc[0] += (double)bf16_lo(w.x); acc[1] += (double)bf16_hi(w.x);
    acc[2] += (double)bf16_lo(w.y); acc[3] += (double)bf16_hi(w.y);
    acc[4] += (double)bf16_lo(w.z); acc[5] += (double)bf16_hi(w.z);
    acc[6] += (double)bf16_lo(w.w); acc[7] += (double)bf16_hi(w.w);
}

__device__ __forceinline__ uint4 round8(const double (&acc)[8])
{
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = bf16_from_f64(acc[e] * (1.0 / kPoolK));
    return make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                      o[6] | (o[7] << 16));
}

// One workgroup = 16 keys x 16 channel chunks of 8.  Each thread sums the 32
// tokens of its key for its 8 channels in fp64 (exact for bf16 inputs), then
// scales by 1/32 (exact) and rounds once.  Keys [n_c(prev), n_c(L)) are
// written, prev = valid_len[s] or 0 for a full rebuild.
__global__ __launch_bounds__(256) void kc_build_kernel(
    const uint16_t* __restrict__ k_pool, uint16_t* __restrict__ kc_pool,
    const int32_t* __restrict__ table, int max_blocks, int Lmax, int Hkv,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ valid_len)
{
    const int s = blockIdx.z, g = blockIdx.y;
    const int L = seq_len(cu_k, s, Lmax);
    int prev = valid_len ? valid_len[s] : 0;
    prev = prev < 0 ? 0 : prev;
    const int j0 = dev_num_keys(prev), j1 = dev_num_keys(L);
    const int jl = threadIdx.x >> 4, cc = threadIdx.x & 15;
    const int32_t* trow = table + (size_t)s * max_blocks;
    for (int j = j0 + (int)blockIdx.x * 16 + jl; j < j1; j += (int)gridDim.x * 16) {
        double acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0;
        for (int i = 0; i < kPoolK; ++i) {
            const int t = j * kPoolS + i;
            acc8(acc, ldg16(k_pool + ((size_t)trow[t / BS] * Hkv + g) * BS * D + k_chunk(t % BS, cc)));
        }
        *reinterpret_cast<uint4*>(kc_page(kc_pool, trow, Hkv, g, j) + kc_chunk(j % SL, cc)) = round8(acc);
    }
}

hipError_t launch_kc_build(const Plan& pl, const nosa_paged_kv& kv, const int32_t* cu_k,
                           const int32_t* valid_len, int grid_x, hipStream_t stream)
{
    dim3 grid(grid_x, pl.Hkv, pl.B);
    hipLaunchKernelGGL(kc_build_kernel, grid, dim3(256), 0, stream, kv.k_pool, kv.kc_pool,
                       kv.block_table, kv.max_blocks_per_seq, pl.Lmax, pl.Hkv, cu_k, valid_len);
    return hipGetLastError();
}

// LDS for combining the four wave states of a workgroup.
struct CombineLds {
    float m[4][16], l[4][16];
    float o[4][16][D + 4];
};

// Merge the four waves' states in LDS and store one (m, l, o) partial per
// head of the group at partial slot `split`.  Must be called by all 256
// threads.  Heads with no data get m = -inf, l = 0, o = 0.
__device__ void store_wg_partial(CombineLds& sh, const AttnState& A, int G, size_t head_row0,
                                 int nsplit, int split, float* __restrict__ po,
                                 float2* __restrict__ pml)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    float l = A.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (wave < 4) {  // a 512-thread caller has folded waves 4..7 in already
        if (kq == 0) {
            sh.m[wave][r] = A.m;
            sh.l[wave][r] = l;
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.o[wave][4 * kq + i][nt * 16 + r] = A.o[nt][i];
    }
    __syncthreads();
    const int h = tid >> 4, c0 = (tid & 15) * 8;
    if (h < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.m[w][h]);
        float wt[4], Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wt[w] = (M == -INFINITY || sh.m[w][h] == -INFINITY) ? 0.f : fexp2(sh.m[w][h] - M);
            Lsum += wt[w] * sh.l[w][h];
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[e] += wt[w] * sh.o[w][h][c0 + e];
        }
        const size_t prow = (head_row0 + h) * nsplit + split;
        float4* dst = reinterpret_cast<float4*>(po + prow * D + c0);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if ((tid & 15) == 0) pml[prow] = make_float2(M, Lsum);
    }
}

// Eight-wave version of store_wg_partial: waves 4..7 first fold their state
// into waves 0..3 through LDS, then the four-wave combine runs.  Must be
// called by all 512 threads.
__device__ void store_wg_partial8(CombineLds& sh, AttnState& A, int G, size_t head_row0,
                                  int nsplit, int split, float* __restrict__ po,
                                  float2* __restrict__ pml)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    __shared__ float m_lo[4][16];
    float l = A.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (wave >= 4) {
        if (kq == 0) {
            sh.m[wave - 4][r] = A.m;
            sh.l[wave - 4][r] = l;
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.o[wave - 4][4 * kq + i][nt * 16 + r] = A.o[nt][i];
    } else if (kq == 0) {
        m_lo[wave][r] = A.m;
    }
    __syncthreads();
    if (wave < 4) {
        // rows of this lane's accumulators: heads 4kq + i; of its (m, l): head r
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * kq + i;
            const float ma = m_lo[wave][h], mb = sh.m[wave][h];
            const float M = fmaxf(ma, mb);
            const float wa = (M == -INFINITY || ma == -INFINITY) ? 0.f : fexp2(ma - M);
            const float wb = (M == -INFINITY || mb == -INFINITY) ? 0.f : fexp2(mb - M);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                A.o[nt][i] = A.o[nt][i] * wa + sh.o[wave][h][nt * 16 + r] * wb;
        }
        const float ma = A.m, mb = sh.m[wave][r];
        const float M = fmaxf(ma, mb);
        const float wa = (M == -INFINITY || ma == -INFINITY) ? 0.f : fexp2(ma - M);
        const float wb = (M == -INFINITY || mb == -INFINITY) ? 0.f : fexp2(mb - M);
        A.l = l * wa + sh.l[wave][r] * wb;  // already summed over the lane groups
        A.m = M;
    }
    __syncthreads();
    // four-wave combine (the l above is complete: keep the lane-group sum from
    // adding it four times)
    if (wave < 4 && kq != 0) A.l = 0.f;
    store_wg_partial(sh, A, G, head_row0, nsplit, split, po, pml);
}

// Block importance of the pair into sI[0 .. nb): mean over the keys
// overlapping block b (keys 4b-1 .. 4b+3 that exist) of
// sigma[j] = sum_h 2^(z_h[j] - lse_h).  Thread tid computes whole blocks
// b = tid + i NT from their five keys (key 4b-1 is also its left neighbour's
// last key), so no block needs a second contribution; the order key of each
// block it computed is returned in keys[i] (i < kSelKeyRounds, 0 past nb).
// z (in LDS or global memory, at least 4 max_nb + 4 entries per head; keys
// at or past nc are never read) was written by this workgroup (call after a
// barrier).  Also writes scores_out.  All NT threads; ends with a barrier.
template <int NT>
__device__ __forceinline__ void pool_pair(const float* __restrict__ zg, int zstride, const float* lse,
                                          int G, int nc, int nb, float* sI,
                                          float* __restrict__ scores_out, int max_nb,
                                          uint32_t (&keys)[kSelKeyRounds])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kSelKeyRounds; ++i) keys[i] = 0u;
#pragma unroll 1
    for (int i = 0, b = tid; b < nb; ++i, b += NT) {
        const int j0 = 4 * b;
        float sg[4] = {0.f, 0.f, 0.f, 0.f}, sp = 0.f;
#pragma unroll 1
        for (int h0 = 0; h0 < G; h0 += 8) {
            float4 zz[8];
            float zp[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (h0 + u < G) {
                    const float* zr = zg + (size_t)(h0 + u) * zstride;
                    zz[u] = *reinterpret_cast<const float4*>(zr + j0);
                    zp[u] = b > 0 ? zr[j0 - 1] : 0.f;
                }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (h0 + u < G) {
                    const float lh = lse[h0 + u];
                    sg[0] += fexp2(zz[u].x - lh);
                    sg[1] += fexp2(zz[u].y - lh);
                    sg[2] += fexp2(zz[u].z - lh);
                    sg[3] += fexp2(zz[u].w - lh);
                    sp += fexp2(zp[u] - lh);
                }
        }
        const int jlo = max(j0 - 1, 0), jhi = min(j0 + 3, nc - 1);
        float sum = (b > 0 && j0 - 1 < nc) ? sp : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j0 + e < nc) sum += sg[e];
        const float I = jlo <= jhi ? sum / (float)(jhi - jlo + 1) : -INFINITY;
        sI[b] = I;
        if (scores_out) scores_out[b] = I;
#pragma unroll
        for (int r = 0; r < kSelKeyRounds; ++r)
            if (r == i) keys[r] = order_key(I);
    }
    if (scores_out)
        for (int b = nb + tid; b < max_nb; b += NT) scores_out[b] = -INFINITY;
    __syncthreads();
}

// --------------------------------------------------------------- step 1 ---

constexpr int kPairWaves = kStep1Waves;  // waves of a step-1 workgroup (512 threads)
constexpr int kPairThreads = kPairWaves * 64;

struct Step1Args {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    uint16_t* kc_pool;
    const int32_t* table;
    const int32_t* cu_k;
    int max_blocks, Lmax, B, Hq, Hkv, G;
    float scale_log2;
    int win_groups;  // window workgroups per pair (0 = none), one page per wave
    int append;      // pool the key completed by the current token
    float* z;        // [B][Hq][zstride] logits (log2 units), private to the pair's workgroup
    int zstride;
    int zl_stride;   // logits kept in LDS instead, [G][zl_stride] (0 = in z)
    int do_select, topk, wblocks, max_nb, max_sel, top_span;
    float* scores_out;  // [pairs][max_nb] or null
    int32_t* sel_out;   // [pairs][max_sel] or null
    int32_t* cnt_out;   // [pairs] or null
    int2* selpg;        // [pairs][top_span] or null
    float* po;
    float2* pml;
    int nsplit;  // partial slots per head
};

// LDS of a step-1 workgroup (dynamic): the block importance, the page ids
// and the logits of the pair (pair workgroups) or the wave states (window
// workgroups).
__host__ __device__ inline size_t step1_z_offset(int max_nb)
{
    const size_t b = (size_t)max_nb * (sizeof(float) + sizeof(int32_t));
    return (b + 15) / 16 * 16;
}
inline size_t step1_lds_bytes(int max_nb, size_t zbytes)
{
    const size_t pair = step1_z_offset(max_nb) + zbytes;
    return pair > sizeof(CombineLds) ? pair : sizeof(CombineLds);
}
constexpr size_t kStep1StaticLds = 10 * 1024;  // bound on the kernel's static LDS

struct PairLds {
    float m[kPairWaves][kMaxGroup], s[kPairWaves][kMaxGroup];
    SelectLds sel;
};

// The per-pair workgroup: scores every pooled key of one (sequence, KV head)
// -- tiles of 16 keys strided over its eight waves, T tiles' loads in flight
// per wave -- with per-wave (max, sum exp2) per head, keeps the logits in the
// workspace (read back only by this workgroup), then pools block importance
// and selects.  The wave owning the key completed by the current token
// (tokens L-32 .. L-1) pools it from K first, stores it and substitutes it
// into its MFMA operand.
template <int T, bool ZL>
__device__ void pair_part(const Step1Args& a, int s, int g, char* smem)
{
    __shared__ PairLds sh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int L = seq_len(a.cu_k, s, a.Lmax);
    const int nc = dev_num_keys(L);
    const int nb = (L + BS - 1) / BS;
    const int32_t* trow = a.table + (size_t)s * a.max_blocks;
    const size_t head_row0 = (size_t)s * a.Hq + g * a.G;
    const size_t pair = (size_t)s * a.Hkv + g;
    float* sI = reinterpret_cast<float*>(smem);
    int32_t* spg = reinterpret_cast<int32_t*>(smem + sizeof(float) * a.max_nb);
    // logits of head h, key j: zb[h * zs + j], in LDS or in the workspace
    const int zs = ZL ? a.zl_stride : a.zstride;
    float* zb = ZL ? reinterpret_cast<float*>(smem + step1_z_offset(a.max_nb))
                   : a.z + head_row0 * a.zstride;
    // The block-table row goes to LDS first (four loads in flight per
    // thread), so no key load below waits on a table load: loads complete in
    // order, so a table load issued behind other loads would wait for them.
    // It is read up to the host bound max_nb (<= max_blocks_per_seq), so its
    // loads and the query's do not wait for the length; entries past nb are
    // never used.
    for (int b0 = tid; b0 < a.max_nb; b0 += 4 * kPairThreads) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = b0 + u * kPairThreads;
            v[u] = b < a.max_nb ? trow[b] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (b0 + u * kPairThreads < a.max_nb) spg[b0 + u * kPairThreads] = v[u];
    }

    select_lds_clear<kPairThreads>(sh.sel);
    bf16x8 qb[4];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
    __syncthreads();
    const int jn = nc - 1;
    const bool appending = a.append && L >= kPoolK && (L - kPoolK) % kPoolS == 0;
    const int ntiles = (nc + 15) / 16;
    // The wave whose batch holds key jn pools it and stores it before its
    // first batch, which then loads it like every other key.
    const bool app_mine = appending && (jn / 16) % kPairWaves == wave;
    if (app_mine) {
        const int tr = lane >> 4, cc = lane & 15;  // 4 token phases x 16 channel chunks
        // tokens 16jn + tr + 4i, i < 8: their pages first, then all loads
        int kpg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int b = (jn * kPoolS + tr + 4 * i) / BS;
            kpg[i] = spg[b];
        }
        uint4 kr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = jn * kPoolS + tr + 4 * i;
            kr[i] = ldg16(a.k_pool + ((size_t)kpg[i] * a.Hkv + g) * BS * D + k_chunk(t % BS, cc));
        }
        double acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc8(acc, kr[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += __shfl_xor(acc[e], 16);
            acc[e] += __shfl_xor(acc[e], 32);
        }
        const uint4 appkey = round8(acc);  // channels 8cc .. 8cc+7, same in every phase
        if (tr == 0) {
            const int pj = spg[jn / SL];
            *reinterpret_cast<uint4*>(a.kc_pool + ((size_t)pj * a.Hkv + g) * SL * D + kc_chunk(jn % SL, cc)) = appkey;
        }
        // the key has reached L2 before this wave loads its tiles below (no
        // other wave reads this page in this launch)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_waitcnt(0);
    }
    float m_run = -INFINITY, s_run = 0.f;  // head r, over this lane's keys
    // tile i of the pair (keys 16i .. 16i + 15) goes to wave i % 8, T tiles
    // of a wave per batch: tiles wave + 8 (bT + t), t < T
    for (int b0 = wave; b0 < ntiles; b0 += kPairWaves * T) {
        // page ids of this lane's keys for the whole batch before any key
        // load; rows past the last key load that key again (their logits are
        // masked below), so the loads need no branch
        int pg[T], kr[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int key = (b0 + kPairWaves * t) * 16 + r;
            kr[t] = key < nc ? key : nc - 1;
            pg[t] = spg[kr[t] / SL];
        }
        uint4 kv[T][4];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint16_t* kp = a.kc_pool + ((size_t)pg[t] * a.Hkv + g) * SL * D;
#pragma unroll
            for (int st = 0; st < 4; ++st) kv[t][st] = ldg16(kp + kc_chunk(kr[t] % SL, st * 4 + kq));
        }
        // every load of the batch is in flight before the first use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int key0 = (b0 + kPairWaves * t) * 16;
            if (key0 >= nc) continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(kv[t][st]), qb[st], acc);
            float zv[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + kq * 4 + i;
                zv[i] = key < nc ? acc[i] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, zv[i]);
            }
            if (r < a.G)
                *reinterpret_cast<float4*>(zb + r * zs + key0 + kq * 4) =
                    make_float4(zv[0], zv[1], zv[2], zv[3]);
            if (tmax != -INFINITY) {
                const float mn = fmaxf(m_run, tmax);
                float add = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) add += fexp2(zv[i] - mn);
                s_run = s_run * fexp2(m_run - mn) + add;
                m_run = mn;
            }
        }
    }
    // per-wave partials of every head -> LDS -> per-head log2-sum-exp2
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m_run, off), so = __shfl_xor(s_run, off);
        const float mn = fmaxf(m_run, mo);
        s_run = mn == -INFINITY ? 0.f : s_run * fexp2(m_run - mn) + so * fexp2(mo - mn);
        m_run = mn;
    }
    if (kq == 0 && r < a.G) {
        sh.m[wave][r] = m_run;
        sh.s[wave][r] = s_run;
    }
    if (!ZL) __builtin_amdgcn_s_waitcnt(0);  // this wave's logits have reached L2
    __syncthreads();
    if (tid < a.G) {
        // all sixteen LDS reads first, then independent exponentials
        float mw[kPairWaves], sw[kPairWaves];
#pragma unroll
        for (int w = 0; w < kPairWaves; ++w) {
            mw[w] = sh.m[w][tid];
            sw[w] = sh.s[w][tid];
        }
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kPairWaves; ++w)
            if (sw[w] > 0.f) m = fmaxf(m, mw[w]);
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kPairWaves; ++w)
            if (sw[w] > 0.f) acc += sw[w] * fexp2(mw[w] - m);
        sh.sel.lse[tid] = m + log2f(acc);
    }
    __syncthreads();
    uint32_t keys[kSelKeyRounds];
    pool_pair<kPairThreads>(zb, zs, sh.sel.lse, a.G, nc, nb, sI,
                            a.scores_out ? a.scores_out + pair * a.max_nb : nullptr, a.max_nb, keys);
    if (!a.do_select) return;
    select_blocks_wg<kPairWaves, true>(keys, sI, nb, a.wblocks, a.topk, sh.sel,
                                 a.sel_out ? a.sel_out + pair * a.max_sel : nullptr,
                                 a.cnt_out ? a.cnt_out + pair : nullptr, a.max_sel,
                                 a.selpg ? a.selpg + pair * a.top_span : nullptr, nullptr,
                                 a.top_span, trow, spg);
}

// Window workgroup: wave w attends window slot 8*grp + w, slot x being block
// nb - min(nb, wblocks) + x, and the workgroup stores one partial.
__device__ void window_part(const Step1Args& a, int s, int g, int grp, char* smem)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int L = seq_len(a.cu_k, s, a.Lmax);
    const int nb = (L + BS - 1) / BS;
    const int wn = nb < a.wblocks ? nb : a.wblocks;
    AttnState A;
    attn_init(A);
    bf16x8 qb[4];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
    const int slot = grp * kPairWaves + wave;
    if (slot < wn) {
        const int b = nb - wn + slot;
        const int page = a.table[(size_t)s * a.max_blocks + b];
        const uint16_t* kb = a.k_pool + ((size_t)page * a.Hkv + g) * BS * D;
        const uint16_t* vb = a.v_pool + ((size_t)page * a.Hkv + g) * D * BS;
        attend_page(kb, vb, L - b * BS, qb, a.scale_log2, r, kq, A);
    }
    store_wg_partial8(*reinterpret_cast<CombineLds*>(smem), A, a.G, (size_t)s * a.Hq + g * a.G,
                      a.nsplit, grp, a.po, a.pml);
}

template <int T, bool ZL>
__global__ __launch_bounds__(512) void step1_kernel(Step1Args a)
{
    extern __shared__ __align__(16) char smem[];
    // pair workgroups first: they carry the launch's critical path
    const int npairs = a.B * a.Hkv;
    int wg = blockIdx.x;
    if (wg < npairs) {
        pair_part<T, ZL>(a, wg / a.Hkv, wg % a.Hkv, smem);
    } else {
        wg -= npairs;
        const int pair = wg / a.win_groups, grp = wg % a.win_groups;
        window_part(a, pair / a.Hkv, pair % a.Hkv, grp, smem);
    }
}

// --------------------------------------------------------------- step 2 ---

struct Step2Args {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* table;
    const int32_t* cu_k;
    int max_blocks, Lmax, B, Hq, Hkv, G;
    float scale_log2;
    int groups;         // workgroups per pair
    int rounds;         // blocks per wave
    const int2* selpg;  // decode mode: [pairs][span] (block, page), -1 padded
    const int32_t* sel; // attend mode: [pairs][max_sel] block ids
    const int32_t* cnt; //              [pairs]
    int span, max_sel;
    float* po;
    float2* pml;
    int nsplit, split0;  // partial slots per head; this kernel writes [split0, split0+groups)
};

// Combination of the nsplit partials (m_i, l_i, o_i) of each head row into
// out = sum_i 2^(m_i - M) o_i / L and lse = (M + log2 L) ln 2, with
// M = max_i m_i and L = sum_i 2^(m_i - M) l_i (empty rows: out 0, lse -inf).
// One workgroup of 128 threads per row, thread c = channel c; partials are
// taken 32 at a time with every load of a batch in flight, the running
// (M, L, acc) rescaled between batches.  A launch of its own, so the
// partials of every workgroup of the step are complete when it starts.
constexpr int kMergeBatch = 32;

__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ po,
                                                    const float2* __restrict__ pml, int nsplit,
                                                    float* __restrict__ out, float* __restrict__ lse)
{
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const float2* ml = pml + row * nsplit;
    const float* op = po + row * nsplit * D + c;
    float M = -INFINITY, L = 0.f, acc = 0.f;
#pragma unroll 1
    for (int i0 = 0; i0 < nsplit; i0 += kMergeBatch) {
        float2 v[kMergeBatch];
        float o[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const bool ok = i0 + u < nsplit;
            v[u] = ok ? ml[i0 + u] : make_float2(-INFINITY, 0.f);
            o[u] = ok ? op[(size_t)(i0 + u) * D] : 0.f;
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) Mb = fmaxf(Mb, v[u].x);
        if (Mb == -INFINITY) continue;
        const float r = M == -INFINITY ? 0.f : fexp2(M - Mb);
        L *= r;
        acc *= r;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const float w = v[u].x == -INFINITY ? 0.f : fexp2(v[u].x - Mb);
            L += w * v[u].y;
            acc += w * o[u];
        }
        M = Mb;
    }
    const bool empty = !(L > 0.f);
    out[row * D + c] = empty ? 0.f : acc / L;
    if (lse && c == 0) lse[row] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
}

static hipError_t launch_merge(const Plan& pl, const Workspace& w, int nsplit, float* out, float* lse,
                               hipStream_t stream)
{
    const int rows = pl.B * pl.Hq;
    if (rows > 0)
        hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(D), 0, stream, w.po, w.pml, nsplit, out,
                           lse);
    return hipGetLastError();
}

// Workgroup = kStep2Waves (4) waves; wave w handles entries
// (grp*rounds + rr)*4 + w of the pair's list, rr < rounds, one 64-token
// block at a time.
static_assert(kStep2Waves == 4, "store_wg_partial combines four waves");
template <bool kDecode, int R>
__global__ __launch_bounds__(kStep2Waves * 64) void step2_kernel(Step2Args a)
{
    __shared__ CombineLds sh;
    const int pair = blockIdx.x / a.groups, grp = blockIdx.x % a.groups;
    const int s = pair / a.Hkv, g = pair % a.Hkv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int L = seq_len(a.cu_k, s, a.Lmax);
    const int nb = (L + BS - 1) / BS;
    const int32_t* trow = a.table + (size_t)s * a.max_blocks;
    int n = 0;
    if (!kDecode) n = min(a.cnt[pair], a.max_sel);
    AttnState A;
    attn_init(A);
    bf16x8 qb[4];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int idx = (grp * R + rr) * kStep2Waves + wave;
        int b = -1, page = -1;
        if (kDecode) {
            if (idx < a.span) {
                const int2 e = a.selpg[(size_t)pair * a.span + idx];
                b = e.x;
                page = e.y;
            }
        } else if (idx < n) {
            b = a.sel[(size_t)pair * a.max_sel + idx];
            if (b >= 0 && b < nb) page = trow[b];
        }
        if (b < 0 || b >= nb) continue;
        const uint16_t* kb = a.k_pool + ((size_t)page * a.Hkv + g) * BS * D;
        const uint16_t* vb = a.v_pool + ((size_t)page * a.Hkv + g) * D * BS;
        attend_page(kb, vb, L - b * BS, qb, a.scale_log2, r, kq, A);
    }
    store_wg_partial(sh, A, a.G, (size_t)s * a.Hq + g * a.G, a.nsplit, a.split0 + grp, a.po, a.pml);
}

// ------------------------------------------------------ select (alone) ---

// Selection from given importance: one workgroup per row of the importance
// (sequence, or sequence x q-block, times KV head).  For a decode row the
// blocks are those of the L tokens; for q-block r of a chunk of Lq queries
// they end at the block of the q-block's last query, L - Lq + min(64r + 64, Lq) - 1.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores_in,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ cnt,
                                                     const int32_t* __restrict__ cu_k,
                                                     const int32_t* __restrict__ cu_q, int Lqmax,
                                                     int max_qblk, int Lmax, int Hkv, int max_nb,
                                                     int max_sel, int topk, int wblocks)
{
    extern __shared__ __align__(16) char smem[];
    __shared__ SelectLds sh;
    float* sI = reinterpret_cast<float*>(smem);
    const int g = blockIdx.x, sr = blockIdx.y;
    const int s = sr / max_qblk, qb = sr % max_qblk;
    const int L = seq_len(cu_k, s, Lmax);
    int nb = (L + BS - 1) / BS;
    if (cu_q) {
        int Lq = cu_q[s + 1] - cu_q[s];
        Lq = Lq < 0 ? 0 : (Lq > Lqmax ? Lqmax : Lq);
        Lq = Lq < L ? Lq : L;
        const int left = Lq - 64 * qb;
        nb = left > 0 ? (L - Lq + 64 * qb + (left < 64 ? left : 64) - 1) / BS + 1 : 0;
    }
    const size_t pair = (size_t)sr * Hkv + g;
    for (int b = threadIdx.x; b < nb; b += 256) sI[b] = scores_in[pair * max_nb + b];
    select_lds_clear<256>(sh);
    __syncthreads();
    uint32_t keys[kSelKeyRounds];
    select_blocks_wg<4, false>(keys, sI, nb, wblocks, topk, sh, sel + pair * max_sel, cnt + pair, max_sel,
                        nullptr, nullptr, 0, nullptr);
}

// ---------------------------------------------------------- launchers ---

template <bool kDecode>
static hipError_t launch_step2(const Step2Args& b, int grid, hipStream_t stream)
{
    switch (b.rounds) {
        case 1: hipLaunchKernelGGL((step2_kernel<kDecode, 1>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
        case 2: hipLaunchKernelGGL((step2_kernel<kDecode, 2>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
        case 3: hipLaunchKernelGGL((step2_kernel<kDecode, 3>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
        case 4: hipLaunchKernelGGL((step2_kernel<kDecode, 4>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
        case 6: hipLaunchKernelGGL((step2_kernel<kDecode, 6>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
        default: hipLaunchKernelGGL((step2_kernel<kDecode, 8>), dim3(grid), dim3(kStep2Waves * 64), 0, stream, b); break;
    }
    return hipGetLastError();
}

static Step1Args step1_args(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                            const int32_t* cu_k, const Workspace& w)
{
    Step1Args a{};
    a.q = q;
    a.k_pool = kv.k_pool;
    a.v_pool = kv.v_pool;
    a.kc_pool = kv.kc_pool;
    a.table = kv.block_table;
    a.cu_k = cu_k;
    a.max_blocks = kv.max_blocks_per_seq;
    a.Lmax = pl.Lmax;
    a.B = pl.B;
    a.Hq = pl.Hq;
    a.Hkv = pl.Hkv;
    a.G = pl.G;
    a.scale_log2 = pl.scale_log2;
    a.z = w.z;
    a.zstride = pl.zstride;
    a.topk = pl.topk;
    a.wblocks = pl.wblocks;
    a.max_nb = pl.max_nb;
    a.max_sel = pl.max_sel;
    a.top_span = pl.top_span;
    a.po = w.po;
    a.pml = w.pml;
    a.nsplit = pl.nsplit;
    return a;
}

// Largest LDS a workgroup may use on the current device (queried once per
// device).
static size_t device_lds_limit()
{
    static size_t cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        cached[dev] = (size_t)v;
    }
    return cached[dev];
}

template <int T, bool ZL>
static void launch_step1_t(dim3 grid, size_t lds, const Step1Args& a, hipStream_t stream)
{
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&step1_kernel<T, ZL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((step1_kernel<T, ZL>), grid, dim3(kPairThreads), lds, stream, a);
}

static hipError_t launch_step1(const Plan& pl, Step1Args a, hipStream_t stream)
{
    const int npairs = pl.B * pl.Hkv;
    dim3 grid(npairs * (1 + a.win_groups));
    // logits in LDS when they fit beside everything else
    // the scoring writes whole tiles of 16 keys, the pooling reads keys up to
    // 4 max_nb + 3 (never past n_c, but the float4 covering them)
    const int zneed = (pl.max_nc + 15) / 16 * 16 > 4 * pl.max_nb + 4 ? (pl.max_nc + 15) / 16 * 16
                                                                    : 4 * pl.max_nb + 4;
    const int zls = zneed + 4;
    const size_t zbytes = (size_t)pl.G * zls * sizeof(float);
    const size_t limit = device_lds_limit();
    if (step1_lds_bytes(pl.max_nb, 0) + kStep1StaticLds > limit) return hipErrorInvalidValue;
    const bool zl = step1_lds_bytes(pl.max_nb, zbytes) + kStep1StaticLds <= limit;
    a.zl_stride = zl ? zls : 0;
    const size_t lds = step1_lds_bytes(pl.max_nb, zl ? zbytes : 0);
#define NOSA_STEP1(T)                                           \
    (zl ? launch_step1_t<T, true>(grid, lds, a, stream)         \
        : launch_step1_t<T, false>(grid, lds, a, stream))
    switch (pl.score_tiles) {
        case 1: NOSA_STEP1(1); break;
        case 2: NOSA_STEP1(2); break;
        case 3: NOSA_STEP1(3); break;
        case 5: NOSA_STEP1(5); break;
        case 7: NOSA_STEP1(7); break;
        case 9: NOSA_STEP1(9); break;
        default: NOSA_STEP1(12); break;
    }
#undef NOSA_STEP1
    return hipGetLastError();
}

hipError_t launch_scores_only(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                              const int32_t* cu_k, const Workspace& w, float* scores_out,
                              hipStream_t stream)
{
    Step1Args a = step1_args(pl, kv, q, cu_k, w);
    a.win_groups = 0;
    a.append = 0;
    a.do_select = 0;
    a.scores_out = scores_out;
    return launch_step1(pl, a, stream);
}

hipError_t launch_decode(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const Workspace& w, float* out, float* lse,
                         int32_t* sel_out, int32_t* cnt_out, float* scores_out,
                         hipStream_t stream)
{
    Step1Args a = step1_args(pl, kv, q, cu_k, w);
    a.win_groups = pl.win_groups;
    a.append = 1;
    a.do_select = 1;
    a.scores_out = scores_out;
    a.sel_out = sel_out;
    a.cnt_out = cnt_out;
    a.selpg = w.selpg;
    hipError_t e = launch_step1(pl, a, stream);
    if (e != hipSuccess) return e;

    Step2Args b{};
    b.q = q;
    b.k_pool = kv.k_pool;
    b.v_pool = kv.v_pool;
    b.table = kv.block_table;
    b.cu_k = cu_k;
    b.max_blocks = kv.max_blocks_per_seq;
    b.Lmax = pl.Lmax;
    b.B = pl.B;
    b.Hq = pl.Hq;
    b.Hkv = pl.Hkv;
    b.G = pl.G;
    b.scale_log2 = pl.scale_log2;
    b.groups = pl.top_groups;
    b.rounds = pl.top_rounds;
    b.selpg = w.selpg;
    b.span = pl.top_span;
    b.po = w.po;
    b.pml = w.pml;
    b.nsplit = pl.nsplit;
    b.split0 = pl.win_groups;
    e = launch_step2<true>(b, pl.B * pl.Hkv * pl.top_groups, stream);
    if (e != hipSuccess) return e;
    return launch_merge(pl, w, pl.nsplit, out, lse, stream);
}

hipError_t launch_attend(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const int32_t* sel, const int32_t* cnt,
                         const Workspace& w, float* out, float* lse, hipStream_t stream)
{
    Step2Args b{};
    b.q = q;
    b.k_pool = kv.k_pool;
    b.v_pool = kv.v_pool;
    b.table = kv.block_table;
    b.cu_k = cu_k;
    b.max_blocks = kv.max_blocks_per_seq;
    b.Lmax = pl.Lmax;
    b.B = pl.B;
    b.Hq = pl.Hq;
    b.Hkv = pl.Hkv;
    b.G = pl.G;
    b.scale_log2 = pl.scale_log2;
    b.groups = pl.attend_groups;
    b.rounds = pl.attend_rounds;
    b.sel = sel;
    b.cnt = cnt;
    b.max_sel = pl.max_sel;
    b.po = w.po;
    b.pml = w.pml;
    b.nsplit = pl.attend_groups;
    b.split0 = 0;
    hipError_t e = launch_step2<false>(b, pl.B * pl.Hkv * pl.attend_groups, stream);
    if (e != hipSuccess) return e;
    return launch_merge(pl, w, pl.attend_groups, out, lse, stream);
}

hipError_t launch_select(const Plan& pl, const int32_t* cu_k, const int32_t* cu_q, int max_seqlen_q,
                         const float* scores_in, int32_t* sel, int32_t* cnt, hipStream_t stream)
{
    const size_t lds = sizeof(float) * (size_t)(pl.max_nb > 0 ? pl.max_nb : 1);
    const int max_qblk = cu_q ? ceil_div(max_seqlen_q, 64) : 1;
    hipLaunchKernelGGL(select_kernel, dim3(pl.Hkv, pl.B * max_qblk), dim3(256), lds, stream,
                       scores_in, sel, cnt, cu_k, cu_q, max_seqlen_q, max_qblk, pl.Lmax, pl.Hkv,
                       pl.max_nb, pl.max_sel, pl.topk, pl.wblocks);
    return hipGetLastError();
}

}  // namespace nosa
