// nosa_prefill.hip -- CDNA4 (gfx950) kernels of the chunked sparse prefill:
// a chunk of Lq queries at the end of a sequence's context, taken in query
// blocks of 64 consecutive queries from the chunk start.  For every
// (sequence, query block, KV head) -- a "pair" below -- the method runs as in
// decode with the query block in place of the single query
// [page "NOSA技术架构解析", section 1.3: the fully sparse mode also prefills
// sparsely; page "NOSA-1B 性能基准全解析", sections 三.2-三.3 for the steps]:
//   * pooled-key scores of every query of the block and every head of the
//     group, softmax per (query, head) over the keys that query can see
//     (window end 16j + 32 <= p + 1), summed over the block's queries and
//     the group's heads, mean-pooled into 64-token block importance;
//   * top-k over the blocks before the window, the window being the 16 blocks
//     ending at the block of the query block's last query;
//   * exact attention of every query over the kept blocks, causal (t <= p).
// Kernels: pf_score_kernel<1> (per-row (max, sum exp2) partials per key
// split), pf_score_kernel<2> (column sums of exp2(z - lse_row) per key),
// pf_pool_kernel (block importance), the shared selector, pf_attend_kernel
// or, for launches of one workgroup per CU or fewer, pf_attend_halves_kernel.
// All contractions run on v_mfma_f32_16x16x32_bf16 with rows = (query, head)
// pairs of the block in tiles of 16.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nosa_device.h"

namespace nosa {

// Timeline build (NOSA_TIMELINE, the benchmark's timeline mode; the NOSA
// library has none of this): thread 0 of each workgroup of the prefill
// launches (0: scoring pass 1, 1: pass 2, 2: attention, 3: pooling)
// stamps the wall clock when the workgroup
// starts and when it leaves the kernel, and records its XCD and its
// hardware id (CU, SIMD, wave slot), in pf_tl[launch][workgroup][0 .. 3].
#ifdef NOSA_TIMELINE
constexpr int kPfTlGroups = 8192;
__device__ unsigned long long pf_tl[4][kPfTlGroups][4];
struct PfTlScope {
    int launch;
    __device__ explicit PfTlScope(int l) : launch(l)
    {
        __builtin_amdgcn_sched_barrier(0);
        if (threadIdx.x == 0 && blockIdx.x < kPfTlGroups) {
            pf_tl[launch][blockIdx.x][0] = wall_clock64();
            pf_tl[launch][blockIdx.x][2] = (unsigned)__builtin_amdgcn_s_getreg(30740);  // XCC_ID
            pf_tl[launch][blockIdx.x][3] = (unsigned)__builtin_amdgcn_s_getreg(63492);  // HW_ID
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __device__ ~PfTlScope()
    {
        __builtin_amdgcn_sched_barrier(0);
        if (threadIdx.x == 0 && blockIdx.x < kPfTlGroups) pf_tl[launch][blockIdx.x][1] = wall_clock64();
    }
};
#define PF_TL_SCOPE(launch) PfTlScope pf_tl_scope_(launch)
#else
#define PF_TL_SCOPE(launch) \
    do {                    \
    } while (0)
#endif

constexpr int kQB = 64;   // queries per query block
constexpr int kChunk = kPfChunk;                       // pooled keys staged in LDS at a time
constexpr int kMaxSpan = kPfChunk * kPfMaxSpanChunks;  // pooled keys per scoring workgroup at most
constexpr int kPfFoldSplits = 16;  // key splits up to which pass 2 merges the row partials itself
constexpr float kPfRescale = 8.f;  // exponent headroom before the attention rescales (log2)

struct PfArgs {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const uint16_t* kc_pool;
    const int32_t* table;
    const int32_t* cu_k;
    const int32_t* cu_q;
    const int32_t* qbase;  // [B] first q / out row of each sequence, or null: cu_q
    int max_blocks, Lmax, Lqmax, B, Hq, Hkv, G, max_qblk;
    float scale_log2;
    float inv_g;     // 1 / G (rounded)
    int rows;        // 64 * G rows per pair: row = query * G + head
    int row_groups;  // workgroups over the rows of a pair
    int key_splits;  // workgroups over the pooled keys of a pair
    int span;        // pooled keys per such workgroup, a multiple of kChunk
    int zlen;        // key_splits * span
    float2* part;    // [pairs][rows][key_splits] per-row (max, sum exp2)
    float* rlse;     // [pairs][rows] lse (log2 units) of each row's scoring softmax
    float* colsum;   // [pairs][row_groups][zlen] per-key sums over a row group
    float* scores;   // [pairs][max_nb] block importance
    int max_nb;
    const int32_t* sel;  // [pairs][max_sel]
    const int32_t* cnt;  // [pairs]
    int max_sel;
    float* out;  // [total_q][Hq][D]
    float* lse;  // [total_q][Hq] or null
};

// Geometry of one pair.
struct PfPair {
    int s, r, g;
    int L, Lq, q0;   // KV length, chunk length, first q row of the sequence
    int p0, nq;      // position of the block's first query, queries in the block
    int nck;         // pooled keys visible to the block's last query
    int nb;          // blocks up to the block of the last query
    bool empty;
};

__device__ __forceinline__ PfPair pf_pair(const PfArgs& a, int pair)
{
    PfPair P;
    P.g = pair % a.Hkv;
    const int sr = pair / a.Hkv;
    P.s = sr / a.max_qblk;
    P.r = sr % a.max_qblk;
    P.L = seq_len(a.cu_k, P.s, a.Lmax);
    int Lq = a.cu_q[P.s + 1] - a.cu_q[P.s];
    Lq = Lq < 0 ? 0 : (Lq > a.Lqmax ? a.Lqmax : Lq);
    P.Lq = Lq < P.L ? Lq : P.L;
    P.q0 = a.qbase ? a.qbase[P.s] : a.cu_q[P.s];
    P.p0 = P.L - P.Lq + kQB * P.r;
    const int left = P.Lq - kQB * P.r;
    P.nq = left < kQB ? left : kQB;
    P.empty = P.nq <= 0;
    const int p_last = P.p0 + (P.nq > 0 ? P.nq : 1) - 1;
    P.nck = dev_num_keys(p_last + 1);
    P.nb = p_last / BS + 1;
    return P;
}

// ------------------------------------------------------------- scoring ---

// The pooled-key pages of a workgroup's span go through LDS a chunk of
// kChunk keys (32 pages) at a time, in two buffers: chunk c + 1 is copied by
// direct global-to-LDS loads while chunk c is multiplied.  Each 1 KB page is
// padded to kPfPageStride uint4, so a key tile's operand reads (16 keys over
// four pages, four chunks) fall on distinct banks in every group of eight
// lanes.
constexpr int kPfPageStride = (1024 + 64) / 16;
constexpr int kChunkPages = kChunk / SL;

struct PfScoreLds {
    float lse[32 * 16];                  // per row of the workgroup (pass 2)
    float ksum[2][4][kChunk];            // per chunk parity, wave and key (pass 2)
    int32_t pages[kMaxSpan / SL];        // page of each group of SL pooled keys of the span
};
typedef uint4 PfChunkBuf[kChunkPages][kPfPageStride];

// max(a, b, c) without canonicalising the operands (NaN propagates, which
// the products never are); gfx950 issues it as one v_maximum3_f32.
// Waits until every global-to-LDS copy this wave has issued has written the
// LDS.  Such a copy is counted by the vector-memory counter, and a barrier
// does not wait for it; every wave therefore waits for its own copies before
// the barrier after which the other waves read them (the compiler waits only
// where the same wave reads what it copied).
__device__ __forceinline__ void wait_lds_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// lse (log2 units) of one row's scoring softmax from its n pass-1 partials
// (max, sum exp2), merged in split order 16 at a time (a batch's loads all in
// flight); +inf for a row without visible keys (pass 2 then adds nothing).
__device__ __forceinline__ float row_lse(const float2* __restrict__ pp, int n)
{
    float m = -INFINITY, acc = 0.f;
    for (int i0 = 0; i0 < n; i0 += 16) {
        float2 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = i0 + u < n ? pp[i0 + u] : make_float2(-INFINITY, 0.f);
        float mb = m;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (v[u].y > 0.f) mb = fmaxf(mb, v[u].x);
        if (mb == -INFINITY) continue;
        acc = m == -INFINITY ? 0.f : acc * fexp2(m - mb);
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (v[u].y > 0.f) acc += v[u].y * fexp2(v[u].x - mb);
        m = mb;
    }
    return acc > 0.f ? m + log2f(acc) : INFINITY;
}

// Wave priority from a workgroup's progress through its steps (done of
// total, wave-uniform): 3 in the first half, 2 to three quarters, 1 to seven
// eighths, 0 in the last eighth.  Two workgroups share each CU, and at equal
// priority a SIMD issues the older wave first: the first-dispatched
// workgroup of every CU would finish well ahead of the other, which then runs
// alone on the CU.  Ranking the waves by progress lets the one behind catch
// up at each threshold, so they part only in the last eighth.
__device__ __forceinline__ void progress_priority(int done, int total)
{
    if (2 * done < total)
        __builtin_amdgcn_s_setprio(3);
    else if (4 * done < 3 * total)
        __builtin_amdgcn_s_setprio(2);
    else if (8 * done < 7 * total)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Workgroup = 4 waves x RTW row tiles of 16 rows, over the `span` pooled keys
// of one key split.  PASS 1 writes per-row (max, sum exp2) over the split's
// visible keys; PASS 2 writes, for every key, sum over the workgroup's rows of
// exp2(z - lse_row) (lse from pf_lse_kernel), in a fixed order.
template <int PASS, int RTW>
__global__ __launch_bounds__(256, 2) void pf_score_kernel(PfArgs a)
{
    PF_TL_SCOPE(PASS - 1);
    __shared__ PfScoreLds sh;
    // the two chunk buffers are distinct objects: a read of one is then known
    // not to wait for the copy in flight into the other
    __shared__ PfChunkBuf kc_even, kc_odd;
    const int per_pair = a.row_groups * a.key_splits;
    const int pair = blockIdx.x / per_pair;
    const int rg = (blockIdx.x % per_pair) / a.key_splits;
    const int ks = blockIdx.x % a.key_splits;
    const PfPair P = pf_pair(a, pair);
    if (P.empty) return;  // nothing of the pair is read (the pooling skips it)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, kq = lane >> 4;
    const int key_lo = ks * a.span;
    const int key_hi = min(key_lo + a.span, P.nck);
    const int nchunks = key_hi > key_lo ? (key_hi - key_lo + kChunk - 1) / kChunk : 0;
    const int32_t* trow = a.table + (size_t)P.s * a.max_blocks;
    const int row_tile0 = (rg * 4 + wave) * RTW;  // first row tile of this wave
    const int wg_row0 = rg * 4 * RTW * 16;        // first row of the workgroup
    // page ids of the span's pooled keys (page 0 past key_hi: read, masked)
    for (int x = tid; x < nchunks * kChunkPages; x += 256) {
        const int key = key_lo + SL * x;
        sh.pages[x] = key < key_hi ? trow[key / SL] : 0;
    }
    if (PASS == 2) {
        // lse of every row of the workgroup (+inf past the pair's rows: the
        // row adds exp2(-inf) = 0), from pf_lse_kernel or, with few key
        // splits, from the partials here
        for (int x = tid; x < 4 * RTW * 16; x += 256) {
            const int row = wg_row0 + x;
            const size_t pr = (size_t)pair * a.rows + row;
            float l = INFINITY;
            if (row < a.rows) l = a.rlse ? a.rlse[pr] : row_lse(a.part + pr * a.key_splits, a.key_splits);
            sh.lse[x] = l;
        }
    }
    __syncthreads();
    // chunk c into buffer c & 1: wave w copies pages w, w + 4, ..., each page
    // one 1 KB load straight into LDS
    const uint16_t* kc_lane = a.kc_pool + (size_t)P.g * SL * D + lane * 8;
    const size_t page_elems = (size_t)a.Hkv * SL * D;
    auto copy_chunk = [&](int c, uint4* __restrict__ dst) {
#pragma unroll
        for (int i = 0; i < kChunkPages / 4; ++i) {
            const int x = wave + 4 * i;
            const int pg = __builtin_amdgcn_readfirstlane(sh.pages[c * kChunkPages + x]);
            __builtin_amdgcn_global_load_lds(kc_lane + (size_t)pg * page_elems,
                                             (__attribute__((address_space(3))) void*)(dst + x * kPfPageStride), 16,
                                             0, 0);
        }
    };
    if (nchunks > 0) copy_chunk(0, &kc_even[0][0]);

    // query operand of the wave's row tiles; a row without a query (past the
    // block's queries or the pair's rows) loads the block's last query: its
    // products are masked by position (pass 1) or weighted by
    // exp2(-lse) = 0 (pass 2).  qi = row / G from a float reciprocal: exact,
    // the quotient being at least 1 / (2G) from an integer.
    bf16x8 qb[RTW][4];
    int qpos[RTW];  // query position of this lane's row r in each tile (-1: none)
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
        const int row = (row_tile0 + u) * 16 + r;
        const int qi = (int)(((float)row + 0.5f) * a.inv_g), h = row - qi * a.G;
        const bool ok = row < a.rows && qi < P.nq;
        qpos[u] = ok ? P.p0 + qi : -1;
        const uint16_t* qr =
            a.q + ((size_t)(P.q0 + kQB * P.r + min(qi, P.nq - 1)) * a.Hq + P.g * a.G + h) * D + kq * 8;
#pragma unroll
        for (int st = 0; st < 4; ++st) qb[u][st] = as_bf16x8(ldg16(qr + st * 32));
    }
    // The wave's rows ascend with the query: every row holds a query when its
    // last row does, and its first row's query is the earliest.
    const int wave_row_last = (row_tile0 + RTW) * 16 - 1;
    const bool wave_full = wave_row_last < a.rows && wave_row_last / a.G < P.nq;
    const int wave_p0 = P.p0 + row_tile0 * 16 / a.G;
    const float sc = a.scale_log2;
    // Is the pair of key tiles from kt (32 keys) visible to every row of the
    // wave?  Then no element is tested (key < n_c(p + 1)  <=>  16 key + 32 <=
    // p + 1); tiles near the diagonal, the span's end and absent rows take
    // the tested path.
    auto pair_fast = [&](int kt) {
        return wave_full && kt + 32 <= key_hi && (kt + 31) * kPoolS + kPoolK <= wave_p0 + 1;
    };
    // Operand of the key tile from kt in the chunk from c0 (buffer cb): lane r
    // holds key kt + r, chunk 4 st + kq.  kt - c0 is a multiple of 16, so the
    // key sits in staged page (kt - c0) / SL + r / SL, slot r % SL; every tile
    // of the chunk lies inside its staged pages.
    const int kl = (r / SL) * kPfPageStride + kq * SL + r % SL;
    auto load_tile = [&](const uint4* __restrict__ buf, int rel, uint4 (&kf)[4]) {
        const uint4* kp = buf + kl + (rel / SL) * kPfPageStride;
#pragma unroll
        for (int st = 0; st < 4; ++st) kf[st] = kp[st * 4 * SL];
    };

    if (PASS == 1) {
        // Products as (key, row) tiles: lane r holds row r, keys 4 kq + i.
        // Running state per row of every tile: a reference m_raw (a maximum
        // of raw products; the scale is positive) and s_run = sum of
        // exp2((z - m_raw) * scale), the scale folded into the exponent's fma.
        // The first pair of key tiles visible to the whole wave sets the
        // reference to the row maxima; later such pairs keep it (no maximum
        // is taken) unless a chunk's sums stop being finite -- a product more
        // than 2^128 above the reference -- when the chunk is done again
        // from its checkpoint with the maximum updated at every pair.
        float m_raw[RTW], s_run[RTW];
#pragma unroll
        for (int u = 0; u < RTW; ++u) {
            m_raw[u] = -INFINITY;
            s_run[u] = 0.f;
        }
        auto tested = [&](int kt, const uint4 (&kf)[4]) {
#pragma unroll
            for (int u = 0; u < RTW; ++u) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) c = mfma16(as_bf16x8(kf[st]), qb[u][st], c);
                float z[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kj = kt + 4 * kq + i;
                    const bool vis = qpos[u] >= 0 && kj < key_hi && kj * kPoolS + kPoolK <= qpos[u] + 1;
                    z[i] = vis ? c[i] : -INFINITY;
                }
                const float tmax = vmax3(vmax3(z[0], z[1], z[2]), z[3], -INFINITY);
                if (tmax != -INFINITY) {
                    const float mx = vmax3(m_raw[u], tmax, -INFINITY);
                    const float nm = -(mx * sc);
                    const float e = (fexp2(fmaf(z[0], sc, nm)) + fexp2(fmaf(z[1], sc, nm))) +
                                    (fexp2(fmaf(z[2], sc, nm)) + fexp2(fmaf(z[3], sc, nm)));
                    s_run[u] = fmaf(s_run[u], fexp2(fmaf(m_raw[u], sc, nm)), e);
                    m_raw[u] = mx;
                }
            }
        };
        // a visible pair with the maximum updated (sets the reference)
        auto pair_max = [&](const uint4 (&kf0)[4], const uint4 (&kf1)[4]) {
#pragma unroll
            for (int u = 0; u < RTW; ++u) {
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) s0 = mfma16(as_bf16x8(kf0[st]), qb[u][st], s0);
#pragma unroll
                for (int st = 0; st < 4; ++st) s1 = mfma16(as_bf16x8(kf1[st]), qb[u][st], s1);
                const float mx =
                    vmax3(vmax3(vmax3(vmax3(m_raw[u], s0[0], s0[1]), s0[2], s0[3]), s1[0], s1[1]), s1[2], s1[3]);
                const float nm = -(mx * sc);
                const float e0 = (fexp2(fmaf(s0[0], sc, nm)) + fexp2(fmaf(s0[1], sc, nm))) +
                                 (fexp2(fmaf(s0[2], sc, nm)) + fexp2(fmaf(s0[3], sc, nm)));
                const float e1 = (fexp2(fmaf(s1[0], sc, nm)) + fexp2(fmaf(s1[1], sc, nm))) +
                                 (fexp2(fmaf(s1[2], sc, nm)) + fexp2(fmaf(s1[3], sc, nm)));
                s_run[u] = fmaf(s_run[u], fexp2(fmaf(m_raw[u], sc, nm)), e0 + e1);
                m_raw[u] = mx;
            }
        };
        // a visible pair against the fixed reference
        auto pair_ref = [&](const uint4 (&kf0)[4], const uint4 (&kf1)[4]) {
#pragma unroll
            for (int u = 0; u < RTW; ++u) {
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) s0 = mfma16(as_bf16x8(kf0[st]), qb[u][st], s0);
#pragma unroll
                for (int st = 0; st < 4; ++st) s1 = mfma16(as_bf16x8(kf1[st]), qb[u][st], s1);
                const float nm = -(m_raw[u] * sc);
                const float e0 = (fexp2(fmaf(s0[0], sc, nm)) + fexp2(fmaf(s0[1], sc, nm))) +
                                 (fexp2(fmaf(s0[2], sc, nm)) + fexp2(fmaf(s0[3], sc, nm)));
                const float e1 = (fexp2(fmaf(s1[0], sc, nm)) + fexp2(fmaf(s1[1], sc, nm))) +
                                 (fexp2(fmaf(s1[2], sc, nm)) + fexp2(fmaf(s1[3], sc, nm)));
                s_run[u] += e0 + e1;
            }
        };
        bool have_ref = false;  // wave-uniform
        auto chunk = [&](int c, const uint4* __restrict__ cur, uint4* __restrict__ nxt) {
            wait_lds_copies();
            __syncthreads();  // chunk c in LDS; every wave done with chunk c - 1
            progress_priority(c, nchunks);
            if (c + 1 < nchunks) copy_chunk(c + 1, nxt);
            const int c0 = key_lo + c * kChunk, c1 = min(c0 + kChunk, key_hi);
            float m_chk[RTW], s_chk[RTW];
#pragma unroll
            for (int u = 0; u < RTW; ++u) {
                m_chk[u] = m_raw[u];
                s_chk[u] = s_run[u];
            }
            const bool ref_chk = have_ref;
            auto pass = [&](bool careful) {
                uint4 kf0[4], kf1[4];
                load_tile(cur, 0, kf0);
                load_tile(cur, 16, kf1);
                for (int kt = c0; kt < c1; kt += 32) {
                    if (pair_fast(kt)) {
                        if (have_ref && !careful) {
                            pair_ref(kf0, kf1);
                        } else {
                            pair_max(kf0, kf1);
                            have_ref = true;
                        }
                    } else {
                        tested(kt, kf0);
                        if (kt + 16 < key_hi) tested(kt + 16, kf1);
                    }
                    // the next pair of the chunk (the last pair reads itself again)
                    const int nx = min(kt - c0 + 32, kChunk - 32);
                    load_tile(cur, nx, kf0);
                    load_tile(cur, nx + 16, kf1);
                }
            };
            pass(false);
            bool bad = false;
#pragma unroll
            for (int u = 0; u < RTW; ++u) bad = bad || !(s_run[u] < INFINITY);
            if (__ballot(bad) != 0) {  // rare: from the checkpoint, maximum at every pair
#pragma unroll
                for (int u = 0; u < RTW; ++u) {
                    m_raw[u] = m_chk[u];
                    s_run[u] = s_chk[u];
                }
                have_ref = ref_chk;
                pass(true);
            }
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, &kc_even[0][0], &kc_odd[0][0]);
            if (c + 1 < nchunks) chunk(c + 1, &kc_odd[0][0], &kc_even[0][0]);
        }
        // per row: combine the four lanes (kq) that hold its keys, in log2
        // units: the halves swapped and merged, then the odd and even rows
        auto merge = [](float m, float s, float mo, float so, float& mr, float& sr) {
            const float mn = fmaxf(m, mo);
            sr = mn == -INFINITY ? 0.f : s * fexp2(m - mn) + so * fexp2(mo - mn);
            mr = mn;
        };
        auto swap32 = [](float x) {
            return __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        };
        auto swap16 = [](float x) {
            return __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        };
        float2* prow = a.part + ((size_t)pair * a.rows + row_tile0 * 16 + r) * a.key_splits + ks;
#pragma unroll
        for (int u = 0; u < RTW; ++u) {
            float m = m_raw[u] * sc, s = s_run[u];
            const auto hm = swap32(m), hs = swap32(s);
            merge(__uint_as_float(hm[0]), __uint_as_float(hs[0]), __uint_as_float(hm[1]), __uint_as_float(hs[1]), m, s);
            const auto qm = swap16(m), qs = swap16(s);
            merge(__uint_as_float(qm[0]), __uint_as_float(qs[0]), __uint_as_float(qm[1]), __uint_as_float(qs[1]), m, s);
            const int row = (row_tile0 + u) * 16 + r;
            if (kq == 0 && row < a.rows) prow[(size_t)u * 16 * a.key_splits] = make_float2(m, s);
        }
    } else {
        // Products as (row, key) tiles (operands swapped): lane r holds key r,
        // rows 4 kq + e, so a key's sum over rows adds within the lane and
        // then over the four lanes of the key.  The lse of those rows (the
        // four of a lane are adjacent in LDS) is read per tile.
        const float4* lse4 = reinterpret_cast<const float4*>(sh.lse) + wave * RTW * 4 + kq;
        auto neg_lse = [&](int u, float (&nl)[4]) {
            const float4 l = lse4[u * 4];
            nl[0] = -l.x;
            nl[1] = -l.y;
            nl[2] = -l.z;
            nl[3] = -l.w;
        };
        // row (query qi = row / G, position p0 + qi) sees key j when
        // 16 j + 32 <= p0 + qi + 1, i.e. when row >= (16 j + 31 - p0) G
        const int row_l = row_tile0 * 16 + 4 * kq;  // the lane's first row
        auto tested = [&](int kt, const uint4 (&kf)[4]) {
            const int key = kt + r;
            const int rmin = key < key_hi ? (key * kPoolS + kPoolK - 1 - P.p0) * a.G : 0x7fffffff;
            float cs = 0.f;
#pragma unroll
            for (int u = 0; u < RTW; ++u) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) c = mfma16(qb[u][st], as_bf16x8(kf[st]), c);
                float nl[4];
                neg_lse(u, nl);
#pragma unroll
                for (int e = 0; e < 4; ++e) cs += row_l + 16 * u + e >= rmin ? fexp2(fmaf(c[e], sc, nl[e])) : 0.f;
            }
            return cs;
        };
        // sum over the four lanes of a key (lanes r, r + 16, r + 32, r + 48):
        // the halves swapped and added, then the odd and even rows
        auto lanes4_sum = [](float x) {
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
            const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            return __uint_as_float(q[0]) + __uint_as_float(q[1]);
        };
        // one key tile at a time
        auto step = [&](int kt, int rel, int cb, const uint4 (&kf)[4]) {
            float cs = 0.f;
            if (wave_full && kt + 16 <= key_hi && (kt + 15) * kPoolS + kPoolK <= wave_p0 + 1) {
#pragma unroll
                for (int u = 0; u < RTW; ++u) {
                    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 4; ++st) c = mfma16(qb[u][st], as_bf16x8(kf[st]), c);
                    float nl[4];
                    neg_lse(u, nl);
#pragma unroll
                    for (int e = 0; e < 4; ++e) cs += fexp2(fmaf(c[e], sc, nl[e]));
                }
            } else {
                cs = tested(kt, kf);
            }
            cs = lanes4_sum(cs);
            if (kq == 0) sh.ksum[cb][wave][rel + r] = cs;
        };
        // a chunk's column sums leave once every wave has written them
        float* dst = a.colsum + ((size_t)pair * a.row_groups + rg) * a.zlen;
        auto store_chunk = [&](int c) {
            const int x = tid, kj = key_lo + c * kChunk + x;
            if (x < kChunk && kj < key_hi) {
                const int cb = c & 1;
                dst[kj] = ((sh.ksum[cb][0][x] + sh.ksum[cb][1][x]) + sh.ksum[cb][2][x]) + sh.ksum[cb][3][x];
            }
        };
        auto chunk = [&](int c, const uint4* __restrict__ cur, uint4* __restrict__ nxt) {
            wait_lds_copies();
            __syncthreads();  // chunk c in LDS; every wave done with chunk c - 1
            progress_priority(c, nchunks);
            if (c + 1 < nchunks) copy_chunk(c + 1, nxt);
            if (c > 0) store_chunk(c - 1);
            const int c0 = key_lo + c * kChunk, c1 = min(c0 + kChunk, key_hi), cb = c & 1;
            for (int kt = c0; kt < c1; kt += 16) {
                uint4 kf[4];
                load_tile(cur, kt - c0, kf);
                step(kt, kt - c0, cb, kf);
            }
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, &kc_even[0][0], &kc_odd[0][0]);
            if (c + 1 < nchunks) chunk(c + 1, &kc_odd[0][0], &kc_even[0][0]);
        }
        __syncthreads();
        if (nchunks > 0) store_chunk(nchunks - 1);
    }
}

// lse of every row's scoring softmax (row_lse), one thread per (pair, row);
// used when the pairs have many key splits.
__global__ __launch_bounds__(256) void pf_lse_kernel(PfArgs a, int total)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const PfPair P = pf_pair(a, t / a.rows);
    a.rlse[t] = P.empty ? INFINITY : row_lse(a.part + (size_t)t * a.key_splits, a.key_splits);
}

// Block importance of a pair: sigma[j] = sum over row groups (fixed order) of
// the column sums; importance of block b = mean of sigma over the keys 4b-1 ..
// 4b+3 that the block's last query sees.  A workgroup per (pair, 256 blocks):
// thread t takes block b = 256 s + t, sums its own keys 4b .. 4b+3 (one
// 16-byte load per row group, all in flight together) and takes key 4b-1 from
// its left neighbour through LDS; thread 0 of a later slice sums that key
// itself, in the same order, so every sigma[j] is one fixed sum.  The loads
// need only the workspace bounds (keys past n_c are masked afterwards), so they
// leave before the pair's lengths are in.
constexpr int kPoolBlocks = 256;

__global__ __launch_bounds__(256) void pf_pool_kernel(PfArgs a, int slices)
{
    PF_TL_SCOPE(3);
    __shared__ float key_w[kPoolBlocks];
    const int tid = threadIdx.x;
    const int pair = blockIdx.x / slices;
    const int b = (blockIdx.x - pair * slices) * kPoolBlocks + tid;
    const int j0 = 4 * b;
    const float* cs = a.colsum + (size_t)pair * a.row_groups * a.zlen;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float left = 0.f;  // sigma[j0 - 1], summed here by thread 0 of a later slice
    const bool own = j0 < a.zlen, edge = tid == 0 && b > 0 && j0 - 1 < a.zlen;
    for (int q0 = 0; q0 < a.row_groups; q0 += 8) {
        float4 w[8];
        float e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool in = q0 + k < a.row_groups;
            const float* row = cs + (size_t)(q0 + k) * a.zlen;
            w[k] = in && own ? *reinterpret_cast<const float4*>(row + j0) : make_float4(0.f, 0.f, 0.f, 0.f);
            e[k] = in && edge ? row[j0 - 1] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (q0 + k >= a.row_groups) break;
            v.x += w[k].x;
            v.y += w[k].y;
            v.z += w[k].z;
            v.w += w[k].w;
            left += e[k];
        }
    }
    key_w[tid] = v.w;
    const PfPair P = pf_pair(a, pair);
    const int nb = P.empty ? 0 : P.nb;
    const int nck = P.empty ? 0 : P.nck;
    __syncthreads();
    if (tid > 0) left = key_w[tid - 1];
    float I = -INFINITY;
    if (b < nb) {
        const int jlo = max(j0 - 1, 0), jhi = min(j0 + 3, P.nck - 1);
        if (jlo <= jhi) {
            const float mine = j0 < nck ? (v.x + (j0 + 1 < nck ? v.y : 0.f)) +
                                              ((j0 + 2 < nck ? v.z : 0.f) + (j0 + 3 < nck ? v.w : 0.f))
                                        : 0.f;
            const float prev = b > 0 && j0 - 1 < nck ? left : 0.f;
            I = (mine + prev) / (float)(jhi - jlo + 1);
        }
    }
    if (b < a.max_nb) a.scores[(size_t)pair * a.max_nb + b] = I;
}

// ------------------------------------------------------------ attention ---

// A K and a V page in LDS, in the pages' own operand order (a straight copy):
// the fragment of QK^T tile t, k-step st is run 4t + st, that of PV k-step
// u, channel tile nt is run 8u + nt, lane l at byte 16 l of its run, so a
// wave's fragment read is 1 KB of consecutive LDS.
typedef uint16_t PfPageBuf[BS * D];

// One wave's rows of a row group: two row tiles of 16 (query, head) rows, the
// query operand of each, and the online-softmax state of each row (lane r of
// each tile): m_run, the reference point of the exponentials (log2 units),
// l_run, the lane's part of sum 2^(z - m_run), and O^T (lane: row r, channels
// 16 nt + 4 kq + e).  The reference moves only when a row's maximum passes it
// by more than kPfRescale, so exponentials stay below 2^kPfRescale and the
// accumulators are rarely rescaled; any reference gives the same quotient
// O / l and lse = m + log2 l.
struct PfAttnRows {
    bf16x8 qb[2][4];
    int qpos[2];  // query position of the row (-1: no query)
    int qrow[2];  // its row of q, out and lse (-1: no query)
    float m_run[2], l_run[2];
    f32x4 o[2][8];
};

// The pair's (block, page) list into LDS (entries outside the pair's blocks
// become (-1, 0)); returns the number of entries.
__device__ __forceinline__ int pf_attn_list(const PfArgs& a, const PfPair& P, int pair, int2* list,
                                            int tid, int nt)
{
    const int32_t* trow = a.table + (size_t)P.s * a.max_blocks;
    const int n = P.empty ? 0 : min(a.cnt[pair], a.max_sel);
    const int32_t* sl = a.sel + (size_t)pair * a.max_sel;
    for (int x = tid; x < n; x += nt) {
        int b = sl[x];
        if (b < 0 || b >= P.nb) b = -1;
        list[x] = make_int2(b, b >= 0 ? trow[b] : 0);
    }
    return n;
}

// Query operands of row tiles tile0 and tile0 + 1 of the pair, and an empty
// softmax state.
__device__ __forceinline__ void pf_attn_rows_init(PfAttnRows& R, const PfArgs& a, const PfPair& P,
                                                  int tile0, int r, int kq)
{
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int row = (tile0 + u) * 16 + r;
        const int qi = row / a.G, h = row % a.G;
        const bool ok = !P.empty && row < a.rows && qi < P.nq;
        R.qpos[u] = ok ? P.p0 + qi : -1;
        R.qrow[u] = ok ? (P.q0 + kQB * P.r + qi) * a.Hq + P.g * a.G + h : -1;
        const uint16_t* qr = a.q + (size_t)(ok ? R.qrow[u] : 0) * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 w = ok ? ldg16(qr + st * 32 + kq * 8) : make_uint4(0, 0, 0, 0);
            R.qb[u][st] = as_bf16x8(w);
        }
        R.m_run[u] = -INFINITY;
        R.l_run[u] = 0.f;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) R.o[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Smallest query position of the wave's rows (pages entirely at or before it
// need no causal mask), wave-uniform.
__device__ __forceinline__ int pf_attn_pmin(const PfAttnRows& R)
{
    int pmin = min(R.qpos[0] < 0 ? 0x7fffffff : R.qpos[0], R.qpos[1] < 0 ? 0x7fffffff : R.qpos[1]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) pmin = min(pmin, __shfl_xor(pmin, off));
    return __builtin_amdgcn_readfirstlane(pmin);
}

// Page idx of the list into LDS by the four waves wq = 0 .. 3 of a page's
// readers: wave wq copies the 1 KB runs wq, wq + 4, wq + 8, wq + 12 of the K
// and of the V page (past the list, page 0 is copied and never used).
__device__ __forceinline__ void pf_copy_page(const PfArgs& a, const PfPair& P, const int2* list, int n,
                                             int idx, int wq, int lane, uint16_t* __restrict__ kd,
                                             uint16_t* __restrict__ vd)
{
    const int page = __builtin_amdgcn_readfirstlane(idx < n ? list[idx].y : 0);
    const size_t base = ((size_t)page * a.Hkv + P.g) * BS * D + lane * 8;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
        const int c = __builtin_amdgcn_readfirstlane(wq) + 4 * c4;
        __builtin_amdgcn_global_load_lds(a.k_pool + base + c * 512,
                                         (__attribute__((address_space(3))) void*)(kd + c * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a.v_pool + base + c * 512,
                                         (__attribute__((address_space(3))) void*)(vd + c * 512), 16, 0, 0);
    }
}

// maximum over the four lanes of a row (lanes r, r + 16, r + 32, r + 48)
__device__ __forceinline__ float lanes4_max(float x)
{
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = vmax3(__uint_as_float(h[0]), __uint_as_float(h[1]), -INFINITY);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax3(__uint_as_float(q[0]), __uint_as_float(q[1]), -INFINITY);
}

// The wave's rows over block b_cur, whose K and V pages are in LDS (kc, vc):
// rows_full = every row of the workgroup holds a query, pmin = the wave's
// smallest query position.
__device__ __forceinline__ void pf_attn_page(PfAttnRows& R, const PfPair& P, float sc, bool rows_full,
                                             int pmin, int lane, const uint16_t* __restrict__ kc,
                                             const uint16_t* __restrict__ vc, int b_cur)
{
    const int kq = lane >> 4;
    // S^T = K q^T, raw products: lane holds row r, keys of tile t as
    // mapped by the K page layout; K fragments from LDS, shared
    float x[2][4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        bf16x8 kf[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
            kf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(kc + ((t * 4 + st) * 64 + lane) * 8));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) acc = mfma16(kf[st], R.qb[u][st], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[u][t][i] = acc[i];
        }
    }
    if (!(rows_full && b_cur * BS + BS - 1 <= pmin && b_cur * BS + BS <= P.L)) {
        // causal and length mask (page near the diagonal, the sequence
        // end, or rows without a query)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = b_cur * BS + 32 * (t >> 1) + 8 * kq + 4 * (t & 1) + i;
                    if (!(R.qpos[u] >= 0 && tk <= R.qpos[u] && tk < P.L)) x[u][t][i] = -INFINITY;
                }
    }
    bf16x8 pa[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float bm = vmax3(vmax3(x[u][0][0], x[u][0][1], x[u][0][2]), x[u][0][3], -INFINITY);
#pragma unroll
        for (int t = 1; t < 4; ++t) bm = vmax3(vmax3(bm, x[u][t][0], x[u][t][1]), x[u][t][2], x[u][t][3]);
        bm = lanes4_max(bm) * sc;  // the row's maximum, log2 units
        if (__ballot(bm > R.m_run[u] + kPfRescale) != 0) {
            const float m_new = fmaxf(R.m_run[u], bm);
            // 1 for an unmoved row (also one still at -inf), 0 from -inf
            const float alpha = m_new == R.m_run[u] ? 1.f : fexp2(R.m_run[u] - m_new);
            R.l_run[u] *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) R.o[u][nt][e] *= alpha;
            R.m_run[u] = m_new;
        }
        // a row with nothing visible yet (m_run = -inf) has every z = -inf
        const float nm = R.m_run[u] == -INFINITY ? 0.f : -R.m_run[u];
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = fexp2(fmaf(x[u][t][i], sc, nm));
                x[u][t][i] = e;
                psum += e;
            }
        R.l_run[u] += psum;
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pa[u][uu][i] = (__bf16)x[u][2 * uu][i];
                pa[u][uu][4 + i] = (__bf16)x[u][2 * uu + 1][i];
            }
    }
    // O^T += V^T P^T (operands swapped): lane holds row r, channels
    // 16 nt + 4 kq + e; V fragments from LDS, shared by both row tiles
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4*>(vc + ((uu * 8 + nt) * 64 + lane) * 8));
#pragma unroll
            for (int u = 0; u < 2; ++u) R.o[u][nt] = mfma16(vf, pa[u][uu], R.o[u][nt]);
        }
}

// A row's sum of 2^(z - m_run) over its four lanes.
__device__ __forceinline__ float pf_row_sum(float l)
{
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    return l;
}

// Workgroups are dealt to the eight XCDs round-robin by index, so index b is
// mapped to the logical workgroup (b % 8) * per_xcd + b / 8: the attn_groups
// workgroups of a pair, which read the same pages, run on one XCD and share
// its L2.  Indices past the last logical workgroup exit at once.
__device__ __forceinline__ int pf_attn_lid(int per_xcd)
{
    return (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
}

// Workgroup = 4 waves x 2 row tiles (128 rows) of one pair; loops over the
// pair's kept pages, each staged once through LDS for all 8 row tiles.  The
// (block, page) list goes to LDS first; page i + 1 is copied by direct
// global-to-LDS loads into the other buffer while page i is computed, so one
// barrier per page suffices (the two buffers are distinct objects: a read
// of one is known not to wait for the copy into the other).  For launches of
// more than kPfSplitGroups workgroups (two or more per CU).
__global__ __launch_bounds__(256, 2) void pf_attend_kernel(PfArgs a, int attn_groups, int total,
                                                        int per_xcd)
{
    PF_TL_SCOPE(2);
    __shared__ PfPageBuf k_even, v_even, k_odd, v_odd;
    extern __shared__ __align__(16) char smem[];
    int2* list = reinterpret_cast<int2*>(smem);  // [max_sel] (block, page)
    const int lid = pf_attn_lid(per_xcd);
    if (lid >= total) return;
    const int pair = lid / attn_groups, ag = lid % attn_groups;
    const PfPair P = pf_pair(a, pair);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = pf_attn_list(a, P, pair, list, tid, 256);
    PfAttnRows R;
    pf_attn_rows_init(R, a, P, (ag * 4 + wave) * 2, lane & 15, lane >> 4);
    __syncthreads();  // the list
    const bool rows_full = __syncthreads_and(R.qpos[0] >= 0 && R.qpos[1] >= 0);
    const int pmin = pf_attn_pmin(R);
    const float sc = a.scale_log2;
    if (n > 0) pf_copy_page(a, P, list, n, 0, wave, lane, k_even, v_even);
    auto step = [&](int idx, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    uint16_t* __restrict__ kn, uint16_t* __restrict__ vn) {
        wait_lds_copies();
        __syncthreads();  // page idx in LDS; every wave done with page idx - 1
        progress_priority(idx, n);
        if (idx + 1 < n) pf_copy_page(a, P, list, n, idx + 1, wave, lane, kn, vn);
        const int b = list[idx].x;
        if (b >= 0) pf_attn_page(R, P, sc, rows_full, pmin, lane, kc, vc, b);
    };
    for (int idx = 0; idx < n; idx += 2) {
        step(idx, k_even, v_even, k_odd, v_odd);
        if (idx + 1 < n) step(idx + 1, k_odd, v_odd, k_even, v_even);
    }
    // normalise and store: lane holds O[row r][channels 16 nt + 4 kq + e]
    const int kq = lane >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float l = pf_row_sum(R.l_run[u]);
        if (R.qrow[u] < 0) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (kq == 0 && a.lse) a.lse[R.qrow[u]] = l > 0.f ? (R.m_run[u] + log2f(l)) * kLn2 : -INFINITY;
        float* dst = a.out + (size_t)R.qrow[u] * D + 4 * kq;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *reinterpret_cast<float4*>(dst + nt * 16) =
                make_float4(R.o[u][nt][0] * inv, R.o[u][nt][1] * inv, R.o[u][nt][2] * inv, R.o[u][nt][3] * inv);
    }
}

// Static LDS of pf_attend_halves_kernel, rounded up: eight page buffers, half
// 1's row states and alignment (the pick list comes on top, dynamically).
constexpr size_t kPfHalvesLds = 8 * sizeof(PfPageBuf) + 4096;

// For launches of at most kPfSplitGroups workgroups (one per CU or fewer, so
// one row group's pages would be a latency-bound chain): workgroup = 8 waves
// over the same 128 rows as pf_attend_kernel's, waves 0-3 (half 0) attending
// the first n/2 kept pages and waves 4-7 (half 1) the rest, each half double
// buffered in its own four page buffers.  Every wave runs the same number of
// steps -- that of half 1, the longer half -- and of barriers, all outside
// the branch on the half; a step past a half's last page only waits at the
// barrier.  At the end half 1 leaves each row's (m, l) and O^T in LDS, and
// half 0 combines the two states (a row's weights 2^(m_k - M), M the larger
// reference), normalises and stores.  The two halves of a row group thus
// share one CU and end together, and no partial goes through memory.
__global__ __launch_bounds__(512, 1) void pf_attend_halves_kernel(PfArgs a, int attn_groups, int total,
                                                               int per_xcd)
{
    PF_TL_SCOPE(2);
    __shared__ PfPageBuf k_even0, v_even0, k_odd0, v_odd0, k_even1, v_even1, k_odd1, v_odd1;
    __shared__ float2 ml1[4][2][16];  // half 1's (m_run, row sum) per wave, row tile, row
    extern __shared__ __align__(16) char smem[];
    int2* list = reinterpret_cast<int2*>(smem);  // [max_sel] (block, page)
    const int lid = pf_attn_lid(per_xcd);
    if (lid >= total) return;
    const int pair = lid / attn_groups, ag = lid % attn_groups;
    const PfPair P = pf_pair(a, pair);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, wq = wave & 3;
    const int r = lane & 15, kq = lane >> 4;
    const int n = pf_attn_list(a, P, pair, list, tid, 512);
    PfAttnRows R;
    pf_attn_rows_init(R, a, P, (ag * 4 + wq) * 2, r, kq);
    __syncthreads();  // the list
    const bool rows_full = __syncthreads_and(R.qpos[0] >= 0 && R.qpos[1] >= 0);
    const int pmin = pf_attn_pmin(R);
    const float sc = a.scale_log2;
    const int i0 = half ? n / 2 : 0, i1 = half ? n : n / 2;  // this half's list entries
    const int steps = n - n / 2;                             // half 1's count, >= half 0's
    // step j of this half without its barrier: the next page's copy, then
    // entry i0 + j (if the half has it) from kc, vc
    auto work = [&](int j, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    uint16_t* __restrict__ kn, uint16_t* __restrict__ vn) {
        const int idx = i0 + j;
        if (idx + 1 < i1) pf_copy_page(a, P, list, n, idx + 1, wq, lane, kn, vn);
        if (idx < i1) {
            const int b = list[idx].x;
            if (b >= 0) pf_attn_page(R, P, sc, rows_full, pmin, lane, kc, vc, b);
        }
    };
    // one copy of the step for both halves, on pointers selected by the half
    // (two inlined copies, one per half, would not fit the registers); each
    // pointer is one of two distinct buffers, so a read of the current page
    // is still known not to wait for the copy into the other
    uint16_t* const ke = half ? k_even1 : k_even0;
    uint16_t* const ve = half ? v_even1 : v_even0;
    uint16_t* const ko = half ? k_odd1 : k_odd0;
    uint16_t* const vo = half ? v_odd1 : v_odd0;
    if (i1 > i0) pf_copy_page(a, P, list, n, i0, wq, lane, ke, ve);
    for (int j = 0; j < steps; j += 2) {
        wait_lds_copies();
        __syncthreads();  // step j's page in LDS; every wave done with step j - 1
        work(j, ke, ve, ko, vo);
        if (j + 1 < steps) {
            wait_lds_copies();
            __syncthreads();
            work(j + 1, ko, vo, ke, ve);
        }
    }
    float lsum[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) lsum[u] = pf_row_sum(R.l_run[u]);
    wait_lds_copies();
    __syncthreads();  // every wave done with the page buffers
    // half 1's O^T of wave wq in its page buffer wq: float4 (u * 8 + nt) * 64 + lane
    uint16_t* hand = wq == 0 ? k_even1 : wq == 1 ? v_even1 : wq == 2 ? k_odd1 : v_odd1;
    float4* h4 = reinterpret_cast<float4*>(hand);
    if (half) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                h4[(u * 8 + nt) * 64 + lane] = make_float4(R.o[u][nt][0], R.o[u][nt][1], R.o[u][nt][2], R.o[u][nt][3]);
            if (kq == 0) ml1[wq][u][r] = make_float2(R.m_run[u], lsum[u]);
        }
    }
    __syncthreads();  // half 1's states in LDS
    if (half) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (R.qrow[u] < 0) continue;
        const float2 p1 = ml1[wq][u][r];
        const float m0 = R.m_run[u];
        const float M = fmaxf(m0, p1.x);
        const float w0 = m0 == -INFINITY ? 0.f : fexp2(m0 - M);
        const float w1 = p1.x == -INFINITY ? 0.f : fexp2(p1.x - M);
        const float L = w0 * lsum[u] + w1 * p1.y;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        if (kq == 0 && a.lse) a.lse[R.qrow[u]] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
        float* dst = a.out + (size_t)R.qrow[u] * D + 4 * kq;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const float4 o1 = h4[(u * 8 + nt) * 64 + lane];
            *reinterpret_cast<float4*>(dst + nt * 16) =
                make_float4((w0 * R.o[u][nt][0] + w1 * o1.x) * inv, (w0 * R.o[u][nt][1] + w1 * o1.y) * inv,
                            (w0 * R.o[u][nt][2] + w1 * o1.z) * inv, (w0 * R.o[u][nt][3] + w1 * o1.w) * inv);
        }
    }
}

// ---------------------------------------------------------- launchers ---

static PfArgs pf_args(const Plan& pl, const PfPlan& pf, const nosa_paged_kv* kv,
                      const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k)
{
    PfArgs a{};
    a.q = q;
    if (kv) {
        a.k_pool = kv->k_pool;
        a.v_pool = kv->v_pool;
        a.kc_pool = kv->kc_pool;
        a.table = kv->block_table;
        a.max_blocks = kv->max_blocks_per_seq;
    }
    a.cu_k = cu_k;
    a.cu_q = cu_q;
    a.Lmax = pl.Lmax;
    a.Lqmax = pf.max_seqlen_q;
    a.B = pl.B;
    a.Hq = pl.Hq;
    a.Hkv = pl.Hkv;
    a.G = pl.G;
    a.max_qblk = pf.max_qblk;
    a.scale_log2 = pl.scale_log2;
    a.rows = pf.rows;
    a.row_groups = pf.row_groups;
    a.key_splits = pf.key_splits;
    a.span = pf.span;
    a.zlen = pf.key_splits * pf.span;
    a.inv_g = (float)(1.0 / pl.G);
    a.max_nb = pl.max_nb;
    a.max_sel = pl.max_sel;
    return a;
}

hipError_t launch_pf_scores(const Plan& pl, const PfPlan& pf, const nosa_paged_kv& kv,
                            const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k,
                            void* ws, float* scores, hipStream_t stream, const int32_t* qbase)
{
    PfArgs a = pf_args(pl, pf, &kv, q, cu_q, cu_k);
    a.qbase = qbase;
    a.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + pf.off_part);
    a.colsum = reinterpret_cast<float*>(static_cast<char*>(ws) + pf.off_colsum);
    // the rows' lse by its own kernel only when pass 2 would merge many
    // partials per row
    a.rlse = pf.key_splits > kPfFoldSplits ? reinterpret_cast<float*>(static_cast<char*>(ws) + pf.off_rlse)
                                            : nullptr;
    a.scores = scores;
    const dim3 grid(pf.npairs * pf.row_groups * pf.key_splits);
#define NOSA_PF(PASS, R) hipLaunchKernelGGL((pf_score_kernel<PASS, R>), grid, dim3(256), 0, stream, a)
    for (int pass = 1; pass <= 2; ++pass) {
        switch (pf.rtw) {
            case 1: if (pass == 1) NOSA_PF(1, 1); else NOSA_PF(2, 1); break;
            case 2: if (pass == 1) NOSA_PF(1, 2); else NOSA_PF(2, 2); break;
            case 4: if (pass == 1) NOSA_PF(1, 4); else NOSA_PF(2, 4); break;
            default: if (pass == 1) NOSA_PF(1, 8); else NOSA_PF(2, 8); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (pass == 1 && a.rlse) {
            const int total = pf.npairs * pf.rows;
            hipLaunchKernelGGL(pf_lse_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, a, total);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
#undef NOSA_PF
    const int slices = (pl.max_nb + kPoolBlocks - 1) / kPoolBlocks;
    if (slices == 0 || pf.npairs == 0) return hipSuccess;
    hipLaunchKernelGGL(pf_pool_kernel, dim3(pf.npairs * slices), dim3(256), 0, stream, a, slices);
    return hipGetLastError();
}

hipError_t launch_pf_attend(const Plan& pl, const PfPlan& pf, const nosa_paged_kv& kv,
                            const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k,
                            const int32_t* sel, const int32_t* cnt, float* out, float* lse,
                            hipStream_t stream, const int32_t* qbase)
{
    PfArgs a = pf_args(pl, pf, &kv, q, cu_q, cu_k);
    a.qbase = qbase;
    a.sel = sel;
    a.cnt = cnt;
    a.out = out;
    a.lse = lse;
    const size_t lds = (size_t)(pl.max_sel > 0 ? pl.max_sel : 1) * sizeof(int2);
    const int total = pf.npairs * pf.attn_groups;
    const int per_xcd = (total + 7) / 8;
    // the halves of each row group on one 8-wave workgroup when the launch
    // would not give every CU two workgroups (and the pick list fits beside
    // its page buffers)
    if (total <= kPfSplitGroups && kPfHalvesLds + lds <= kPfLdsBytes)
        hipLaunchKernelGGL(pf_attend_halves_kernel, dim3(8 * per_xcd), dim3(512), lds, stream, a,
                           pf.attn_groups, total, per_xcd);
    else
        hipLaunchKernelGGL(pf_attend_kernel, dim3(8 * per_xcd), dim3(256), lds, stream, a,
                           pf.attn_groups, total, per_xcd);
    return hipGetLastError();
}

// ------------------------------------------------- whole-prompt prefill ---
//
// A prompt is processed in chunks of C queries (C a multiple of 64): chunk c
// of sequence s is its queries cC .. min(cC + C, L_s) - 1 against its first
// min(cC + C, L_s) tokens, which is the chunk convention of the entry points
// above with the query blocks of the whole prompt (64 from its start).  Per
// chunk: the bookkeeping arrays, the pooled keys completed by its tokens,
// importance, selection and attention, which read the queries from and write
// the outputs to the prompt's own rows (qbase).

// cu_k_c / cu_q_c: the chunk's context lengths and query counts as
// cumulative arrays; valid_c: tokens already pooled (cC, capped by L_s);
// qbase_c: the prompt row of the chunk's first query.
__global__ __launch_bounds__(64) void chunk_setup_kernel(const int32_t* __restrict__ cu, int B,
                                                         int Lmax, int c, int C,
                                                         int32_t* __restrict__ cu_k_c,
                                                         int32_t* __restrict__ cu_q_c,
                                                         int32_t* __restrict__ valid_c,
                                                         int32_t* __restrict__ qbase_c)
{
    if (threadIdx.x != 0) return;
    int k = 0, q = 0;
    cu_k_c[0] = 0;
    cu_q_c[0] = 0;
    for (int s = 0; s < B; ++s) {
        const int L = seq_len(cu, s, Lmax);
        const long long e = (long long)(c + 1) * C, b = (long long)c * C;
        const int end = e < L ? (int)e : L, start = b < L ? (int)b : L;
        k += end;
        q += end - start;
        cu_k_c[s + 1] = k;
        cu_q_c[s + 1] = q;
        valid_c[s] = start;
        qbase_c[s] = cu[s] + start;
    }
}

hipError_t launch_chunk_setup(const int32_t* cu, int B, int Lmax, int c, int C, int32_t* cu_k_c,
                              int32_t* cu_q_c, int32_t* valid_c, int32_t* qbase_c,
                              hipStream_t stream)
{
    hipLaunchKernelGGL(chunk_setup_kernel, dim3(1), dim3(64), 0, stream, cu, B, Lmax, c, C, cu_k_c,
                       cu_q_c, valid_c, qbase_c);
    return hipGetLastError();
}

}  // namespace nosa

#ifdef NOSA_TIMELINE
// Readout of the prefill launches' stamps (not part of the NOSA C ABI).
extern "C" {

// Copies launch `launch`'s stamps ([8192][4] unsigned 64-bit) to host memory.
int nosa_timeline_read_prefill(int launch, unsigned long long* host)
{
    if (launch < 0 || launch > 3 || !host) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(nosa::pf_tl), sizeof(nosa::pf_tl[0]),
                                    (size_t)launch * sizeof(nosa::pf_tl[0]), hipMemcpyDeviceToHost);
}

// Zeroes every prefill stamp (synchronous).
int nosa_timeline_clear_prefill(void)
{
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(nosa::pf_tl));
    if (e != hipSuccess) return (int)e;
    e = hipMemset(p, 0, sizeof(nosa::pf_tl));
    if (e != hipSuccess) return (int)e;
    return (int)hipDeviceSynchronize();
}

}  // extern "C"
#endif
