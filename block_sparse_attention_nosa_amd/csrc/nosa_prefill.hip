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
// pf_pool_kernel (block importance), the shared selector, pf_attend_kernel.
// All contractions run on v_mfma_f32_16x16x32_bf16 with rows = (query, head)
// pairs of the block in tiles of 16.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nosa_device.h"

namespace nosa {

constexpr int kQB = 64;   // queries per query block
constexpr int kKPS = 256; // pooled keys per split of the scoring passes

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
    int rows;        // 64 * G rows per pair: row = query * G + head
    int row_groups;  // workgroups over the rows of a pair
    int key_splits;  // workgroups over the pooled keys of a pair
    int zlen;        // key_splits * kKPS
    float2* part;    // [pairs][rows][key_splits] per-row (max, sum exp2)
    float* colsum;   // [pairs][row_groups][zlen] per-key sums over a row group
    float* scores;   // [pairs][max_nb] block importance
    int max_nb;
    const int32_t* sel;  // [pairs][max_sel]
    const int32_t* cnt;  // [pairs]
    int max_sel;
    float* out;  // [total_q][Hq][D]
    float* lse;  // [total_q][Hq] or null
    // attention split over two workgroups per row group (ksplit = 2): each
    // attends half of the kept pages and leaves unnormalised partials
    int ksplit;
    int rp;       // rows per pair in the partials: min(64, Lqmax) * G
    float* po;    // [pairs][rp][2][D]
    float2* pml;  // [pairs][rp][2] (max, sum) in log2 units
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

struct PfScoreLds {
    float lse[32 * 16];          // per row of the workgroup (pass 2)
    float ksum[4][kKPS];         // per wave, per key of the split (pass 2)
    int32_t pages[kKPS / SL];    // page of each group of SL pooled keys of the split
};

// Sum over the 16 lanes of each row of 16 (DPP shifts within the row; the
// total lands in lane 15 of the row).
template <int CTRL, int BANK_MASK>
__device__ __forceinline__ float dpp_row_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf,
                                                                 BANK_MASK, true));
}

__device__ __forceinline__ float row16_sum_to_last(float x)
{
    x += dpp_row_f<0x111, 0xf>(x);  // row_shr:1
    x += dpp_row_f<0x112, 0xf>(x);  // row_shr:2
    x += dpp_row_f<0x114, 0xe>(x);  // row_shr:4, lanes 4..15
    x += dpp_row_f<0x118, 0xc>(x);  // row_shr:8, lanes 8..15
    return x;
}

// Workgroup = 4 waves x RTW row tiles of 16 rows, over the kKPS pooled keys of
// one split.  PASS 1 writes per-row (max, sum exp2) over the split's visible
// keys; PASS 2 writes, for every key, sum over the workgroup's rows of
// exp2(z - lse_row) (lse from the pass-1 partials), in a fixed order.
template <int PASS, int RTW>
__global__ __launch_bounds__(256) void pf_score_kernel(PfArgs a)
{
    __shared__ PfScoreLds sh;
    const int per_pair = a.row_groups * a.key_splits;
    const int pair = blockIdx.x / per_pair;
    const int rg = (blockIdx.x % per_pair) / a.key_splits;
    const int ks = blockIdx.x % a.key_splits;
    const PfPair P = pf_pair(a, pair);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int key_lo = ks * kKPS;
    const int key_hi = min(key_lo + kKPS, P.nck);
    const int32_t* trow = a.table + (size_t)P.s * a.max_blocks;
    const int row_tile0 = (rg * 4 + wave) * RTW;  // first row tile of this wave
    const int wg_row0 = rg * 4 * RTW * 16;        // first row of the workgroup
    // page ids of the split's pooled keys first: a table load queued behind
    // key loads would wait for them
    for (int x = tid; x < kKPS / SL; x += 256) {
        const int key = key_lo + SL * x;
        sh.pages[x] = key < key_hi ? trow[key / SL] : 0;
    }
    if (PASS == 1) __syncthreads();

    if (PASS == 2) {
        // lse of every row of the workgroup from the pass-1 partials
        // (partials read 16 at a time, all loads of a batch in flight, then
        // combined; a loop-carried load chain would wait on each)
        for (int x = tid; x < 4 * RTW * 16; x += 256) {
            const int row = wg_row0 + x;
            float m = -INFINITY, acc = 0.f;
            if (row < a.rows && !P.empty) {
                const float2* pp = a.part + ((size_t)pair * a.rows + row) * a.key_splits;
                for (int i0 = 0; i0 < a.key_splits; i0 += 16) {
                    float2 v[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        v[u] = i0 + u < a.key_splits ? pp[i0 + u] : make_float2(-INFINITY, 0.f);
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
            }
            sh.lse[x] = acc > 0.f ? m + log2f(acc) : INFINITY;  // +inf: row contributes 0
        }
        __syncthreads();  // also publishes the page ids
    }

    // query operand of the wave's row tiles; rows of absent queries are zero
    bf16x8 qb[RTW][4];
    int qpos[RTW];  // query position of this lane's row r in each tile (-1: none)
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
        const int row = (row_tile0 + u) * 16 + r;
        const int qi = row / a.G, h = row % a.G;
        const bool ok = !P.empty && row < a.rows && qi < P.nq;
        qpos[u] = ok ? P.p0 + qi : -1;
        const uint16_t* qr = a.q + ((size_t)(P.q0 + kQB * P.r + (ok ? qi : 0)) * a.Hq + P.g * a.G + h) * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 w = ok ? ldg16(qr + st * 32 + kq * 8) : make_uint4(0, 0, 0, 0);
            qb[u][st] = as_bf16x8(w);
        }
    }
    // per row tile: does every row hold a query, and the first query position
    // (the rows of a tile are 16 consecutive (query, head) pairs)
    bool all_vis[RTW];
    int tile_p0[RTW];
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
        all_vis[u] = __ballot(qpos[u] < 0) == 0;  // wave-uniform
        int p = qpos[u] < 0 ? 0x7fffffff : qpos[u];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) p = min(p, __shfl_xor(p, off));
        tile_p0[u] = __builtin_amdgcn_readfirstlane(p);
    }
    float lse_r[RTW];
    if (PASS == 2) {
#pragma unroll
        for (int u = 0; u < RTW; ++u) lse_r[u] = sh.lse[(wave * RTW + u) * 16 + r];
    }
    float m_run[RTW], s_run[RTW];
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
        m_run[u] = -INFINITY;
        s_run[u] = 0.f;
    }

    // Two key tiles in flight: the loads of tile kt + 16 are issued before
    // tile kt is computed.  Rows past key_hi load the last key again (their
    // logits are masked).
    auto load_tile = [&](int kt, uint4 (&kf)[4]) {
        const int key = min(kt + r, key_hi - 1);
        const uint16_t* kp = a.kc_pool + ((size_t)sh.pages[(key - key_lo) / SL] * a.Hkv + P.g) * SL * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) kf[st] = ldg16(kp + kc_chunk(key % SL, st * 4 + kq));
    };
    auto tile = [&](int kt, const uint4 (&kf)[4]) {
        float colacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < RTW; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(kf[st]), qb[u][st], acc);
            // visible: key < n_c(p + 1)  <=>  16 * key + 32 <= p + 1; when every
            // key of the tile is visible to every row of the tile (the common
            // case) the per-element test is skipped
            float zz[4];
            float tmax = -INFINITY;
            if (all_vis[u] && kt + 16 <= key_hi && (kt + 15) * kPoolS + kPoolK <= tile_p0[u] + 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zz[i] = acc[i] * a.scale_log2;
                    tmax = fmaxf(tmax, zz[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kj = kt + 4 * kq + i;
                    const bool vis = qpos[u] >= 0 && kj < key_hi && kj * kPoolS + kPoolK <= qpos[u] + 1;
                    zz[i] = vis ? acc[i] * a.scale_log2 : -INFINITY;
                    tmax = fmaxf(tmax, zz[i]);
                }
            }
            if (PASS == 1) {
                if (tmax != -INFINITY) {
                    const float mn = fmaxf(m_run[u], tmax);
                    float add = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) add += fexp2(zz[i] - mn);
                    s_run[u] = s_run[u] * fexp2(m_run[u] - mn) + add;
                    m_run[u] = mn;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) colacc[i] += fexp2(zz[i] - lse_r[u]);
            }
        }
        if (PASS == 2) {
            // sum over the 16 rows (lanes r) of each key; lane r == 15 holds it
#pragma unroll
            for (int i = 0; i < 4; ++i) colacc[i] = row16_sum_to_last(colacc[i]);
            if (r == 15)
#pragma unroll
                for (int i = 0; i < 4; ++i) sh.ksum[wave][kt - key_lo + 4 * kq + i] = colacc[i];
        }
    };
    // (the loads are issued unconditionally -- past key_hi they repeat the
    // last key -- so no branch makes the compiler wait for all of them)
    if (key_lo < key_hi) {
        uint4 kfa[4], kfb[4];
        load_tile(key_lo, kfa);
        for (int kt = key_lo; kt < key_hi; kt += 32) {
            load_tile(kt + 16, kfb);
            tile(kt, kfa);
            load_tile(kt + 32, kfa);
            if (kt + 16 < key_hi) tile(kt + 16, kfb);
        }
    }

    if (PASS == 1) {
#pragma unroll
        for (int u = 0; u < RTW; ++u) {
            float m = m_run[u], s = s_run[u];
#pragma unroll
            for (int off = 16; off < 64; off <<= 1) {
                const float mo = __shfl_xor(m, off), so = __shfl_xor(s, off);
                const float mn = fmaxf(m, mo);
                s = mn == -INFINITY ? 0.f : s * fexp2(m - mn) + so * fexp2(mo - mn);
                m = mn;
            }
            const int row = (row_tile0 + u) * 16 + r;
            if (kq == 0 && row < a.rows)
                a.part[((size_t)pair * a.rows + row) * a.key_splits + ks] = make_float2(m, s);
        }
    } else {
        __syncthreads();
        float* dst = a.colsum + ((size_t)pair * a.row_groups + rg) * a.zlen + key_lo;
        for (int x = tid; x < kKPS; x += 256) {
            const int kj = key_lo + x;
            float v = 0.f;
            if (kj < key_hi) v = ((sh.ksum[0][x] + sh.ksum[1][x]) + sh.ksum[2][x]) + sh.ksum[3][x];
            dst[x] = v;
        }
    }
}

// Block importance of a pair: sigma[j] = sum over row groups (fixed order) of
// the column sums; importance of block b = mean of sigma over the keys 4b-1 ..
// 4b+3 that the block's last query sees.  One workgroup per pair.
__global__ __launch_bounds__(256) void pf_pool_kernel(PfArgs a)
{
    extern __shared__ __align__(16) char smem[];
    float* sI = reinterpret_cast<float*>(smem);
    const int pair = blockIdx.x;
    const PfPair P = pf_pair(a, pair);
    const int tid = threadIdx.x;
    float* out = a.scores + (size_t)pair * a.max_nb;
    const int nb = P.empty ? 0 : P.nb;
    for (int b = tid; b < nb; b += 256) sI[b] = 0.f;
    __syncthreads();
    const float* cs = a.colsum + (size_t)pair * a.row_groups * a.zlen;
    for (int j0 = 4 * tid; j0 < (P.empty ? 0 : P.nck); j0 += 4 * 256) {
        float sg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = 0.f;
            for (int q = 0; q < a.row_groups; ++q) v += cs[(size_t)q * a.zlen + j0 + e];
            sg[e] = j0 + e < P.nck ? v : 0.f;
        }
        const int b = j0 >> 2;
        atomicAdd(&sI[b], (sg[0] + sg[1]) + (sg[2] + sg[3]));
        if (j0 + 3 < P.nck && b + 1 < nb) atomicAdd(&sI[b + 1], sg[3]);
    }
    __syncthreads();
    for (int b = tid; b < a.max_nb; b += 256) {
        float I = -INFINITY;
        if (b < nb) {
            const int jlo = max(4 * b - 1, 0), jhi = min(4 * b + 3, P.nck - 1);
            if (jlo <= jhi) I = sI[b] / (float)(jhi - jlo + 1);
        }
        out[b] = I;
    }
}

// ------------------------------------------------------------ attention ---

// A K and a V page in LDS, in the pages' own operand order (a straight copy):
// the fragment of QK^T tile t, k-step st is run 4t + st, that of PV k-step
// u, channel tile nt is run 8u + nt, lane l at byte 16 l of its run, so a
// wave's fragment read is 1 KB of consecutive LDS.
struct PfAttnLds {
    uint16_t k[2][BS * D];
    uint16_t v[2][BS * D];
};

// Workgroup = 4 waves x 2 row tiles (128 rows) of one pair; loops over the
// pair's kept pages, each staged once through LDS for all 8 row tiles.  The
// (block, page) list goes to LDS first; page i + 1's loads are issued before
// page i is computed and land in the other LDS buffer after it, so one
// barrier per page suffices.
//
// Workgroups are dealt to the eight XCDs round-robin by index, so index b is
// mapped to the logical workgroup (b % 8) * per_xcd + b / 8: the attn_groups
// workgroups of a pair, which read the same pages, run on one XCD and share
// its L2.  Indices past the last logical workgroup exit at once.
//
// With ksplit = 2 (a launch that would not give every CU two workgroups:
// one workgroup's pages are then a latency-bound chain), logical workgroup
// 2w + k attends the k-th half of row group w's pages and stores its
// unnormalised partial; pf_merge_kernel combines the two.
__global__ __launch_bounds__(256, 2) void pf_attend_kernel(PfArgs a, int attn_groups, int total,
                                                        int per_xcd)
{
    __shared__ PfAttnLds sh;
    extern __shared__ __align__(16) char smem[];
    int2* list = reinterpret_cast<int2*>(smem);  // [max_sel] (block, page)
    const int lid_k = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (lid_k >= total * a.ksplit) return;
    const int lid = lid_k / a.ksplit, ks = lid_k % a.ksplit;
    const int pair = lid / attn_groups, ag = lid % attn_groups;
    const PfPair P = pf_pair(a, pair);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int32_t* trow = a.table + (size_t)P.s * a.max_blocks;
    const int n = P.empty ? 0 : min(a.cnt[pair], a.max_sel);
    const int32_t* sl = a.sel + (size_t)pair * a.max_sel;
    for (int x = tid; x < n; x += 256) {
        int b = sl[x];
        if (b < 0 || b >= P.nb) b = -1;
        list[x] = make_int2(b, b >= 0 ? trow[b] : 0);
    }

    bf16x8 qb[2][4];
    int qpos[2];
    int qrow[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int row = ((ag * 4 + wave) * 2 + u) * 16 + r;
        const int qi = row / a.G, h = row % a.G;
        const bool ok = !P.empty && row < a.rows && qi < P.nq;
        qpos[u] = ok ? P.p0 + qi : -1;
        qrow[u] = ok ? (P.q0 + kQB * P.r + qi) * a.Hq + P.g * a.G + h : -1;
        const uint16_t* qr = a.q + (size_t)(ok ? qrow[u] : 0) * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 w = ok ? ldg16(qr + st * 32 + kq * 8) : make_uint4(0, 0, 0, 0);
            qb[u][st] = as_bf16x8(w);
        }
    }
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4 o[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) o[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // the list

    // thread tid moves the 16-byte chunks tid + 256c (c < 4) of a K and a V
    // page: the same offsets in global memory and in LDS
    uint4 stk[4], stv[4];
    // (unconditional loads: past the list, or for a dropped entry, page 0 is
    // read and never used; a branch around the loads makes the compiler wait
    // for every outstanding load at the loop head)
    auto fetch = [&](int idx, uint4 (&k4)[4], uint4 (&v4)[4]) {
        const int page = idx < n ? list[idx].y : 0;
        const uint16_t* kb = a.k_pool + ((size_t)page * a.Hkv + P.g) * BS * D;
        const uint16_t* vb = a.v_pool + ((size_t)page * a.Hkv + P.g) * D * BS;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = tid + 256 * c;
            k4[c] = ldg16(kb + ch * 8);
            v4[c] = ldg16(vb + ch * 8);
        }
    };
    auto stash = [&](int buf, const uint4 (&k4)[4], const uint4 (&v4)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = tid + 256 * c;
            *reinterpret_cast<uint4*>(&sh.k[buf][ch * 8]) = k4[c];
            *reinterpret_cast<uint4*>(&sh.v[buf][ch * 8]) = v4[c];
        }
    };
    // every row of the workgroup holds a query, and the smallest position:
    // pages entirely at or before it need no causal mask
    const bool rows_full = __syncthreads_and(qpos[0] >= 0 && qpos[1] >= 0);
    int pmin = min(qpos[0] < 0 ? 0x7fffffff : qpos[0], qpos[1] < 0 ? 0x7fffffff : qpos[1]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) pmin = min(pmin, __shfl_xor(pmin, off));
    pmin = __builtin_amdgcn_readfirstlane(pmin);  // per wave (its own rows)
    auto compute = [&](int buf, int b_cur) {
        // S^T = K q^T for both row tiles: K fragments from LDS, shared
        float x[2][4][4];
        float bmax[2] = {-INFINITY, -INFINITY};
        const bool full = rows_full && b_cur * BS + BS - 1 <= pmin && b_cur * BS + BS <= P.L;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 kf[4];
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(&sh.k[buf][((t * 4 + st) * 64 + lane) * 8]));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) acc = mfma16(kf[st], qb[u][st], acc);
                if (full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[u][t][i] = acc[i] * a.scale_log2;
                        bmax[u] = fmaxf(bmax[u], x[u][t][i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = b_cur * BS + 32 * (t >> 1) + 8 * kq + 4 * (t & 1) + i;
                        const bool vis = qpos[u] >= 0 && tk <= qpos[u] && tk < P.L;
                        x[u][t][i] = vis ? acc[i] * a.scale_log2 : -INFINITY;
                        bmax[u] = fmaxf(bmax[u], x[u][t][i]);
                    }
                }
            }
        }
        bf16x8 pa[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float bm = bmax[u];
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float m_new = fmaxf(m_run[u], bm);
            // a row with nothing visible yet keeps m = -inf and adds nothing
            const float alpha = m_new == -INFINITY ? 1.f : fexp2(m_run[u] - m_new);
            float psum = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = m_new == -INFINITY ? 0.f : fexp2(x[u][t][i] - m_new);
                    x[u][t][i] = e;
                    psum += e;
                }
            l_run[u] = l_run[u] * alpha + psum;
            // the accumulators are rescaled only when some row's maximum moved
            if (__ballot(m_new != m_run[u]) != 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * kq + i);
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) o[u][nt][i] *= ai;
                }
            }
            m_run[u] = m_new;
#pragma unroll
            for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pa[u][uu][i] = (__bf16)x[u][2 * uu][i];
                    pa[u][uu][4 + i] = (__bf16)x[u][2 * uu + 1][i];
                }
        }
        // O += P V: V fragments from LDS, shared by both row tiles
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const bf16x8 vf =
                    as_bf16x8(*reinterpret_cast<const uint4*>(&sh.v[buf][((uu * 8 + nt) * 64 + lane) * 8]));
#pragma unroll
                for (int u = 0; u < 2; ++u) o[u][nt] = mfma16(pa[u][uu], vf, o[u][nt]);
            }
    };

    // this workgroup's pages: all, or half of them
    const int i0 = n * ks / a.ksplit, i1 = n * (ks + 1) / a.ksplit;
    if (i1 > i0) {
        fetch(i0, stk, stv);
        stash(0, stk, stv);
        __syncthreads();
    }
    for (int idx = i0; idx < i1; ++idx) {
        const int buf = (idx - i0) & 1;
        fetch(idx + 1, stk, stv);  // in flight while page idx is computed
        const int b = list[idx].x;
        if (b >= 0) compute(buf, b);
        if (idx + 1 < i1) stash(buf ^ 1, stk, stv);
        __syncthreads();
    }
    if (a.ksplit > 1) {  // unnormalised partial of this half, rows holding a query
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float l = l_run[u];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            const int row0 = ((ag * 4 + wave) * 2 + u) * 16;  // the row tile in the pair
            const size_t pr0 = (size_t)pair * a.rp + row0;
            if (kq == 0 && qpos[u] >= 0) a.pml[(pr0 + r) * 2 + ks] = make_float2(m_run[u], l);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (__shfl(qpos[u], 4 * kq + i) < 0) continue;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
                    a.po[((pr0 + 4 * kq + i) * 2 + ks) * D + nt * 16 + r] = o[u][nt][i];
            }
        }
        return;
    }

    // normalise and store: lane holds O[rows 4kq + i][channels 16nt + r]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float l = l_run[u];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (kq == 0 && qrow[u] >= 0 && a.lse)
            a.lse[qrow[u]] = l > 0.f ? (m_run[u] + log2f(l)) * 0.69314718055994531f : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float inv_i = __shfl(inv, 4 * kq + i);
            const int row_i = __shfl(qrow[u], 4 * kq + i);
            if (row_i < 0) continue;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) a.out[(size_t)row_i * D + nt * 16 + r] = o[u][nt][i] * inv_i;
        }
    }
}

// The two halves of a split attention: row x of row group w from partials
// (m_k, l_k, o_k), k < 2, in log2 units: out = sum 2^(m_k - M) o_k / L,
// L = sum 2^(m_k - M) l_k, lse = (M + log2 L) ln 2; a row that saw nothing
// gets 0 and -inf.  Workgroup (w, y): rows 8y .. 8y + 7 of row group w, a
// thread per (row, 4 channels).
__global__ __launch_bounds__(256) void pf_merge_kernel(PfArgs a, int attn_groups, int total)
{
    const int lid = blockIdx.x;
    if (lid >= total) return;
    const int pair = lid / attn_groups, ag = lid % attn_groups;
    const PfPair P = pf_pair(a, pair);
    const int row = ag * 128 + (int)blockIdx.y * 8 + (threadIdx.x >> 5), c4 = threadIdx.x & 31;
    const int qi = row / a.G, h = row % a.G;
    if (P.empty || row >= a.rows || qi >= P.nq) return;  // rows past the block's queries
    const size_t pr = (size_t)pair * a.rp + row;
    const float2 p0 = a.pml[pr * 2], p1 = a.pml[pr * 2 + 1];
    const float4 o0 = reinterpret_cast<const float4*>(a.po + (pr * 2) * D)[c4];
    const float4 o1 = reinterpret_cast<const float4*>(a.po + (pr * 2 + 1) * D)[c4];
    const float M = fmaxf(p0.x, p1.x);
    const float w0 = p0.x == -INFINITY ? 0.f : fexp2(p0.x - M);
    const float w1 = p1.x == -INFINITY ? 0.f : fexp2(p1.x - M);
    const float L = w0 * p0.y + w1 * p1.y;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t qrow = (size_t)(P.q0 + kQB * P.r + qi) * a.Hq + P.g * a.G + h;
    reinterpret_cast<float4*>(a.out + qrow * D)[c4] =
        make_float4((w0 * o0.x + w1 * o1.x) * inv, (w0 * o0.y + w1 * o1.y) * inv,
                    (w0 * o0.z + w1 * o1.z) * inv, (w0 * o0.w + w1 * o1.w) * inv);
    if (a.lse && c4 == 0) a.lse[qrow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
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
    a.zlen = pf.key_splits * kKPS;
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
    }
#undef NOSA_PF
    const size_t lds = sizeof(float) * (size_t)(pl.max_nb > 0 ? pl.max_nb : 1);
    hipLaunchKernelGGL(pf_pool_kernel, dim3(pf.npairs), dim3(256), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_pf_attend(const Plan& pl, const PfPlan& pf, const nosa_paged_kv& kv,
                            const nosa_bf16* q, const int32_t* cu_q, const int32_t* cu_k,
                            const int32_t* sel, const int32_t* cnt, float* out, float* lse,
                            void* ws, size_t ws_bytes, hipStream_t stream, const int32_t* qbase)
{
    PfArgs a = pf_args(pl, pf, &kv, q, cu_q, cu_k);
    a.qbase = qbase;
    a.sel = sel;
    a.cnt = cnt;
    a.out = out;
    a.lse = lse;
    const size_t lds = (size_t)(pl.max_sel > 0 ? pl.max_sel : 1) * sizeof(int2);
    const int total = pf.npairs * pf.attn_groups;
    // split the pages of each row group over two workgroups when the launch
    // has at most kPfSplitGroups of them and the workspace holds the partials
    a.ksplit = total <= kPfSplitGroups && ws && ws_bytes >= pf.bytes_split ? 2 : 1;
    if (a.ksplit > 1) {
        a.rp = pf.split_rows;
        a.po = reinterpret_cast<float*>(static_cast<char*>(ws) + pf.off_po);
        a.pml = reinterpret_cast<float2*>(static_cast<char*>(ws) + pf.off_pml);
    }
    const int per_xcd = (total * a.ksplit + 7) / 8;
    hipLaunchKernelGGL(pf_attend_kernel, dim3(8 * per_xcd), dim3(256), lds, stream, a, pf.attn_groups,
                       total, per_xcd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ksplit == 1 || total == 0) return e;
    hipLaunchKernelGGL(pf_merge_kernel, dim3(total, 16), dim3(256), 0, stream, a, pf.attn_groups,
                       total);
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
