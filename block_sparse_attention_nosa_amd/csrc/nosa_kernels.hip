// nosa_kernels.hip -- CDNA4 (gfx950) kernels of the NOSA sparse decode step.
//
// A decode step is three launches on the caller's stream:
//   score : workgroup (pair, chunk) scores 64 T pooled keys of one (sequence,
//           KV head) pair on MFMA and leaves per-chunk softmax partials; the
//           chunk holding the key completed by the current token pools it
//           from K first and stores it;
//   top   : per pair, "top" workgroups each recompute the pair's selection
//           from those partials (log-sum-exp, block importance, top-k) and
//           attend their slice of the picks, while "window" workgroups attend
//           the local window, which needs no selection;
//   merge : combines the (m, l, o) partials of every head into out / lse.
// Kernel boundaries order every hand-off: no workgroup reads another
// workgroup's output within a launch, so there are no counters, fences or
// zero-filled buffers.  The stand-alone entry points reuse the pieces:
// kc_build (pooled keys), score + top in importance-only mode, select (from
// given importance), attend (given block lists) + merge.
//
// Sources: page "NOSA-1B 性能基准全解析" (sections 三.2 local window and TopK
// blocks, 三.3 two-stage attention with kernel 32 / stride 16 pooling, 三.4 the
// mean-pool kernel), page "NOSA-1B 模型家族全景" (core principle: compressed
// attention filters KV blocks, CIS score mean pooling), page "NOSA技术架构解析"
// (section 2.1: paged KV pool; section 5.1: importance scores kept in fp32).
//
// Shared device helpers (MFMA operand layout, one-page attention, the
// selector) are in nosa_device.h.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "nosa_device.h"

namespace nosa {

// Timeline build: compiled with NOSA_TIMELINE, a library of its own for the
// benchmark's timeline mode (the NOSA library has none of this).  Thread 0
// of a workgroup stamps the constant-rate wall clock at points of its
// launch (0: scoring, 1: selection + attention, 2: merge) into
// tl_stamps[launch][workgroup][point]; point 7 holds the workgroup's role.
// The scheduling barriers keep each stamp between the instructions around
// it.
#ifdef NOSA_TIMELINE
constexpr int kTlGroups = 8192;
__device__ unsigned long long tl_stamps[3][kTlGroups][16];
#define NOSA_TL(launch, point)                                                           \
    do {                                                                                 \
        __builtin_amdgcn_sched_barrier(0);                                               \
        if (threadIdx.x == 0 && blockIdx.x < kTlGroups)                                  \
            tl_stamps[launch][blockIdx.x][point] = wall_clock64();                       \
        __builtin_amdgcn_sched_barrier(0);                                               \
    } while (0)
// point 7: the role; 13: the XCD (hardware register XCC_ID); 14: HW_ID
// (compute unit, shader array and engine of the wave); 15 (selection: set
// when a digit level after the first runs) is cleared here, so that every
// step of a replay leaves its own value, not one of an earlier step
#define NOSA_TL_ROLE(launch, role)                                                       \
    do {                                                                                 \
        if (threadIdx.x == 0 && blockIdx.x < kTlGroups) {                                \
            tl_stamps[launch][blockIdx.x][7] = (role);                                   \
            tl_stamps[launch][blockIdx.x][13] = (unsigned)__builtin_amdgcn_s_getreg(30740); \
            tl_stamps[launch][blockIdx.x][14] = (unsigned)__builtin_amdgcn_s_getreg(63492); \
            tl_stamps[launch][blockIdx.x][15] = 0;                                       \
        }                                                                                \
    } while (0)
#else
#define NOSA_TL(launch, point) \
    do {                       \
    } while (0)
#define NOSA_TL_ROLE(launch, role) \
    do {                           \
    } while (0)
#endif

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

// Pooled keys from whole K pages.  Key j pools tokens [16 j, 16 j + 32):
// 16-token groups j and j + 1, so keys 4b, 4b+1, 4b+2 lie inside page b and
// key 4b+3 takes the last group of page b and the first of page b+1.  A wave
// owns `ppw` consecutive pages of one (sequence, KV head) and streams them:
// it reads each page once, a contiguous kilobyte per load instruction (the
// pages are stored in operand order), the next page's loads in flight while
// the current one is summed (block-table entries read a page ahead of those),
// and puts each page into its own 16 KB of LDS token-major.  Lane (u, c8)
// sums channels 8 c8 .. 8 c8 + 7 of group u of the page over its 16 tokens in
// ascending order in fp64; key 4b + u is its group sum plus that of lane
// (u + 1, c8) (one lane rotation), key 4b - 1 the previous page's last group
// sum plus this page's first.  Each fp64 sum of bf16 values here is exact
// while a key's nonzero values span at most 2^40 in magnitude (they are
// multiples of the smallest one's last bit, and 32 of them fit 53 bits), so
// the mean, scaled by 1/32 and rounded once to bf16, is then the exact one,
// bit for bit whatever the order of the additions.  After the wave's last
// page, lanes u = 0 read the first group of the next page for the last key.
// Keys [n_c(prev), n_c(L)) are written, prev = valid_len[s] or 0 for a full
// build.  Long runs per wave keep a page of loads in flight from start to
// end (a wave fills and drains its pipeline once); the grid is sized to
// about four waves per SIMD (two resident at a time, two workgroups per CU),
// so that the second half of the waves starts as the first ones end.
//
// LDS slot of (token x, chunk c8): 16 x + (c8 ^ swz(x)), swz(x) = (x & 3) |
// ((x & 8) >> 1).  A wave's store of one operand run (lanes: 16 tokens x 4
// chunks) and its loads of one token per lane group (16 chunks) then touch
// eight different 16-byte bank groups in every group of eight lanes.
constexpr int kKcMinPagesPerWave = 2;
constexpr int kKcTargetWaves = 4096;

__device__ __forceinline__ int kc_lds_slot(int x, int c8)
{
    return 16 * x + (c8 ^ ((x & 3) | ((x & 8) >> 1)));
}

__global__ __launch_bounds__(256, 2) void kc_build_kernel(
    const uint16_t* __restrict__ k_pool, uint16_t* __restrict__ kc_pool,
    const int32_t* __restrict__ table, int max_blocks, int Lmax, int Hkv,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ valid_len, int ppw)
{
    __shared__ uint4 tile[4][BS * D / 8];  // a page per wave, 16 KB
    const int s = blockIdx.z, g = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int L = seq_len(cu_k, s, Lmax);
    int prev = valid_len ? valid_len[s] : 0;
    prev = prev < 0 ? 0 : (prev > L ? L : prev);
    const int j0 = dev_num_keys(prev), j1 = dev_num_keys(L);
    if (j0 >= j1) return;  // (whole workgroup)
    const int b_lo = j0 / SL, b_hi = (j1 - 1) / SL;  // pages holding the first token of a new key
    const int ntask = (b_hi - b_lo) / ppw + 1;
    const int32_t* trow = table + (size_t)s * max_blocks;
    const int u = lane >> 4, c8 = lane & 15;         // group u of the page, chunk c8
    const int r16 = lane & 15, kq4 = lane >> 4;      // this lane's token and chunk in a stored run
    const int nbr = (lane + 16) & 63;                // lane (u + 1, c8), (0, c8) for u = 3
    uint4* t = tile[wave];
    for (int task = (int)blockIdx.x * 4 + wave; task < ntask; task += (int)gridDim.x * 4) {
        const int b0 = b_lo + task * ppw;
        const int npg = min(ppw, b_hi + 1 - b0);  // pages b0 .. b0 + npg - 1
        const int jsp = 4 * (b0 + npg - 1) + 3;   // the last page's key 4b+3
        const bool spill = jsp >= j0 && jsp < j1;  // then page b0 + npg exists
        // table entry of the task's page i (the spill page for i = npg when
        // it exists; unused ones are clamped to the first page)
        auto pid = [&](int i) {
            return trow[b0 + ((i < npg || (i == npg && spill)) ? i : 0)];
        };
        // The four keys of page bb (lane (u, c8): key 4 bb + u, chunk c8, in
        // `own`) as one contiguous 1 KB store: lane l writes slot l & 3 of
        // chunk l >> 2, taken from lane (l & 3, l >> 2) by a rotation of
        // lanes; keys outside [j0, j1) are left as they are.  The page's id
        // comes from the entries above (a table load here would wait, in
        // order, behind the prefetched page).
        auto store_page = [&](int bb, int page, uint4 own) {
            const int src = (lane & 3) * 16 + (lane >> 2);
            const uint4 val = make_uint4(__shfl(own.x, src), __shfl(own.y, src),
                                         __shfl(own.z, src), __shfl(own.w, src));
            const int j = 4 * bb + (lane & 3);
            if (j >= j0 && j < j1)
                *reinterpret_cast<uint4*>(kc_pool + ((size_t)page * Hkv + g) * SL * D + lane * 8) = val;
        };
        auto rotate = [&](const double (&a)[8], double (&b)[8]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = __shfl(a[e], nbr);
        };
        int p_prev = 0, p_cur = pid(0), p_n1 = pid(1);
        double carry[8];  // lanes u = 3: the previous page's last group sum
#pragma unroll
        for (int e = 0; e < 8; ++e) carry[e] = 0.0;
        uint4 kprev = make_uint4(0, 0, 0, 0);  // lanes u < 3: key 4 (b - 1) + u, rounded
        uint4 v[16];
        {
            const uint16_t* pg = k_pool + ((size_t)p_cur * Hkv + g) * BS * D + lane * 8;
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = ldg16_stream(pg + r * 512);
        }
        for (int q = 0; q < npg; ++q) {
            // The tile is the wave's own: LDS operations of a wave execute in
            // program order, so only the compiler must keep the lanes' reads
            // of one page and the writes of the next in order (a memory
            // clobber).
            asm volatile("" ::: "memory");
#pragma unroll
            for (int r = 0; r < 16; ++r)
                t[kc_lds_slot(qk_row_token(r >> 2, r16), 4 * (r & 3) + kq4)] = v[r];
            if (q + 1 < npg) {  // the next page into the freed buffer
                const uint16_t* pg = k_pool + ((size_t)p_n1 * Hkv + g) * BS * D + lane * 8;
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = ldg16_stream(pg + r * 512);
            } else if (spill && u == 0) {  // the next page's first group, chunk c8
                const uint16_t* pg = k_pool + ((size_t)p_n1 * Hkv + g) * BS * D;
#pragma unroll
                for (int x = 0; x < 16; ++x) v[x] = ldg16(pg + k_chunk(x, c8));
            }
            const int p_n2 = pid(q + 2);
            asm volatile("" ::: "memory");
            double gs[8], nb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gs[e] = 0.0;
#pragma unroll 8
            for (int k = 0; k < 16; ++k) acc8(gs, t[kc_lds_slot(16 * u + k, c8)]);
            rotate(gs, nb);
            // this lane's key: 4b + u (groups u and u + 1), or for u = 3 key
            // 4b - 1 (the previous page's last group and this page's first)
#pragma unroll
            for (int e = 0; e < 8; ++e) nb[e] = (u < 3 ? gs[e] : carry[e]) + nb[e];
            if (u == 3) {
#pragma unroll
                for (int e = 0; e < 8; ++e) carry[e] = gs[e];
            }
            const uint4 kr = round8(nb);
            const int b = b0 + q;
            if (q > 0) store_page(b - 1, p_prev, u < 3 ? kprev : kr);  // page b - 1 is complete
            kprev = kr;
            if (q + 1 == npg) {  // page b: key 4b + 3 with the next page's first group
                uint4 k3 = kr;
                if (spill) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) gs[e] = 0.0;
                    if (u == 0) {
#pragma unroll
                        for (int x = 0; x < 16; ++x) acc8(gs, v[x]);
                    }
                    rotate(gs, nb);
#pragma unroll
                    for (int e = 0; e < 8; ++e) nb[e] = carry[e] + nb[e];
                    k3 = round8(nb);
                }
                store_page(b, p_cur, u < 3 ? kr : k3);
            }
            p_prev = p_cur;
            p_cur = p_n1;
            p_n1 = p_n2;
        }
    }
}

// Pages per wave for a build whose pairs each hold up to max_pages pages of
// new keys: enough that the launch has about kKcTargetWaves waves.
static int kc_pages_per_wave(const Plan& pl, int max_pages)
{
    const long long total = (long long)pl.B * pl.Hkv * (max_pages > 0 ? max_pages : 1);
    const long long ppw = (total + kKcTargetWaves - 1) / kKcTargetWaves;
    return (int)(ppw < kKcMinPagesPerWave ? kKcMinPagesPerWave : (ppw > (1 << 20) ? (1 << 20) : ppw));
}

// max_pages: an upper bound of the pages holding a new key's first token per
// (sequence, KV head) (a grid-stride loop covers whatever the grid misses).
hipError_t launch_kc_build(const Plan& pl, const nosa_paged_kv& kv, const int32_t* cu_k,
                           const int32_t* valid_len, int max_pages, hipStream_t stream)
{
    const int ppw = kc_pages_per_wave(pl, max_pages);
    const int tasks = ceil_div(max_pages > 0 ? max_pages : 1, ppw);
    dim3 grid(ceil_div(tasks, 4), pl.Hkv, pl.B);
    hipLaunchKernelGGL(kc_build_kernel, grid, dim3(256), 0, stream, kv.k_pool, kv.kc_pool,
                       kv.block_table, kv.max_blocks_per_seq, pl.Lmax, pl.Hkv, cu_k, valid_len,
                       ppw);
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

// One page attended by the four waves of a workgroup, each loading a quarter
// of it (8 KB: a CU keeps only about 28 KB of loads in flight, so a wave that
// issues a whole 32 KB page stalls until most of it has arrived).  Wave w computes S for QK tile w (16 tokens, all heads); the
// page maximum per head and P go through LDS; then wave w computes P V for
// channel tiles 2w and 2w+1 over all 64 tokens.  Stores the page's (m, l, o)
// partial per head at slot `split` (m, l in log2 units, o unnormalised).
// All 256 threads; `limit` = tokens of the page that exist (>= 1).
struct SplitPageLds {
    float m[4][kMaxGroup], l[4][kMaxGroup];
    uint4 p[2][64];  // PV A operand per k-step and lane (8 bf16)
};

template <bool STREAM>
__device__ void attend_page_split4(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                   int limit, const bf16x8 (&qb)[4], float scale_log2, int G,
                                   size_t head_row0, int nsplit, int split, float* __restrict__ po,
                                   float2* __restrict__ pml, SplitPageLds& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int lane8 = lane * 8;
    uint4 ka[4], va[2][2];
    if constexpr (STREAM) {
#pragma unroll
        for (int st = 0; st < 4; ++st) ka[st] = ldg16_stream(kb + (wave * 4 + st) * 512 + lane8);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j) va[u][j] = ldg16_stream(vb + (u * 8 + 2 * wave + j) * 512 + lane8);
    } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) ka[st] = ldg16(kb + (wave * 4 + st) * 512 + lane8);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j) va[u][j] = ldg16(vb + (u * 8 + 2 * wave + j) * 512 + lane8);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(ka[st]), qb[st], acc);
    // lane (r, kq): head r, tokens 32 (w >> 1) + 8 kq + 4 (w & 1) + i
    float x[4], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = 32 * (wave >> 1) + 8 * kq + 4 * (wave & 1) + i;
        x[i] = tok < limit ? acc[i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (kq == 0) sh.m[wave][r] = mx;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.m[w][r]);  // finite: token 0 exists
    float ps = 0.f;
    uint32_t pk[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = fexp2(x[i] - M);
#pragma unroll
    for (int i = 0; i < 4; ++i) ps += x[i];
    {
        bf16x8 t;
        t[0] = (__bf16)x[0];
        t[1] = (__bf16)x[1];
        t[2] = (__bf16)x[2];
        t[3] = (__bf16)x[3];
        const uint4 w4 = __builtin_bit_cast(uint4, t);
        pk[0] = w4.x;
        pk[1] = w4.y;
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    if (kq == 0) sh.l[wave][r] = ps;
    // elements 4 (w & 1) .. +3 of the k-step (w >> 1) operand of this lane
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(&sh.p[wave >> 1][lane]) + 8 * (wave & 1)) =
        make_uint2(pk[0], pk[1]);
    __syncthreads();
    f32x4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const bf16x8 pa = as_bf16x8(sh.p[u][lane]);
#pragma unroll
        for (int j = 0; j < 2; ++j) o[j] = mfma16(pa, as_bf16x8(va[u][j]), o[j]);
    }
    // o[j][i]: head 4 kq + i, channel 16 (2w + j) + r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * kq + i;
        if (h < G) {
            float* dst = po + ((head_row0 + h) * nsplit + split) * D + 32 * wave + r;
            dst[0] = o[0][i];
            dst[16] = o[1][i];
        }
    }
    if (wave == 0 && kq == 0 && r < G) {
        const float L = sh.l[0][r] + sh.l[1][r] + sh.l[2][r] + sh.l[3][r];
        pml[(head_row0 + r) * nsplit + split] = make_float2(M, L);
    }
}

// Page of window block b of sequence s: block-table entry, or with a ring of
// `ring` recent pages per sequence (offloaded KV), ring slot b % ring.
__device__ __forceinline__ int window_page(const int32_t* table, int max_blocks, int ring, int s,
                                           int b)
{
    return ring > 0 ? s * ring + b % ring : table[(size_t)s * max_blocks + b];
}

// Window slot x of pair (s, g): block nb - wn + x, wn = min(nb, wblocks),
// attended by the four waves together, its partial at slot split0 + x (an
// empty partial past wn).  All 256 threads.
__device__ void store_empty_partial(int G, size_t head_row0, int nsplit, int split,
                                    float* __restrict__ po, float2* __restrict__ pml);
template <bool STREAM>
__device__ void window_slot(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* table, int ring, const int32_t* cu_k, int max_blocks, int Lmax,
                            int Hq, int Hkv, int G, float scale_log2, int wblocks, int s, int g,
                            int x, int nsplit, int split0, float* po, float2* pml,
                            SplitPageLds& sh)
{
    const int lane = threadIdx.x & 63, r = lane & 15, kq = lane >> 4;
    const int L = seq_len(cu_k, s, Lmax);
    const int nb = (L + BS - 1) / BS;
    const int wn = nb < wblocks ? nb : wblocks;
    const size_t head_row0 = (size_t)s * Hq + g * G;
    if (x < wn) {
        bf16x8 qb[4];
        load_q(q, Hq, s, g * G, G, r, kq, qb);
        const int b = nb - wn + x;
        const int page = window_page(table, max_blocks, ring, s, b);
        attend_page_split4<STREAM>(k_pool + ((size_t)page * Hkv + g) * BS * D,
                           v_pool + ((size_t)page * Hkv + g) * D * BS, L - b * BS, qb, scale_log2, G,
                           head_row0, nsplit, split0 + x, po, pml, sh);
    } else {
        store_empty_partial(G, head_row0, nsplit, split0 + x, po, pml);
    }
}

// Window slots 4 j .. 4 j + 3 of pair (s, g), a page per wave (blocks
// nb - wn + 4 j + wave, wn = min(nb, wblocks); waves past wn attend
// nothing), the four wave states combined into the partial at slot
// split0 + j.  All 256 threads.
__device__ __forceinline__ void window_group(const uint16_t* q, const uint16_t* k_pool,
                                             const uint16_t* v_pool,
                             const int32_t* table, int ring, const int32_t* cu_k, int max_blocks,
                             int Lmax, int Hq, int Hkv, int G, float scale_log2, int wblocks, int s,
                             int g, int j, int nsplit, int split0, float* po, float2* pml,
                             CombineLds& sh, bool stream)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, kq = lane >> 4;
    const int L = seq_len(cu_k, s, Lmax);
    const int nb = (L + BS - 1) / BS;
    const int wn = nb < wblocks ? nb : wblocks;
    const int x = 4 * j + wave;
    AttnState A;
    attn_init(A);
    if (x < wn) {  // wave-uniform
        bf16x8 qb[4];
        load_q(q, Hq, s, g * G, G, r, kq, qb);
        const int b = nb - wn + x;
        const int page = window_page(table, max_blocks, ring, s, b);
        attend_page(k_pool + ((size_t)page * Hkv + g) * BS * D, v_pool + ((size_t)page * Hkv + g) * D * BS,
                    L - b * BS, qb, scale_log2, r, kq, A, stream);
    }
    store_wg_partial(sh, A, G, (size_t)s * Hq + g * G, nsplit, split0 + j, po, pml);
}

// An empty partial (m = -inf, l = 0, o = 0) at slot `split`; all 256 threads.
__device__ void store_empty_partial(int G, size_t head_row0, int nsplit, int split,
                                    float* __restrict__ po, float2* __restrict__ pml)
{
    for (int x = threadIdx.x; x < G * (D / 4); x += 256) {
        const int h = x / (D / 4), c4 = x % (D / 4);
        reinterpret_cast<float4*>(po + ((head_row0 + h) * nsplit + split) * D)[c4] =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if ((int)threadIdx.x < G) pml[(head_row0 + threadIdx.x) * nsplit + split] = make_float2(-INFINITY, 0.f);
}

// --------------------------------------------------------------- scoring ---
//
// Launch 1 of a decode step.  Workgroup (pair, c) scores pooled keys
// [CK c, CK (c + 1)), CK = 64 T, of one (sequence, KV head) pair: wave w takes
// tiles wT .. wT + T - 1 of 16 keys, every load in flight before the first
// MFMA, so a short context is spread over many CUs (one CU streams only about
// 100 GB/s).  Relative to the chunk's own per-head maximum m_h of
// z_h[j] = scale log2(e) q_h . Kc_j it leaves, for every head h of the group:
//   cml[pair][h][c]   = (m_h, sum over the chunk's keys of 2^(z_h[j] - m_h))
//   bpart[pair][b][h] = sum over keys 4b-1 .. 4b+3 inside the chunk of
//                       2^(z_h[j] - m_h), for the chunk's CK/4 blocks b
//   spill[pair][h][c] = 2^(z_h[j] - m_h) of the chunk's last key j, which is
//                       key 4b-1 of the first block b of the next chunk.
// These are exact rescalings of the per-head softmax terms: the selection
// multiplies them by 2^(m_h - lse_h) once every chunk's (m, sum) is known.
// The chunk holding the key completed by the current token (tokens L-32 ..
// L-1) pools it from K first (fp64 sum, one bf16 rounding), stores it to the
// pooled-key page and substitutes it into its MFMA operand in registers.
//
// The local window needs no selection, so its pages (one four-wave
// workgroup each, window_slot) ride in whichever launch has room: here,
// after the npairs * nchunks scoring workgroups, when the attention launch
// would need more than two workgroups per CU (the scoring reads little from
// HBM, so the window streams alongside it); otherwise in the attention
// launch, beside the selection, which reads nothing from HBM either.

struct ScoreArgs {
    const uint16_t* q;
    const uint16_t* k_pool;  // window pages and the tokens of the appended key
    const uint16_t* v_pool;  // (the recent-page ring when ring > 0)
    uint16_t* kc_pool;
    const int32_t* table;
    int ring;                // recent pages per sequence (offloaded KV), else 0
    const int32_t* cu_k;
    int max_blocks, num_pages, Lmax, Hq, Hkv, G, gp;
    float scale_log2;
    int append;  // pool the key completed by the current token
    int stream_kc;  // stream the pooled-key loads (non-temporal)
    int nchunks, nbk;
    float2* cml;
    float* spill;
    float* bpart;
    int nscore;                   // scoring workgroups = pairs * ceil(nchunks / CPW)
    int wslots, wblocks, split0;  // window pages per pair (0: none); partial slot of slot 0
    int wgroups;                  // window workgroups per pair: wslots (a page each) or
                                  // ceil(wslots / 4) (a page per wave, T = 8 only)
    int nsplit;
    float* po;
    float2* pml;
};

// Dynamic LDS of the scoring launch: a chunk's logits, [G][CK + 4] floats,
// or a window page's exchange, or the four wave states of a window group.
inline size_t score_lds_bytes(int T, int G, bool per_wave)
{
    size_t z = (size_t)G * (64 * T + 4) * sizeof(float);
    if (z < sizeof(SplitPageLds)) z = sizeof(SplitPageLds);
    if (per_wave && z < sizeof(CombineLds)) z = sizeof(CombineLds);
    return z;
}

// This lane's pooled keys of T tiles of 16 (tile t: page pgj[t], keys
// kwj + 16 t + r), as MFMA operands; page ids clamped into the pool.
// Streamed (non-temporal) when a step's pooled keys are too many to stay
// cached until the next step (stream: wave-uniform).
template <int T>
__device__ __forceinline__ void load_chunk_keys(uint4 (&kv)[T][4], const int (&pgj)[T], int kwj,
                                                const uint16_t* kc_pool, int num_pages, int Hkv,
                                                int g, int r, int kq, bool stream)
{
    const uint16_t* kp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int p = min(max(pgj[t], 0), num_pages - 1);
        kp[t] = kc_pool + ((size_t)p * Hkv + g) * SL * D;
    }
    if (stream) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kv[t][st] = ldg16_stream(kp[t] + kc_chunk((kwj + t * 16 + r) % SL, st * 4 + kq));
    } else {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kv[t][st] = ldg16(kp[t] + kc_chunk((kwj + t * 16 + r) % SL, st * 4 + kq));
    }
}

// CPW: chunks per scoring workgroup (1 or 2; 2 only with T = 8).  With two,
// the second chunk's keys are requested into the key registers as soon as
// the first chunk's MFMAs have read them, so they stream while the first
// chunk's logits go through LDS and its partials are stored: a long context
// is then scored in one dispatch round of workgroups whose loads keep HBM
// busy, instead of two rounds that all load, then all compute, together
// (and two such workgroups must fit on a CU: the launch bounds say so).
template <int T, int CPW>
__global__ __launch_bounds__(kScoreWaves * 64, CPW) void score_kernel(ScoreArgs a)
{
    constexpr int CK = 64 * T;  // keys per chunk: kScoreWaves waves x T tiles x 16
    constexpr int CB = CK / 4;  // blocks per chunk
    constexpr int ZS = CK + 4;  // LDS row stride of the logits
    static_assert(kScoreWaves == 4, "a chunk is four waves of T tiles");
    extern __shared__ __align__(16) char smem[];
    float* zl = reinterpret_cast<float*>(smem);  // [G][ZS]
    __shared__ float wm[kScoreWaves][kMaxGroup], wsum[kScoreWaves][kMaxGroup];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    // The counts that place the workgroup and its first loads, as scalar
    // registers through an empty asm: read in the first batch of argument
    // loads, not in later batches that each wait for the one before.
    int nscore = a.nscore, nchunks = a.nchunks, Hkv = a.Hkv, max_blocks = a.max_blocks;
    int stream_kc = a.stream_kc;
    asm("" : "+s"(nscore), "+s"(nchunks), "+s"(Hkv), "+s"(max_blocks), "+s"(stream_kc));
    // Scoring workgroups are dealt to the eight XCDs (round-robin by index)
    // so that a pair's chunks run on one XCD, the one its attention
    // workgroups use in the next launch: slot b is scoring workgroup
    // (b % 8) * spx + b / 8 (spx = ceil(nscore / 8); past nscore: idle).
    const int spx = (nscore + 7) >> 3;
    NOSA_TL(0, 0);
    if ((int)blockIdx.x >= 8 * spx) {  // window workgroup
        NOSA_TL_ROLE(0, 1);
        const int w = (int)blockIdx.x - 8 * spx;
        const int pair = w / a.wgroups;
        if constexpr (T == 8) {
            if (a.wgroups != a.wslots) {  // a page per wave
                window_group(a.q, a.k_pool, a.v_pool, a.table, a.ring, a.cu_k, a.max_blocks, a.Lmax,
                             a.Hq, a.Hkv, a.G, a.scale_log2, a.wblocks, pair / a.Hkv, pair % a.Hkv,
                             w % a.wgroups, a.nsplit, a.split0, a.po, a.pml,
                             *reinterpret_cast<CombineLds*>(smem), true);
                NOSA_TL(0, 2);
                return;
            }
        }
        window_slot<true>(a.q, a.k_pool, a.v_pool, a.table, a.ring, a.cu_k, a.max_blocks, a.Lmax,
                          a.Hq, a.Hkv, a.G, a.scale_log2, a.wblocks, pair / a.Hkv, pair % a.Hkv,
                          w % a.wgroups, a.nsplit, a.split0, a.po, a.pml,
                          *reinterpret_cast<SplitPageLds*>(smem));
        NOSA_TL(0, 2);
        return;
    }
    const int sid = ((int)blockIdx.x & 7) * spx + ((int)blockIdx.x >> 3);
    if (sid >= nscore) return;  // (whole workgroup)
    NOSA_TL_ROLE(0, 0);
    const int cpp = (nchunks + CPW - 1) / CPW;  // scoring workgroups per pair
    const int pair = sid / cpp, c0 = (sid % cpp) * CPW;
    const int s = pair / Hkv, g = pair % Hkv;
    const int32_t* trow = a.table + (size_t)s * max_blocks;
    // Table entries of this lane's keys in a chunk (the row has max_blocks
    // entries; those past the sequence may hold anything, so the page ids
    // are clamped into the pool: their keys are masked).  The first chunk's
    // are issued before the length is known, with the query.
    int pg[T];
    auto table_entries = [&](int cj) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int blk = (cj * CK + wave * T * 16 + t * 16 + r) / SL;
            pg[t] = trow[blk < max_blocks ? blk : max_blocks - 1];
        }
    };
    table_entries(c0);
    bf16x8 qb[4];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
    const int L = seq_len(a.cu_k, s, a.Lmax);
    const int nc = dev_num_keys(L);
    // The table entries are taken as an operand here so that their loads
    // stay ahead of the exit test below (they would otherwise move after
    // it, one more memory round trip before the keys can be requested).
    asm volatile("" ::"v"(pg[0]));
    if (c0 * CK >= nc) return;  // the pair has no key in these chunks (whole workgroup)
    uint4 kv[T][4];
    load_chunk_keys<T>(kv, pg, c0 * CK + wave * T * 16, a.kc_pool, a.num_pages, Hkv, g, r, kq,
                       stream_kc != 0);
    const int jn = nc - 1;
    const bool appending = a.append && L >= kPoolK && (L - kPoolK) % kPoolS == 0;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
    const int c = c0 + j;
    const int k0 = c * CK;
    if (c >= nchunks || k0 >= nc) break;  // (whole workgroup)
    const int kw = k0 + wave * T * 16;  // first key of this wave
    if (appending && jn >= kw && jn < kw + T * 16) {  // wave-uniform
        const int tr = lane >> 4, cc = lane & 15;  // 4 token phases x 16 channel chunks
        // tokens 16 jn + tr + 4i, i < 8
        int kpg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            kpg[i] = window_page(a.table, a.max_blocks, a.ring, s, (jn * kPoolS + tr + 4 * i) / BS);
        uint4 kt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = jn * kPoolS + tr + 4 * i;
            kt[i] = ldg16(a.k_pool + ((size_t)kpg[i] * a.Hkv + g) * BS * D + k_chunk(t % BS, cc));
        }
        double acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc8(acc, kt[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] += __shfl_xor(acc[e], 16);
            acc[e] += __shfl_xor(acc[e], 32);
        }
        const uint4 appkey = round8(acc);  // channels 8cc .. 8cc+7, same in every phase
        const int ta = (jn - kw) / 16, ra = (jn - kw) % 16;
        const int jb = jn / SL;  // key jn's page
        const int ppg = trow[jb < max_blocks ? jb : max_blocks - 1];
        if (tr == 0)
            *reinterpret_cast<uint4*>(a.kc_pool + ((size_t)ppg * a.Hkv + g) * SL * D +
                                      kc_chunk(jn % SL, cc)) = appkey;
        // MFMA operand of key jn: lane (ra, kq), k-step st holds chunk 4 st + kq
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int src = st * 4 + kq;
            const uint4 v = make_uint4(__shfl(appkey.x, src), __shfl(appkey.y, src),
                                       __shfl(appkey.z, src), __shfl(appkey.w, src));
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (t == ta && r == ra) kv[t][st] = v;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // logits -> LDS; this lane's (max, sum 2^(z - max)) for head r
    float m_l = -INFINITY, s_l = 0.f;
    float zv[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(kv[t][st]), qb[st], acc);
        const int key0 = kw + t * 16 + kq * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zv[t][i] = key0 + i < nc ? acc[i] * a.scale_log2 : -INFINITY;
            m_l = fmaxf(m_l, zv[t][i]);
        }
        if (r < a.G)
            *reinterpret_cast<float4*>(zl + r * ZS + (wave * T + t) * 16 + kq * 4) =
                make_float4(zv[t][0], zv[t][1], zv[t][2], zv[t][3]);
    }
    if (j == 0) NOSA_TL(0, 1);  // the first chunk's keys in and multiplied
    const bool next = j + 1 < CPW && c + 1 < nchunks && k0 + CK < nc;  // (whole workgroup)
    if (next) table_entries(c + 1);  // the next chunk's, now that kv is free
    if (m_l != -INFINITY) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_l += fexp2(zv[t][i] - m_l);
    }
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m_l, off), so = __shfl_xor(s_l, off);
        const float mn = fmaxf(m_l, mo);
        s_l = mn == -INFINITY ? 0.f : s_l * fexp2(m_l - mn) + so * fexp2(mo - mn);
        m_l = mn;
    }
    if (kq == 0 && r < a.G) {
        wm[wave][r] = m_l;
        wsum[wave][r] = s_l;
    }
    __syncthreads();
    if (next)  // its keys stream while this chunk's block sums and partials are made
        load_chunk_keys<T>(kv, pg, k0 + CK + wave * T * 16, a.kc_pool, a.num_pages, Hkv, g, r, kq,
                           stream_kc != 0);
    // per (block, head): the block's keys in this chunk, relative to the
    // chunk maximum (finite: key k0 exists for every head)
    const size_t prow = (size_t)pair * a.nbk + (size_t)c * CB;
    const size_t crow = (size_t)pair * a.G * a.nchunks + c;  // + h * nchunks
    for (int idx = tid; idx < a.gp * CB; idx += kScoreWaves * 64) {
        const int h = idx % a.gp, bb = idx / a.gp;
        if (h >= a.G) {  // padding of the row to gp heads: exact zeros
            a.bpart[(prow + bb) * a.gp + h] = 0.f;
            continue;
        }
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w) m = fmaxf(m, wm[w][h]);
        const float4 z4 = *reinterpret_cast<const float4*>(zl + h * ZS + 4 * bb);
        float part = fexp2(z4.x - m) + fexp2(z4.y - m) + fexp2(z4.z - m) + fexp2(z4.w - m);
        if (bb > 0) part += fexp2(zl[h * ZS + 4 * bb - 1] - m);
        a.bpart[(prow + bb) * a.gp + h] = part;
        if (bb == CB - 1) a.spill[crow + (size_t)h * a.nchunks] = fexp2(z4.w - m);
    }
    if (tid < a.G) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w) m = fmaxf(m, wm[w][tid]);
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w)
            if (wsum[w][tid] > 0.f) sum += wsum[w][tid] * fexp2(wm[w][tid] - m);
        a.cml[crow + (size_t)tid * a.nchunks] = make_float2(m, sum);
    }
    if (j + 1 < CPW) __syncthreads();  // zl, wm and wsum are rewritten by the next chunk
    }
    NOSA_TL(0, 2);
}


// ----------------------------------------------- selection + attention ---
//
// Launch 2 of a decode step: `groups` four-wave top workgroups per pair.
// Every one recomputes the pair's selection from the scoring partials --
// per-head log-sum-exp over the chunks, block importance, top-k -- a few
// microseconds of LDS work (latency, not bandwidth) that replaces a hand-off
// between workgroups (a kernel boundary is cheaper on this chip than any
// in-launch hand-off with counters); it then attends its slice of the picks,
// one page per wave (picks 4 R k .. 4 R (k+1) - 1), and stores one partial
// at slot k.  Slots groups .. nsplit - 1 hold the window pages' partials,
// from `wslots` window workgroups per pair in this launch or the scoring
// launch (window_slot).
//
// Block importance: I[b] = mean over keys j of 4b-1 .. 4b+3 below n_c of
// sum_h 2^(z_h[j] - lse_h) -- the softmax over the pooled keys per query
// head, summed over the group, pooled over the keys whose window overlaps
// block b (page "NOSA-1B 模型家族全景", core principle, CIS score mean pooling;
// page "NOSA-1B 性能基准全解析" section 三.3).

constexpr int kMaxRounds = 8;  // top-k blocks per wave (compiled limit of the plan)
constexpr int kFetch = 1 << 30;      // slot_of flag: the pick is read from host memory

struct TopArgs {
    const uint16_t* q;
    const uint16_t* k_pool;  // top-k pages (host pools when offloaded)
    const uint16_t* v_pool;
    const uint16_t* wk;      // window pages: the pools, or the recent-page ring
    const uint16_t* wv;
    int ring;                // recent pages per sequence (offloaded KV), else 0
    int num_pages;
    // offloaded KV: the block cache of each pair, `cap` pages; map[pair][slot]
    // = block held, used[pair][slot] = sequence length when it was last
    // picked (read); map_next / used_next = both after this step (written by
    // workgroup 0 of the pair, installed by the merge launch)
    uint16_t* cache_k;
    uint16_t* cache_v;
    const int32_t* map;
    const int32_t* used;
    int32_t* map_next;
    int32_t* used_next;
    int32_t* fetch_out;      // [pairs] picks read from host memory, or null
    int cap;
    const int32_t* table;
    const int32_t* cu_k;
    int max_blocks, Lmax, Hq, Hkv, G, gp;
    float scale_log2;
    int chunk_keys, cb_shift, nchunks, nbk;  // cb_shift = log2(chunk_keys / 4)
    const float2* cml;
    const float* spill;
    const float* bpart;
    int topk, wblocks, max_nb, max_sel;
    int groups, rounds;  // top workgroups per pair; top-k blocks per wave
    int wslots;          // window slots (pages) per pair in this launch (0: none)
    int wgroups;         // window workgroups per pair: wslots or ceil(wslots / 4)
    int nsplit;          // partial slots per head
    int4 disp;           // top / window workgroups per XCD, top / window workgroups of the
                         // launch (one argument, so one scalar load gates the early exit)
    int scores_only;     // importance only (no selection, no attention)
    int stream;          // the host's choice of instantiation: page loads streamed
    float* scores_out;   // [pairs][max_nb] or null (workgroup 0 of a pair writes)
    int32_t* sel_out;    // [pairs][max_sel] or null (workgroup 0 of a pair writes)
    int32_t* cnt_out;    // [pairs] or null
    float* po;
    float2* pml;
};

struct alignas(16) TopLds {
    union {
        struct {
            float f[kMaxChunks][kMaxGroup];   // 2^(m_ch - lse_h): chunk partials -> softmax weights
            float fs[kMaxChunks][kMaxGroup];  // f[c][h] * spill[c][h]
            SelectLds sel;
        };
        SplitPageLds page;  // window workgroups
        struct {            // offloaded KV, after the selection
            int4 age[kMaxCacheSlots / 4];  // eviction order key per slot (free slots)
            int freeslot[kMaxCacheSlots];  // free slots, least recently picked first
            int misspick[kMaxCacheSlots];  // picks not in the cache in pick order
        } miss;
    };
    CombineLds comb;
    // (block, page) of this workgroup's picks (the pair's every pick when the
    // KV is offloaded)
    int2 list[kMaxCacheSlots];
    int slot_of[kMaxCacheSlots];  // offloaded KV: cache slot per pick (| kFetch)
    int ocnt[2][kStep2Waves];
};
static_assert(kMaxCacheSlots >= kStep2Waves * kMaxRounds, "list of a top workgroup");

// Dynamic LDS of a top workgroup: the block-table row, and the importance
// of blocks past the register rounds.
inline size_t top_lds_bytes(int max_nb, int krb)
{
    const size_t row = ((size_t)max_nb * sizeof(int32_t) + 15) / 16 * 16;
    return row + (max_nb > krb * 256 ? (size_t)max_nb * sizeof(float) : 16);
}

// Importance of block b from its partial row (heads 4u .. 4u+3 in bv[u];
// the padding heads G .. 4 GP4 - 1 carry zero sums and zero weights).
// Straight-line: both LDS rows are read whatever b is (indexes clamped into
// the 64 rows) and the terms that do not apply are dropped afterwards, so
// the reads of several blocks can be in flight together.
template <int GP4>
__device__ __forceinline__ float block_importance(int b, int nc, int cb_shift, int nvalid, int G,
                                                  const float4 (&bv)[GP4], const TopLds& sh)
{
    const int c = b >> cb_shift;
    const int cr = c < kMaxChunks ? c : kMaxChunks - 1;
    const int cp = c > 0 ? (c <= kMaxChunks ? c - 1 : kMaxChunks - 1) : 0;
    float own = 0.f, spill = 0.f;
#pragma unroll
    for (int u = 0; u < GP4; ++u) {
        const float4 f4 = *reinterpret_cast<const float4*>(&sh.f[cr][4 * u]);
        const float4 s4 = *reinterpret_cast<const float4*>(&sh.fs[cp][4 * u]);
        const float v[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
        const float f[4] = {f4.x, f4.y, f4.z, f4.w};
        const float q[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // heads past G: zero weights and zero sums
            own += f[e] * v[e];
            spill += q[e];
        }
    }
    // key 4b-1 lies in the previous chunk when b starts a chunk
    const bool first = b > 0 && (b & ((1 << cb_shift) - 1)) == 0 && 4 * b - 1 < nc;
    const float sum = (c < nvalid ? own : 0.f) + (first ? spill : 0.f);
    const int jlo = 4 * b - 1 > 0 ? 4 * b - 1 : 0;
    const int jhi = 4 * b + 3 < nc - 1 ? 4 * b + 3 : nc - 1;
    return jlo <= jhi ? sum / (float)(jhi - jlo + 1) : -INFINITY;
}

// Global-memory (address space 1) views of the chunk partials: a kernel
// argument pointer that has passed through an asm statement is otherwise a
// flat pointer, and flat loads also hold up every wait for scalar loads.
typedef float gf2 __attribute__((ext_vector_type(2)));
typedef float gf4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) gf2* GlobalF2;
typedef const __attribute__((address_space(1))) float* GlobalF1;
typedef const __attribute__((address_space(1))) gf4* GlobalF4;
typedef const __attribute__((address_space(1))) int32_t* GlobalI1;

// KRB: candidate rounds of 256 blocks whose importance stays in registers
// (1, 2, 4 or 8; blocks past KRB * 256 go through LDS, only when KRB = 8).
// GP4: float4 loads per block of the partial row (G <= 4 GP4).
// OFF: offloaded KV.  The window pages come from the ring of recent pages in
// device memory; the top-k picks from the pair's block cache.  Every top
// workgroup of the pair derives the same slot assignment from the cache map
// and the selection: picks already cached keep their slot; the others take
// the free slots (those whose block was not picked), least recently picked
// first, and are read from host memory, attended and written into their slot
// in one pass.
// Cached blocks lie before the window, so they are complete and never change.
template <int KRB, int GP4, bool OFF, bool STREAM>
__global__ __launch_bounds__(kStep2Waves * 64, 2) void top_kernel(TopArgs a)
{
    constexpr int NT = kStep2Waves * 64;
    static_assert(KRB <= kSelKeyRounds, "register rounds of the selector");
    extern __shared__ __align__(16) char smem[];
    __shared__ TopLds sh;
    // Workgroups are dealt to the XCDs round-robin by index.  XCD x runs top
    // workgroups x * tpx .. x * tpx + tpx - 1 first, then window workgroups
    // x * wpx .. x * wpx + wpx - 1: the same pairs, so the top workgroups of
    // a pair (which read the same partials) share an L2, and the CUs each
    // get one top workgroup before any gets a second.
    const int xcd = (int)(blockIdx.x % 8), pos = (int)(blockIdx.x / 8);
    int4 disp = a.disp;  // tpx, wpx, ntop, nwin
    // The empty asm takes the four counts as scalar registers, so they are
    // read together, in the one batch of argument loads that gates the
    // early exit, instead of one dependent scalar load after another (not
    // volatile: such an asm touches no memory, so the uniform loads after
    // it stay scalar loads).
    asm("" : "+s"(disp.x), "+s"(disp.y), "+s"(disp.z), "+s"(disp.w));
    const bool window = pos >= disp.x;
    const int lid = window ? xcd * disp.y + (pos - disp.x) : xcd * disp.x + pos;
    if (lid >= (window ? disp.w : disp.z)) return;  // whole workgroup
    NOSA_TL(1, 0);
    NOSA_TL_ROLE(1, window ? 1 : 0);
    // the chunk partials' addresses, in the argument batch that follows (a
    // load of their own later would also wait for the sequence bounds)
    GlobalF2 cml = (GlobalF2)a.cml;
    GlobalF1 spill = (GlobalF1)a.spill;
    GlobalF4 bpart4 = (GlobalF4)a.bpart;
    asm("" : "+s"(cml), "+s"(spill), "+s"(bpart4));
    if (window && a.wgroups == a.wslots) {  // one window page, the four waves together
        const int pair = lid / a.wgroups;
        window_slot<STREAM>(a.q, a.wk, a.wv, a.table, a.ring, a.cu_k, a.max_blocks, a.Lmax, a.Hq,
                            a.Hkv, a.G, a.scale_log2, a.wblocks, pair / a.Hkv, pair % a.Hkv,
                            lid % a.wgroups, a.nsplit, a.groups, a.po, a.pml, sh.page);
        NOSA_TL(1, 5);
        return;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    // window workgroup j (a page per wave: slots 4 j + wave) or top workgroup k
    const int pair = window ? lid / a.wgroups : lid / a.groups;
    const int k = window ? lid % a.wgroups : lid % a.groups;
    const int s = pair / a.Hkv, g = pair % a.Hkv;
    const int32_t* trow = a.table + (size_t)s * a.max_blocks;
    const size_t head_row0 = (size_t)s * a.Hq + g * a.G;
    // the sequence's bounds, read here (scalar loads) and used only after
    // the top workgroups' first loads are issued
    const int cu0 = a.cu_k[s], cu1 = a.cu_k[s + 1];

    bf16x8 qb[4];
    int rounds = 1, lbase = 0;
    int L, nb, nc;  // sequence length, its blocks and pooled keys
    if (window) {
        L = seq_len_of(cu0, cu1, a.Lmax);
        nb = (L + BS - 1) / BS;
        nc = dev_num_keys(L);
        // this wave's window page as a one-entry list; the attention below
        // is the top workgroups' own
        const int wn = nb < a.wblocks ? nb : a.wblocks;
        const int x = 4 * k + wave;
        int2 e = make_int2(-1, -1);
        if (x < wn)
            e = make_int2(nb - wn + x, window_page(a.table, a.max_blocks, a.ring, s, nb - wn + x));
        if (lane == 0) sh.list[wave] = e;
        load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
        __syncthreads();
    } else {
    // ---- top workgroup k: the pair's selection, then picks 4 R k .. 4 R (k+1) - 1
    int32_t* spg = reinterpret_cast<int32_t*>(smem);  // block-table row
    float* sI = reinterpret_cast<float*>(smem + ((size_t)a.max_nb * sizeof(int32_t) + 15) / 16 * 16);
    const int CK = a.chunk_keys;

    // Loads, in the order they are needed (they complete in order, so each
    // wait below covers only what was issued before), none of them waiting
    // for the sequence length (read after them): chunk partials (lane = chunk, heads wave + 4u;
    // chunks past the pair's last are masked later), this thread's importance
    // partials and block-table entries, the query.  Every address is clamped
    // in range, so no load needs a branch.
    float2 cv[4];
    float sv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int h = wave + 4 * u < a.G ? wave + 4 * u : a.G - 1;
        const size_t o = ((size_t)pair * a.G + h) * a.nchunks + (lane < a.nchunks ? lane : 0);
        const gf2 c2 = cml[o];
        cv[u] = make_float2(c2.x, c2.y);
        sv[u] = spill[o];
    }
    float4 bv[KRB][GP4];
#pragma unroll
    for (int i = 0; i < KRB; ++i) {
        const int b = i * NT + tid < a.nbk ? i * NT + tid : a.nbk - 1;
        GlobalF4 src = bpart4 + ((size_t)pair * a.nbk + b) * a.gp / 4;  // gp is a multiple of 4
#pragma unroll
        for (int u = 0; u < GP4; ++u) {
            const gf4 x = src[u * 4 < a.gp ? u : 0];
            bv[i][u] = make_float4(x.x, x.y, x.z, x.w);
        }
    }
    int tv[KRB];
#pragma unroll
    for (int i = 0; i < KRB; ++i) tv[i] = trow[i * NT + tid < a.max_nb ? i * NT + tid : a.max_nb - 1];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
    int cb = -1, cu = 0;  // offloaded KV: block in cache slot tid, length at its last pick
    if (OFF) {
        if (tid < a.cap) {
            cb = a.map[(size_t)pair * a.cap + tid];
            cu = a.used[(size_t)pair * a.cap + tid];
        }
        sh.slot_of[tid] = -1;
    }
    // nothing above waits for the length, which arrives while those loads
    // are in flight
    __builtin_amdgcn_sched_barrier(0);
    L = seq_len_of(cu0, cu1, a.Lmax);
    nb = (L + BS - 1) / BS;
    nc = dev_num_keys(L);
    const int nvalid = (nc + CK - 1) / CK;  // chunks holding keys of this pair, <= 64
    NOSA_TL(1, 12);  // the sequence bounds in
    select_lds_clear<NT>(sh.sel);
    // per-head log2-sum-exp2 over the chunks, then each chunk's weight
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int h = wave + 4 * u;
        if (h >= a.G) {  // heads G .. 4 GP4 - 1 read by block_importance: zero weights
            if (h < 4 * GP4) {
                sh.f[lane][h] = 0.f;
                sh.fs[lane][h] = 0.f;
            }
            continue;
        }
        const bool ok = lane < nvalid;
        const float m = ok ? cv[u].x : -INFINITY;
        const float M = wave_max_f(m);
        const float S = wave_sum_f(ok ? cv[u].y * fexp2(m - M) : 0.f);
        const float lse = M + log2f(S);
        const float f = ok ? fexp2(m - lse) : 0.f;
        sh.f[lane][h] = f;
        sh.fs[lane][h] = ok ? f * sv[u] : 0.f;
    }
    NOSA_TL(1, 6);  // this wave's log-sum-exp (its loads in)
#pragma unroll
    for (int i = 0; i < KRB; ++i)
        if (i * NT + tid < a.max_nb) spg[i * NT + tid] = tv[i];
    __syncthreads();
    NOSA_TL(1, 1);  // log-sum-exp and chunk weights
    uint32_t keys[kSelKeyRounds];
#pragma unroll
    for (int i = 0; i < kSelKeyRounds; ++i) keys[i] = 0u;
    float* so = a.scores_out && k == 0 ? a.scores_out + (size_t)pair * a.max_nb : nullptr;
#pragma unroll
    for (int i = 0; i < KRB; ++i) {
        if (i * NT >= nb) break;  // rounds wholly past the sequence
        const int b = i * NT + tid;
        const float I = block_importance<GP4>(b, nc, a.cb_shift, nvalid, a.G, bv[i], sh);
        keys[i] = b < nb ? order_key(I) : 0u;
        if (so && b < nb) so[b] = I;
    }
    // contexts past KRB * 256 blocks: the rest of the row and of the
    // importance through LDS
    for (int b = KRB * NT + tid; b < a.max_nb; b += NT) {
        spg[b] = trow[b];
        if (b >= nb) continue;
        float4 bw[GP4];
        const int bc = b < a.nbk ? b : a.nbk - 1;
        const float4* src = reinterpret_cast<const float4*>(a.bpart + ((size_t)pair * a.nbk + bc) * a.gp);
#pragma unroll
        for (int u = 0; u < GP4; ++u) bw[u] = src[u * 4 < a.gp ? u : 0];
        const float I = block_importance<GP4>(b, nc, a.cb_shift, nvalid, a.G, bw, sh);
        sI[b] = I;
        if (so) so[b] = I;
    }
    if (so)
        for (int b = nb + tid; b < a.max_nb; b += NT) so[b] = -INFINITY;
    if (a.scores_only) return;
    const int ncand = nb > a.wblocks ? nb - a.wblocks : 0;
    const bool in_regs = ncand <= KRB * NT;  // every candidate's key is in keys[]
    if (in_regs) select_wave_range<NT, kSelKeyRounds>(keys, ncand, sh.sel);
    __syncthreads();  // sI, the rest of the row, the key ranges
    NOSA_TL(1, 2);  // block importance
    const int lo = k * a.rounds * kStep2Waves;
    select_blocks_wg<kStep2Waves, true>(keys, sI, nb, a.wblocks, a.topk, sh.sel,
                                        a.sel_out && k == 0 ? a.sel_out + (size_t)pair * a.max_sel : nullptr,
                                        a.cnt_out && k == 0 ? a.cnt_out + pair : nullptr, a.max_sel,
                                        sh.list, OFF ? 0 : lo, OFF ? kMaxCacheSlots : a.rounds * kStep2Waves,
                                        spg, in_regs, [](int m) { NOSA_TL(1, 8 + m); });
    __syncthreads();  // the list
    NOSA_TL(1, 3);  // selection
    rounds = a.rounds;
    if (OFF) {
        // picks 0 .. npk - 1 in sh.list, ascending block ids
        lbase = lo;
        const int npk = a.topk < ncand ? a.topk : ncand;
        bool hit = false;
        if (cb >= 0 && cb < ncand) {  // is slot tid's block a pick?  binary search
            int x0 = 0, x1 = npk;
            while (x0 < x1) {
                const int mid = (x0 + x1) >> 1;
                if (sh.list[mid].x < cb) x0 = mid + 1;
                else x1 = mid;
            }
            if (x0 < npk && sh.list[x0].x == cb) {
                sh.slot_of[x0] = tid;
                hit = true;
            }
        }
        __syncthreads();
        const bool fre = tid < a.cap && !hit;
        const bool mis = tid < npk && sh.slot_of[tid] < 0;
        // eviction order of the free slots: empty ones, then by the length
        // at the last pick, then by slot
        const int age = fre ? (cb < 0 ? INT_MIN : cu) : INT_MAX;
        reinterpret_cast<int*>(sh.miss.age)[tid] = age;
        const uint64_t bm = __ballot(mis);
        if (lane == 0) sh.ocnt[1][wave] = (int)__popcll(bm);
        __syncthreads();
        int rm = lanes_below(bm), nmiss = 0;
#pragma unroll
        for (int w = 0; w < kStep2Waves; ++w) {
            if (w < wave) rm += sh.ocnt[1][w];
            nmiss += sh.ocnt[1][w];
        }
        int rf = 0;  // rank of a free slot in eviction order
        if (nmiss > 0) {  // (workgroup-uniform: every pick cached skips the assignment)
            if (fre) {
                for (int u4 = 0; u4 < kMaxCacheSlots / 4; ++u4) {
                    const int4 v = sh.miss.age[u4];
                    const int u = 4 * u4;
                    rf += (v.x < age || (v.x == age && u < tid)) + (v.y < age || (v.y == age && u + 1 < tid)) +
                          (v.z < age || (v.z == age && u + 2 < tid)) + (v.w < age || (v.w == age && u + 3 < tid));
                }
            }
            if (fre && rf < nmiss) sh.miss.freeslot[rf] = tid;
            if (mis) sh.miss.misspick[rm] = tid;
            __syncthreads();
            // cap >= topk, so there are at least as many free slots as misses
            if (mis) sh.slot_of[tid] = sh.miss.freeslot[rm] | kFetch;
        }
        if (k == 0) {
            if (tid < a.cap) {
                const bool fill = fre && rf < nmiss;
                a.map_next[(size_t)pair * a.cap + tid] = fill ? sh.list[sh.miss.misspick[rf]].x : cb;
                a.used_next[(size_t)pair * a.cap + tid] = hit || fill ? L : cu;
            }
            if (tid == 0 && a.fetch_out) a.fetch_out[pair] = nmiss;
        }
        if (nmiss > 0) __syncthreads();  // slot_of (the hits' entries were set two barriers ago)
    }
    }
    AttnState A;
    attn_init(A);
#pragma unroll 1
    for (int rr = 0; rr < rounds; ++rr) {
        const int p = lbase + rr * kStep2Waves + wave;
        const int2 e = p < kMaxCacheSlots ? sh.list[p] : make_int2(-1, -1);
        if (e.x < 0) continue;
        const uint16_t* kb;
        const uint16_t* vb;
        if (window) {
            kb = a.wk + ((size_t)e.y * a.Hkv + g) * BS * D;
            vb = a.wv + ((size_t)e.y * a.Hkv + g) * D * BS;
        } else if (OFF) {
            const int so = sh.slot_of[p];
            const size_t unit = (size_t)pair * a.cap + (so & (kFetch - 1));
            uint16_t* ck = a.cache_k + unit * BS * D;
            uint16_t* cv = a.cache_v + unit * BS * D;
            if (so & kFetch) {  // from host memory, kept in the cache slot
                const int pg = min(max(e.y, 0), a.num_pages - 1);
                const int lane8 = (16 * kq + r) * 8;
                PageRegs pr;
                load_page(a.k_pool + ((size_t)pg * a.Hkv + g) * BS * D,
                          a.v_pool + ((size_t)pg * a.Hkv + g) * D * BS, lane8, pr, STREAM);
                __builtin_amdgcn_sched_barrier(0);
                store_page(ck, cv, lane8, pr);
                attend_loaded(pr, L - e.x * BS, qb, a.scale_log2, r, kq, A);
                continue;
            }
            kb = ck;
            vb = cv;
        } else {
            kb = a.k_pool + ((size_t)e.y * a.Hkv + g) * BS * D;
            vb = a.v_pool + ((size_t)e.y * a.Hkv + g) * D * BS;
        }
        attend_page(kb, vb, L - e.x * BS, qb, a.scale_log2, r, kq, A, STREAM);
    }
    NOSA_TL(1, 4);  // pages attended
    store_wg_partial(sh.comb, A, a.G, head_row0, a.nsplit, window ? a.groups + k : k, a.po, a.pml);
    NOSA_TL(1, 5);
}

// ------------------------------------------------ attention (alone) ---

struct AttendArgs {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* table;
    const int32_t* cu_k;
    int max_blocks, Lmax, Hq, Hkv, G;
    float scale_log2;
    int groups;          // workgroups per pair
    const int32_t* sel;  // [pairs][max_sel] block ids
    const int32_t* cnt;  // [pairs]
    int max_sel;
    int stream;          // the host's choice of instantiation: page loads streamed
    float* po;
    float2* pml;
};

// Combination of the nsplit partials (m_i, l_i, o_i) of each head row into
// out = sum_i 2^(m_i - M) o_i / L and lse = (M + log2 L) ln 2, with
// M = max_i m_i and L = sum_i 2^(m_i - M) l_i (empty rows: out 0, lse -inf).
// One workgroup of 128 threads per row, thread c = channel c; partials are
// taken 32 at a time with every load of a batch in flight (the (m, l) pairs
// a lane each, their maximum and weighted sum by wave reductions, the
// weights read back lane by lane for the channel sums), the running
// (M, L, acc) rescaled between batches.  A launch of its own, so the
// partials of every workgroup of the step are complete when it starts.
// With offloaded KV the row of each group's first head also installs the
// pair's new cache map and pick lengths (map_next -> map, used_next -> used,
// `cap` entries each): every workgroup of the attention launch has read the
// old ones by now.
constexpr int kMergeBatch = 32;

__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ po,
                                                    const float2* __restrict__ pml, int nsplit,
                                                    float* __restrict__ out, float* __restrict__ lse,
                                                    const int32_t* __restrict__ map_next,
                                                    const int32_t* __restrict__ used_next,
                                                    int32_t* __restrict__ map,
                                                    int32_t* __restrict__ used, int cap, int G,
                                                    size_t rows)
{
    // the empty asm reads every argument in one batch of scalar loads (not
    // the count first for the loop test, then the rest); as its operands
    // are inputs only, the pointers stay global ones
    asm volatile("" ::"s"(po), "s"(pml), "s"(nsplit), "s"(out), "s"(lse), "s"(map_next),
                 "s"(used_next), "s"(map), "s"(used), "s"(cap), "s"(G), "s"(rows));
    // head rows dealt to the XCDs like the attention workgroups' pairs (a
    // pair's rows on the XCD whose L2 holds its partials): slot b is row
    // (b % 8) * rpx + b / 8, rpx = gridDim.x / 8 (past the last row: idle)
    const int rpx = (int)gridDim.x >> 3;
    const size_t row = (size_t)(((int)blockIdx.x & 7) * rpx + ((int)blockIdx.x >> 3));
    if (row >= rows) return;  // (whole workgroup)
    NOSA_TL(2, 0);
    NOSA_TL_ROLE(2, 0);
    const int c = threadIdx.x, lane = c & 63;
    const float2* ml = pml + row * nsplit;
    const float* op = po + row * nsplit * D + c;
    float M = -INFINITY, L = 0.f, acc = 0.f;
#pragma unroll 1
    for (int i0 = 0; i0 < nsplit; i0 += kMergeBatch) {
        // partial i0 + u of the batch: its (m, l) in lane u (and u + 32) of
        // each wave, its o value of channel c in o[u]; straight-line loads,
        // indexes past nsplit read the last partial again and are masked
        const int iu = i0 + (lane & (kMergeBatch - 1));
        float2 v = ml[iu < nsplit ? iu : nsplit - 1];
        float o[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) o[u] = op[(size_t)(i0 + u < nsplit ? i0 + u : nsplit - 1) * D];
        if (iu >= nsplit) v = make_float2(-INFINITY, 0.f);
        if (i0 == 0 && map && row % G == 0) {  // after the first loads are in flight
            const size_t pair = row / G;
            for (int x = c; x < cap; x += D) {
                map[pair * cap + x] = map_next[pair * cap + x];
                used[pair * cap + x] = used_next[pair * cap + x];
            }
        }
        const float Mb = fmaxf(M, wave_max_f(v.x));
        if (Mb == -INFINITY) continue;
        const float r = M == -INFINITY ? 0.f : fexp2(M - Mb);
        const float w = v.x == -INFINITY ? 0.f : fexp2(v.x - Mb);  // 0 for masked partials
        L = L * r + wave_sum_f(lane < kMergeBatch ? w * v.y : 0.f);
        acc *= r;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
            acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)) * o[u];
        M = Mb;
    }
    const bool empty = !(L > 0.f);
    out[row * D + c] = empty ? 0.f : acc / L;
    if (lse && c == 0) lse[row] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    NOSA_TL(2, 1);
}

static hipError_t launch_merge(const Plan& pl, const Workspace& w, int nsplit, float* out, float* lse,
                               hipStream_t stream, const Offload* off = nullptr)
{
    const int rows = pl.B * pl.Hq;
    if (rows > 0)
        hipLaunchKernelGGL(merge_kernel, dim3(8 * ceil_div(rows, 8)), dim3(D), 0, stream, w.po,
                           w.pml, nsplit, out, lse, off ? off->map_next : nullptr,
                           off ? off->used_next : nullptr, off ? off->cache_map : nullptr,
                           off ? off->cache_used : nullptr, off ? off->cap : 0, pl.G,
                           (size_t)rows);
    return hipGetLastError();
}

// Attention over given block lists: workgroup = kStep2Waves (4) waves; the
// entries are dealt round-robin to the pair's workgroups (wave w of
// workgroup grp takes entries (rr*4 + w)*groups + grp, rr < R), so every
// workgroup gets the same number of pages, give or take one; one 64-token
// block at a time, and the workgroup stores one partial per head at slot grp.
static_assert(kStep2Waves == 4, "store_wg_partial combines four waves");
template <int R, bool STREAM>
__global__ __launch_bounds__(kStep2Waves * 64) void attend_kernel(AttendArgs a)
{
    __shared__ CombineLds sh;
    // the placement counts and the index arrays in the first batch of
    // argument loads (an empty asm that takes them as scalar registers; the
    // arrays as global-memory pointers, so their loads stay global ones)
    int groups = a.groups, Hkv = a.Hkv, max_sel = a.max_sel, Lmax = a.Lmax, max_blocks = a.max_blocks;
    GlobalI1 cuk = (GlobalI1)a.cu_k, cnt = (GlobalI1)a.cnt, sel = (GlobalI1)a.sel,
             table = (GlobalI1)a.table;
    asm("" : "+s"(groups), "+s"(Hkv), "+s"(max_sel), "+s"(Lmax), "+s"(max_blocks), "+s"(cuk),
        "+s"(cnt), "+s"(sel), "+s"(table));
    const int pair = blockIdx.x / groups, grp = blockIdx.x % groups;
    const int s = pair / Hkv, g = pair % Hkv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    // The query and every round's list entry are requested with the length
    // and the count (indexes clamped into the row, checked once all are
    // in), then every round's table entry: two memory round trips before
    // the first page, whatever R.
    bf16x8 qb[4];
    load_q(a.q, a.Hq, s, g * a.G, a.G, r, kq, qb);
    GlobalI1 srow = sel + (size_t)pair * max_sel;
    int bl[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int idx = (rr * kStep2Waves + wave) * groups + grp;
        bl[rr] = max_sel > 0 ? srow[idx < max_sel ? idx : max_sel - 1] : -1;  // (no list: no read)
    }
    const int cu0 = cuk[s], cu1 = cuk[s + 1], npick = cnt[pair];  // one wait for the three
    const int L = seq_len_of(cu0, cu1, Lmax);
    const int nb = (L + BS - 1) / BS;
    GlobalI1 trow = table + (size_t)s * max_blocks;
    const int n = min(npick, max_sel);
    int pl[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int idx = (rr * kStep2Waves + wave) * groups + grp;
        if (idx >= n || bl[rr] < 0 || bl[rr] >= nb) bl[rr] = -1;  // no page this round
        pl[rr] = trow[bl[rr] >= 0 ? bl[rr] : 0];
    }
    AttnState A;
    attn_init(A);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int b = bl[rr], page = pl[rr];
        if (b < 0) continue;
        const uint16_t* kb = a.k_pool + ((size_t)page * a.Hkv + g) * BS * D;
        const uint16_t* vb = a.v_pool + ((size_t)page * a.Hkv + g) * D * BS;
        attend_page(kb, vb, L - b * BS, qb, a.scale_log2, r, kq, A, STREAM);
    }
    store_wg_partial(sh, A, a.G, (size_t)s * a.Hq + g * a.G, groups, grp, a.po, a.pml);
}

// ------------------------------------------------------ select (alone) ---

// Selection from given importance: one workgroup per row of the importance
// (sequence, or sequence x q-block, times KV head).  For a decode row the
// blocks are those of the L tokens; for q-block r of a chunk of Lq queries
// they end at the block of the q-block's last query, L - Lq + min(64r + 64, Lq) - 1.
constexpr int kSelThreads = 512;  // eight waves: a row of up to 4096 blocks in registers

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores_in,
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
    // the scores in batches of kSelKeyRounds per thread, every load of a
    // batch in flight before the first is used; the first batch's order keys
    // go to the selector in registers, every score to LDS
    const float* row = scores_in + pair * max_nb;
    uint32_t keys[kSelKeyRounds];
    for (int b0 = 0; b0 < nb; b0 += kSelKeyRounds * kSelThreads) {
        float v[kSelKeyRounds];
#pragma unroll
        for (int i = 0; i < kSelKeyRounds; ++i) {
            const int b = b0 + i * kSelThreads + (int)threadIdx.x;
            v[i] = b < nb ? row[b] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kSelKeyRounds; ++i) {
            const int b = b0 + i * kSelThreads + (int)threadIdx.x;
            if (b < nb) sI[b] = v[i];
            if (b0 == 0) keys[i] = order_key(v[i]);
        }
    }
    if (nb <= 0) {
#pragma unroll
        for (int i = 0; i < kSelKeyRounds; ++i) keys[i] = 0u;
    }
    select_lds_clear<kSelThreads>(sh);
    __syncthreads();
    select_blocks_wg<kSelThreads / 64, true>(keys, sI, nb, wblocks, topk, sh, sel + pair * max_sel, cnt + pair,
                              max_sel, nullptr, 0, 0, nullptr);
}

// ---------------------------------------------------------- launchers ---

// Device-side input checks (nosa_check_inputs).  check_clear_kernel zeroes
// the flags (a kernel, not a memset, so that a captured graph replays it
// like the rest); then workgroup s of check_inputs_kernel tests sequence s:
// its cu_seqlens entries and length (every thread, the same loads), and the
// block-table entries of the blocks its clamped length holds (a thread per
// entry), and ORs the bits found into *flags.  The table row is read only up
// to nb(min(L_s, Lmax)) <= max_blocks entries.
__global__ void check_clear_kernel(int32_t* flags) { *flags = 0; }

__global__ __launch_bounds__(256) void check_inputs_kernel(const int32_t* __restrict__ cu_k,
                                                           const int32_t* __restrict__ cu_q,
                                                           const int32_t* __restrict__ table,
                                                           int max_blocks, int num_pages, int Lmax,
                                                           int Lqmax, int32_t* __restrict__ flags)
{
    const int s = blockIdx.x;
    int f = 0;
    const int k0 = cu_k[s], k1 = cu_k[s + 1];
    if ((s == 0 && k0 != 0) || k1 < k0) f |= NOSA_CHECK_CU_K;
    const long long Ls = (long long)k1 - k0;
    if (Ls < 1 || Ls > Lmax) f |= NOSA_CHECK_LEN_K;
    const int L = Ls < 0 ? 0 : (Ls > Lmax ? Lmax : (int)Ls);
    if (cu_q) {
        const int q0 = cu_q[s], q1 = cu_q[s + 1];
        const long long Lq = (long long)q1 - q0;
        if ((s == 0 && q0 != 0) || Lq < 0 || Lq > Lqmax || Lq > L) f |= NOSA_CHECK_CU_Q;
    }
    const int nb = (L + BS - 1) / BS;
    const int32_t* row = table + (size_t)s * max_blocks;
    for (int b = threadIdx.x; b < nb; b += blockDim.x) {
        const int pg = row[b];
        if (pg < 0 || pg >= num_pages) f |= NOSA_CHECK_TABLE;
    }
    if (f) atomicOr(flags, f);
}

hipError_t launch_check_inputs(const int32_t* cu_k, const int32_t* cu_q, const int32_t* table,
                               int max_blocks, int num_pages, int Lmax, int Lqmax, int batch,
                               int32_t* flags, hipStream_t stream)
{
    hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, stream, flags);
    if (batch > 0)
        hipLaunchKernelGGL(check_inputs_kernel, dim3(batch), dim3(256), 0, stream, cu_k, cu_q, table,
                           max_blocks, num_pages, Lmax, Lqmax, flags);
    return hipGetLastError();
}

// Per-device attribute caches: an attribute is read once per device and kept
// in an atomic slot (0 = not read yet), so concurrent first calls on several
// threads at worst read it twice and store the same value.
constexpr int kMaxDevices = 64;

static int device_attribute(std::atomic<int>* slots, hipDeviceAttribute_t attr, int fallback)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
    int v = slots[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
    slots[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Largest LDS a workgroup may use on the current device.
static size_t device_lds_limit()
{
    static std::atomic<int> cached[kMaxDevices];
    return (size_t)device_attribute(cached, hipDeviceAttributeMaxSharedMemoryPerBlock, 64 * 1024);
}

// Compute units of the current device.
static int device_cus()
{
    static std::atomic<int> cached[kMaxDevices];
    return device_attribute(cached, hipDeviceAttributeMultiprocessorCount, 256);
}

// Scratch of nosa_decode_step_static: the decode step's partials for callers
// that cannot allocate.  Every device the library runs on holds its own copy
// from module load until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, read once per device with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr)
{
    static std::atomic<void*> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

// A step's pooled keys and its K and V pages are mostly read again at the
// next step.  Where a step reads more of either than an eighth of the 256 MB
// Infinity Cache (so that a model's layers could not keep theirs there), the
// loads are streamed (non-temporal) and leave the caches to what is reused;
// below that they are ordinary loads, which the next step may find cached.
constexpr long long kStreamBytes = 32LL << 20;
static int stream_keys(const Plan& pl)
{
    return (long long)pl.B * pl.Hkv * pl.max_nc * D * 2 > kStreamBytes ? 1 : 0;
}
static int stream_pages(const Plan& pl)
{
    const int pages = pl.max_sel < pl.max_nb ? pl.max_sel : pl.max_nb;
    return (long long)pl.B * pl.Hkv * pages * BS * D * 2 * 2 > kStreamBytes ? 1 : 0;
}

// wgroups > 0: also the window workgroups, wgroups per pair (pl.wslots: a
// page each; fewer: a page per wave, score_tiles = 8 only), their partials
// at slots top_groups .. of nsplit.
static hipError_t launch_score(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                               const int32_t* cu_k, const Workspace& w, int append, int wgroups,
                               int nsplit, hipStream_t stream, const Offload* off = nullptr)
{
    ScoreArgs a{};
    a.q = q;
    a.k_pool = off ? off->k_recent : kv.k_pool;
    a.v_pool = off ? off->v_recent : kv.v_pool;
    a.ring = off ? off->recent : 0;
    a.kc_pool = kv.kc_pool;
    a.table = kv.block_table;
    a.cu_k = cu_k;
    a.max_blocks = kv.max_blocks_per_seq;
    a.num_pages = kv.num_pages;
    a.Lmax = pl.Lmax;
    a.Hq = pl.Hq;
    a.Hkv = pl.Hkv;
    a.G = pl.G;
    a.gp = pl.gp;
    a.scale_log2 = pl.scale_log2;
    a.append = append;
    a.stream_kc = stream_keys(pl);
    a.nchunks = pl.nchunks;
    a.nbk = pl.nbk;
    a.cml = w.cml;
    a.spill = w.spill;
    a.bpart = w.bpart;
    // two chunks per workgroup (8 tiles only) when the chunks would
    // otherwise take more than one dispatch round of two workgroups per CU
    const long long pairs = (long long)pl.B * pl.Hkv;
    const int cpw = pl.score_tiles == 8 && pairs * pl.nchunks > 2LL * device_cus() ? 2 : 1;
    a.nscore = (int)(pairs * ceil_div(pl.nchunks, cpw));
    a.wslots = wgroups > 0 ? pl.wslots : 0;
    a.wgroups = wgroups > 0 ? wgroups : 1;
    a.wblocks = pl.wblocks;
    a.split0 = pl.top_groups;
    a.nsplit = nsplit;
    a.po = w.po;
    a.pml = w.pml;
    const bool per_wave = wgroups > 0 && wgroups != pl.wslots;
    if (per_wave && pl.score_tiles != 8) return hipErrorInvalidValue;
    const dim3 grid(8 * ceil_div(a.nscore, 8) + pl.B * pl.Hkv * (wgroups > 0 ? wgroups : 0)),
        block(kScoreWaves * 64);
    const size_t lds = score_lds_bytes(pl.score_tiles, pl.G, per_wave);  // <= 16 x 516 floats
    switch (pl.score_tiles) {
        case 1: hipLaunchKernelGGL((score_kernel<1, 1>), grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL((score_kernel<2, 1>), grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL((score_kernel<4, 1>), grid, block, lds, stream, a); break;
        default:
            if (cpw == 2) hipLaunchKernelGGL((score_kernel<8, 2>), grid, block, lds, stream, a);
            else hipLaunchKernelGGL((score_kernel<8, 1>), grid, block, lds, stream, a);
            break;
    }
    return hipGetLastError();
}

static TopArgs top_args(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                        const int32_t* cu_k, const Workspace& w)
{
    TopArgs a{};
    a.stream = stream_pages(pl);
    a.q = q;
    a.k_pool = kv.k_pool;
    a.v_pool = kv.v_pool;
    a.wk = kv.k_pool;
    a.wv = kv.v_pool;
    a.num_pages = kv.num_pages;
    a.table = kv.block_table;
    a.cu_k = cu_k;
    a.max_blocks = kv.max_blocks_per_seq;
    a.Lmax = pl.Lmax;
    a.Hq = pl.Hq;
    a.Hkv = pl.Hkv;
    a.G = pl.G;
    a.gp = pl.gp;
    a.scale_log2 = pl.scale_log2;
    a.chunk_keys = pl.chunk_keys;
    a.cb_shift = 31 - __builtin_clz((unsigned)(pl.chunk_keys / 4));
    a.nchunks = pl.nchunks;
    a.nbk = pl.nbk;
    a.cml = w.cml;
    a.spill = w.spill;
    a.bpart = w.bpart;
    a.topk = pl.topk;
    a.wblocks = pl.wblocks;
    a.max_nb = pl.max_nb;
    a.max_sel = pl.max_sel;
    a.po = w.po;
    a.pml = w.pml;
    return a;
}

template <int KRB, int GP4, bool OFF, bool STREAM>
static void launch_top_t(dim3 grid, size_t lds, const TopArgs& a, hipStream_t stream)
{
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&top_kernel<KRB, GP4, OFF, STREAM>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((top_kernel<KRB, GP4, OFF, STREAM>), grid, dim3(kStep2Waves * 64), lds, stream, a);
}

// Offloaded KV: always streamed (its picks come from host memory).
template <int KRB, int GP4>
static void launch_top_s(dim3 grid, size_t lds, const TopArgs& a, hipStream_t stream)
{
    if (a.cap > 0) launch_top_t<KRB, GP4, true, true>(grid, lds, a, stream);
    else if (a.stream) launch_top_t<KRB, GP4, false, true>(grid, lds, a, stream);
    else launch_top_t<KRB, GP4, false, false>(grid, lds, a, stream);
}

template <int KRB>
static void launch_top_k(dim3 grid, size_t lds, int gp4, const TopArgs& a, hipStream_t stream)
{
    switch (gp4) {
        case 1: launch_top_s<KRB, 1>(grid, lds, a, stream); break;
        case 2: launch_top_s<KRB, 2>(grid, lds, a, stream); break;
        default: launch_top_s<KRB, 4>(grid, lds, a, stream); break;
    }
}

// Grid: eight XCDs x (tpx top + wpx window workgroups); see top_kernel.
static hipError_t launch_top(const Plan& pl, TopArgs a, hipStream_t stream)
{
    const int nr = ceil_div(pl.max_nb, kStep2Waves * 64);
    const int krb = nr <= 1 ? 1 : nr <= 2 ? 2 : nr <= 4 ? 4 : 8;
    const size_t lds = top_lds_bytes(pl.max_nb, krb);
    if (lds + sizeof(TopLds) > device_lds_limit()) return hipErrorInvalidValue;
    const int ntop = pl.B * pl.Hkv * a.groups, nwin = pl.B * pl.Hkv * a.wgroups;
    a.disp = make_int4(ceil_div(ntop, 8), ceil_div(nwin, 8), ntop, nwin);
    const dim3 grid(8 * (a.disp.x + a.disp.y));
    const int gp4 = pl.gp / 4;
    switch (krb) {
        case 1: launch_top_k<1>(grid, lds, gp4, a, stream); break;
        case 2: launch_top_k<2>(grid, lds, gp4, a, stream); break;
        case 4: launch_top_k<4>(grid, lds, gp4, a, stream); break;
        default: launch_top_k<8>(grid, lds, gp4, a, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_scores_only(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                              const int32_t* cu_k, const Workspace& w, float* scores_out,
                              hipStream_t stream)
{
    hipError_t e = launch_score(pl, kv, q, cu_k, w, 0, 0, pl.nsplit, stream);
    if (e != hipSuccess) return e;
    TopArgs a = top_args(pl, kv, q, cu_k, w);
    a.groups = 1;
    a.rounds = 1;
    a.scores_only = 1;
    a.scores_out = scores_out;
    return launch_top(pl, a, stream);
}

hipError_t launch_decode(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const Workspace& w, float* out, float* lse,
                         int32_t* sel_out, int32_t* cnt_out, float* scores_out,
                         hipStream_t stream, const Offload* off)
{
    // The window pages (known before any selection) go beside the selection
    // when the attention launch then fits on the chip at once (two
    // workgroups per CU): a page per workgroup if that fits, else a page per
    // wave, if need be with up to four top-k pages per wave instead of fewer
    // (fewer top workgroups: the window pages then stream while the
    // selection runs, when HBM is otherwise idle); otherwise beside the
    // scoring, a page per workgroup.
    const long long pairs = (long long)pl.B * pl.Hkv, room = 2LL * device_cus();
    const int per_wave = ceil_div(pl.wslots, 4);
    int groups = pl.top_groups, rounds = pl.top_rounds, wg_top = 0;
    if (pairs * (groups + pl.wslots) <= room) {
        wg_top = pl.wslots;
    } else if (pairs * (groups + per_wave) <= room) {
        wg_top = per_wave;
    } else {
        for (int r = rounds + 1; r <= 4 && wg_top == 0; ++r) {
            const int gr = ceil_div(pl.top_span > 0 ? pl.top_span : 1, kStep2Waves * r);
            if (pairs * (gr + per_wave) <= room) {
                groups = gr;
                rounds = r;
                wg_top = per_wave;
            }
        }
    }
    // Beside the scoring, the 8-tile scoring kernel (long contexts) takes
    // the window a page per wave: four times the bytes in flight per
    // workgroup slot of a launch whose slots its registers limit to two per
    // CU; the others a page per workgroup.
    const int wg_score = wg_top > 0 || pl.wslots == 0 ? 0 : (pl.score_tiles == 8 ? per_wave : pl.wslots);
    // partials per head: the top workgroups', then one per window workgroup
    // (at most top_groups + wslots, the workspace's)
    const int nsplit = groups + (wg_top > 0 ? wg_top : (wg_score > 0 ? wg_score : pl.wslots));
    hipError_t e = launch_score(pl, kv, q, cu_k, w, 1, wg_score, nsplit, stream, off);
    if (e != hipSuccess) return e;
    TopArgs a = top_args(pl, kv, q, cu_k, w);
    if (off) {
        a.k_pool = off->k_host;
        a.v_pool = off->v_host;
        a.wk = off->k_recent;
        a.wv = off->v_recent;
        a.ring = off->recent;
        a.cache_k = off->cache_k;
        a.cache_v = off->cache_v;
        a.map = off->cache_map;
        a.used = off->cache_used;
        a.map_next = off->map_next;
        a.used_next = off->used_next;
        a.fetch_out = off->fetch_out;
        a.cap = off->cap;
    }
    a.groups = groups;
    a.rounds = rounds;
    a.wslots = wg_top > 0 ? pl.wslots : 0;
    a.wgroups = wg_top;
    a.nsplit = nsplit;
    a.scores_out = scores_out;
    a.sel_out = sel_out;
    a.cnt_out = cnt_out;
    e = launch_top(pl, a, stream);
    if (e != hipSuccess) return e;
    return launch_merge(pl, w, nsplit, out, lse, stream, off);
}

template <int R>
static void launch_attend_r(dim3 grid, dim3 block, const AttendArgs& b, hipStream_t stream)
{
    if (b.stream) hipLaunchKernelGGL((attend_kernel<R, true>), grid, block, 0, stream, b);
    else hipLaunchKernelGGL((attend_kernel<R, false>), grid, block, 0, stream, b);
}

hipError_t launch_attend(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const int32_t* sel, const int32_t* cnt,
                         const Workspace& w, float* out, float* lse, hipStream_t stream)
{
    AttendArgs b{};
    b.stream = stream_pages(pl);
    b.q = q;
    b.k_pool = kv.k_pool;
    b.v_pool = kv.v_pool;
    b.table = kv.block_table;
    b.cu_k = cu_k;
    b.max_blocks = kv.max_blocks_per_seq;
    b.Lmax = pl.Lmax;
    b.Hq = pl.Hq;
    b.Hkv = pl.Hkv;
    b.G = pl.G;
    b.scale_log2 = pl.scale_log2;
    b.groups = pl.attend_groups;
    b.sel = sel;
    b.cnt = cnt;
    b.max_sel = pl.max_sel;
    b.po = w.po;
    b.pml = w.pml;
    const dim3 grid(pl.B * pl.Hkv * pl.attend_groups), block(kStep2Waves * 64);
    switch (pl.attend_rounds) {
        case 1: launch_attend_r<1>(grid, block, b, stream); break;
        case 2: launch_attend_r<2>(grid, block, b, stream); break;
        case 3: launch_attend_r<3>(grid, block, b, stream); break;
        case 4: launch_attend_r<4>(grid, block, b, stream); break;
        case 6: launch_attend_r<6>(grid, block, b, stream); break;
        default: launch_attend_r<8>(grid, block, b, stream); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(pl, w, pl.attend_groups, out, lse, stream);
}

hipError_t launch_select(const Plan& pl, const int32_t* cu_k, const int32_t* cu_q, int max_seqlen_q,
                         const float* scores_in, int32_t* sel, int32_t* cnt, hipStream_t stream)
{
    const size_t lds = sizeof(float) * (size_t)(pl.max_nb > 0 ? pl.max_nb : 1);
    const int max_qblk = cu_q ? ceil_div(max_seqlen_q, 64) : 1;
    hipLaunchKernelGGL(select_kernel, dim3(pl.Hkv, pl.B * max_qblk), dim3(kSelThreads), lds, stream,
                       scores_in, sel, cnt, cu_k, cu_q, max_seqlen_q, max_qblk, pl.Lmax, pl.Hkv,
                       pl.max_nb, pl.max_sel, pl.topk, pl.wblocks);
    return hipGetLastError();
}

}  // namespace nosa

#ifdef NOSA_TIMELINE
// Readout of the timeline build's stamps (not part of the NOSA C ABI).
extern "C" {

// Copies launch `launch`'s stamps ([8192][16] unsigned 64-bit) to host memory.
int nosa_timeline_read(int launch, unsigned long long* host)
{
    if (launch < 0 || launch > 2 || !host) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(nosa::tl_stamps), sizeof(nosa::tl_stamps[0]),
                                    (size_t)launch * sizeof(nosa::tl_stamps[0]), hipMemcpyDeviceToHost);
}

// Zeroes every stamp (synchronous).
int nosa_timeline_clear(void)
{
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(nosa::tl_stamps));
    if (e != hipSuccess) return (int)e;
    e = hipMemset(p, 0, sizeof(nosa::tl_stamps));
    if (e != hipSuccess) return (int)e;
    return (int)hipDeviceSynchronize();
}

// The wall clock's rate in kHz, or 0 on an error.
int nosa_timeline_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
#endif
