// nosa_device.h -- device code shared by the decode kernels (nosa_kernels.hip)
// and the chunked-prefill kernels (nosa_prefill.hip): bf16 and MFMA helpers,
// page layouts, one-page attention on MFMA and the workgroup top-k selector.
// Internal; compiled into libnosa.so only.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Operand layout (wave64, lane l,
// r = l % 16, kq = l / 16): A supplies A[r][8kq .. 8kq+7], B supplies
// B[8kq .. 8kq+7][r], the accumulator holds D[4kq + i][r] for i = 0..3.  The
// contraction index may be permuted freely as long as A and B agree; the
// kernels map k-step st, lane group kq to channels 32st + 8kq .. +7 so that
// four lane groups read 64 contiguous bytes of a row.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "nosa_internal.h"

namespace nosa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int BS = kBlock;
constexpr int SL = kSlots;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int dev_num_keys(int L) { return L >= kPoolK ? (L - kPoolK) / kPoolS + 1 : 0; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x with the hardware instruction (results below 2^-126 flush to zero,
// which no softmax weight or sum here is sensitive to).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// The same load with the non-temporal hint, for data streamed once per use
// whose volume across a model's layers is far beyond the caches (the K and V
// pages of a large decode step, every K page of a pooled-key build): the
// stream then leaves the L2 and the Infinity Cache to what is reused or
// written -- the partials, pooled keys and tables of the step, the pooled
// keys a build writes.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const void* p)
{
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------- page layouts ---
// Every page of every pool is stored in the order the MFMA operands are
// loaded, so that one 16-byte-per-lane load instruction of a wave reads 1 KB
// of contiguous memory (lane l at byte 16 l) instead of sixteen 64-byte
// pieces of sixteen rows.  Offsets below are in bf16 elements from the start
// of the page of one KV head and address 8 consecutive elements.

// K page (64 tokens x 128 channels): 16 blocks of 1 KB; block 4t + st is the
// A operand of QK^T tile t, k-step st: lane 16 kq + m holds channels
// 32 st + 8 kq .. +7 of token qk_row_token(t, m).  Offset of channels
// 8 c8 .. 8 c8 + 7 of token x:
__device__ __forceinline__ int k_chunk(int x, int c8)
{
    const int t = 2 * (x >> 5) + ((x >> 2) & 1), m = 4 * ((x >> 3) & 3) + (x & 3);
    return (((t * 4 + (c8 >> 2)) * 4 + (c8 & 3)) * 16 + m) * 8;
}

// V page (64 tokens x 128 channels): 16 blocks of 1 KB; block 8u + nt is the
// B operand of PV k-step u (tokens 32u .. 32u + 31), channel tile nt: lane
// 16 kq + r holds tokens 32u + 8kq .. +7 of channel 16 nt + r.  Offset of
// tokens 8 x8 .. 8 x8 + 7 of channel c:
__device__ __forceinline__ int v_chunk(int c, int x8)
{
    return ((((x8 >> 2) * 8 + (c >> 4)) * 4 + (x8 & 3)) * 16 + (c & 15)) * 8;
}

// Pooled-key page (4 keys x 128 channels, 1 KB): channel chunk major,
// [16 chunks][4 slots][8].  Offset of channels 8 c8 .. 8 c8 + 7 of slot j:
__device__ __forceinline__ int kc_chunk(int slot, int c8) { return (c8 * SL + slot) * 8; }

// Start of the pooled-key page holding key j of KV head g of a sequence.
__device__ __forceinline__ uint16_t* kc_page(uint16_t* kc_pool, const int32_t* trow, int Hkv, int g,
                                             int j)
{
    return kc_pool + ((size_t)trow[j / SL] * Hkv + g) * SL * D;
}

// Length of sequence s clamped to [0, Lmax], Lmax = min(host bound, what a
// block-table row addresses): a device length above the host-side bound can
// then never index past the table, the workspace rows or the LDS arrays.
__device__ __forceinline__ int seq_len_of(int cu0, int cu1, int Lmax)
{
    int L = cu1 - cu0;
    L = L < 0 ? 0 : L;
    return L < Lmax ? L : Lmax;
}

__device__ __forceinline__ int seq_len(const int32_t* cu_k, int s, int Lmax)
{
    return seq_len_of(cu_k[s], cu_k[s + 1], Lmax);
}

// ------------------------------------------------------ block attention ---

// Row order of the K tile inside the QK^T MFMA.  Tile t = 2u + v, row
// m = 4c + i holds token 32u + 8c + 4v + i.  With this order the
// accumulator of lane (r, kq) ends up holding, for head r, the tokens
// 32u + 8kq + 0..7 across tiles 2u and 2u+1: exactly the A operand of the
// PV MFMA over the 32 tokens of k-step u.
__device__ __forceinline__ int qk_row_token(int t, int m)
{
    return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

// Query operand of one KV head's group: B[channel][head r] (heads >= G zero).
__device__ __forceinline__ void load_q(const uint16_t* q, int Hq, int s, int h0, int G, int r,
                                       int kq, bf16x8 (&qb)[4])
{
    const uint16_t* qh = q + ((size_t)s * Hq + h0 + (r < G ? r : 0)) * D;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        uint4 w = ldg16(qh + st * 32 + kq * 8);
        if (r >= G) w = make_uint4(0, 0, 0, 0);
        qb[st] = as_bf16x8(w);
    }
}

struct AttnState {
    float m, l;
    f32x4 o[8];
};

__device__ __forceinline__ void attn_init(AttnState& A)
{
    A.m = -INFINITY;
    A.l = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) A.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One wave attends one 64-token page: S^T = K q^T (4 tiles x 4 k-steps), fp32
// online softmax in log2 units, O += P V (2 k-steps x 8 channel tiles).
// `limit` = tokens of the page that exist (tokens >= limit are masked).
// The MFMA operands of one page (32 loads of 16 bytes per lane).
struct PageRegs {
    uint4 k[4][4], v[2][8];
};

// Issues every load of a page: operand blocks in lane order (k_chunk /
// v_chunk), 1 KB per load, streamed (non-temporal) when `stream` (uniform).
// `lane8` is the lane's element offset in a block, (16 kq + r) * 8 (0 makes
// every lane read the block's first 16 bytes).
__device__ __forceinline__ void load_page(const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int lane8, PageRegs& p,
                                          bool stream)
{
    if (stream) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st) p.k[t][st] = ldg16_stream(kb + (t * 4 + st) * 512 + lane8);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) p.v[u][nt] = ldg16_stream(vb + (u * 8 + nt) * 512 + lane8);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st) p.k[t][st] = ldg16(kb + (t * 4 + st) * 512 + lane8);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) p.v[u][nt] = ldg16(vb + (u * 8 + nt) * 512 + lane8);
    }
}

// The page held in p back to memory at kb / vb, in the same order (a copy of
// a page into another pool).
__device__ __forceinline__ void store_page(uint16_t* __restrict__ kb, uint16_t* __restrict__ vb,
                                           int lane8, const PageRegs& p)
{
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int st = 0; st < 4; ++st)
            *reinterpret_cast<uint4*>(kb + (t * 4 + st) * 512 + lane8) = p.k[t][st];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *reinterpret_cast<uint4*>(vb + (u * 8 + nt) * 512 + lane8) = p.v[u][nt];
}

__device__ __forceinline__ void attend_loaded(const PageRegs& p, int limit, const bf16x8 (&qb)[4],
                                              float scale_log2, int r, int kq, AttnState& A);

__device__ __forceinline__ void attend_page(const uint16_t* __restrict__ kb,
                                            const uint16_t* __restrict__ vb, int limit,
                                            const bf16x8 (&qb)[4], float scale_log2, int r,
                                            int kq, AttnState& A, bool stream)
{
    PageRegs p;
    load_page(kb, vb, (16 * kq + r) * 8, p, stream);
    // Keep every load of the page in flight before the first use: a wave that
    // attends one page pays one memory latency instead of one per few loads.
    __builtin_amdgcn_sched_barrier(0);
    attend_loaded(p, limit, qb, scale_log2, r, kq, A);
}

// Online-softmax update of A with one page whose operands are in p.
__device__ __forceinline__ void attend_loaded(const PageRegs& p, int limit, const bf16x8 (&qb)[4],
                                              float scale_log2, int r, int kq, AttnState& A)
{
    const auto& ka = p.k;
    const auto& va = p.v;
    float x[4][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(ka[t][st]), qb[st], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 32 * (t >> 1) + 8 * kq + 4 * (t & 1) + i;
            x[t][i] = tok < limit ? acc[i] * scale_log2 : -INFINITY;
            bmax = fmaxf(bmax, x[t][i]);
        }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(A.m, bmax);
    const float alpha = fexp2(A.m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[t][i] = fexp2(x[t][i] - m_new);
            psum += x[t][i];
        }
    A.l = A.l * alpha + psum;
    A.m = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * kq + i);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) A.o[nt][i] *= ai;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        bf16x8 pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pa[i] = (__bf16)x[2 * u][i];
            pa[4 + i] = (__bf16)x[2 * u + 1][i];
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) A.o[nt] = mfma16(pa, as_bf16x8(va[u][nt]), A.o[nt]);
    }
}

// ------------------------------------------------------------ selection ---

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x);

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of lanes of this wave below the calling lane whose bit is set.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

constexpr int kSelMaxRounds = kMaxBlocks / 256;  // candidate rounds of a 4-wave selector
constexpr int kSelKeyRounds = 8;                  // candidate rounds whose keys stay in registers

struct alignas(16) SelectLds {
    float lse[kMaxGroup];
    int hist0[1024];                  // digit counts, first level (10-bit digits)
    int hist[3][256];                 // digit counts, later levels (zero before the selector runs)
    int cnt[2][kSelMaxRounds][8];     // per (round, wave): tied candidates, taken candidates
    uint32_t mm[2][8];                // per wave: smallest, largest candidate key
};

// Zeroes the digit counts; all NT threads, and a barrier before the selector.
template <int NT>
__device__ __forceinline__ void select_lds_clear(SelectLds& sh)
{
    int4* h0 = reinterpret_cast<int4*>(sh.hist0);
    for (int i = threadIdx.x; i < 256; i += NT) h0[i] = make_int4(0, 0, 0, 0);
    int* h = &sh.hist[0][0];
    for (int i = threadIdx.x; i < 3 * 256; i += NT) h[i] = 0;
}

// Smallest and largest order key of this thread's candidates (i*NT + tid <
// ncand, i < KR, keys in registers) reduced over the wave and stored for
// wave `wave` in sh.mm; the selector reads them after the caller's next
// barrier (range_known).
template <int NT, int KR>
__device__ __forceinline__ void select_wave_range(const uint32_t (&keys)[KR], int ncand, SelectLds& sh)
{
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < KR; ++i)
        if (i * NT + (int)threadIdx.x < ncand) {
            lo = min(lo, keys[i]);
            hi = max(hi, keys[i]);
        }
    lo = ~wave_max_u32(~lo);
    hi = wave_max_u32(hi);
    if ((threadIdx.x & 63) == 0) {
        sh.mm[0][threadIdx.x >> 6] = lo;
        sh.mm[1][threadIdx.x >> 6] = hi;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 within each row of 16 lanes, then the last lane of row 0 is
// added to rows 1 and 3 and the last lane of row 1 to rows 2 and 3.  A lane
// that a move does not write receives 0.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xe, true);   // row_shr:4, lanes 4..15
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xc, true);   // row_shr:8, lanes 8..15
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Wave-wide reductions with DPP moves (the pattern of wave_incl_scan; a
// lane that a move does not reach keeps the identity), read from lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    int v = (int)x;
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, true));
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, true));
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
    v = max((unsigned)v, (unsigned)__builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max_f(float x)
{
    constexpr int kNegInf = (int)0xff800000u;
    int v = __float_as_int(x);
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x111, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x112, 0xf, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x114, 0xf, 0xe, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x118, 0xf, 0xc, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x142, 0xa, 0xf, false))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, v, 0x143, 0xc, 0xf, false))));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ float wave_sum_f(float x)
{
    int v = __float_as_int(x);
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// Top-min(topk, ncand) of the candidates [0, ncand) by (importance desc, block
// asc) with the window [ncand, nb) always kept.  Writes, when non-null:
//   sel_out[0 .. max_sel): every kept block ascending, -1 padded; *cnt_out;
//   list[0 .. list_n): (block, pages[block]) of top-k picks list_lo ..
//                      list_lo + list_n - 1 in ascending block order,
//                      (-1, -1) past the last pick (list may be in LDS).
// Must be called by all NW*64 threads, the digit counts zeroed and a barrier
// passed since; sI holds the importance in LDS (read only for candidates past
// the register rounds when KEYS_GIVEN); `pages` is the block-table row (LDS
// or global).  With KEYS_GIVEN the caller passes the order keys of its
// candidates i*NT + tid, i < KR, in keys[] (those rounds are then not read
// from sI).  With range_known every candidate is in registers and the caller
// stored each wave's key range with select_wave_range before its last
// barrier.  No barrier at the end: the caller synchronises before reading
// what was written to LDS.
//
// The k-th largest order key is found by a radix search over u = key - kmin,
// kmin and kmax being the smallest and largest candidate key: the first
// digit is the top 10 bits of the range kmax - kmin (so the candidates spread
// over its 1024 values however narrow their range), each later digit the
// next 8 bits below.  A level is one LDS histogram of the digit over the
// candidates that share the prefix found so far, one barrier, and a scan of
// the 256 counts by every wave; the search stops as soon as the candidates
// sharing the prefix are exactly the ones still needed, which for distinct
// keys usually happens at the first level.  The taken candidates are then
// compacted in ascending order from per-wave ballot counts (one barrier, two
// when tied keys straddle the cut).
// Mark, called with 0 .. 3 as the selector passes its stages (the range
// known, the first digit found, the last digit found, the compaction's
// counts shared), and with 7 when a digit level after the first runs: a
// hook for instrumented builds, a no-op by default.
struct NoMark {
    __device__ void operator()(int) const {}
};

template <int NW, bool KEYS_GIVEN, class Mark = NoMark>
__device__ __forceinline__ void select_blocks_wg(uint32_t (&keys)[kSelKeyRounds], const float* sI, int nb,
                                                 int wblocks, int topk, SelectLds& sh,
                                                 int32_t* __restrict__ sel_out, int32_t* __restrict__ cnt_out,
                                                 int max_sel, int2* list, int list_lo, int list_n,
                                                 const int32_t* pages, bool range_known = false,
                                                 Mark mark = Mark())
{
    static_assert(NW >= 4 && NW <= 8, "per-round counts are sized for 4 to 8 waves");
    constexpr int NT = NW * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ncand = nb > wblocks ? nb - wblocks : 0;
    const int kk = topk < ncand ? topk : ncand;
    const bool partial = kk > 0 && kk < ncand;
    const int rounds = (ncand + NT - 1) / NT;  // <= kMaxBlocks / 256 = kSelMaxRounds
    // candidate keys of this thread (candidate round*NT + tid), first KR rounds
    constexpr int KR = kSelKeyRounds;
    if (!KEYS_GIVEN) {
        // all KR reads issued together; indexes clamped into [0, ncand) (sI
        // has at least one entry), lanes past ncand are masked wherever keys
        // are used
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int b = i * NT + tid;
            keys[i] = order_key(sI[b < ncand ? b : (ncand > 0 ? ncand - 1 : 0)]);
        }
    }
    // f(i, key) for every candidate round i < rounds: the register rounds
    // unrolled (constant indexes into keys[]), later ones read from sI
    auto for_rounds = [&](auto&& f) {
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            if (i >= rounds) return;
            f(i, keys[i]);
        }
        for (int i = KR; i < rounds; ++i) {
            const int b = i * NT + tid;
            f(i, b < ncand ? order_key(sI[b]) : 0u);
        }
    };
    // Candidates whose u >> shift is above P are taken; of those equal to P,
    // the `need` lowest blocks; there are n_eq of them.  shift = 32: every
    // candidate is equal (P = 0).
    int shift = 32, need = kk, n_eq = kk;
    uint32_t P = 0, kmin = 0;
    if (partial) {
        // range of the candidate keys
        if (!range_known) {
            uint32_t lo = 0xffffffffu, hi = 0u;
            for_rounds([&](int i, uint32_t key) {
                if (i * NT + tid < ncand) {
                    lo = min(lo, key);
                    hi = max(hi, key);
                }
            });
            lo = ~wave_max_u32(~lo);
            hi = wave_max_u32(hi);
            if (lane == 0) {
                sh.mm[0][wave] = lo;
                sh.mm[1][wave] = hi;
            }
            __syncthreads();
        }
        kmin = 0xffffffffu;
        uint32_t kmax = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            kmin = min(kmin, sh.mm[0][w]);
            kmax = max(kmax, sh.mm[1][w]);
        }
        const uint32_t range = kmax - kmin;
        mark(0);
        n_eq = ncand;
        need = kk;
        if (range != 0u) {
            const int bits = 32 - __builtin_clz(range);
            int sh_lo = bits > 10 ? bits - 10 : 0;
            int prev = 32, above = 0;
            // one level: histogram of (u >> sh_lo) & (nd - 1) over the
            // candidates sharing the prefix, then every wave finds the digit
            // holding the kk-th largest; lane l holds digits nd-1-DPL*l
            // downwards (DPL per lane), so the lane prefix sum counts from
            // the top digit down
            auto level_pass = [&](int* hist, auto dpl_tag) -> bool {
                constexpr int DPL = decltype(dpl_tag)::value;
                constexpr int ND = 64 * DPL;
                for_rounds([&](int i, uint32_t key) {
                    const int b = i * NT + tid;
                    const uint32_t u = key - kmin;
                    const bool match = b < ncand && (prev == 32 || (u >> prev) == P);
                    if (match) atomicAdd(&hist[(u >> sh_lo) & (ND - 1)], 1);
                });
                __syncthreads();
                int v[DPL], loc = 0;
#pragma unroll
                for (int j = 0; j < DPL; j += 4) {
                    const int4 c4 = *reinterpret_cast<const int4*>(&hist[ND - DPL * (lane + 1) + DPL - 4 - j]);
                    v[j] = c4.w;
                    v[j + 1] = c4.z;
                    v[j + 2] = c4.y;
                    v[j + 3] = c4.x;
                }
#pragma unroll
                for (int j = 0; j < DPL; ++j) loc += v[j];
                const int incl = wave_incl_scan(loc);
                // first lane whose digits reach kk candidates at or above them
                const uint64_t reach = __ballot(above + incl >= kk);
                const int l0 = (int)__builtin_ctzll(reach);  // exists: all candidates sharing P count
                // in lane l0, the first of its digits (from the top) that reaches kk
                int acc = above + incl - loc, dj = DPL - 1, before = 0, at = 0;
                bool found = false;
#pragma unroll
                for (int j = 0; j < DPL; ++j) {
                    if (!found && acc + v[j] >= kk) {
                        found = true;
                        dj = j;
                        before = acc;
                        at = v[j];
                    }
                    acc += v[j];
                }
                const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(ND - 1 - DPL * lane - dj, l0);
                above = __builtin_amdgcn_readlane(before, l0);
                n_eq = __builtin_amdgcn_readlane(at, l0);
                // the digit's bits below the prefix are the new ones
                const int nbits = prev - sh_lo;  // 1 .. 10
                P = prev == 32 ? digit : (P << nbits) | (digit & ((1u << nbits) - 1u));
                prev = sh_lo;
                shift = sh_lo;
                need = kk - above;
                return n_eq == need || sh_lo == 0;  // taken exactly, or u fully resolved
            };
            const bool done = level_pass(sh.hist0, std::integral_constant<int, 16>{});
            mark(1);
            if (!done) {
#pragma unroll 1
                for (int level = 0; level < 3; ++level) {
                    mark(7);
                    sh_lo = sh_lo > 8 ? sh_lo - 8 : 0;
                    if (level_pass(sh.hist[level], std::integral_constant<int, 4>{})) break;
                }
            }
            mark(2);
        }
    }
    // Ascending compaction: candidate i*NT + tid in round i; per (round,
    // wave) counts through LDS, one barrier per pass.
    const bool ranked = partial && n_eq > need;
    auto prefix = [&](uint32_t key) -> uint32_t {
        return shift < 32 ? (key - kmin) >> shift : 0u;
    };
    if (ranked) {
        for_rounds([&](int i, uint32_t key) {
            const int b = i * NT + tid;
            const bool eq = b < ncand && prefix(key) == P;
            const uint64_t m = __ballot(eq);
            if (lane == 0) sh.cnt[0][i][wave] = (int)__popcll(m);
        });
        __syncthreads();
    }
    uint32_t takebits = 0;
    {
        int eq_base = 0;
        for_rounds([&](int i, uint32_t key) {
            const int b = i * NT + tid;
            const bool valid = b < ncand;
            bool take;
            if (!partial) {
                take = valid && kk > 0;
            } else {
                const uint32_t kp = prefix(key);
                const bool gt = kp > P, eq = kp == P;
                if (ranked) {
                    const uint64_t m = __ballot(valid && eq);
                    int r = eq_base + lanes_below(m);
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        const int c = sh.cnt[0][i][w];
                        if (w < wave) r += c;
                        eq_base += c;
                    }
                    take = valid && (gt || (eq && r < need));
                } else {
                    take = valid && (gt || eq);
                }
            }
            const uint64_t mt = __ballot(take);
            if (lane == 0) sh.cnt[1][i][wave] = (int)__popcll(mt);
            if (take) takebits |= 1u << i;
        });
    }
    __syncthreads();
    mark(3);
    int sel_base = 0;
    for_rounds([&](int i, uint32_t) {
        const bool take = (takebits >> i) & 1u;
        const uint64_t mt = __ballot(take);
        int pos = sel_base + lanes_below(mt);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = sh.cnt[1][i][w];
            if (w < wave) pos += c;
            sel_base += c;
        }
        if (take) {
            const int b = i * NT + tid;
            if (sel_out) sel_out[pos] = b;
            if (list && pos >= list_lo && pos < list_lo + list_n)
                list[pos - list_lo] = make_int2(b, pages[b]);
        }
    });
    const int nsel = sel_base;
    const int total = nsel + (nb - ncand);
    if (sel_out) {
        for (int b = ncand + tid; b < nb; b += NT) sel_out[nsel + (b - ncand)] = b;
        for (int x = total + tid; x < max_sel; x += NT) sel_out[x] = -1;
    }
    if (list)
        for (int x = (nsel > list_lo ? nsel - list_lo : 0) + tid; x < list_n; x += NT)
            list[x] = make_int2(-1, -1);
    if (tid == 0 && cnt_out) *cnt_out = total;
}

}  // namespace nosa
