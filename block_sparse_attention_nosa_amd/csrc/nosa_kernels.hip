// nosa_kernels.hip -- CDNA4 (gfx950) kernels of the NOSA sparse decode step.
//
// Five kernels, launched in this order by a decode step:
//   kc_build  : pooled keys, key j = bf16(mean of K over tokens [16j, 16j+32))
//   scores    : z_h[j] = scale*log2(e) * q_h . Kc_j on MFMA (16 keys x 16 heads
//               per instruction group), per-wave max / sum(exp2) partials
//   select    : per (sequence, KV head) workgroup: per-head log-sum-exp, block
//               importance = mean over overlapping keys of sum_h exp2(z - lse),
//               radix top-k over the candidates, window forced, ascending ids
//   attend    : split-K flash decode over the kept 64-token blocks; QK^T and PV
//               on MFMA with the G query heads of a KV head as the N (resp. M)
//               dimension; fp32 online softmax; per-workgroup (m, l, o) partial
//   merge     : combine the partials into out / lse
//
// Sources: page "NOSA-1B 性能基准全解析" (sections 三.2 local window and TopK
// blocks, 三.3 two-stage attention with kernel 32 / stride 16 pooling, 三.4 the
// mean-pool kernel), page "NOSA-1B 模型家族全景" (core principle: compressed
// attention filters KV blocks, CIS score mean pooling), page "NOSA技术架构解析"
// (section 2.1: paged KV pool; section 5.1: importance scores kept in fp32).
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Operand layout (wave64, lane l,
// r = l % 16, kq = l / 16): A supplies A[r][8kq .. 8kq+7], B supplies
// B[8kq .. 8kq+7][r], the accumulator holds D[4kq + i][r] for i = 0..3.  The
// contraction index may be permuted freely as long as A and B agree; every
// kernel below maps k-step st, lane group kq to channels 32st + 8kq .. +7 so
// that four lane groups read 64 contiguous bytes of a row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nosa_internal.h"

namespace nosa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int BS = kBlock;
constexpr int SL = kSlots;

__device__ __forceinline__ int dev_num_keys(int L) { return L >= kPoolK ? (L - kPoolK) / kPoolS + 1 : 0; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Length of sequence s clamped to [0, Lmax], Lmax = min(host bound, what a
// block-table row addresses): a device length above the host-side bound can
// then never index past the table, the workspace rows or the LDS arrays.
__device__ __forceinline__ int seq_len(const int32_t* cu_k, int s, int Lmax)
{
    int L = cu_k[s + 1] - cu_k[s];
    L = L < 0 ? 0 : L;
    return L < Lmax ? L : Lmax;
}

// ------------------------------------------------------------ kc_build ---

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

// One workgroup = 16 keys x 16 channel chunks of 8.  Each thread sums the 32
// tokens of its key for its 8 channels in fp64 (exact for bf16 inputs), then
// scales by 1/32 (exact) and rounds once.  Keys [n_c(prev), n_c(L)) are
// written, prev = valid_len[s], or L - 1 when appending for the current
// token, or 0 for a full rebuild.
__global__ __launch_bounds__(256) void kc_build_kernel(
    const uint16_t* __restrict__ k_pool, uint16_t* __restrict__ kc_pool,
    const int32_t* __restrict__ table, int max_blocks, int Lmax, int Hkv,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ valid_len, int append_current)
{
    const int s = blockIdx.z, g = blockIdx.y;
    const int L = seq_len(cu_k, s, Lmax);
    int prev = valid_len ? valid_len[s] : (append_current ? L - 1 : 0);
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
            const int page = trow[t / BS];
            const uint4 w = ldg16(k_pool + (((size_t)page * Hkv + g) * BS + (t % BS)) * D + cc * 8);
            acc[0] += (double)bf16_lo(w.x); acc[1] += (double)bf16_hi(w.x);
            acc[2] += (double)bf16_lo(w.y); acc[3] += (double)bf16_hi(w.y);
            acc[4] += (double)bf16_lo(w.z); acc[5] += (double)bf16_hi(w.z);
            acc[6] += (double)bf16_lo(w.w); acc[7] += (double)bf16_hi(w.w);
        }
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = bf16_from_f64(acc[e] * (1.0 / kPoolK));
        uint4 packed;
        packed.x = o[0] | (o[1] << 16);
        packed.y = o[2] | (o[3] << 16);
        packed.z = o[4] | (o[5] << 16);
        packed.w = o[6] | (o[7] << 16);
        const int page = trow[j / SL];
        *reinterpret_cast<uint4*>(kc_pool + (((size_t)page * Hkv + g) * SL + (j % SL)) * D + cc * 8) = packed;
    }
}

hipError_t launch_kc_build(const Plan& pl, const nosa_paged_kv& kv, const int32_t* cu_k,
                           const int32_t* valid_len, bool append_current, int grid_x,
                           hipStream_t stream)
{
    dim3 grid(grid_x, pl.Hkv, pl.B);
    hipLaunchKernelGGL(kc_build_kernel, grid, dim3(256), 0, stream, kv.k_pool, kv.kc_pool,
                       kv.block_table, kv.max_blocks_per_seq, pl.Lmax, pl.Hkv, cu_k, valid_len,
                       append_current ? 1 : 0);
    return hipGetLastError();
}

// -------------------------------------------------------------- scores ---

// Workgroup = 4 waves; wave w of workgroup x scores keys
// [(4x + w) * 16T, (4x + w + 1) * 16T) of one (sequence, KV head) as T MFMA
// tiles: A = 16 pooled keys x 32 channels, B = 32 channels x 16 query heads
// (heads >= G are zero).  z is written in log2 units, per-wave (max, sum exp2)
// go to zpart.
template <int T>
__global__ __launch_bounds__(256) void scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc_pool,
    const int32_t* __restrict__ table, int max_blocks, int Lmax, const int32_t* __restrict__ cu_k,
    int Hq, int Hkv, int G, float scale_log2, float* __restrict__ z, int zstride,
    float2* __restrict__ zpart, int nchunk)
{
    const int s = blockIdx.z, g = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int L = seq_len(cu_k, s, Lmax);
    const int nc = dev_num_keys(L);
    const int chunk = blockIdx.x * 4 + wave;
    const int key0 = chunk * 16 * T;
    const int32_t* trow = table + (size_t)s * max_blocks;

    bf16x8 qb[4];
    {
        const uint16_t* qh = q + ((size_t)s * Hq + g * G + (r < G ? r : 0)) * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 w = ldg16(qh + st * 32 + kq * 8);
            if (r >= G) w = make_uint4(0, 0, 0, 0);
            qb[st] = as_bf16x8(w);
        }
    }
    uint4 a[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int key = key0 + t * 16 + r;
        if (key < nc) {
            const uint16_t* kp = kc_pool + (((size_t)trow[key / SL] * Hkv + g) * SL + key % SL) * D;
#pragma unroll
            for (int st = 0; st < 4; ++st) a[t][st] = ldg16(kp + st * 32 + kq * 8);
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) a[t][st] = make_uint4(0, 0, 0, 0);
        }
    }
    float mx = -INFINITY;
    float zv[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma16(as_bf16x8(a[t][st]), qb[st], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + t * 16 + kq * 4 + i;
            zv[t][i] = key < nc ? acc[i] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, zv[t][i]);
        }
        if (r < G) {
            float4 o = make_float4(zv[t][0], zv[t][1], zv[t][2], zv[t][3]);
            *reinterpret_cast<float4*>(z + ((size_t)s * Hq + g * G + r) * zstride + key0 + t * 16 + kq * 4) = o;
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum += exp2f(zv[t][i] - mx);
    }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (kq == 0 && r < G) zpart[((size_t)s * Hq + g * G + r) * nchunk + chunk] = make_float2(mx, sum);
}

hipError_t launch_scores(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, float* z, float2* zpart, hipStream_t stream)
{
    dim3 grid(pl.score_groups, pl.Hkv, pl.B);
#define NOSA_SCORES(T)                                                                        \
    hipLaunchKernelGGL(scores_kernel<T>, grid, dim3(256), 0, stream, q, kv.kc_pool,           \
                       kv.block_table, kv.max_blocks_per_seq, pl.Lmax, cu_k, pl.Hq, pl.Hkv, pl.G, \
                       pl.scale_log2, z, pl.zstride, zpart, pl.nchunk)
    switch (pl.score_tiles) {
        case 1: NOSA_SCORES(1); break;
        case 2: NOSA_SCORES(2); break;
        case 4: NOSA_SCORES(4); break;
        default: NOSA_SCORES(8); break;
    }
#undef NOSA_SCORES
    return hipGetLastError();
}

// -------------------------------------------------------------- select ---

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of the workgroup; returns this
// thread's prefix and writes the total to *total.  Uses `scratch` (>= 4 ints).
__device__ int block_exclusive_scan(int v, int* scratch, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int t = scratch[w];
        if (w < wave) base += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return base + x - v;
}

// One workgroup per (KV head, sequence).  LDS: the block importances of the
// sequence (max_nb floats) + small tables.
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ z, int zstride, const float2* __restrict__ zpart, int nchunk,
    const float* __restrict__ scores_in, float* __restrict__ scores_out,
    int32_t* __restrict__ sel, int32_t* __restrict__ cnt, const int32_t* __restrict__ cu_k,
    int Lmax, int Hq, int Hkv, int G, int max_nb, int max_sel, int topk, int wblocks)
{
    extern __shared__ float sI[];
    __shared__ float s_lse[kMaxGroup];
    __shared__ int hist[256];
    __shared__ int scan_tmp[8];
    __shared__ int s_digit, s_need;

    const int g = blockIdx.x, s = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = seq_len(cu_k, s, Lmax);
    const int nc = dev_num_keys(L);
    const int nb = (L + BS - 1) / BS;
    const size_t row = (size_t)s * Hkv + g;

    if (z) {
        // per-head log2-sum-exp2 over all keys, from the per-wave partials
        for (int h = wave; h < G; h += 4) {
            const float2* zp = zpart + ((size_t)s * Hq + g * G + h) * nchunk;
            float m = -INFINITY;
            for (int c = lane; c < nchunk; c += 64) m = fmaxf(m, zp[c].x);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            float acc = 0.f;
            if (m != -INFINITY)
                for (int c = lane; c < nchunk; c += 64) {
                    const float2 v = zp[c];
                    if (v.y > 0.f) acc += v.y * exp2f(v.x - m);
                }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) s_lse[h] = m + log2f(acc);
        }
        __syncthreads();
        // block importance: mean over the keys overlapping the block of the
        // group's summed softmax probabilities
        const float* zg = z + ((size_t)s * Hq + g * G) * zstride;
        for (int b = tid; b < nb; b += 256) {
            const int jlo = max(4 * b - 1, 0), jhi = min(4 * b + 3, nc - 1);
            float I = -INFINITY;
            if (jlo <= jhi) {
                float acc = 0.f;
                for (int j = jlo; j <= jhi; ++j) {
                    float sj = 0.f;
                    for (int h = 0; h < G; ++h) sj += exp2f(zg[(size_t)h * zstride + j] - s_lse[h]);
                    acc += sj;
                }
                I = acc / (float)(jhi - jlo + 1);
            }
            sI[b] = I;
            if (scores_out) scores_out[row * max_nb + b] = I;
        }
        if (scores_out)
            for (int b = nb + tid; b < max_nb; b += 256) scores_out[row * max_nb + b] = -INFINITY;
    } else {
        for (int b = tid; b < nb; b += 256) sI[b] = scores_in[row * max_nb + b];
    }
    if (!sel) return;
    __syncthreads();

    const int ncand = nb > wblocks ? nb - wblocks : 0;
    const int kk = topk < ncand ? topk : ncand;
    uint32_t thresh = 0;
    int need = 0;
    const bool partial = kk > 0 && kk < ncand;
    if (partial) {
        // radix select of the kk-th largest key, 8 bits at a time from the top
        uint32_t prefix = 0, pmask = 0;
        need = kk;
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            for (int b = tid; b < ncand; b += 256) {
                const uint32_t key = order_key(sI[b]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
            }
            __syncthreads();
            // reverse the bin order so the exclusive scan is over larger digits
            const int rev = hist[255 - tid];
            int tot;
            const int above_rev = block_exclusive_scan(rev, scan_tmp, &tot);
            // thread tid handles digit 255 - tid: keys with digit > (255 - tid)
            const int digit = 255 - tid;
            if (above_rev < need && above_rev + rev >= need) {
                s_digit = digit;
                s_need = need - above_rev;
            }
            __syncthreads();
            prefix |= (uint32_t)s_digit << shift;
            pmask |= 0xffu << shift;
            need = s_need;
            __syncthreads();
        }
        thresh = prefix;
    }

    // ascending compaction of the chosen candidates; thread tid owns a
    // contiguous run of candidate ids
    const int per = (ncand + 255) / 256;
    const int b0 = min(tid * per, ncand), b1 = min(b0 + per, ncand);
    int eq_before = 0, tot;
    if (partial) {
        int eq = 0;
        for (int b = b0; b < b1; ++b) eq += order_key(sI[b]) == thresh;
        eq_before = block_exclusive_scan(eq, scan_tmp, &tot);
    }
    int nmine = 0;
    {
        int eqr = eq_before;
        for (int b = b0; b < b1; ++b) {
            bool take;
            if (!partial) {
                take = kk > 0;
            } else {
                const uint32_t key = order_key(sI[b]);
                take = key > thresh || (key == thresh && eqr < need);
                eqr += key == thresh;
            }
            nmine += take;
        }
    }
    int nsel;
    int pos = block_exclusive_scan(nmine, scan_tmp, &nsel);
    int32_t* out = sel + row * max_sel;
    {
        int eqr = eq_before;
        for (int b = b0; b < b1; ++b) {
            bool take;
            if (!partial) {
                take = kk > 0;
            } else {
                const uint32_t key = order_key(sI[b]);
                take = key > thresh || (key == thresh && eqr < need);
                eqr += key == thresh;
            }
            if (take) out[pos++] = b;
        }
    }
    const int total = nsel + (nb - ncand);
    for (int b = ncand + tid; b < nb; b += 256) out[nsel + (b - ncand)] = b;
    for (int x = total + tid; x < max_sel; x += 256) out[x] = -1;
    if (tid == 0) cnt[row] = total;
}

hipError_t launch_select(const Plan& pl, const int32_t* cu_k, const float* z,
                         const float2* zpart, const float* scores_in, float* scores_out,
                         int32_t* sel, int32_t* cnt, hipStream_t stream)
{
    dim3 grid(pl.Hkv, pl.B);
    const size_t lds = sizeof(float) * (size_t)(pl.max_nb > 0 ? pl.max_nb : 1);
    hipLaunchKernelGGL(select_kernel, grid, dim3(256), lds, stream, z, pl.zstride, zpart,
                       pl.nchunk, scores_in, scores_out, sel, cnt, cu_k, pl.Lmax,
                       pl.Hq, pl.Hkv, pl.G, pl.max_nb, pl.max_sel, pl.topk, pl.wblocks);
    return hipGetLastError();
}

// -------------------------------------------------------------- attend ---

// Row order of the K tile inside the QK^T MFMA.  Tile t = 2u + v, row
// m = 4c + i holds token 32u + 8c + 4v + i.  With this order the
// accumulator of lane (r, kq) ends up holding, for head r, the tokens
// 32u + 8kq + 0..7 across tiles 2u and 2u+1: exactly the A operand of the
// PV MFMA over the 32 tokens of k-step u.
__device__ __forceinline__ int qk_row_token(int t, int m)
{
    return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

// Workgroup = 4 waves = one split of one (sequence, KV head).  Wave w handles
// the selected blocks split*4R + 4*rr + w, rr < R.  Per block: 16 MFMAs for
// S^T = K q^T (64 tokens x 16 heads), online softmax in fp32, 16 MFMAs for
// O += P V (16 heads x 128 channels).  The four wave partials are merged in
// LDS into one (m, l, o) partial per workgroup.
template <int R>
__global__ __launch_bounds__(256) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ table, int max_blocks,
    int Lmax, const int32_t* __restrict__ cu_k, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ cnt, int max_sel, int Hq, int Hkv, int G, float scale_log2,
    float* __restrict__ po, float2* __restrict__ pml, int nsplit)
{
    __shared__ float sm[4][16], sl[4][16];
    __shared__ float so[4][16][D + 4];

    const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int L = seq_len(cu_k, s, Lmax);
    const int nb = (L + BS - 1) / BS;
    const size_t row = (size_t)s * Hkv + g;
    const int count = min(cnt[row], max_sel);
    const int32_t* mysel = sel + row * max_sel;
    const int32_t* trow = table + (size_t)s * max_blocks;

    bf16x8 qb[4];
    {
        const uint16_t* qh = q + ((size_t)s * Hq + g * G + (r < G ? r : 0)) * D;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint4 w = ldg16(qh + st * 32 + kq * 8);
            if (r >= G) w = make_uint4(0, 0, 0, 0);
            qb[st] = as_bf16x8(w);
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int rr = 0; rr < R; ++rr) {
        const int idx = split * 4 * R + rr * 4 + wave;
        if (idx >= count) break;
        const int b = mysel[idx];
        if (b < 0 || b >= nb) continue;
        const int page = trow[b];
        const uint16_t* kb = k_pool + ((size_t)page * Hkv + g) * BS * D;
        const uint16_t* vb = v_pool + ((size_t)page * Hkv + g) * D * BS;
        uint4 ka[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tok = qk_row_token(t, r);
#pragma unroll
            for (int st = 0; st < 4; ++st) ka[t][st] = ldg16(kb + tok * D + st * 32 + kq * 8);
        }
        uint4 va[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) va[u][nt] = ldg16(vb + (nt * 16 + r) * BS + u * 32 + kq * 8);

        const int limit = L - b * BS;  // tokens of this block that exist
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
        const float m_new = fmaxf(m_run, bmax);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[t][i] = exp2f(x[t][i] - m_new);
                psum += x[t][i];
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * kq + i);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) o[nt][i] *= ai;
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
            for (int nt = 0; nt < 8; ++nt) o[nt] = mfma16(pa, as_bf16x8(va[u][nt]), o[nt]);
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (kq == 0) {
        sm[wave][r] = m_run;
        sl[wave][r] = l_run;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[wave][4 * kq + i][nt * 16 + r] = o[nt][i];
    __syncthreads();

    const int h = tid >> 4, c0 = (tid & 15) * 8;
    if (h < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][h]);
        float wt[4], Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wt[w] = (M == -INFINITY || sm[w][h] == -INFINITY) ? 0.f : exp2f(sm[w][h] - M);
            Lsum += wt[w] * sl[w][h];
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[e] = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[e] += wt[w] * so[w][h][c0 + e];
        }
        const size_t prow = ((size_t)s * Hq + g * G + h) * nsplit + split;
        float4* dst = reinterpret_cast<float4*>(po + prow * D + c0);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if ((tid & 15) == 0) pml[prow] = make_float2(M, Lsum);
    }
}

hipError_t launch_attend(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* q,
                         const int32_t* cu_k, const int32_t* sel, const int32_t* cnt,
                         float* po, float2* pml, hipStream_t stream)
{
    dim3 grid(pl.nsplit, pl.Hkv, pl.B);
#define NOSA_ATTEND(R)                                                                        \
    hipLaunchKernelGGL(attend_kernel<R>, grid, dim3(256), 0, stream, q, kv.k_pool, kv.v_pool, \
                       kv.block_table, kv.max_blocks_per_seq, pl.Lmax, cu_k, sel, cnt,        \
                       pl.max_sel,                                                            \
                       pl.Hq, pl.Hkv, pl.G, pl.scale_log2, po, pml, pl.nsplit)
    switch (pl.attn_rounds) {
        case 1: NOSA_ATTEND(1); break;
        case 2: NOSA_ATTEND(2); break;
        case 3: NOSA_ATTEND(3); break;
        default: NOSA_ATTEND(4); break;
    }
#undef NOSA_ATTEND
    return hipGetLastError();
}

// --------------------------------------------------------------- merge ---

// One workgroup of 128 threads (one per channel) per (query head, sequence).
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ po,
                                                    const float2* __restrict__ pml, int nsplit,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse, int Hq)
{
    const int h = blockIdx.x, s = blockIdx.y, c = threadIdx.x;
    const size_t rowq = (size_t)s * Hq + h;
    const float2* ml = pml + rowq * nsplit;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[i].x);
    float acc = 0.f, Lsum = 0.f;
    if (M != -INFINITY)
        for (int i = 0; i < nsplit; ++i) {
            const float2 v = ml[i];
            if (v.x == -INFINITY) continue;
            const float w = exp2f(v.x - M);
            Lsum += w * v.y;
            acc += w * po[(rowq * nsplit + i) * D + c];
        }
    const bool empty = !(Lsum > 0.f);
    out[rowq * D + c] = empty ? 0.f : acc / Lsum;
    if (lse && c == 0) lse[rowq] = empty ? -INFINITY : (M + log2f(Lsum)) * 0.69314718055994531f;
}

hipError_t launch_merge(const Plan& pl, const float* po, const float2* pml, float* out,
                        float* lse, hipStream_t stream)
{
    dim3 grid(pl.Hq, pl.B);
    hipLaunchKernelGGL(merge_kernel, grid, dim3(D), 0, stream, po, pml, pl.nsplit, out, lse,
                       pl.Hq);
    return hipGetLastError();
}

}  // namespace nosa
