// nosa_front.hip -- the attention front end of a decode step on gfx950: the
// QKV projection of each sequence's current token, the rotary encoding of q
// and k, and the write of k and v into the token's page slot, in one launch
// (page "NOSA技术架构解析", section 2.1: NOSI fuses the projection, the rotary
// encoding and the importance scoring to cut the launches of a decode step).
//
// The projection reads the whole weight matrix once per step, (Hq + 2 Hkv) x
// 128 rows of `hidden` bf16 (10.5 MB for 16 / 2 heads and hidden 2048), for a
// handful of tokens: it is bound by HBM, not by the matrix cores, so the
// launch is laid out to stream the weights over many CUs.  A workgroup owns a
// tile of 16 output rows of one head -- rows 8j .. 8j+7 and 64+8j .. 64+8j+7,
// the eight channel pairs that the rotary encoding turns together -- for 16
// tokens, and its eight waves split the hidden dimension in runs of 256.
// The weights are stored packed in MFMA operand order (nosa_pack_qkv_weights):
// for tile T, run kb and k-step t, the 64 lanes' 16-byte operands lie in one
// contiguous kilobyte, so every load instruction of a wave reads 1 KB in one
// piece.  Lane 16 grp + m of k-step t holds row m, hidden channels
// 256 kb + 32 t + 8 grp .. +7, and the activations are read with the same
// channel order.  The projection of one head cannot be fused into the
// scoring launch: every scoring workgroup of a (sequence, KV head) would have
// to read the G heads' weights again.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

constexpr int kFrontWaves = 8;   // waves of a front-end workgroup (split the hidden dimension)
constexpr int kFrontRows = 16;   // output rows per workgroup: 8 rotary pairs
constexpr int kFrontTokens = 16; // tokens per workgroup (MFMA N)

// Output row of local row m (0 .. 15) of tile T = 8 head + j.
__device__ __forceinline__ int front_row(int T, int m)
{
    const int head = T >> 3, j = T & 7;
    return head * D + (m < 8 ? 8 * j + m : 64 + 8 * j + (m - 8));
}

struct FrontArgs {
    const uint16_t* x;      // [B][hidden]
    const uint16_t* w;      // packed: [tiles][hidden / 256][8][64 lanes][8]
    const float* inv_freq;  // [64] or null: then freq
    double freq[D / 2];     // theta^(-2i / 128), computed on the host
    const int32_t* cu_k;
    const int32_t* table;
    int max_blocks, Lmax, B, hidden, Hq, Hkv;
    uint16_t* k_pool;
    uint16_t* v_pool;
    uint16_t* q_out;        // [B][Hq][128]
};

// bf16 round-to-nearest-even of a finite float.
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(kFrontWaves * 64) void front_kernel(FrontArgs a)
{
    __shared__ float part[kFrontWaves][kFrontRows][kFrontTokens + 1];
    __shared__ float sum[kFrontRows][kFrontTokens + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, grp = lane >> 4;  // MFMA operand row / column, k group
    const int head = blockIdx.x >> 3, j = blockIdx.x & 7;
    const int tok0 = blockIdx.y * kFrontTokens;
    const int tok = min(tok0 + m, a.B - 1);  // token of column m (columns past the batch unused)
    // Thread (token c, pair p) of the first 128 writes channels i and i + 64
    // of token b.  Its position is loaded before the weights, so that the
    // rotation is computed while they are in flight, and its page slot after
    // them (needed only at the end).
    const int c = (tid >> 3) & 15, p = tid & 7;
    const int b = tok0 + c, i = 8 * j + p;
    const bool lead = tid < 8 * kFrontTokens && b < a.B;
    const int L = lead ? seq_len(a.cu_k, b, a.Lmax) : 0;
    const int nkb = a.hidden / 256;  // runs of 256 hidden channels, dealt to the waves
    const uint16_t* wt = a.w + (size_t)blockIdx.x * nkb * 8 * 512 + lane * 8;
    const uint16_t* xr = a.x + (size_t)tok * a.hidden + 8 * grp;
    int kb = wave;
    uint4 wv[8], xv[8];
    if (kb < nkb) {
#pragma unroll
        for (int t = 0; t < 8; ++t) wv[t] = ldg16(wt + ((size_t)kb * 8 + t) * 512);
#pragma unroll
        for (int t = 0; t < 8; ++t) xv[t] = ldg16(xr + kb * 256 + 32 * t);
    }
    const int pos = L - 1;
    const bool live = lead && pos >= 0;
    float s32 = 0.f, c32 = 1.f;
    if (live && head < a.Hq + a.Hkv) {
        // angle pos * f in fp64, reduced to [-pi, pi] by subtracting the
        // nearest multiple of 2 pi (Cody and Waite: 2 pi as a double plus its
        // remainder, each product exact inside a fused multiply-add), then
        // sine and cosine of the small remainder in fp32
        const double f = a.inv_freq ? (double)a.inv_freq[i] : a.freq[i];
        const double ang = (double)pos * f;
        const double kk = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
        double red = fma(-kk, 6.283185307179586, ang);      // 2 pi rounded to double
        red = fma(-kk, 2.4492935982947064e-16, red);        // 2 pi minus that double
        sincosf((float)red, &s32, &c32);
    }
    const int page = live && head >= a.Hq ? a.table[(size_t)b * a.max_blocks + pos / BS] : 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    while (kb < nkb) {
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = mfma16(as_bf16x8(wv[t]), as_bf16x8(xv[t]), acc);
        kb += kFrontWaves;
        if (kb < nkb) {
#pragma unroll
            for (int t = 0; t < 8; ++t) wv[t] = ldg16(wt + ((size_t)kb * 8 + t) * 512);
#pragma unroll
            for (int t = 0; t < 8; ++t) xv[t] = ldg16(xr + kb * 256 + 32 * t);
        }
    }
    // lane (m, grp) holds rows 4 grp + i of token column m
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wave][4 * grp + e][m] = acc[e];
    __syncthreads();
    if (tid < kFrontRows * kFrontTokens) {
        const int rr = tid / kFrontTokens, cc = tid % kFrontTokens;
        float sm = 0.f;
#pragma unroll
        for (int w = 0; w < kFrontWaves; ++w) sm += part[w][rr][cc];
        sum[rr][cc] = sm;
    }
    __syncthreads();
    if (!live) return;
    float lo = sum[p][c], hi = sum[p + 8][c];
    if (head < a.Hq + a.Hkv) {  // q and k heads: rotary encoding
        const float nlo = lo * c32 - hi * s32, nhi = hi * c32 + lo * s32;
        lo = nlo;
        hi = nhi;
    }
    const uint16_t blo = bf16_rne(lo), bhi = bf16_rne(hi);
    if (head < a.Hq) {
        uint16_t* qo = a.q_out + ((size_t)b * a.Hq + head) * D;
        qo[i] = blo;
        qo[i + 64] = bhi;
        return;
    }
    const int x = pos % BS;
    if (head < a.Hq + a.Hkv) {
        uint16_t* kp = a.k_pool + ((size_t)page * a.Hkv + (head - a.Hq)) * BS * D;
        kp[k_chunk(x, i / 8) + i % 8] = blo;
        kp[k_chunk(x, (i + 64) / 8) + (i + 64) % 8] = bhi;
    } else {
        uint16_t* vp = a.v_pool + ((size_t)page * a.Hkv + (head - a.Hq - a.Hkv)) * D * BS;
        vp[v_chunk(i, x / 8) + x % 8] = blo;
        vp[v_chunk(i + 64, x / 8) + x % 8] = bhi;
    }
}

// Packs row-major weights [(Hq + 2 Hkv) * 128][hidden] into the operand
// order above: one thread per 16-byte operand.
__global__ __launch_bounds__(256) void pack_qkv_kernel(const uint16_t* __restrict__ w,
                                                       uint16_t* __restrict__ packed, int hidden,
                                                       long long n16)
{
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n16) return;
    const int nkb = hidden / 256;
    const int lane = (int)(idx & 63), t = (int)((idx >> 6) & 7);
    const long long rest = idx >> 9;  // T * nkb + kb
    const int kb = (int)(rest % nkb), T = (int)(rest / nkb);
    const int m = lane & 15, grp = lane >> 4;
    const uint16_t* src = w + (size_t)front_row(T, m) * hidden + 256 * kb + 32 * t + 8 * grp;
    *reinterpret_cast<uint4*>(packed + (size_t)idx * 8) = ldg16(src);
}

hipError_t launch_pack_qkv(int Hq, int Hkv, int hidden, const nosa_bf16* w, nosa_bf16* packed,
                           hipStream_t stream)
{
    const long long n16 = (long long)(Hq + 2 * Hkv) * D * hidden / 8;
    if (n16 > 0)
        hipLaunchKernelGGL(pack_qkv_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0,
                           stream, w, packed, hidden, n16);
    return hipGetLastError();
}

hipError_t launch_front(const Plan& pl, const nosa_paged_kv& kv, const nosa_bf16* x,
                        const nosa_bf16* w, int hidden, float theta, const float* inv_freq,
                        const int32_t* cu_k, nosa_bf16* q_out, hipStream_t stream)
{
    FrontArgs a{};
    a.x = x;
    a.w = w;
    a.inv_freq = inv_freq;
    for (int i = 0; i < D / 2; ++i) a.freq[i] = pow((double)theta, -2.0 * i / D);
    a.cu_k = cu_k;
    a.table = kv.block_table;
    a.max_blocks = kv.max_blocks_per_seq;
    a.Lmax = pl.Lmax;
    a.B = pl.B;
    a.hidden = hidden;
    a.Hq = pl.Hq;
    a.Hkv = pl.Hkv;
    a.k_pool = const_cast<uint16_t*>(kv.k_pool);
    a.v_pool = const_cast<uint16_t*>(kv.v_pool);
    a.q_out = q_out;
    const dim3 grid((pl.Hq + 2 * pl.Hkv) * 8, ceil_div(pl.B, kFrontTokens));
    hipLaunchKernelGGL(front_kernel, grid, dim3(kFrontWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nosa
