// probe_chip.hip -- machine probes of the benchmark's --chip-probes mode
// (measurement only; not part of the NOSA library or its C ABI): the costs
// on this chip that the library's design rests on.
//   * nosa_probe_mix: the instruction mix of a prefill scoring step (per wave
//     and iteration 64 v_mfma_f32_16x16x32_bf16 and, per product, an fma, an
//     exp2 and an add), with the MFMAs alone, the VALU work alone, both
//     dependent (the VALU work reads the MFMA results, as in the kernel) and
//     both independent -- how far the VALU and the matrix core overlap;
//   * nosa_probe_lds_read: LDS read bandwidth, each wave reading 1 KB of
//     consecutive LDS per ds_read_b128;
//   * nosa_probe_handoff: partials of 16 workgroups handed to the last of
//     them inside one launch (device-scope release/acquire, or coherent
//     stores and loads with no fence) against a second launch;
//   * nosa_probe_chase: the latency of a dependent load (vector and scalar
//     loads) with its lines in the XCD's L2, in the Infinity Cache, or in
//     HBM only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// MODE 0: MFMA + dependent VALU, 1: MFMA only, 2: VALU only, 3: MFMA + VALU
// on values that do not wait for the MFMAs.  Two workgroups of 4 waves per
// CU: two waves per SIMD, as in the scoring kernels.
template <int MODE>
__global__ __launch_bounds__(256, 2) void mix_kernel(float* __restrict__ sink, int iters, float sc)
{
    const int lane = threadIdx.x & 63;
    bf16x8 qb[8][4], kf0[4], kf1[4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[u][st][e] = (__bf16)(0.01f * ((lane + u + st + e) & 7));
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kf0[st][e] = (__bf16)(0.02f * ((lane + st + e) & 3));
            kf1[st][e] = (__bf16)(0.03f * ((lane + st * e) & 3));
        }
    float s_run[8], ref[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        s_run[u] = 0.f;
        ref[u] = 0.1f * u;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            if (MODE != 2) {
#pragma unroll
                for (int st = 0; st < 4; ++st) s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf0[st], qb[u][st], s0, 0, 0, 0);
#pragma unroll
                for (int st = 0; st < 4; ++st) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1[st], qb[u][st], s1, 0, 0, 0);
            }
            if (MODE == 1) {
                s_run[u] += s0[0] + s1[3];
                continue;
            }
            // the products the VALU work reads: the MFMA results, or values
            // carried from the previous iteration (no MFMA to wait for)
            f32x4 z0 = s0, z1 = s1;
            if (MODE >= 2) {
                const float c = s_run[u] * 0.5f;
                z0 = f32x4{c, c + 1.f, c + 2.f, c + 3.f};
                z1 = f32x4{c + 4.f, c + 5.f, c + 6.f, c + 7.f};
            }
            const float nm = -(ref[u] * sc);
            float e = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                e += __builtin_amdgcn_exp2f(fmaf(z0[i], sc, nm)) + __builtin_amdgcn_exp2f(fmaf(z1[i], sc, nm));
            s_run[u] = (s_run[u] + e) * 1e-3f + (MODE == 3 ? (s0[0] + s1[3]) * 1e-30f : 0.f);
        }
    }
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) t += s_run[u];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
}

// Each wave reads the 32 runs of 1 KB of a 32 KB LDS buffer per iteration.
__global__ __launch_bounds__(256, 2) void lds_read_kernel(uint32_t* __restrict__ sink, int iters)
{
    __shared__ uint4 buf[2048];
    for (int i = threadIdx.x; i < 2048; i += 256) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint4 v = buf[((j + 8 * w + it) & 31) * 64 + lane];
            acc = (acc ^ v.x) + (v.y ^ v.z) + v.w;
        }
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Hand-off: workgroup b writes a 4 KB partial (every element b + 1), then the
// last of its group of 16 to arrive sums the group's 16 partials into out
// (expected 16 * 17 / 2 + 16 * 16 * g... written as the sum itself, checked
// on the host) and resets the group's counter.
constexpr int kHandGroup = 16;
template <int MODE>
__global__ __launch_bounds__(256) void handoff_kernel(float* __restrict__ part, int* __restrict__ counter,
                                                      float* __restrict__ out)
{
    __shared__ int last;
    const int b = blockIdx.x, g = b / kHandGroup, t = threadIdx.x;
    float* p = part + (size_t)b * 1024 + 4 * t;
    if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = (float)(b + 1);
        __syncthreads();
        if (t == 0)
            last = __hip_atomic_fetch_add(&counter[g], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                   kHandGroup - 1;
    } else {
        // coherent stores (they bypass the non-coherent caches), all of them
        // completed before the count: no cache write-back or invalidation
#pragma unroll
        for (int e = 0; e < 4; ++e) __hip_atomic_store(p + e, (float)(b + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        if (t == 0)
            last = __hip_atomic_fetch_add(&counter[g], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   kHandGroup - 1;
    }
    __syncthreads();
    if (!last) return;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kHandGroup; ++j) {
        const float* q = part + (size_t)(g * kHandGroup + j) * 1024 + 4 * t;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s[e] += MODE == 0 ? q[e] : __hip_atomic_load(q + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(size_t)g * 1024 + 4 * t + e] = s[e];
    if (t == 0) counter[g] = 0;
}

__global__ __launch_bounds__(256) void handoff_write_kernel(float* __restrict__ part)
{
    float* p = part + (size_t)blockIdx.x * 1024 + 4 * threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = (float)(blockIdx.x + 1);
}

__global__ __launch_bounds__(256) void handoff_sum_kernel(const float* __restrict__ part, float* __restrict__ out)
{
    const int g = blockIdx.x, t = threadIdx.x;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kHandGroup; ++j) {
        const float* q = part + (size_t)(g * kHandGroup + j) * 1024 + 4 * t;
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += q[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(size_t)g * 1024 + 4 * t + e] = s[e];
}

// A chain of dependent loads through next[] (a cycle through the array),
// timed inside the launch with the constant-rate wall clock: `warm` hops from
// `warm_start` first (untimed: they bring the timed hops' lines into the
// caches when warm_start == start), then `steps` hops from `start`, timed.
// With VECTOR, every lane of one wave follows the chain (the index comes
// from memory, so the loads are vector loads, the lanes' addresses
// coinciding); else a uniform index (scalar loads).  out[0] = the chain's end,
// out[1] = the timed hops' wall-clock ticks.
template <bool VECTOR>
__global__ void chase_kernel(const int* __restrict__ next, int warm_start, int warm, int start,
                             int steps, const int* __restrict__ zero, long long* __restrict__ out)
{
    if (VECTOR) {
        int i = warm_start + zero[threadIdx.x];
        for (int s = 0; s < warm; ++s) i = next[i];
        asm volatile("" ::"v"(i));
        i = start + zero[threadIdx.x];
        asm volatile("" : "+v"(i));
        const long long t0 = wall_clock64();
        for (int s = 0; s < steps; ++s) i = next[i];
        asm volatile("" ::"v"(i));
        const long long t1 = wall_clock64();
        if (threadIdx.x == 0) {
            out[0] = i;
            out[1] = t1 - t0;
        }
    } else {
        int i = warm_start;
        for (int s = 0; s < warm; ++s) i = next[i];
        asm volatile("" ::"s"(i));
        i = start;
        asm volatile("" : "+s"(i));
        const long long t0 = wall_clock64();
        for (int s = 0; s < steps; ++s) i = next[i];
        asm volatile("" ::"s"(i));
        const long long t1 = wall_clock64();
        if (threadIdx.x == 0) {
            out[0] = i;
            out[1] = t1 - t0;
        }
    }
}

}  // namespace

extern "C" {

// The instruction-mix probe (mode 0 .. 3 as above) with `workgroups`
// workgroups of 256 threads for `iters` iterations; sink: workgroups * 256
// floats.  Returns the hipError_t of the launch.
int nosa_probe_mix(int mode, int workgroups, int iters, float* sink, void* stream)
{
    if (!sink || workgroups <= 0 || iters < 0 || mode < 0 || mode > 3) return (int)hipErrorInvalidValue;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float sc = 0.1275f;
    switch (mode) {
        case 0: hipLaunchKernelGGL(mix_kernel<0>, dim3(workgroups), dim3(256), 0, s, sink, iters, sc); break;
        case 1: hipLaunchKernelGGL(mix_kernel<1>, dim3(workgroups), dim3(256), 0, s, sink, iters, sc); break;
        case 2: hipLaunchKernelGGL(mix_kernel<2>, dim3(workgroups), dim3(256), 0, s, sink, iters, sc); break;
        default: hipLaunchKernelGGL(mix_kernel<3>, dim3(workgroups), dim3(256), 0, s, sink, iters, sc); break;
    }
    return (int)hipGetLastError();
}

// LDS read probe: `workgroups` workgroups of 4 waves, each wave reading 32 KB
// of LDS per iteration; sink: workgroups * 256 words.
int nosa_probe_lds_read(int workgroups, int iters, uint32_t* sink, void* stream)
{
    if (!sink || workgroups <= 0 || iters < 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(lds_read_kernel, dim3(workgroups), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), sink,
                       iters);
    return (int)hipGetLastError();
}

// Hand-off probe over groups * 16 workgroups: mode 0 device-scope
// release/acquire, 1 coherent stores and loads, 2 two launches.  part:
// groups * 16 * 1024 floats; counter: groups ints, zero before the first
// call (each group's last workgroup resets its counter); out: groups * 1024
// floats.
int nosa_probe_handoff(int mode, int groups, float* part, int* counter, float* out, void* stream)
{
    if (!part || !counter || !out || groups <= 0 || mode < 0 || mode > 2) return (int)hipErrorInvalidValue;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid(groups * kHandGroup);
    if (mode == 0) hipLaunchKernelGGL(handoff_kernel<0>, grid, dim3(256), 0, s, part, counter, out);
    else if (mode == 1) hipLaunchKernelGGL(handoff_kernel<1>, grid, dim3(256), 0, s, part, counter, out);
    else {
        hipLaunchKernelGGL(handoff_write_kernel, grid, dim3(256), 0, s, part);
        hipLaunchKernelGGL(handoff_sum_kernel, dim3(groups), dim3(256), 0, s, part, out);
    }
    return (int)hipGetLastError();
}

// Dependent-load probe (chase_kernel above): one wave; zero: 64 device
// ints, all zero; out: 2 device long longs.  Returns the hipError_t of the
// launch.
int nosa_probe_chase(const int* next, int warm_start, int warm, int start, int steps, int vector,
                     const int* zero, long long* out, void* stream)
{
    if (!next || !zero || !out || steps < 0 || warm < 0) return (int)hipErrorInvalidValue;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (vector)
        hipLaunchKernelGGL(chase_kernel<true>, dim3(1), dim3(64), 0, s, next, warm_start, warm, start,
                           steps, zero, out);
    else
        hipLaunchKernelGGL(chase_kernel<false>, dim3(1), dim3(64), 0, s, next, warm_start, warm, start,
                           steps, zero, out);
    return (int)hipGetLastError();
}

// The wall clock's rate in kHz (chase_kernel's ticks), or 0 on an error.
int nosa_probe_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
