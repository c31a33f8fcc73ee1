// probe_ceiling.hip -- read-bandwidth ceilings of the device, for the
// benchmark's --ceiling mode (measurement only; not part of the NOSA library
// or its C ABI).  One kernel reads whole pages of page_bytes (a multiple of
// 1 KB) in a given order, each wave one page at a time with every load of the
// page in flight (16 bytes per lane per load, so each load instruction reads
// one contiguous kilobyte, the access pattern of the decode kernels), and
// folds what it read into one word per wave so no load can be dropped.  The
// identity order measures a stream read, a random permutation of 32 KB pages
// the page gather of sparse attention.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kPageLoads = 32;  // 32 KB pages: 32 loads of 1 KB per wave

__global__ __launch_bounds__(256) void read_pages_kernel(const uint4* __restrict__ src,
                                                         const int32_t* __restrict__ order,
                                                         int npages, uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const int nwaves = (int)(gridDim.x * (blockDim.x >> 6));
    uint32_t acc = 0;
    for (int i = wave; i < npages; i += nwaves) {
        const uint4* p = src + (size_t)order[i] * (kPageLoads * 64) + lane;
        uint4 v[kPageLoads];
#pragma unroll
        for (int j = 0; j < kPageLoads; ++j) v[j] = p[j * 64];
#pragma unroll
        for (int j = 0; j < kPageLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    sink[(size_t)wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Reads npages pages of 32 KB of src (device) in the order given by
// order[0 .. npages) (device int32, page indexes), with `workgroups`
// workgroups of 256 threads; sink (device) receives workgroups * 4 * 64
// words.  Returns the hipError_t of the launch.
int nosa_probe_read_pages(const void* src, const int32_t* order, int npages, int workgroups,
                          uint32_t* sink, void* stream)
{
    if (!src || !order || !sink || npages < 0 || workgroups <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_pages_kernel, dim3(workgroups), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(src),
                       order, npages, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
