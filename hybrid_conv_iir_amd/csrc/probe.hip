// HBM probes: a streaming read kernel that measures the practical read
// ceiling next to the published peak, and a plain copy kernel of known size
// against which hardware byte counters are calibrated.
#include "hci_internal.h"

namespace hci {

constexpr int kProbeBlocks = 256 * 2;   // 8 waves per CU on a 256-CU part (the sweep optimum)
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const uint4* __restrict__ src, size_t n16,
                                                              float* __restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = load_nt(src + i), b = load_nt(src + i + stride);
        const uint4 c = load_nt(src + i + 2 * stride), d = load_nt(src + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t red[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kProbeThreads / 64; ++w) r ^= red[w];
        sink[blockIdx.x] = __uint_as_float(r & 0x007fffffu);
    }
}

__global__ __launch_bounds__(kProbeThreads) void k_probe_copy(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                              size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int probe_blocks() { return kProbeBlocks; }

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t st)
{
    hipLaunchKernelGGL(k_probe_read, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                       (const uint4*)src, bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t st)
{
    hipLaunchKernelGGL(k_probe_copy, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                       (uint4*)dst, (const uint4*)src, bytes / 16);
    return hipGetLastError();
}

}  // namespace hci
