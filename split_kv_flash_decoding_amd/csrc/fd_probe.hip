// HBM probes: a streaming read and a plain copy (see include/fd_probe.h).
// Grid-stride loops over 16-byte words; a fixed grid of FD_PROBE_SINK_FLOATS
// work-groups of 256 threads keeps many loads in flight on every compute unit.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"
#include "fd_probe.h"

namespace fdp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, uint64_t n,
                                                        float* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 x = src[i];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)(red[0] & 0xffffu);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                        uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace fdp

using namespace fd;

extern "C" {

fd_status fd_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
    clear_error();
    if (!src || !sink || bytes == 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_read needs 16-byte aligned src, sink and a size multiple of 16");
    hipLaunchKernelGGL(fdp::read_kernel, dim3(FD_PROBE_SINK_FLOATS), dim3(fdp::kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const fdp::u32x4*>(src),
                       (uint64_t)(bytes / 16), sink);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FD_ERR_HIP, "probe_read launch: %s", hipGetErrorString(e));
    return FD_OK;
}

fd_status fd_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    clear_error();
    if (!src || !dst || bytes == 0 || (bytes & 15) ||
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_copy needs 16-byte aligned pointers and a size multiple of 16");
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return fail(FD_ERR_INVALID_ARGUMENT, "probe_copy ranges overlap");
    hipLaunchKernelGGL(fdp::copy_kernel, dim3(FD_PROBE_SINK_FLOATS), dim3(fdp::kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<fdp::u32x4*>(dst),
                       static_cast<const fdp::u32x4*>(src), (uint64_t)(bytes / 16));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FD_ERR_HIP, "probe_copy launch: %s", hipGetErrorString(e));
    return FD_OK;
}

}  // extern "C"
