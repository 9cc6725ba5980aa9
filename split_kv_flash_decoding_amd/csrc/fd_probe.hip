// HBM probes: a streaming read and a plain copy (see include/fd_probe.h).
// A fixed grid of FD_PROBE_SINK_FLOATS work-groups of 256 threads; each
// work-group streams one contiguous slice with non-temporal 16-byte loads,
// eight in flight per thread (the fastest of the read patterns measured on
// MI355X: about 7.1 TB/s on a 2 GiB buffer).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"
#include "fd_probe.h"

namespace fdp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, uint64_t n,
                                                        float* __restrict__ sink) {
    const uint64_t per = (n + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = (uint64_t)blockIdx.x * per;
    const uint64_t b1 = b0 + per < n ? b0 + per : n;
    uint32_t acc = 0;
    uint64_t i = b0 + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < b1; i += kThreads) {
        const u32x4 x = __builtin_nontemporal_load(src + i);
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
