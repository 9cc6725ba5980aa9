// HBM probes (see include/fd_probe.h): a streaming read, a read of two
// row-major buffers in the decode kernels' pattern, and a plain copy.
// The streaming read: a fixed grid of FD_PROBE_SINK_FLOATS work-groups of 256
// threads; each work-group streams one contiguous slice with non-temporal
// 16-byte loads, eight in flight per thread (measured on MI355X over a 1 GiB
// K and a 1 GiB V buffer, one after the other: about 6.5 TB/s).

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

// Two buffers a and b of `rows` rows of `row_bytes` bytes, read the way the
// decode kernels read a token-major K and V cache: one work-group of eight
// waves per (chunk of chunk_rows rows, column block of block_bytes), column
// blocks fastest; every wave instruction reads 1 KB of one row (16 bytes per
// lane), and a stage is 4 rows of a and 4 of b, the next stage's eight loads
// in flight while the current one is consumed. ACROSS = false: the waves take
// stages w, w + 8, ... of the chunk in a 1 KB column block (the head-rows
// kernel); ACROSS = true: wave w takes every stage of column w of an 8 KB
// block (the head-columns kernel). Rows past the chunk re-read its last row.
// ROTATE (head rows only): a full chunk c starts at stage (7 c mod n) 8 of its
// n 8 stages and wraps round, the head-rows kernel's traversal of a 16-bit
// cache.
constexpr int kRowWaves = 8;
template <bool ACROSS, bool ROTATE = false>
__global__ __launch_bounds__(64 * kRowWaves) void read_rows_kernel(const uint8_t* __restrict__ a,
                                                                   const uint8_t* __restrict__ b, int64_t rows,
                                                                   int row_bytes, int block_bytes, int chunk_rows,
                                                                   float* __restrict__ sink) {
    const int nblk = row_bytes / block_bytes;
    const int blk = blockIdx.x % nblk;
    const int64_t r0 = (int64_t)(blockIdx.x / nblk) * chunk_rows;
    const int64_t r1 = r0 + chunk_rows < rows ? r0 + chunk_rows : rows;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)blk * block_bytes + (ACROSS ? wave * 1024 : 0) + lane * 16;
    const int nst = (int)((r1 - r0 + 3) / 4);
    const int step = ACROSS ? 1 : kRowWaves;
    int rot = 0;
    if (ROTATE && nst % kRowWaves == 0) rot = (int)((blockIdx.x / nblk * 7) % (nst / kRowWaves)) * kRowWaves;
    auto load = [&](int st_, u32x4* x) {
        const int st = st_ + rot < nst ? st_ + rot : st_ + rot - nst;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int64_t r = r0 + 4 * st + u;
            r = r < r1 ? r : r1 - 1;
            x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a + r * row_bytes + col));
            x[4 + u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + r * row_bytes + col));
        }
    };
    uint32_t acc = 0;
    auto use = [&](const u32x4* x) {
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    };
    u32x4 x[8], y[8];
    int st = ACROSS ? 0 : wave;
    if (st < nst) load(st, x);
    while (st < nst) {
        if (st + step < nst) load(st + step, y);
        use(x);
        st += step;
        if (st >= nst) break;
        if (st + step < nst) load(st + step, x);
        use(y);
        st += step;
    }
    // A store the compiler cannot rule out keeps the loads; it practically
    // never happens.
    if (acc == 0x9e3779b9u) sink[blockIdx.x % FD_PROBE_SINK_FLOATS] = (float)threadIdx.x;
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

fd_status fd_probe_read_rows(const void* a, const void* b, int64_t rows, int32_t row_bytes, int32_t block_bytes,
                             int32_t chunk_rows, int32_t waves_across, float* sink, void* stream) {
    clear_error();
    if (!a || !b || !sink || ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15))
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_read_rows needs 16-byte aligned a, b and a sink");
    if (rows < 1 || chunk_rows < 1 || row_bytes < 1024 || row_bytes % 1024)
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_read_rows: rows %lld, chunk_rows %d, row_bytes %d (a multiple "
                    "of 1024)", (long long)rows, chunk_rows, row_bytes);
    if (waves_across < 0 || waves_across > 2)
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_read_rows: waves_across %d is not 0, 1 or 2", waves_across);
    const int32_t want_block = waves_across == 1 ? 1024 * fdp::kRowWaves : 1024;
    if (block_bytes != want_block || row_bytes % block_bytes)
        return fail(FD_ERR_INVALID_ARGUMENT, "probe_read_rows: block_bytes must be %d and divide row_bytes %d",
                    want_block, row_bytes);
    const int64_t wgs = (rows + chunk_rows - 1) / chunk_rows * (row_bytes / block_bytes);
    if (wgs > INT32_MAX) return fail(FD_ERR_INVALID_ARGUMENT, "probe_read_rows: too many work-groups");
    const uint8_t* pa = static_cast<const uint8_t*>(a);
    const uint8_t* pb = static_cast<const uint8_t*>(b);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (waves_across == 1)
        hipLaunchKernelGGL(fdp::read_rows_kernel<true>, dim3((uint32_t)wgs), dim3(64 * fdp::kRowWaves), 0, hs, pa,
                           pb, rows, row_bytes, block_bytes, chunk_rows, sink);
    else if (waves_across == 2)
        hipLaunchKernelGGL((fdp::read_rows_kernel<false, true>), dim3((uint32_t)wgs), dim3(64 * fdp::kRowWaves), 0,
                           hs, pa, pb, rows, row_bytes, block_bytes, chunk_rows, sink);
    else
        hipLaunchKernelGGL(fdp::read_rows_kernel<false>, dim3((uint32_t)wgs), dim3(64 * fdp::kRowWaves), 0, hs, pa,
                           pb, rows, row_bytes, block_bytes, chunk_rows, sink);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FD_ERR_HIP, "probe_read_rows launch: %s", hipGetErrorString(e));
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
