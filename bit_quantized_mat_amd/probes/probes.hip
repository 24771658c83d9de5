// probes.hip -- calibration kernels for the benchmark (not part of the C ABI).
//
// bqm_probe_empty: a kernel that does nothing, for the fixed cost of one
// dispatch. bqm_probe_read: streams a buffer once with 16-byte loads and
// writes one dword per workgroup, for the HBM read rate that any kernel of the
// same grid can reach on the same number of bytes. bqm_probe_copy: copies a
// buffer with 16-byte loads and stores, a transfer of known size against which
// the memory counters (bytes fetched from and written to HBM) are scaled.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void empty_kernel() {}

__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ src, uint64_t n16,
                                                   uint32_t *__restrict__ out)
{
    uint32_t x = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int m = 32; m >= 1; m >>= 1)
        x ^= __shfl_xor(x, m, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src,
                                                   uint4 *__restrict__ dst, uint64_t n16)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int bqm_probe_empty(int grid, void *stream)
{
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// buf: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned);
// out: device buffer of `grid` dwords.
__attribute__((visibility("default"))) int bqm_probe_read(const void *buf, uint64_t bytes,
                                                          uint32_t *out, int grid, void *stream)
{
    if (!buf || !out || grid < 1 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0)
        return -2;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)buf, bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// src, dst: device buffers of `bytes` bytes each (a multiple of 16, 16-byte
// aligned, not overlapping).
__attribute__((visibility("default"))) int bqm_probe_copy(const void *src, void *dst,
                                                          uint64_t bytes, int grid, void *stream)
{
    if (!src || !dst || grid < 1 || bytes % 16 != 0 || (((uintptr_t)src | (uintptr_t)dst) & 15u))
        return -2;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)src, (uint4 *)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
