// probes.hip -- calibration kernels for the benchmark (not part of the C ABI).
//
// bqm_probe_empty: a kernel that does nothing, for the fixed cost of one
// dispatch. bqm_probe_read: streams a buffer once with 16-byte loads and
// writes one dword per workgroup, for the HBM read rate that any kernel of the
// same grid can reach on the same number of bytes. bqm_probe_copy: copies a
// buffer with 16-byte loads and stores, a transfer of known size against which
// the memory counters (bytes fetched from and written to HBM) are scaled.
// bqm_probe_valu: long chains of one vector ALU instruction kind per lane, for
// the device's vector-ALU issue rate (lane operations per second) on the
// instruction kinds the TQ1_0 decode is made of.
#include <hip/hip_runtime.h>

#include <chrono>
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

// Eight independent dependency chains per lane, four steps of each per loop
// iteration: 32 instructions of the chosen kind per iteration and wave (the
// loop counter lives in scalar registers). Kinds: 0 v_dot4_i32_i8, 1
// v_mad_u32_u24, 2 v_pk_mul_lo_u16, 3 v_perm_b32.
typedef unsigned short probe_u16x2 __attribute__((ext_vector_type(2)));

template <int KIND>
__device__ __forceinline__ uint32_t valu_step(uint32_t a, uint32_t b)
{
    if (KIND == 0)
        return (uint32_t)__builtin_amdgcn_sdot4((int)a, (int)b, (int)a, false);
    if (KIND == 1)
        return __umul24(a, 0x9e37u) + b;
    if (KIND == 2) {
        probe_u16x2 x = __builtin_bit_cast(probe_u16x2, a), y = __builtin_bit_cast(probe_u16x2, b);
        return __builtin_bit_cast(uint32_t, (probe_u16x2)(x * y));
    }
    return __builtin_amdgcn_perm(a, b, 0x07050301u);
}

template <int KIND>
__global__ __launch_bounds__(256) void valu_kernel(int iters, uint32_t seed,
                                                   uint32_t *__restrict__ out)
{
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        a[k] = seed ^ (t * 2654435761u + 97u * k);
        b[k] = seed + 0x01010101u * (k + 1) + t;
    }
    for (int i = 0; i < iters; i++) {
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int k = 0; k < 8; k++) {
                a[k] = valu_step<KIND>(a[k], b[k]);
                // an empty statement that keeps each step one instruction: the
                // compiler would otherwise merge consecutive steps algebraically
                asm volatile("" : "+v"(a[k]));
            }
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < 8; k++)
        x ^= a[k];
    out[t] = x;
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

// out: device buffer of grid * 256 dwords. Each wave issues 32 * iters
// instructions of the kind chosen (0 dot4, 1 mad_u24, 2 pk_mul_lo_u16, 3 perm).
__attribute__((visibility("default"))) int bqm_probe_valu(int kind, int iters, uint32_t *out,
                                                          int grid, void *stream)
{
    if (!out || grid < 1 || iters < 1 || kind < 0 || kind > 3)
        return -2;
    const dim3 g(grid), b(256);
    switch (kind) {
    case 0: hipLaunchKernelGGL(valu_kernel<0>, g, b, 0, (hipStream_t)stream, iters, 12345u, out); break;
    case 1: hipLaunchKernelGGL(valu_kernel<1>, g, b, 0, (hipStream_t)stream, iters, 12345u, out); break;
    case 2: hipLaunchKernelGGL(valu_kernel<2>, g, b, 0, (hipStream_t)stream, iters, 12345u, out); break;
    default: hipLaunchKernelGGL(valu_kernel<3>, g, b, 0, (hipStream_t)stream, iters, 12345u, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Eager stepping through the C ABI with no Python in the loop: `iters`
// calls of fn (the signature of mmvq_tq1_0_f32) on the weight copies
// w_base + (i mod R) * w_stride, enqueued back to back on the stream. Writes
// the host time per call spent enqueueing (enqueue_us) and the wall time per
// call until the stream drains (wall_us). Returns fn's first nonzero status.
typedef int (*bqm_f32_fn)(const void *, const float *, float *, int64_t, int64_t, int32_t,
                          void *);
__attribute__((visibility("default"))) int bqm_probe_eager(void *fn, const uint8_t *w_base,
                                                           uint64_t w_stride, int R,
                                                           const float *x, float *y, int64_t N,
                                                           int64_t K, int32_t T, int iters,
                                                           void *stream, double *enqueue_us,
                                                           double *wall_us)
{
    if (!fn || !w_base || R < 1 || iters < 1 || !enqueue_us || !wall_us)
        return -2;
    const bqm_f32_fn f = reinterpret_cast<bqm_f32_fn>(fn);
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return -5;
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < iters; i++) {
        const int rc = f(w_base + (uint64_t)(i % R) * w_stride, x, y, N, K, T, stream);
        if (rc)
            return rc;
    }
    const auto t1 = std::chrono::steady_clock::now();
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return -5;
    const auto t2 = std::chrono::steady_clock::now();
    *enqueue_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / iters;
    *wall_us = std::chrono::duration<double, std::micro>(t2 - t0).count() / iters;
    return 0;
}

}  // extern "C"
