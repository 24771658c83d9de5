// mmvq_staged.hip -- TQ1_0 x Q8_1 mat-vec for one to eight activation columns
// (the decode and small-batch shapes) on gfx950.
//
// Dedicated kernel that consumes whole 256-element blocks and walks packed
// bytes rather than elements ("CUDA: TQ1_0 mat-vec is load-bound by the
// per-32-element chunk contract", "Proposed approach", option 1): every packed
// byte is loaded from HBM once and all of its digits are expanded in registers
// (tq1_decode.hpp).
//
// Thread mapping: Lr lanes share an output row (Lr = the largest power of two
// dividing the row's block count, at most 64); lane i of the row takes blocks
// i, i+Lr, ... Consecutive lanes therefore read consecutive 54-byte blocks,
// and a wave's weight loads cover one contiguous stretch of rows.
//
// Activations: the workgroup copies the Q8_1 column into LDS once per chunk of
// up to 128 blocks, transposed so that dword j of all eight sub-blocks of a
// 256-element block sits together, and precomputes each sub-block's fp32
// scale and -sum(q). Every row of the workgroup reuses the staged copy.
#include "mmvq_staged.hpp"

namespace bqm {

// Plain product: T columns of a [T][K/32] activation matrix, y [T][N].
template <int TC, bool ISUMS>
__global__ __launch_bounds__(256) void mmvq_staged_kernel(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ a,
                                                          float *__restrict__ y,
                                                          int32_t *__restrict__ isums, int64_t N,
                                                          int nb, int T, int lr_log2, int chunk)
{
    extern __shared__ uint4 act_lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    const int nblk = nb * 8;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * nblk * kQ81BlockBytes);
    uint32_t col_off[TC];
    float *out[TC];
#pragma unroll
    for (int t = 0; t < TC; t++) {
        col_off[t] = (uint32_t)t * nblk * kQ81BlockBytes;
        out[t] = ISUMS ? nullptr : y + (int64_t)t * N;
    }
    staged_rows<TC, ISUMS>(rw, ra, col_off, out, isums, reinterpret_cast<uint32_t *>(act_lds),
                           row, row < N, N, nb, T, lr_log2, chunk);
}

int lanes_per_row_log2(int64_t nb)
{
    // smallest power of two (<= 64) not below the row's block count; lanes
    // beyond the count stay idle and add zeros in the butterfly
    int l = 0;
    while (l < 6 && (1ll << l) < nb)
        l++;
    return l;
}

size_t lds_budget()
{
    // dynamic LDS per workgroup this device allows, cached per device
    static size_t cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return kLdsDefault;
    if (!cached[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = (int)kLdsDefault;
        cached[dev] = (size_t)v < kLdsMax ? (size_t)v : kLdsMax;
    }
    return cached[dev];
}

bool staged_supported(int64_t K, int32_t T)
{
    if (T < 1 || T > kStagedMaxCols)
        return false;
    const int nb = (int)(K / kTq1BlockElems);
    return staged_chunk(nb, lanes_per_row_log2(nb), T, lds_budget()) > 0;
}

template <int TC>
static void launch_staged_tc(const uint8_t *w, const uint8_t *a, float *y, int32_t *isums,
                             int64_t N, int nb, int T, int lr, int chunk, dim3 grid, size_t lds,
                             hipStream_t stream)
{
    allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_staged_kernel<TC, true>), lds);
    allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_staged_kernel<TC, false>), lds);
    if (isums)
        hipLaunchKernelGGL((mmvq_staged_kernel<TC, true>), grid, dim3(256), lds, stream, w, a,
                           nullptr, isums, N, nb, T, lr, chunk);
    else
        hipLaunchKernelGGL((mmvq_staged_kernel<TC, false>), grid, dim3(256), lds, stream, w, a,
                           y, nullptr, N, nb, T, lr, chunk);
}

int launch_mmvq_staged(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                       int64_t K, int32_t T, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = staged_chunk(nb, lr, T, lds_budget());
    const int64_t rows_per_wg = 4 * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
    const size_t lds = (size_t)T * chunk * kActStride * 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    // column-capacity ladder: a call pays for the next rung up, never for 8
    if (T == 1)
        launch_staged_tc<1>(wp, ap, y, isums, N, nb, T, lr, chunk, grid, lds, stream);
    else if (T == 2)
        launch_staged_tc<2>(wp, ap, y, isums, N, nb, T, lr, chunk, grid, lds, stream);
    else if (T <= 4)
        launch_staged_tc<4>(wp, ap, y, isums, N, nb, T, lr, chunk, grid, lds, stream);
    else
        launch_staged_tc<8>(wp, ap, y, isums, N, nb, T, lr, chunk, grid, lds, stream);
    return check_launch();
}

}  // namespace bqm
