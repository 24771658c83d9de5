// mmvq_staged.hip -- TQ1_0 x Q8_1 mat-vec for one to eight activation columns
// (the decode and small-batch shapes) on gfx950.
//
// Dedicated kernel that consumes whole 256-element blocks and walks packed
// bytes rather than elements ("CUDA: TQ1_0 mat-vec is load-bound by the
// per-32-element chunk contract", "Proposed approach", option 1): every packed
// byte is loaded from HBM once and all of its digits are expanded in registers
// (tq1_decode.hpp).
//
// Thread mapping: Lr lanes share an output row (Lr = the smallest power of
// two, at most 64, not below the row's block count); lane i of the row takes
// blocks i, i+Lr, ... Consecutive lanes therefore read consecutive 54-byte
// blocks, and a wave's weight loads cover one contiguous stretch of rows.
//
// Activations: the workgroup copies the Q8_1 column into LDS once per chunk of
// up to 128 blocks, transposed so that dword j of all eight sub-blocks of a
// 256-element block sits together, and precomputes each sub-block's fp32
// scale and -sum(q). Every row of the workgroup reuses the staged copy.
#include <atomic>
#include <mutex>

#include "mmvq_staged.hpp"

namespace bqm {

// Plain product: T columns of a [T][K/32] Q8_1 activation matrix (F32: of
// a [T][K] fp32 matrix, quantized while staging), y [T][N].
template <int TC, bool ISUMS, bool F32, int WPG>
__global__ __launch_bounds__(64 * WPG) void mmvq_staged_kernel(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ a,
                                                          float *y, const float *resid,
                                                          int32_t *__restrict__ isums, int64_t N,
                                                          int nb, int T, int lr_log2, int chunk)
{
    extern __shared__ uint4 act_lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * WPG + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    const int nblk = nb * 8;
    const uint32_t col_bytes = F32 ? (uint32_t)nb * kTq1BlockElems * 4 : (uint32_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    uint32_t col_off[TC];
    float *out[TC];
#pragma unroll
    for (int t = 0; t < TC; t++) {
        col_off[t] = (uint32_t)t * col_bytes;
        out[t] = ISUMS ? nullptr : y + (int64_t)t * N;
    }
    staged_rows<TC, ISUMS, F32>(rw, ra, col_off, out, resid, isums,
                                reinterpret_cast<uint32_t *>(act_lds),
                                row, row < N, N, nb, T, lr_log2, chunk, 64 * WPG);
}

// Gate-up pair with the SiLU-gated epilogue: y[t][n] = silu(g) * u, where g
// and u are row n of the gate matrix wg and of the up matrix wu against
// column t, one or two columns (F32: fp32 columns, quantized while staging).
// Waves come in pairs over the same rows: the even wave of a pair runs the
// plain staged product on the gate rows and the odd one on the up rows (each
// in the plain product's fp32 order, so g and u are bitwise mmvq_tq1_0's);
// the odd wave hands its sums over through LDS, and after one barrier the
// even wave's row lanes store silu(g) * u. Both waves share the workgroup's
// staged columns.
template <int TC, bool F32, int WPG>
__global__ __launch_bounds__(64 * WPG) void mmvq_glu_kernel(const uint8_t *__restrict__ wg,
                                                       const uint8_t *__restrict__ wu,
                                                       const uint8_t *__restrict__ a, float *y,
                                                       int64_t N, int nb, int T, int lr_log2,
                                                       int chunk)
{
    static_assert(WPG % 2 == 0, "waves come in gate-up pairs");
    extern __shared__ uint4 act_lds[];
    __shared__ float up_sums[WPG / 2][TC][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int pair = wave >> 1;
    const bool up = wave & 1;
    const int64_t row =
        ((int64_t)blockIdx.x * (WPG / 2) + pair) * (64 >> lr_log2) + (lane >> lr_log2);
    const int nblk = nb * 8;
    const uint32_t col_bytes = F32 ? (uint32_t)nb * kTq1BlockElems * 4 : (uint32_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(up ? wu : wg, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    uint32_t col_off[TC];
    float *out[TC];
#pragma unroll
    for (int t = 0; t < TC; t++) {
        col_off[t] = (uint32_t)t * col_bytes;
        out[t] = nullptr;
    }
    float g[TC];
    auto store = [&](int t, float v) {
        if (up)
            up_sums[pair][t][lane >> lr_log2] = v;
        else
            g[t] = v;
    };
    staged_rows<TC, false, F32>(rw, ra, col_off, out, nullptr, nullptr,
                                reinterpret_cast<uint32_t *>(act_lds), row, row < N, N, nb, T,
                                lr_log2, chunk, 64 * WPG, store);
    __syncthreads();
    if (!up && row < N && (lane & ((1 << lr_log2) - 1)) == 0) {
#pragma unroll
        for (int t = 0; t < TC; t++)
            if (t < T)
                y[(int64_t)t * N + row] =
                    g[t] / (1.0f + expf(-g[t])) * up_sums[pair][t][lane >> lr_log2];
    }
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

// Host-side caches of this file. Each is safe to use from several host
// threads at once: the per-device attribute caches are arrays of atomics
// (a value is computed by whichever thread first asks and every thread
// computes the same value), and the occupancy cache sits behind a mutex.
size_t lds_budget()
{
    // dynamic LDS per workgroup this device allows, cached per device
    static std::atomic<size_t> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return kLdsDefault;
    size_t v = cached[dev].load(std::memory_order_relaxed);
    if (!v) {
        int a = 0;
        if (hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            a <= 0)
            a = (int)kLdsDefault;
        v = (size_t)a < kLdsMax ? (size_t)a : kLdsMax;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int compute_units()
{
    // compute units of the current device, cached per device
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (!v) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int resident_workgroups(const void *kernel, int threads, size_t lds)
{
    // workgroups of this kernel the whole device holds at once; remembered
    // for every (kernel, block size, dynamic LDS, device) asked about. The
    // library launches a fixed set of kernels at a handful of block sizes and
    // LDS sizes per kernel, so the table stays small; past kMaxEntries (never
    // reached by the launchers here) further queries are answered uncached.
    struct Entry {
        const void *kernel;
        int threads, dev;
        size_t lds;
        int count;
    };
    constexpr int kMaxEntries = 256;
    static std::mutex mu;
    static Entry cache[kMaxEntries];
    static int used;
    int dev = 0;
    (void)hipGetDevice(&dev);
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; i++) {
            const Entry &e = cache[i];
            if (e.kernel == kernel && e.threads == threads && e.lds == lds && e.dev == dev)
                return e.count;
        }
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int count = per_cu * compute_units();
    std::lock_guard<std::mutex> lock(mu);
    if (used < kMaxEntries)
        cache[used++] = Entry{kernel, threads, dev, lds, count};
    return count;
}

bool staged_supported(int64_t K, int32_t T)
{
    if (T < 1 || T > kStagedMaxCols)
        return false;
    const int nb = (int)(K / kTq1BlockElems);
    return staged_chunk(nb, lanes_per_row_log2(nb), T, lds_budget()) > 0;
}

template <int TC, bool F32, int WPG>
static void launch_staged_tc(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                             int32_t *isums,
                             int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                             hipStream_t stream)
{
    const int64_t rows_per_wg = WPG * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(64 * WPG);
    if (isums && !F32) {
        allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_staged_kernel<TC, true, false, WPG>), lds);
        hipLaunchKernelGGL((mmvq_staged_kernel<TC, true, false, WPG>), grid, block, lds, stream, w,
                           a, nullptr, nullptr, isums, N, nb, T, lr, chunk);
    } else {
        allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_staged_kernel<TC, false, F32, WPG>), lds);
        hipLaunchKernelGGL((mmvq_staged_kernel<TC, false, F32, WPG>), grid, block, lds, stream, w,
                           a, y, r, nullptr, N, nb, T, lr, chunk);
    }
}

// Waves per workgroup: eight unless that puts more waves on the busiest SIMD
// than four do (rounds of workgroups per compute unit times waves per
// workgroup); eight halve the staging per row.
static int staged_waves(int64_t N, int lr)
{
    const int64_t cu = compute_units(), rows4 = 4 * (64 >> lr);
    const int64_t r4 = ((N + rows4 - 1) / rows4 + cu - 1) / cu;
    const int64_t r8 = ((N + 2 * rows4 - 1) / (2 * rows4) + cu - 1) / cu;
    return 2 * r8 <= r4 ? 8 : 4;
}

int staged_workgroup_waves(int64_t N, int lr)
{
    // a grid whose one-wave workgroups all fit one per compute unit takes
    // them, spreading its few waves over the device (256 x 1024: 2.56 ->
    // 2.47 us, fused 2.99 -> 2.88 us)
    const int64_t rows4 = 4 * (64 >> lr);
    if ((N + rows4 - 1) / rows4 * 4 <= compute_units())
        return 1;
    return staged_waves(N, lr);
}

template <int TC, bool F32>
static void launch_staged_w(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                            int32_t *isums,
                            int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                            hipStream_t stream)
{
    const int wpg = staged_workgroup_waves(N, lr);
    if (wpg == 1)
        launch_staged_tc<TC, F32, 1>(w, a, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    else if (wpg == 8)
        launch_staged_tc<TC, F32, 8>(w, a, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    else
        launch_staged_tc<TC, F32, 4>(w, a, y, r, isums, N, nb, T, lr, chunk, lds, stream);
}

template <bool F32>
static int launch_staged(const void *w, const void *a, float *y, const float *r,
                         int32_t *isums, int64_t N, int64_t K, int32_t T, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = staged_chunk(nb, lr, T, lds_budget());
    const size_t lds = (size_t)T * chunk * kActStride * 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    // column-capacity ladder: a call pays for the next rung up, never for 8
    if (T == 1)
        launch_staged_w<1, F32>(wp, ap, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    else if (T == 2)
        launch_staged_w<2, F32>(wp, ap, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    else if (T <= 4)
        launch_staged_w<4, F32>(wp, ap, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    else
        launch_staged_w<8, F32>(wp, ap, y, r, isums, N, nb, T, lr, chunk, lds, stream);
    return check_launch();
}

int launch_mmvq_staged(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                       int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_staged<false>(w, a, y, r, isums, N, K, T, stream);
}

int launch_mmvq_staged_f32(const void *w, const float *x, float *y, int64_t N, int64_t K,
                           int32_t T, hipStream_t stream, const float *r)
{
    return launch_staged<true>(w, x, y, r, nullptr, N, K, T, stream);
}

template <int TC, bool F32, int WPG>
static void launch_glu_tc(const uint8_t *wg, const uint8_t *wu, const uint8_t *a, float *y,
                          int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                          hipStream_t stream)
{
    const int64_t rows_per_wg = WPG / 2 * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(64 * WPG);
    allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_glu_kernel<TC, F32, WPG>), lds);
    hipLaunchKernelGGL((mmvq_glu_kernel<TC, F32, WPG>), grid, block, lds, stream, wg, wu, a, y, N,
                       nb, T, lr, chunk);
}

template <int TC, bool F32>
static void launch_glu_w(const uint8_t *wg, const uint8_t *wu, const uint8_t *a, float *y,
                         int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                         hipStream_t stream)
{
    // the workgroup shapes of the plain kernel on the 2N rows of both
    // matrices, with pairs of waves in place of single ones
    const int wpg = staged_workgroup_waves(2 * N, lr);
    if (wpg == 1)
        launch_glu_tc<TC, F32, 2>(wg, wu, a, y, N, nb, T, lr, chunk, lds, stream);
    else if (wpg == 8)
        launch_glu_tc<TC, F32, 8>(wg, wu, a, y, N, nb, T, lr, chunk, lds, stream);
    else
        launch_glu_tc<TC, F32, 4>(wg, wu, a, y, N, nb, T, lr, chunk, lds, stream);
}

int launch_mmvq_glu(const void *wg, const void *wu, const void *a, float *y, int64_t N, int64_t K,
                    int32_t T, bool f32, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = staged_chunk(nb, lr, T, lds_budget());
    if (T < 1 || T > kGluMaxCols || chunk == 0)
        return BQM_ERR_SHAPE;
    const size_t lds = (size_t)T * chunk * kActStride * 4;
    const uint8_t *g = static_cast<const uint8_t *>(wg), *u = static_cast<const uint8_t *>(wu);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (T == 1 && f32)
        launch_glu_w<1, true>(g, u, ap, y, N, nb, T, lr, chunk, lds, stream);
    else if (T == 1)
        launch_glu_w<1, false>(g, u, ap, y, N, nb, T, lr, chunk, lds, stream);
    else if (f32)
        launch_glu_w<2, true>(g, u, ap, y, N, nb, T, lr, chunk, lds, stream);
    else
        launch_glu_w<2, false>(g, u, ap, y, N, nb, T, lr, chunk, lds, stream);
    return check_launch();
}

}  // namespace bqm
