// mmvq_tq2.hip -- TQ2_0 weights on gfx950: packing, and the product with
// Q8_1 activations.
//
// TQ2_0 is the second ternary type named by "CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract", "Upstream state"; the
// layout this library reads (2-bit digit fields, 66-byte blocks) is stated in
// include/bqm.h and tq2_decode.hpp. The product definition and the Q8_1
// activations are those of TQ1_0, and so is the design: each lane owns whole
// 256-element blocks and spends every packed byte it loads on all four of its
// fields ("Upstream state": one load per packed byte, every digit expanded in
// place), with the activations staged in LDS once per workgroup.
//
// Dispatch: the staged kernel below for one and two columns (the field
// extraction is one mask per field, so a lane's arithmetic stays under its
// share of the HBM time); from three columns the matrix-core kernels, which
// take the format as a policy (Tq2Tile): the register-operand kernel for rows
// of 5 to 16 blocks, else the LDS-resident one where the columns fit, else the
// streamed one (14336 x 4096: staged 9.7, 10.9, 20.7, 24.3 us at 3, 4, 6, 8
// columns, the register-operand kernel 10.0 to 10.1 us at each).
#include "mmvq_staged.hpp"
#include "tq2_decode.hpp"

namespace bqm {

// ---------------------------------------------------------------------------
// Packing: one thread per output byte. Byte p < 64 of block g holds the
// digits trit + 1 of elements 128 (p / 32) + 32 f + p % 32 in fields f = 0..3;
// bytes 64, 65 copy the fp16 scale, little endian.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void tq2_pack_kernel(const int8_t *__restrict__ trits,
                                                       const uint16_t *__restrict__ d,
                                                       uint8_t *__restrict__ w,
                                                       int64_t total_bytes)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_bytes)
        return;
    const int64_t g = i / kTq2BlockBytes;            // global block index n * nb + B
    const int p = (int)(i - g * kTq2BlockBytes);      // byte within the block
    uint32_t out;
    if (p < 64) {
        const int8_t *e = trits + g * kTq1BlockElems + 128 * (p >> 5) + (p & 31);
        out = 0;
#pragma unroll
        for (int f = 0; f < 4; f++)
            out |= (uint32_t)(e[32 * f] + 1) << (2 * f);
    } else {
        const uint32_t h = d[g];
        out = p == 64 ? (h & 0xffu) : (h >> 8);
    }
    w[i] = (uint8_t)out;
}

int launch_tq2_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
                    hipStream_t stream)
{
    const int64_t total = N * (K / kTq1BlockElems) * kTq2BlockBytes;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(tq2_pack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, trits, d,
                       static_cast<uint8_t *>(w), total);
    return check_launch();
}

// ---------------------------------------------------------------------------
// Staged product.
// ---------------------------------------------------------------------------

constexpr int kTq2StagedMaxCols = 2;

// Exact sub-block sums of one block against TC staged columns (column t at
// ab0 + t * col_stride, in mmvq_staged.hpp's layout: dword j of sub-blocks
// 4h .. 4h + 3 at [8j + 4h], -sum q of sub-block b at [72 + b]); columns at or
// past T are skipped. qs dword 8h + j meets dword j of sub-blocks 4h + f, one
// field each; the four scaled fields are formed once and serve every column.
template <int TC>
__device__ __forceinline__ void tq2_sums_staged(const RawBlock2 &raw,
                                                const uint32_t *__restrict__ ab0, int col_stride,
                                                int T, int (&isum)[TC][8])
{
    int acc[TC][8];
#pragma unroll
    for (int t = 0; t < TC; t++)
#pragma unroll
        for (int b = 0; b < 8; b++)
            acc[t][b] = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t w = raw2_dword(raw, 8 * h + j);
            uint32_t f[4];
#pragma unroll
            for (int k = 0; k < 4; k++)
                f[k] = tq2_field_scaled(w, k);
#pragma unroll
            for (int t = 0; t < TC; t++) {
                if (TC == 1 || t < T) {
                    const uint4 q =
                        *reinterpret_cast<const uint4 *>(ab0 + t * col_stride + 8 * j + 4 * h);
                    acc[t][4 * h] = sdot4(f[0], q.x, acc[t][4 * h]);
                    acc[t][4 * h + 1] = sdot4(f[1], q.y, acc[t][4 * h + 1]);
                    acc[t][4 * h + 2] = sdot4(f[2], q.z, acc[t][4 * h + 2]);
                    acc[t][4 * h + 3] = sdot4(f[3], q.w, acc[t][4 * h + 3]);
                }
            }
        }
    }
    // sum(u q) = acc / 4^f exactly (an arithmetic shift of an exact
    // multiple), and the trit sum is sum(u q) - sum(q)
#pragma unroll
    for (int t = 0; t < TC; t++)
#pragma unroll
        for (int b = 0; b < 8; b++)
            isum[t][b] = (acc[t][b] >> tq2_field_shift(b & 3)) +
                         (int)ab0[t * col_stride + 72 + b];
}

// Thread mapping as in the TQ1_0 staged kernel: Lr = 1 << lr_log2 lanes per
// output row, lane i of a row takes blocks i, i + Lr, ... of each chunk of
// `chunk` blocks, whose T activation columns the workgroup stages first.
template <int TC, bool ISUMS, int WPG>
__global__ __launch_bounds__(64 * WPG) void mmvq_tq2_staged_kernel(
    const uint8_t *__restrict__ w, const uint8_t *__restrict__ a, float *y, const float *resid,
    int32_t *__restrict__ isums, int64_t N, int nb, int T, int lr_log2, int chunk)
{
    extern __shared__ uint4 act_lds[];
    uint32_t *act = reinterpret_cast<uint32_t *>(act_lds);
    constexpr int nthreads = 64 * WPG;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t row = ((int64_t)blockIdx.x * WPG + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    const bool row_ok = row < N;
    const int Lr = 1 << lr_log2, sub = lane & (Lr - 1);
    const int nblk = nb * 8;
    const uint32_t col_bytes = (uint32_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq2BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    const uint32_t row_off = (uint32_t)((row_ok ? row : 0) * nb * kTq2BlockBytes);
    float acc[TC];
#pragma unroll
    for (int t = 0; t < TC; t++)
        acc[t] = 0.0f;

    for (int B0 = 0; B0 < nb; B0 += chunk) {
        const int end = min(B0 + chunk, nb);
        const int cb = end - B0;
        const int first = B0 + sub;
        if (B0 > 0)
            __syncthreads();  // readers of the previous chunk are done
        // the first column's first staging batch, then this lane's first
        // weight block (every lane issues it, at kTq2IdleOffset without a
        // block), so that the weights' HBM latency overlaps the staging and the
        // staging waits for its own batch only; the fences keep the compiler
        // from reordering the two
        StageBatch<false> head;
        stage_load<false>(head, ra, 0u, B0, cb, 0, tid, nthreads);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        RawBlock2 cur = load_raw_block2(rw, row_ok && first < end
                                                ? row_off + (uint32_t)first * kTq2BlockBytes
                                                : kTq2IdleOffset);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_sched_barrier(0);
        stage_column<false>(act, ra, 0u, B0, cb, tid, nthreads, &head);
#pragma unroll
        for (int t = 1; t < TC; t++)
            if (t < T)
                stage_column<false>(act + t * cb * kActStride, ra, (uint32_t)t * col_bytes, B0, cb,
                                    tid, nthreads, nullptr);
        __syncthreads();
        if (row_ok) {
            for (int B = first; B < end; B += Lr) {
                if (B != first)
                    cur = load_raw_block2(rw, row_off + (uint32_t)B * kTq2BlockBytes);
                const uint32_t *ab = act + (B - B0) * kActStride;
                int isum[TC][8];
                tq2_sums_staged<TC>(cur, ab, cb * kActStride, T, isum);
                const float dw = f16_bits_to_f32(raw2_scale_bits(cur));
#pragma unroll
                for (int t = 0; t < TC; t++) {
                    if (t < T) {
                        if (ISUMS) {
                            int32_t *dst = isums + ((int64_t)t * N + row) * nblk + 8 * B;
#pragma unroll
                            for (int b = 0; b < 8; b++)
                                dst[b] = isum[t][b];
                        } else {
                            // the library's fixed fp32 order (block_dot_f32)
                            float da[8];
#pragma unroll
                            for (int b = 0; b < 8; b++)
                                da[b] = __uint_as_float(ab[t * cb * kActStride + 64 + b]);
                            acc[t] = fmaf(dw, block_dot_f32(isum[t], da), acc[t]);
                        }
                    }
                }
            }
        }
    }
    if (!ISUMS) {
        // butterfly over the Lr lanes of the row (every lane of the wave takes part)
#pragma unroll
        for (int t = 0; t < TC; t++)
            acc[t] = row_sum(acc[t], lr_log2);
        if (row_ok && sub == 0) {
#pragma unroll
            for (int t = 0; t < TC; t++) {
                if (t < T) {
                    const int64_t oi = (int64_t)t * N + row;
                    y[oi] = resid ? acc[t] + resid[oi] : acc[t];
                }
            }
        }
    }
}

template <int TC, int WPG>
static void launch_tq2_staged_tc(const uint8_t *w, const uint8_t *a, float *y, int32_t *isums,
                                 int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                                 hipStream_t stream)
{
    const int64_t rows_per_wg = WPG * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(64 * WPG);
    if (isums) {
        allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_tq2_staged_kernel<TC, true, WPG>),
                          lds);
        hipLaunchKernelGGL((mmvq_tq2_staged_kernel<TC, true, WPG>), grid, block, lds, stream, w,
                           a, nullptr, nullptr, isums, N, nb, T, lr, chunk);
    } else {
        allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_tq2_staged_kernel<TC, false, WPG>),
                          lds);
        hipLaunchKernelGGL((mmvq_tq2_staged_kernel<TC, false, WPG>), grid, block, lds, stream, w,
                           a, y, nullptr, nullptr, N, nb, T, lr, chunk);
    }
}

template <int TC>
static void launch_tq2_staged_w(const uint8_t *w, const uint8_t *a, float *y, int32_t *isums,
                                int64_t N, int nb, int T, int lr, int chunk, size_t lds,
                                hipStream_t stream)
{
    const int wpg = staged_workgroup_waves(N, lr);
    if (wpg == 1)
        launch_tq2_staged_tc<TC, 1>(w, a, y, isums, N, nb, T, lr, chunk, lds, stream);
    else if (wpg == 8)
        launch_tq2_staged_tc<TC, 8>(w, a, y, isums, N, nb, T, lr, chunk, lds, stream);
    else
        launch_tq2_staged_tc<TC, 4>(w, a, y, isums, N, nb, T, lr, chunk, lds, stream);
}

int launch_mmvq_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N, int64_t K,
                    int32_t T, hipStream_t stream)
{
    if (T > kTq2StagedMaxCols) {
        if (mfma_reg_supported(K, T))
            return launch_mmvq_mfma_reg_tq2(w, a, y, isums, N, K, T, stream);
        if (mfma_resident_supported(K, T))
            return launch_mmvq_mfma_resident_tq2(w, a, y, isums, N, K, T, stream);
        return launch_mmvq_mfma_tq2(w, a, y, isums, N, K, T, stream);
    }
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    // two columns of 64 blocks take 43,008 bytes: always within the budget
    const int chunk = staged_chunk(nb, lr, T, lds_budget());
    if (chunk == 0)
        return BQM_ERR_SHAPE;
    const size_t lds = (size_t)T * chunk * kActStride * 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (T == 1)
        launch_tq2_staged_w<1>(wp, ap, y, isums, N, nb, T, lr, chunk, lds, stream);
    else
        launch_tq2_staged_w<2>(wp, ap, y, isums, N, nb, T, lr, chunk, lds, stream);
    return check_launch();
}

}  // namespace bqm
