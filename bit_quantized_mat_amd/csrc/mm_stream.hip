// mm_stream.hip -- TQ1_0 x Q8_1 product for many activation columns (prefill
// batches, T well beyond 32) on gfx950, matrix cores, K streamed block by
// block.
//
// The many-column product is the contraction the matrix cores are for: per
// 32-element Q8_1 sub-block, a 16-row tile of weight digits times 16
// activation columns is one v_mfma_i32_16x16x32_i8 whose int32 results are
// the exact sub-block sums (operand layouts and the digit decode:
// mfma_common.hpp). A workgroup owns 64 rows (one 16-row tile per wave) and
// 16 NCT columns. It walks K one 256-element block at a time: the block's
// activations for its columns are copied into LDS in the B-operand layout,
// each wave decodes its rows' block once, and the decoded operands meet all
// NCT column tiles. The weights are read once per column group; the
// activations once per row group, from L2.
//
// fp32 order: per block and column, s = d_a[0] isum[0], then fma over the
// sub-blocks as everywhere in this library, then acc + d_w s over the blocks in
// order, with the running sum folded into an outer sum every kFoldBlocks
// blocks. The error stays within about (kFoldBlocks + 9 + nb / kFoldBlocks)
// units of fp32 rounding of the sum of |terms|; the order differs from the
// single-column product's lane-group tree, so results agree with it within
// that bound, not bit for bit.
#include "mfma_common.hpp"

namespace bqm {

constexpr int kMmCols = 4;         // 16-column tiles per workgroup (64 columns)
constexpr int kMmAhead = 2;        // staging tasks per thread per block
constexpr int kFoldBlocks = 64;

// LDS per block, in dwords: bq [ct][b][lane] x 2, then the fp16 sub-block
// scales of each column, [c] x 4 dwords; two of each, for consecutive blocks.
constexpr int kMmBqDwords = kMmCols * 8 * 128;
constexpr int kMmDahDwords = kMmCols * 16 * 4;

// One 64-row group of a workgroup against its columns c0 .. c0 + 16 kMmCols - 1.
__device__ __forceinline__ void row_group(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ra,
                                          float *__restrict__ y, int64_t N, int nb, int T, int c0,
                                          int64_t rgroup, uint32_t *bq, uint32_t *dah)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int kg = lane >> 4;                   // decode lane: row lane % 16, K group kg
    const QhLaneMuls qm = qh_lane_muls(kg);
    const int col = lane & 15, rg = lane >> 4;  // output lane: column col, rows 4rg..4rg+3
    const int nblk = nb * 8;
    const uint32_t col_bytes = (uint32_t)nblk * kQ81BlockBytes;
    // this decode lane's row (rows past N read row 0 and store nothing)
    const int64_t rowA = ((int64_t)rgroup * 4 + wave) * 16 + (lane & 15);
    const uint32_t row_off = (uint32_t)((rowA < N ? rowA : 0) * nb * kTq1BlockBytes);

    float acc[kMmCols][4], outer[kMmCols][4];
#pragma unroll
    for (int ct = 0; ct < kMmCols; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[ct][i] = 0.0f;
            outer[ct][i] = 0.0f;
        }

    // block B's activations for this workgroup's columns: task i = column
    // (i >> 3), sub-block (i & 7); columns past T load at the idle offset
    // (zeros) and stage zeros
    u32x4 v0[kMmAhead], v1[kMmAhead];
    uint32_t ds[kMmAhead];
    // (B = nb: every lane loads at the idle offset, so that the loads are
    // issued unconditionally and the compiler can count them)
    auto issue_stage = [&](int B) {
#pragma unroll
        for (int k = 0; k < kMmAhead; k++) {
            const int i = k * 256 + tid;
            const int c = c0 + (i >> 3), b = i & 7;
            const uint32_t off = c < T && B < nb ? (uint32_t)c * col_bytes +
                                                       (uint32_t)(8 * B + b) * kQ81BlockBytes
                                                 : kIdleLoadOffset;
            v0[k] = ld_b128(ra, off);
            v1[k] = ld_b128(ra, off + 16);
            ds[k] = ld_b32(ra, off + 32);
        }
    };
    // the loads of block B + 1 (activations, then weights) are in flight
    // while block B is multiplied
    issue_stage(0);
    LaneBlock lb = load_lane_block(rw, row_off, kg);
    for (int B = 0; B < nb; B++) {
        const LaneBlock ln = load_lane_block(
            rw, B + 1 < nb ? row_off + (uint32_t)(B + 1) * kTq1BlockBytes : kIdleLoadOffset, kg);
        // block B's copy goes to buffer B & 1: the other buffer may still be
        // read for block B - 1, and every wave finished block B - 2's reads of
        // this one before the previous barrier
        uint32_t *const bqB = bq + (B & 1) * kMmBqDwords;
        uint32_t *const dahB = dah + (B & 1) * kMmDahDwords;
#pragma unroll
        for (int k = 0; k < kMmAhead; k++) {
            const int i = k * 256 + tid;
            const int c = i >> 3, b = i & 7;
            const uint32_t q[8] = {v0[k].x, v0[k].y, v0[k].z, v0[k].w,
                                   v1[k].x, v1[k].y, v1[k].z, v1[k].w};
            const int ct = c >> 4, cc = c & 15;
            uint32_t *dst = bqB + (ct * 8 + b) * 128;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const uint32_t lo = b < 5 ? q[2 * g] : q[g];
                const uint32_t hi = b < 5 ? q[2 * g + 1] : q[4 + g];
                *reinterpret_cast<u32x2 *>(dst + 2 * (16 * g + cc)) = (u32x2){lo, hi};
            }
            reinterpret_cast<uint16_t *>(dahB + c * 4)[b] = (uint16_t)ds[k];
        }
        issue_stage(B + 1);
        __syncthreads();  // block B's copy is complete

        const TileOperands op = decode_lane_block(lb, qm);
        float dw[4];  // block scales of the four rows this output lane holds
#pragma unroll
        for (int i = 0; i < 4; i++)
            dw[i] = __shfl(op.dw, 4 * rg + i, 64);
        // the products of (column tile, sub-block) j + 1 are issued before
        // the fp32 work on those of j, and the B operand of j + 2 is read
        // from LDS meanwhile, so neither waits on the one just issued
        auto bq_at = [&](int j) -> long {
            const u32x2 bv = *reinterpret_cast<const u32x2 *>(bqB + (j >> 3) * 8 * 128 + 2 * lane +
                                                             (j & 7) * 128);
            return (long)(((uint64_t)bv.y << 32) | bv.x);
        };
        auto product = [&](int j, long Bq) -> i32x4 {
            const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x32_i8(kAllMinusOne, Bq,
                                                                        (i32x4){0, 0, 0, 0}, 0, 0, 0);
            return __builtin_amdgcn_mfma_i32_16x16x32_i8(op.A[j & 7], Bq, neg_sum, 0, 0, 0);
        };
        constexpr int kJ = 8 * kMmCols;
        long Bn = bq_at(1);
        i32x4 Cn = product(0, bq_at(0));
        u32x4 dv;
        float s[4];
#pragma unroll
        for (int j = 0; j < kJ; j++) {
            const int ct = j >> 3, b = j & 7;
            const i32x4 C = Cn;
            if (j + 1 < kJ) {
                Cn = product(j + 1, Bn);
                if (j + 2 < kJ)
                    Bn = bq_at(j + 2);
            }
            if (b == 0)
                dv = *reinterpret_cast<const u32x4 *>(dahB + (ct * 16 + col) * 4);
            __builtin_amdgcn_sched_barrier(0);
            const float da = f16_bits_to_f32(dv[b >> 1] >> (16 * (b & 1)));
#pragma unroll
            for (int i = 0; i < 4; i++)
                s[i] = b == 0 ? da * (float)C[i] : fmaf(da, (float)C[i], s[i]);
            if (b == 7) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[ct][i] = fmaf(dw[i], s[i], acc[ct][i]);
            }
        }
        if ((B + 1) % kFoldBlocks == 0) {
#pragma unroll
            for (int ct = 0; ct < kMmCols; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    outer[ct][i] += acc[ct][i];
                    acc[ct][i] = 0.0f;
                }
        }
        lb = ln;
    }
    const int64_t r0 = ((int64_t)rgroup * 4 + wave) * 16 + 4 * rg;
#pragma unroll
    for (int ct = 0; ct < kMmCols; ct++) {
        const int c = c0 + ct * 16 + col;
        if (c < T) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (r0 + i < N)
                    y[(int64_t)c * N + r0 + i] = outer[ct][i] + acc[ct][i];
        }
    }
}

// grid.x: column groups of 16 kMmCols columns; grid.y and grid.z: 64-row
// groups, row group blockIdx.z gridDim.y + blockIdx.y (grid.y stays within
// 65535; the few workgroups past the last row group exit at once).
// Workgroups of one row group are adjacent in dispatch order, so the L2
// serves the row group's weights to its column groups from one HBM read.
// The register budget is that of three waves per SIMD: under the 128
// registers of four, the compiler would funnel every matrix-core product
// through one or two accumulator quads and serialize them. With the products
// issued one (column tile, sub-block) ahead of their fp32 work the kernel
// needs 126, so four waves still fit.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void mm_stream_kernel(
    const uint8_t *__restrict__ w, const uint8_t *__restrict__ a, float *__restrict__ y, int64_t N,
    int nb, int T, int64_t nrowgroups)
{
    __shared__ uint32_t bq[2 * kMmBqDwords];  // two buffers: blocks B and B + 1
    __shared__ uint32_t dah[2 * kMmDahDwords];
    const int64_t rgroup = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    if (rgroup >= nrowgroups)
        return;
    const uint32_t col_bytes = (uint32_t)nb * 8 * kQ81BlockBytes;
    const int c0 = (int)blockIdx.x * 16 * kMmCols;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    row_group(rw, ra, y, N, nb, T, c0, rgroup, bq, dah);
}

int64_t mm_stream_workgroups(int64_t N, int64_t T)
{
    return (N + 63) / 64 * ((T + 16 * kMmCols - 1) / (16 * kMmCols));
}

int launch_mm_stream(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
                     hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int64_t nrowgroups = (N + 63) / 64;
    const int64_t ncolgroups = (T + 16 * kMmCols - 1) / (16 * kMmCols);
    const int64_t gy = nrowgroups < 65535 ? nrowgroups : 65535;
    const dim3 grid((unsigned)ncolgroups, (unsigned)gy, (unsigned)((nrowgroups + gy - 1) / gy));
    hipLaunchKernelGGL(mm_stream_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(a), y, N,
                       nb, (int)T, nrowgroups);
    return check_launch();
}

}  // namespace bqm
