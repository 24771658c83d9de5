// mmvq_t1.hip -- one-column TQ1_0 x Q8_1 mat-vec (the decode shape) on gfx950.
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
#include "launch.hpp"
#include "tq1_decode.hpp"

namespace bqm {

// Staged layout of one 256-element block of activations, in dwords:
//   [8j + c]   dword j of sub-block c's q bytes     (j, c < 8)
//   [64 + c]   fp32 scale of sub-block c
//   [72 + c]   -sum(q) of sub-block c
//   [80..83]   padding (keeps the per-block stride at 16-byte alignment and
//              spreads the blocks of a wave over distinct LDS banks)
constexpr int kActStride = 84;
constexpr int kMaxChunkBlocks = 128;

__device__ __forceinline__ void stage_activations(uint32_t *__restrict__ act,
                                                  __amdgpu_buffer_rsrc_t ra, uint32_t col_off,
                                                  int B0, int cb, int tid, int nthreads)
{
    for (int i = tid; i < cb * 8; i += nthreads) {
        const int bi = i >> 3, c = i & 7;
        const uint32_t off = col_off + (uint32_t)((B0 + bi) * 8 + c) * kQ81BlockBytes;
        const u32x4 v0 = ld_b128(ra, off);
        const u32x4 v1 = ld_b128(ra, off + 16);
        const uint32_t ds = ld_b32(ra, off + 32);
        uint32_t *dst = act + bi * kActStride;
        const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        int sq = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            dst[8 * j + c] = q[j];
            sq = sdot4(0x01010101u, q[j], sq);
        }
        dst[64 + c] = __float_as_uint(f16_bits_to_f32(ds & 0xffffu));
        dst[72 + c] = (uint32_t)(-sq);
    }
}

// Integer sums of one block (raw weights) against the staged activations.
__device__ __forceinline__ void block_sums_staged(const RawBlock &raw,
                                                  const uint32_t *__restrict__ ab, int (&isum)[8])
{
    BlockSums s;
#pragma unroll
    for (int c = 0; c < 8; c++) {
        s.P[c] = (int)ab[72 + c];
        s.N[c] = 0;
    }
    uint32_t q[8][8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint4 lo = *reinterpret_cast<const uint4 *>(ab + 8 * j);
        const uint4 hi = *reinterpret_cast<const uint4 *>(ab + 8 * j + 4);
        q[j][0] = lo.x; q[j][1] = lo.y; q[j][2] = lo.z; q[j][3] = lo.w;
        q[j][4] = hi.x; q[j][5] = hi.y; q[j][6] = hi.z; q[j][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < 8; j++)
        dot_qs_lo(raw_dword(raw, j), q[j][0], q[j][1], q[j][2], q[j][3], q[j][4], s);
#pragma unroll
    for (int i = 0; i < 4; i++)
        dot_qs_hi(raw_dword(raw, 8 + i), q[i][5], q[4 + i][5], q[i][6], q[4 + i][6], q[i][7], s);
    dot_qh(raw_dword(raw, 12), q[4][7], q[5][7], q[6][7], q[7][7], s);
    finish_isums(s, isum);
}

template <bool ISUMS>
__global__ __launch_bounds__(256) void mmvq_t1_kernel(const uint8_t *__restrict__ w,
                                                      const uint8_t *__restrict__ a,
                                                      float *__restrict__ y,
                                                      int32_t *__restrict__ isums, int64_t N,
                                                      int nb, int lr_log2, int chunk)
{
    extern __shared__ uint4 act_lds[];
    uint32_t *act = reinterpret_cast<uint32_t *>(act_lds);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Lr = 1 << lr_log2;
    const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    const int sub = lane & (Lr - 1);
    const bool row_ok = row < N;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)nb * 8 * kQ81BlockBytes);
    const uint32_t row_off = (uint32_t)((row_ok ? row : 0) * nb * kTq1BlockBytes);
    const int nblk = nb * 8;
    float acc = 0.0f;

    for (int B0 = 0; B0 < nb; B0 += chunk) {
        const int end = min(B0 + chunk, nb);
        const int first = B0 + sub;
        // issue this lane's first weight block before staging, so the HBM
        // latency overlaps the activation copy; later blocks of the chunk are
        // loaded into the same registers at the top of their iteration
        RawBlock cur;
        if (row_ok && first < end)
            cur = load_raw_block(rw, row_off + (uint32_t)first * kTq1BlockBytes);
        __syncthreads();  // readers of the previous chunk are done
        stage_activations(act, ra, 0, B0, end - B0, tid, 256);
        __syncthreads();
        if (row_ok) {
            for (int B = first; B < end; B += Lr) {
                if (B != first)
                    cur = load_raw_block(rw, row_off + (uint32_t)B * kTq1BlockBytes);
                const uint32_t *ab = act + (B - B0) * kActStride;
                int isum[8];
                block_sums_staged(cur, ab, isum);
                if (ISUMS) {
                    int32_t *dst = isums + row * nblk + 8 * B;
#pragma unroll
                    for (int b = 0; b < 8; b++)
                        dst[b] = isum[b];
                } else {
                    float da[8];
#pragma unroll
                    for (int b = 0; b < 8; b++)
                        da[b] = __uint_as_float(ab[64 + b]);
                    const float dw = f16_bits_to_f32(raw_scale_bits(cur));
                    acc = fmaf(dw, block_dot_f32(isum, da), acc);
                }
            }
        }
    }
    if (!ISUMS) {
        for (int m = Lr >> 1; m >= 1; m >>= 1)
            acc += __shfl_xor(acc, m, 64);
        if (row_ok && sub == 0)
            y[row] = acc;
    }
}

int lanes_per_row_log2(int64_t nb)
{
    // largest power of two (<= 64) that divides the row's block count
    int l = 0;
    while (l < 6 && nb % (2ll << l) == 0)
        l++;
    return l;
}

int launch_mmvq_t1(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                   int64_t K, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = nb < kMaxChunkBlocks ? nb : kMaxChunkBlocks;  // a multiple of 1 << lr
    const int64_t rows_per_wg = 4 * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
    const size_t lds = (size_t)chunk * kActStride * 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (isums)
        hipLaunchKernelGGL(mmvq_t1_kernel<true>, grid, dim3(256), lds, stream, wp, ap, nullptr,
                           isums, N, nb, lr, chunk);
    else
        hipLaunchKernelGGL(mmvq_t1_kernel<false>, grid, dim3(256), lds, stream, wp, ap, y,
                           nullptr, N, nb, lr, chunk);
    return check_launch();
}

}  // namespace bqm
