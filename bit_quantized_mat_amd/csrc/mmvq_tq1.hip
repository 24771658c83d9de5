// mmvq_tq1.hip -- dispatch of the plain product, and the ungrouped
// expert-routed kernel (one (token, slot) pair per workgroup row), used when
// the grouped kernel's staged activations do not fit its LDS budget.
//
// The ungrouped kernel is byte-major ("CUDA: TQ1_0 mat-vec is load-bound by
// the per-32-element chunk contract", "Upstream state" and "Proposed
// approach"): each thread owns whole 256-element blocks, loads every packed
// byte of a block once, expands all of its base-3 digits in registers, and
// spends each digit against the matching Q8_1 activation bytes. Digit
// u = trit + 1 is in {0,1,2}, so the integer dot uses the unsigned digits and
// subtracts the activation block's sum of q once: sum(t*q) = sum(u*q) - sum(q).
//
// Thread mapping: Lr lanes (a power of two, at most 64) share one output row;
// lane i of a row takes blocks i, i+Lr, ... of that row. A wave thus covers a
// contiguous run of 64 packed blocks per step, so its loads are coalesced.
#include "launch.hpp"
#include "tq1_decode.hpp"

namespace bqm {

// Digits of the four bytes of w, one byte per digit slot:
// out[c] holds digit c of byte k in its byte k.
template <int NDIG>
__device__ __forceinline__ void digits4(uint32_t w, uint32_t (&out)[NDIG])
{
    uint32_t b0 = w & 0xffu, b1 = (w >> 8) & 0xffu, b2 = (w >> 16) & 0xffu, b3 = w >> 24;
#pragma unroll
    for (int c = 0; c < NDIG; c++) {
        const uint32_t q0 = b0 / 3u, q1 = b1 / 3u, q2 = b2 / 3u, q3 = b3 / 3u;
        out[c] = (b0 - 3u * q0) | ((b1 - 3u * q1) << 8) | ((b2 - 3u * q2) << 16) |
                 ((b3 - 3u * q3) << 24);
        b0 = q0;
        b1 = q1;
        b2 = q2;
        b3 = q3;
    }
}

// A decoded TQ1_0 block: U[c][j] = digit c of qs dword j (j < 12);
// H[c] = digit c of the qh dword; dw = fp32 scale.
struct DecodedBlock {
    uint32_t U[5][12];
    uint32_t H[4];
    float dw;
};

// Load the 54-byte block starting at byte offset off (even) and decode it.
// Odd blocks of a row start 2 bytes past a dword boundary: the 14 aligned
// dwords covering the block are realigned with alignbyte.
__device__ __forceinline__ void load_decode_block(__amdgpu_buffer_rsrc_t rw, uint32_t off,
                                                  DecodedBlock &blk)
{
    const uint32_t base = off & ~3u;
    const uint32_t sh = off & 3u;
    uint32_t r[14];
#pragma unroll
    for (int i = 0; i < 12; i += 4) {
        u32x4 v = ld_b128(rw, base + 4 * i);
        r[i] = v.x;
        r[i + 1] = v.y;
        r[i + 2] = v.z;
        r[i + 3] = v.w;
    }
    u32x2 t = ld_b64(rw, base + 48);
    r[12] = t.x;
    r[13] = t.y;
    uint32_t qs[12], qh, dh;
#pragma unroll
    for (int i = 0; i < 12; i++)
        qs[i] = align_bytes(r[i + 1], r[i], sh);
    qh = align_bytes(r[13], r[12], sh);
    dh = sh ? (r[13] >> 16) : (r[13] & 0xffffu);
#pragma unroll
    for (int j = 0; j < 12; j++) {
        uint32_t u[5];
        digits4<5>(qs[j], u);
#pragma unroll
        for (int c = 0; c < 5; c++)
            blk.U[c][j] = u[c];
    }
    digits4<4>(qh, blk.H);
    blk.dw = f16_bits_to_f32(dh);
}

// Exact per-32 sums of one decoded block against activation column t:
// isum[b] for the 8 Q8_1 sub-blocks, and the fp32 scales d_a[b].
// Activation block (column t, sub-block j) starts at byte (t*nblk + j)*36.
__device__ __forceinline__ void block_isums(const DecodedBlock &blk, __amdgpu_buffer_rsrc_t ra,
                                            uint32_t aoff, int (&isum)[8], float (&da)[8])
{
#pragma unroll
    for (int b = 0; b < 8; b++) {
        uint32_t q[9];
        const uint32_t o = aoff + b * kQ81BlockBytes;
        u32x4 v0 = ld_b128(ra, o);
        u32x4 v1 = ld_b128(ra, o + 16);
        q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
        q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
        q[8] = ld_b32(ra, o + 32);
        int s = 0, sq = 0;
#pragma unroll
        for (int j = 0; j < 8; j++)
            sq = sdot4(0x01010101u, q[j], sq);
        if (b < 5) {
            // sub-blocks 0..4: digit b of qs[0..31]
#pragma unroll
            for (int j = 0; j < 8; j++)
                s = sdot4(blk.U[b][j], q[j], s);
        } else if (b < 7) {
            // sub-block 5: digits 0, 1 of qs[32..47]; sub-block 6: digits 2, 3
            const int c0 = 2 * (b - 5);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                s = sdot4(blk.U[c0][8 + j], q[j], s);
                s = sdot4(blk.U[c0 + 1][8 + j], q[4 + j], s);
            }
        } else {
            // sub-block 7: digit 4 of qs[32..47], then digits 0..3 of qh
#pragma unroll
            for (int j = 0; j < 4; j++) {
                s = sdot4(blk.U[4][8 + j], q[j], s);
                s = sdot4(blk.H[j], q[4 + j], s);
            }
        }
        isum[b] = s - sq;
        da[b] = f16_bits_to_f32(q[8] & 0xffffu);
    }
}

// Work description for one output row group: where the weight rows start,
// which activation columns, and where the outputs go.
template <int TC, bool ISUMS>
__device__ __forceinline__ void rows_product(const uint8_t *__restrict__ w, uint64_t w_bytes,
                                             const uint8_t *__restrict__ a, uint64_t a_bytes,
                                             int64_t row, bool row_ok, int nb, int sub, int Lr,
                                             int T, int tcol0, float *__restrict__ y,
                                             int64_t y_col_stride, int32_t *__restrict__ isums,
                                             int64_t N)
{
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, w_bytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, a_bytes);
    const int nblk = nb * 8;
    float acc[TC];
#pragma unroll
    for (int t = 0; t < TC; t++)
        acc[t] = 0.0f;
    if (row_ok) {
        for (int B = sub; B < nb; B += Lr) {
            DecodedBlock blk;
            load_decode_block(rw, (uint32_t)((row * nb + B) * kTq1BlockBytes), blk);
#pragma unroll
            for (int t = 0; t < TC; t++) {
                if (t < T) {
                    int isum[8];
                    float da[8];
                    const uint32_t aoff =
                        (uint32_t)(((int64_t)(tcol0 + t) * nblk + 8 * B) * kQ81BlockBytes);
                    block_isums(blk, ra, aoff, isum, da);
                    if (ISUMS) {
                        int32_t *dst = isums + ((int64_t)t * N + row) * nblk + 8 * B;
#pragma unroll
                        for (int b = 0; b < 8; b++)
                            dst[b] = isum[b];
                    } else {
                        acc[t] = fmaf(blk.dw, block_dot_f32(isum, da), acc[t]);
                    }
                }
            }
        }
    }
    if (!ISUMS) {
        // butterfly over the Lr lanes of the row (all lanes of the wave take part)
#pragma unroll
        for (int t = 0; t < TC; t++) {
            acc[t] = row_sum(acc[t], __builtin_ctz(Lr));  // Lr: a power of two
        }
        if (row_ok && sub == 0) {
#pragma unroll
            for (int t = 0; t < TC; t++)
                if (t < T)
                    y[t * y_col_stride + row] = acc[t];
        }
    }
}

// Whether a call of T < kMfmaMinCols columns that the quad kernel does not
// take (rows of at most 8 blocks, from three columns) goes to the staged
// kernel. From three columns on it does so only when its grid gives the
// device more than one wave per SIMD: with one block per lane and no second
// wave to overlap it, the multi-column work after the weights arrive
// outlasts the matrix-core kernel's (measured on 4096 x 4096 with the two
// kernels alone: 5.6 against 5.3 us at three columns, 6.2 against 5.5 at
// four; at 5120 x 6144 and 14336 x 4096, with more waves, the staged kernel
// is as fast or faster).
static bool use_staged(int64_t N, int64_t K, int32_t T)
{
    if (T >= kMfmaMinCols || !staged_supported(K, T))
        return false;
    if (T < 3 || !mfma_resident_supported(K, T))
        return true;
    const int64_t waves = N * (1ll << lanes_per_row_log2(K / kTq1BlockElems)) / 64;
    return waves > 4ll * compute_units();
}

// Plain product: the quad kernel for three and four columns where it takes
// the shape, the staged kernel for other narrow calls whose activations fit
// its LDS, the matrix-core kernel for everything else. The quad kernel's two
// column groups (five to eight columns) need about 210 registers, two waves
// per SIMD, and lose to the resident matrix-core kernel on Q8_1 input
// (14336 x 4096 at eight columns: 14.2 against 11.4 us); at three and four
// columns they win (8.9 against 11.6 us at four, 4096 x 4096: 5.1 against
// 5.6 us).
int launch_mmvq(const void *w, const void *a, float *y, int32_t *isums, int64_t N, int64_t K,
                int32_t T, hipStream_t stream, const float *r)
{
    if (T >= 3 && T <= 4 && quad_supported(K, T))
        return launch_mmvq_quad(w, a, y, isums, N, K, T, stream, r);
    if (use_staged(N, K, T))
        return launch_mmvq_staged(w, a, y, isums, N, K, T, stream, r);
    if (mfma_reg_supported(K, T))
        return launch_mmvq_mfma_reg(w, a, y, isums, N, K, T, stream, r);
    if (mfma_resident_supported(K, T))
        return launch_mmvq_mfma_resident(w, a, y, isums, N, K, T, stream, r);
    return launch_mmvq_mfma(w, a, y, isums, N, K, T, stream, r);
}

// Many-column product: up to BQM_MMVQ_MAX_COLS columns the plain product.
// Beyond, the K-streaming kernel (mm_stream.hip) once its grid gives the
// device at least 1.5 workgroups per compute unit: each of its workgroups
// walks all of K, so with fewer of them that walk is exposed, and the
// resident kernel over column chunks (whose columns must fit LDS) is faster
// (4096 x 4096 at 64 columns: 16.2 against 45.0 us, at 512: 69.5 against
// 56.9; 14336 x 4096 at 128 columns: 62.1 against 57.2, at 512: 223 against
// 145 us).
int launch_mm(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
              hipStream_t stream)
{
    if (T <= BQM_MMVQ_MAX_COLS)
        return launch_mmvq(w, a, y, nullptr, N, K, (int32_t)T, stream);
    // up to three chunks of 32 columns on rows of 5 to 16 blocks: one plain
    // product per chunk (on the register-operand kernel) beats one launch of
    // the column-chunked or K-streaming kernels there (14336 x 4096: 33 / 64 /
    // 80 / 96 columns 36.3 / 36.0 / 58.2 / 57.5 -> 21.7 / 31.4 / 42.1 / 46.9 us;
    // at 128 columns 57.7 -> 61.8, so not beyond 96)
    if (T <= 3 * BQM_MMVQ_MAX_COLS && mfma_reg_supported(K, BQM_MMVQ_MAX_COLS)) {
        const int64_t col_bytes = K / 32 * kQ81BlockBytes;
        for (int64_t t0 = 0; t0 < T; t0 += BQM_MMVQ_MAX_COLS) {
            const int64_t tc = T - t0 < BQM_MMVQ_MAX_COLS ? T - t0 : BQM_MMVQ_MAX_COLS;
            if (int rc = launch_mmvq(w, static_cast<const uint8_t *>(a) + t0 * col_bytes,
                                     y + t0 * N, nullptr, N, K, (int32_t)tc, stream))
                return rc;
        }
        return BQM_OK;
    }
    if (2 * mm_stream_workgroups(N, T) < 3ll * compute_units() && mm_chunked_supported(K))
        return launch_mm_chunked(w, a, y, N, K, T, stream);
    return launch_mm_stream(w, a, y, N, K, T, stream);
}

// ---------------------------------------------------------------------------
// Expert-routed product, one (token, slot) pair per blockIdx.y: the pair's
// expert matrix times its token's activation column. Used for shapes whose
// staged activations do not fit the grouped kernel's LDS budget.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mmvq_id_tq1_kernel(const uint8_t *__restrict__ w,
                                                          const uint8_t *__restrict__ a,
                                                          const int32_t *__restrict__ ids,
                                                          float *__restrict__ y, int64_t E,
                                                          int64_t N, int nb, int pairs_per_col,
                                                          int lr_log2)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Lr = 1 << lr_log2;
    const int rows_per_wave = 64 >> lr_log2;
    const int64_t row =
        ((int64_t)blockIdx.x * 4 + wave) * rows_per_wave + (lane >> lr_log2);
    const int sub = lane & (Lr - 1);
    const int64_t pair = blockIdx.y;  // t * n_used + s
    const int64_t t = pair / pairs_per_col;  // its activation column
    int e = ids[pair];
    e = e < 0 ? 0 : (e >= E ? (int)E - 1 : e);  // keep accesses inside w for bad ids
    const uint64_t expert_bytes = (uint64_t)N * nb * kTq1BlockBytes;
    const uint64_t col_bytes = (uint64_t)nb * 8 * kQ81BlockBytes;
    rows_product<1, false>(w + e * expert_bytes, expert_bytes, a + t * col_bytes, col_bytes, row,
                           row < N, nb, sub, Lr, 1, 0, y + pair * N, N, nullptr, N);
}

int launch_mmvq_id_pairs(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                         int64_t N, int64_t K, int64_t T, int32_t n_used, int pairs_per_col,
                         hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int64_t rows_per_wg = 4 * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)(T * n_used));
    hipLaunchKernelGGL(mmvq_id_tq1_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(a), ids, y,
                       E, N, nb, pairs_per_col, lr);
    return check_launch();
}

}  // namespace bqm
