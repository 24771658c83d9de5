// mmvq_mfma.hip -- TQ1_0 x Q8_1 product for 9 to 32 activation columns on
// gfx950, with the integer sums on the matrix cores.
//
// With many columns the product is a real contraction: per 32-element Q8_1
// sub-block, a 16-row tile of weight trits times up to 16 activation columns
// is exactly one v_mfma_i32_16x16x32_i8, whose int32 results are the exact
// per-sub-block sums. The decoded trits of a 256-element block feed all
// column tiles; the fp32 scaling uses the same order as the one-column
// kernel, so a column's result does not depend on how many columns the call
// carries (the exactness the multi-column kernel of "cuda: opt-in MMVQ
// activation reuse across output rows" keeps against single-column calls).
//
// Operand layout of v_mfma_i32_16x16x32_i8 (K = 32 = one sub-block):
//   A (weights): lane (r, kg) = (lane % 16, lane / 16) holds 8 trits of row r;
//   B (activations): lane (c, kg) holds the 8 matching q bytes of column c;
//   D: lane (c, rg) holds rows 4rg..4rg+3 of column c.
// The eight K positions of lane group kg are, per sub-block b:
//   b < 5: elements 8kg..8kg+7  (digit b of qs bytes 8kg..8kg+7),
//   b = 5: elements 4kg..4kg+3 and 16+4kg..16+4kg+3 (digits 0, 1 of qs dword
//          8+kg), b = 6 likewise with digits 2, 3, and b = 7: digit 4 of qs
//          dword 8+kg, then digit kg of the qh dword (elements 16+4kg..),
// so every lane decodes two qs dwords of the first 32 bytes, one of the next
// 16 and the qh dword, and the activation operands are plain Q8_1 dwords.
//
// Reduction order: a row's blocks are split into the same Lr lane groups as
// in the staged kernel (block B belongs to group B mod Lr). Each wave of the
// workgroup owns Lr / nw groups, accumulates each group's blocks in order,
// and the groups are then combined by the same xor butterfly, first inside
// the wave and then across waves through LDS.
#include "launch.hpp"
#include "tq1_decode.hpp"

namespace bqm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kMfmaMaxWaves = 8;  // waves per workgroup

// This lane's share of one 54-byte block (see the layout above): qs dwords
// 2kg and 2kg+1, qs dword 8+kg, the qh dword and the fp16 scale, read as the
// aligned dwords that cover them and realigned (odd blocks of a row start two
// bytes past a dword boundary).
struct LaneBlock {
    uint32_t lo0, lo1, hi, qh, dbits;
};

__device__ __forceinline__ LaneBlock load_lane_block(__amdgpu_buffer_rsrc_t rw, uint32_t off, int kg)
{
    const uint32_t sh = off & 3u, base = off - sh;
    const u32x3 l = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 8 * kg, 0, 0);
    const u32x2 h = ld_b64(rw, base + 32 + 4 * kg);
    const u32x2 t = ld_b64(rw, base + 48);
    LaneBlock b;
    b.lo0 = align_bytes(l.y, l.x, sh);
    b.lo1 = align_bytes(l.z, l.y, sh);
    b.hi = align_bytes(h.y, h.x, sh);
    b.qh = align_bytes(t.y, t.x, sh);
    b.dbits = sh ? (t.y >> 16) : (t.y & 0xffffu);
    return b;
}

// Decoded weight operands of one lane for one 16-row tile and block: A[b] is
// the 8-byte trit operand of sub-block b, dw the fp32 scale of the lane's row.
struct TileOperands {
    long A[8];
    float dw;
};

__device__ __forceinline__ TileOperands decode_lane_block(const LaneBlock &lb, int kg)
{
    const QsTrits lo0 = qs_trits(lb.lo0);
    const QsTrits lo1 = qs_trits(lb.lo1);
    const QsTrits hi = qs_trits(lb.hi);
    const QhTrits qh = qh_trits(lb.qh);
    const uint32_t qhk = kg == 0 ? qh.T[0] : kg == 1 ? qh.T[1] : kg == 2 ? qh.T[2] : qh.T[3];
    TileOperands t;
#pragma unroll
    for (int c = 0; c < 5; c++)
        t.A[c] = (long)(((uint64_t)lo1.T[c] << 32) | lo0.T[c]);
    t.A[5] = (long)(((uint64_t)hi.T[1] << 32) | hi.T[0]);
    t.A[6] = (long)(((uint64_t)hi.T[3] << 32) | hi.T[2]);
    t.A[7] = (long)(((uint64_t)qhk << 32) | hi.T[4]);
    t.dw = f16_bits_to_f32(lb.dbits);
    return t;
}

// GPW: butterfly groups per wave (Lr / waves); NT: 16-column tiles (1 or 2);
// R: 16-row tiles per workgroup, which share each block's activation
// operands; ISUMS: write the exact per-sub-block sums instead of outputs.
template <int GPW, int NT, int R, bool ISUMS>
__global__ __launch_bounds__(512) void mmvq_mfma_kernel(const uint8_t *__restrict__ w,
                                                        const uint8_t *__restrict__ a,
                                                        float *__restrict__ y,
                                                        int32_t *__restrict__ isums, int64_t N,
                                                        int nb, int T, int lr_log2)
{
    extern __shared__ float red[];  // [waves][64][R * NT * 4]: cross-wave butterfly
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int Lr = 1 << lr_log2;
    const int kg = lane >> 4;                   // decode lane: row lane % 16, K group kg
    const int col = lane & 15, rg = lane >> 4;  // output lane: column col, rows 4rg..4rg+3
    const int64_t r0 = (int64_t)blockIdx.x * 16 * R;
    const int nblk = nb * 8;
    const uint64_t col_bytes = (uint64_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    // columns past T read as zero (beyond the buffer's range)
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    uint32_t row_off[R];
#pragma unroll
    for (int rt = 0; rt < R; rt++) {
        const int64_t rowA = r0 + 16 * rt + (lane & 15);
        row_off[rt] = (uint32_t)((rowA < N ? rowA : 0) * nb * kTq1BlockBytes);
    }

    float acc[GPW][R][NT][4];
#pragma unroll
    for (int gi = 0; gi < GPW; gi++)
#pragma unroll
        for (int rt = 0; rt < R; rt++)
#pragma unroll
            for (int ct = 0; ct < NT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[gi][rt][ct][i] = 0.0f;

#pragma unroll
    for (int gi = 0; gi < GPW; gi++) {
        const int g = wave + nw * gi;
        for (int B = g; B < nb; B += Lr) {
            // weights of all row tiles first (HBM), then the activations (L2)
            LaneBlock lb[R];
#pragma unroll
            for (int rt = 0; rt < R; rt++)
                lb[rt] = load_lane_block(rw, row_off[rt] + (uint32_t)B * kTq1BlockBytes, kg);
            long Bq[NT][8];
            float da[NT][8];
#pragma unroll
            for (int ct = 0; ct < NT; ct++) {
                const uint32_t cbase = (uint32_t)((uint64_t)(ct * 16 + col) * col_bytes) +
                                       (uint32_t)(8 * B) * kQ81BlockBytes;
#pragma unroll
                for (int b = 0; b < 8; b++) {
                    const uint32_t o = cbase + b * kQ81BlockBytes;
                    uint32_t q0, q1;
                    if (b < 5) {
                        const u32x2 v = ld_b64(ra, o + 8 * kg);
                        q0 = v.x;
                        q1 = v.y;
                    } else {
                        q0 = ld_b32(ra, o + 4 * kg);
                        q1 = ld_b32(ra, o + 16 + 4 * kg);
                    }
                    Bq[ct][b] = (long)(((uint64_t)q1 << 32) | q0);
                    da[ct][b] = f16_bits_to_f32(ld_b32(ra, o + 32) & 0xffffu);
                }
            }
#pragma unroll
            for (int rt = 0; rt < R; rt++) {
                const TileOperands op = decode_lane_block(lb[rt], kg);
                // block scales of the four rows this output lane holds
                float dw[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    dw[i] = __shfl(op.dw, 4 * rg + i, 64);
#pragma unroll
                for (int ct = 0; ct < NT; ct++) {
                    i32x4 C[8];
#pragma unroll
                    for (int b = 0; b < 8; b++)
                        C[b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(op.A[b], Bq[ct][b],
                                                                      (i32x4){0, 0, 0, 0}, 0, 0, 0);
                    const int c = ct * 16 + col;
                    if (ISUMS) {
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int64_t row = r0 + 16 * rt + 4 * rg + i;
                            if (c < T && row < N) {
                                int32_t *dst = isums + ((int64_t)c * N + row) * nblk + 8 * B;
#pragma unroll
                                for (int b = 0; b < 8; b++)
                                    dst[b] = C[b][i];
                            }
                        }
                    } else {
                        // the one-column kernel's fp32 order: s = sum_b da[b] * isum[b]
                        // from b = 0 up, then acc + dw * s
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            float sum = da[ct][0] * (float)C[0][i];
#pragma unroll
                            for (int b = 1; b < 8; b++)
                                sum = fmaf(da[ct][b], (float)C[b][i], sum);
                            acc[gi][rt][ct][i] = fmaf(dw[i], sum, acc[gi][rt][ct][i]);
                        }
                    }
                }
            }
        }
    }
    if (ISUMS)
        return;

    // butterfly over the Lr groups: first the levels that pair groups held by
    // this wave (group g = wave + nw * gi; the partner differs in gi), then
    // the levels across waves through LDS. Each side forms mine + partner, so
    // every group ends with the same value.
#pragma unroll
    for (int m = GPW >> 1; m >= 1; m >>= 1) {
        float nxt[GPW][R][NT][4];
#pragma unroll
        for (int gi = 0; gi < GPW; gi++)
#pragma unroll
            for (int rt = 0; rt < R; rt++)
#pragma unroll
                for (int ct = 0; ct < NT; ct++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        nxt[gi][rt][ct][i] = acc[gi][rt][ct][i] + acc[gi ^ m][rt][ct][i];
#pragma unroll
        for (int gi = 0; gi < GPW; gi++)
#pragma unroll
            for (int rt = 0; rt < R; rt++)
#pragma unroll
                for (int ct = 0; ct < NT; ct++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[gi][rt][ct][i] = nxt[gi][rt][ct][i];
    }
    constexpr int kPer = R * NT * 4;
    float *mine = red + ((size_t)wave * 64 + lane) * kPer;
    for (int m = nw >> 1; m >= 1; m >>= 1) {
#pragma unroll
        for (int rt = 0; rt < R; rt++)
#pragma unroll
            for (int ct = 0; ct < NT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    mine[(rt * NT + ct) * 4 + i] = acc[0][rt][ct][i];
        __syncthreads();
        const float *other = red + ((size_t)(wave ^ m) * 64 + lane) * kPer;
#pragma unroll
        for (int rt = 0; rt < R; rt++)
#pragma unroll
            for (int ct = 0; ct < NT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[0][rt][ct][i] = acc[0][rt][ct][i] + other[(rt * NT + ct) * 4 + i];
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int rt = 0; rt < R; rt++)
#pragma unroll
            for (int ct = 0; ct < NT; ct++) {
                const int c = ct * 16 + col;
                if (c < T) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int64_t row = r0 + 16 * rt + 4 * rg + i;
                        if (row < N)
                            y[(int64_t)c * N + row] = acc[0][rt][ct][i];
                    }
                }
            }
    }
}

template <int GPW, int NT>
static void launch_mfma_gn(const uint8_t *w, const uint8_t *a, float *y, int32_t *isums,
                           int64_t N, int nb, int T, int lr, int nw, hipStream_t stream)
{
    // row tiles sharing each block's activation operands: as many as keep the
    // wave's accumulators (GPW * R * NT sets of four) within eight sets and
    // the activation operands plus accumulators within the register file
    constexpr int Rcap = NT == 1 ? 4 : 2;
    constexpr int Racc = GPW * NT >= 8 ? 1 : 8 / (GPW * NT);
    constexpr int R = Racc < Rcap ? Racc : Rcap;
    const dim3 grid((unsigned)((N + 16 * R - 1) / (16 * R)));
    const size_t lds = (size_t)nw * 64 * R * NT * 4 * sizeof(float);
    if (isums)
        hipLaunchKernelGGL((mmvq_mfma_kernel<GPW, NT, R, true>), grid, dim3(64 * nw), lds,
                           stream, w, a, nullptr, isums, N, nb, T, lr);
    else
        hipLaunchKernelGGL((mmvq_mfma_kernel<GPW, NT, R, false>), grid, dim3(64 * nw), lds,
                           stream, w, a, y, nullptr, N, nb, T, lr);
}

template <int NT>
static void launch_mfma_n(const uint8_t *w, const uint8_t *a, float *y, int32_t *isums,
                          int64_t N, int nb, int T, int lr, hipStream_t stream)
{
    const int Lr = 1 << lr;
    const int nw = Lr < kMfmaMaxWaves ? Lr : kMfmaMaxWaves;
    switch (Lr / nw) {
    case 1: launch_mfma_gn<1, NT>(w, a, y, isums, N, nb, T, lr, nw, stream); break;
    case 2: launch_mfma_gn<2, NT>(w, a, y, isums, N, nb, T, lr, nw, stream); break;
    case 4: launch_mfma_gn<4, NT>(w, a, y, isums, N, nb, T, lr, nw, stream); break;
    default: launch_mfma_gn<8, NT>(w, a, y, isums, N, nb, T, lr, nw, stream); break;
    }
}

int launch_mmvq_mfma(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (T <= 16)
        launch_mfma_n<1>(wp, ap, y, isums, N, nb, T, lr, stream);
    else
        launch_mfma_n<2>(wp, ap, y, isums, N, nb, T, lr, stream);
    return check_launch();
}

}  // namespace bqm
