// mmvq_quad.hip -- TQ1_0 x Q8_1 product for three to eight activation
// columns on gfx950: whole-block decode per lane as in the staged kernel,
// with the sub-block sums on the matrix cores as sixteen independent
// 4 x 4 x 4 products per instruction (v_mfma_i32_4x4x4i8).
//
// Operand layout of v_mfma_i32_4x4x4i8: product g uses lanes 4g .. 4g+3;
// lane 4g+i supplies row i of A (four int8) and column i of B (four int8),
// and receives column i of the 4 x 4 result, row v in accumulator register v.
//
// Thread mapping: a wave owns four consecutive rows. Lane l = 4g + i decodes
// blocks g, g + 16, g + 32, ... of row i; each decoded dword (the digits of
// four consecutive elements) is row i of product g's A operand, and the same
// lane supplies the four matching q bytes of activation column i (4 + i for
// the second column group) as its B operand. So the four lanes of slot g
// work on the same block index of the wave's four rows, and each lane reads
// only its own column's activations from LDS, where a lane of the staged
// kernel reads every column.
//
// Sums: the eight products of a sub-block start from the staged -sum(q) of
// the column (the -1 of every trit) and add u q over its 32 elements, which
// is the exact sub-block sum. The fp32 order is the staged kernel's (s =
// da[0] isum[0], fmaf over b = 1..7, then acc + dw s), and a row's blocks
// fall into the same Lr >= 16 groups (block B in group B mod Lr), combined
// by the same butterfly: groups g + 16 h of one lane first (levels 32 and
// 16), then across the slots. The result is bitwise the staged kernel's.
#include "mmvq_staged.hpp"

namespace bqm {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS stride between staged activation columns, in dwords: the cb staged
// blocks plus padding to 16 modulo 64, so that the four columns read by one
// slot's lanes start on different banks.
__host__ __device__ inline int quad_col_stride(int cb)
{
    const int s = cb * kActStride;
    return s + ((16 - s) & 63);
}

// Blocks staged per pass, as staged_chunk with the padded column stride
// (Lr >= 16 lanes per row here); 0 if nothing fits.
static int quad_chunk(int nb, int lr, int T, size_t budget)
{
    const int Lr = 1 << lr;
    auto fits = [&](int c) { return (size_t)T * quad_col_stride(c) * 4 <= budget; };
    if (nb <= Lr)
        return fits(nb) ? nb : 0;
    int chunk = (nb < kMaxChunkBlocks ? nb : kMaxChunkBlocks) / Lr * Lr;
    while (chunk >= Lr && !fits(chunk))
        chunk -= Lr;
    return chunk >= Lr ? chunk : 0;
}

// CG column groups of four (T <= 4 CG), GPW = Lr / 16 groups per lane, WPG
// waves (4 WPG rows) per workgroup.
template <int CG, int GPW, bool ISUMS, bool F32, int WPG>
__global__ __launch_bounds__(64 * WPG) void mmvq_quad_kernel(const uint8_t *__restrict__ w,
                                                        const uint8_t *__restrict__ a,
                                                        float *y, const float *resid,
                                                        int32_t *__restrict__ isums, int64_t N,
                                                        int nb, int T, int chunk)
{
    extern __shared__ uint4 act_lds[];
    uint32_t *act = reinterpret_cast<uint32_t *>(act_lds);
    const int tid = threadIdx.x, lane = tid & 63;
    const int g = lane >> 2, qi = lane & 3;
    const int64_t row0 = ((int64_t)blockIdx.x * WPG + (tid >> 6)) * 4;  // the wave's first row
    const int64_t row = row0 + qi;                                      // this lane's A row
    const bool row_ok = row < N;
    const int nblk = nb * 8;
    const uint32_t col_bytes = F32 ? (uint32_t)nb * kTq1BlockElems * 4 : (uint32_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    const uint32_t row_off = (uint32_t)((row_ok ? row : 0) * nb * kTq1BlockBytes);
    // this lane's B columns; a column past T reads column T - 1's copy and
    // its results are never stored
    int bcol[CG];
#pragma unroll
    for (int cg = 0; cg < CG; cg++)
        bcol[cg] = 4 * cg + qi < T ? 4 * cg + qi : T - 1;
    float acc[GPW][CG][4];
#pragma unroll
    for (int h = 0; h < GPW; h++)
#pragma unroll
        for (int cg = 0; cg < CG; cg++)
#pragma unroll
            for (int v = 0; v < 4; v++)
                acc[h][cg][v] = 0.0f;

    auto pass = [&](int B0) {
        const int end = min(B0 + chunk, nb);
        const int cb = end - B0;
        const int S = quad_col_stride(cb);
        const int first = B0 + g;
        if (B0 > 0)
            __syncthreads();  // readers of the previous chunk are done
        // first staging batch, then this lane's first weight block (as in the
        // staged kernel: the weights' latency overlaps the activation copy)
        StageBatch<F32> head;
        stage_load<F32>(head, ra, 0, B0, cb, 0, tid, 64 * WPG);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        RawBlock cur = load_raw_block(rw, row_ok && first < end
                                              ? row_off + (uint32_t)first * kTq1BlockBytes
                                              : kIdleLoadOffset);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_sched_barrier(0);
        stage_column<F32>(act, ra, 0, B0, cb, tid, 64 * WPG, &head);
#pragma unroll
        for (int t = 1; t < 4 * CG; t++)
            if (t < T)
                stage_column<F32>(act + t * S, ra, (uint32_t)t * col_bytes, B0, cb, tid, 64 * WPG,
                                  nullptr);
        __syncthreads();
        // the slot's blocks B = first + 16 m; the trip count is the same for
        // every lane (the matrix products need the whole wave), and a slot
        // past the end computes on block B0's activations and keeps nothing
        const int steps = (cb + 15) >> 4;
        for (int m0 = 0; m0 < steps; m0 += GPW) {
#pragma unroll
            for (int h = 0; h < GPW; h++) {
                const int m = m0 + h;
                if (m >= steps)
                    break;  // uniform
                const int B = first + 16 * m;
                const bool have = B < end;
                if (m > 0)
                    cur = load_raw_block(rw, row_ok && have ? row_off + (uint32_t)B * kTq1BlockBytes
                                                            : kIdleLoadOffset);
                const uint32_t *ab[CG];
#pragma unroll
                for (int cg = 0; cg < CG; cg++)
                    ab[cg] = act + bcol[cg] * S + (have ? B - B0 : 0) * kActStride;
                i32x4 D[CG][8];
#pragma unroll
                for (int cg = 0; cg < CG; cg++)
#pragma unroll
                    for (int b = 0; b < 8; b++) {
                        const int n = (int)ab[cg][72 + b];
                        D[cg][b] = (i32x4){n, n, n, n};
                    }
                // digit c of qs dword j < 8: dword j of sub-block c
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const QsDigits u = qs_digits(raw_dword(cur, j));
#pragma unroll
                    for (int cg = 0; cg < CG; cg++) {
                        const uint4 q = *reinterpret_cast<const uint4 *>(ab[cg] + 8 * j);
                        const uint32_t q4 = ab[cg][8 * j + 4];
                        const uint32_t qv[5] = {q.x, q.y, q.z, q.w, q4};
#pragma unroll
                        for (int c = 0; c < 5; c++)
                            D[cg][c] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[c], (int)qv[c],
                                                                          D[cg][c], 0, 0, 0);
                    }
                }
                // digits 0..4 of qs dword 8 + i: dwords i, 4 + i of sub-blocks
                // 5 and 6, dword i of sub-block 7; digit i of qh: dword 4 + i
                // of sub-block 7
                const QhDigits uh = qh_digits(raw_dword(cur, 12));
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const QsDigits u = qs_digits(raw_dword(cur, 8 + i));
#pragma unroll
                    for (int cg = 0; cg < CG; cg++) {
                        const uint4 lo = *reinterpret_cast<const uint4 *>(ab[cg] + 8 * i + 4);
                        const uint4 hi = *reinterpret_cast<const uint4 *>(ab[cg] + 8 * (4 + i) + 4);
                        D[cg][5] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[0], (int)lo.y, D[cg][5], 0, 0, 0);
                        D[cg][5] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[1], (int)hi.y, D[cg][5], 0, 0, 0);
                        D[cg][6] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[2], (int)lo.z, D[cg][6], 0, 0, 0);
                        D[cg][6] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[3], (int)hi.z, D[cg][6], 0, 0, 0);
                        D[cg][7] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)u.U[4], (int)lo.w, D[cg][7], 0, 0, 0);
                        D[cg][7] = __builtin_amdgcn_mfma_i32_4x4x4i8((int)uh.U[i], (int)hi.w, D[cg][7], 0, 0, 0);
                    }
                }
                if (ISUMS) {
#pragma unroll
                    for (int cg = 0; cg < CG; cg++) {
                        const int col = 4 * cg + qi;
#pragma unroll
                        for (int v = 0; v < 4; v++) {
                            const int64_t r = row0 + v;
                            if (have && col < T && r < N) {
                                int32_t *dst = isums + ((int64_t)col * N + r) * nblk + 8 * B;
#pragma unroll
                                for (int b = 0; b < 8; b++)
                                    dst[b] = D[cg][b][v];
                            }
                        }
                    }
                } else {
                    // block scales of the slot's four rows (lane 4g + v holds row v's)
                    const float dw = f16_bits_to_f32(raw_scale_bits(cur));
                    const float dwv[4] = {dpp_move<0x00>(dw), dpp_move<0x55>(dw),
                                          dpp_move<0xaa>(dw), dpp_move<0xff>(dw)};
#pragma unroll
                    for (int cg = 0; cg < CG; cg++) {
                        float s[4];
#pragma unroll
                        for (int b = 0; b < 8; b++) {
                            const float da = __uint_as_float(ab[cg][64 + b]);
#pragma unroll
                            for (int v = 0; v < 4; v++)
                                s[v] = b == 0 ? da * (float)D[cg][b][v]
                                              : fmaf(da, (float)D[cg][b][v], s[v]);
                        }
#pragma unroll
                        for (int v = 0; v < 4; v++)
                            if (have)
                                acc[h][cg][v] = fmaf(dwv[v], s[v], acc[h][cg][v]);
                    }
                }
            }
        }
    };
    if (chunk >= nb) {
        pass(0);
    } else {
        for (int B0 = 0; B0 < nb; B0 += chunk)
            pass(B0);
    }
    if (ISUMS)
        return;
    // group levels inside the lane (h: group g + 16 h), highest first
#pragma unroll
    for (int m = GPW >> 1; m >= 1; m >>= 1) {
        float nxt[GPW][CG][4];
#pragma unroll
        for (int h = 0; h < GPW; h++)
#pragma unroll
            for (int cg = 0; cg < CG; cg++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    nxt[h][cg][v] = acc[h][cg][v] + acc[h ^ m][cg][v];
#pragma unroll
        for (int h = 0; h < GPW; h++)
#pragma unroll
            for (int cg = 0; cg < CG; cg++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    acc[h][cg][v] = nxt[h][cg][v];
    }
    // levels 8, 4, 2, 1 of the slot index g = lane bits 2..5: lane ^ 32 and
    // ^ 16 through the crossbar, then rotations by 8 and 4 inside each 16-lane
    // row (the rotation by 4 reads lane k ^ 4 or, past the previous level,
    // a lane holding the same value)
    float out[CG][4];
#pragma unroll
    for (int cg = 0; cg < CG; cg++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float x = acc[0][cg][v];
            x += __shfl_xor(x, 32, 64);
            x += __shfl_xor(x, 16, 64);
            x += dpp_move<0x128>(x);  // row_ror:8
            x += dpp_move<0x124>(x);  // row_ror:4
            out[cg][v] = x;
        }
    // slot 0 stores: lane i writes column 4 cg + i of the wave's four rows
    if (g == 0) {
#pragma unroll
        for (int cg = 0; cg < CG; cg++) {
            const int col = 4 * cg + qi;
#pragma unroll
            for (int v = 0; v < 4; v++)
                if (col < T && row0 + v < N) {
                    const int64_t o = (int64_t)col * N + row0 + v;
                    y[o] = epilogue(out[cg][v], resid, o);
                }
        }
    }
}

bool quad_supported(int64_t K, int32_t T)
{
    if (T < 3 || T > 8)
        return false;
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    return lr >= 4 && quad_chunk(nb, lr, T, lds_budget()) > 0;
}

// Waves per workgroup: eight (32 rows) unless that puts more waves on the
// busiest SIMD than four do (counted as rounds of workgroups per compute unit
// times waves per workgroup). Eight halves the staging per row, which is the
// activation copy and, on fp32 input, the quantization (14336 x 4096 fp32 at
// eight columns: 22.3 against 24.0 us; 5120 x 6144: 16.0 against 23.2 us);
// four keep every compute unit busy on 4096 rows (4.85 against 5.63 us).
static int quad_waves(int64_t N)
{
    const int64_t cu = compute_units();
    const int64_t r4 = ((N + 15) / 16 + cu - 1) / cu;
    const int64_t r8 = ((N + 31) / 32 + cu - 1) / cu;
    return 2 * r8 <= r4 ? 8 : 4;
}

template <int CG, int GPW, bool F32, int WPG>
static void launch_quad_cg(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                           int32_t *isums,
                           int64_t N, int nb, int T, int chunk, size_t lds, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 4 * WPG - 1) / (4 * WPG))), block(64 * WPG);
    if (isums && !F32) {
        const void *k = reinterpret_cast<const void *>(&mmvq_quad_kernel<CG, GPW, true, false, WPG>);
        allow_dynamic_lds(k, lds);
        hipLaunchKernelGGL((mmvq_quad_kernel<CG, GPW, true, false, WPG>), grid, block, lds, stream,
                           w, a, nullptr, nullptr, isums, N, nb, T, chunk);
    } else {
        const void *k = reinterpret_cast<const void *>(&mmvq_quad_kernel<CG, GPW, false, F32, WPG>);
        allow_dynamic_lds(k, lds);
        hipLaunchKernelGGL((mmvq_quad_kernel<CG, GPW, false, F32, WPG>), grid, block, lds, stream,
                           w, a, y, r, nullptr, N, nb, T, chunk);
    }
}

template <int GPW, bool F32>
static void launch_quad_gpw(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                            int32_t *isums,
                            int64_t N, int nb, int T, int chunk, size_t lds, hipStream_t stream)
{
    const bool two = T > 4, wide = quad_waves(N) == 8;
    if (two)
        wide ? launch_quad_cg<2, GPW, F32, 8>(w, a, y, r, isums, N, nb, T, chunk, lds, stream)
             : launch_quad_cg<2, GPW, F32, 4>(w, a, y, r, isums, N, nb, T, chunk, lds, stream);
    else
        wide ? launch_quad_cg<1, GPW, F32, 8>(w, a, y, r, isums, N, nb, T, chunk, lds, stream)
             : launch_quad_cg<1, GPW, F32, 4>(w, a, y, r, isums, N, nb, T, chunk, lds, stream);
}

template <bool F32>
static int launch_quad(const void *w, const void *a, float *y, const float *r, int32_t *isums,
                       int64_t N, int64_t K, int32_t T, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = quad_chunk(nb, lr, T, lds_budget());
    if (T < 3 || T > 8 || lr < 4 || chunk <= 0)
        return BQM_ERR_SHAPE;
    const size_t lds = (size_t)T * quad_col_stride(chunk) * 4;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    switch (lr) {
    case 4: launch_quad_gpw<1, F32>(wp, ap, y, r, isums, N, nb, T, chunk, lds, stream); break;
    case 5: launch_quad_gpw<2, F32>(wp, ap, y, r, isums, N, nb, T, chunk, lds, stream); break;
    default: launch_quad_gpw<4, F32>(wp, ap, y, r, isums, N, nb, T, chunk, lds, stream); break;
    }
    return check_launch();
}

int launch_mmvq_quad(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_quad<false>(w, a, y, r, isums, N, K, T, stream);
}

int launch_mmvq_quad_f32(const void *w, const float *x, float *y, int64_t N, int64_t K,
                         int32_t T, hipStream_t stream, const float *r)
{
    return launch_quad<true>(w, x, y, r, nullptr, N, K, T, stream);
}

}  // namespace bqm
