// mmvq_mfma.hip -- TQ1_0 (and TQ2_0) x Q8_1 product for many activation
// columns on gfx950, with the integer sums on the matrix cores; activations
// streamed through LDS one block at a time (any K).
//
// With many columns the product is a real contraction: per 32-element Q8_1
// sub-block, a 16-row tile of weight digits times up to 16 activation columns
// is exactly one v_mfma_i32_16x16x32_i8, whose int32 results are the exact
// per-sub-block sums. The decoded digits of a 256-element block feed all
// column tiles; the fp32 scaling uses the same order as the staged kernels,
// so a column's result does not depend on how many columns the call carries
// (the exactness the multi-column kernel of "cuda: opt-in MMVQ activation
// reuse across output rows" keeps against single-column calls).
//
// (operand layouts and the digit decode: mfma_common.hpp)
//
// Activations: for each block it works on, a wave copies the block's Q8_1 data
// of every column (8 x 36 bytes per column) into its own slice of LDS with
// plain coalesced 8-byte loads, then reads each lane's 8-byte B operand and
// the sub-block scale from there. Loading the operands straight from memory
// instead would cost one scattered load per sub-block and column tile, each
// touching 16 cache lines.
//
// Reduction order: a row's blocks are split into the same Lr lane groups as
// in the staged kernel (block B belongs to group B mod Lr). Each wave of the
// workgroup owns Lr / nw groups, accumulates each group's blocks in order,
// and the groups are then combined by the same xor butterfly, first inside
// the wave and then across waves through LDS.
//
// The weight format enters through a policy (Tq1Tile, Tq2Tile; see
// mmvq_mfma_reg.hip).
#include "tq2_decode.hpp"

namespace bqm {

constexpr int kMfmaMaxWaves = 8;     // waves per workgroup
// Fmt: the weight format policy; GPW: butterfly groups per wave (Lr /
// waves); NT: 16-column tiles (1 or 2);
// R: 16-row tiles that share each staged activation block; ISUMS: write the
// exact per-sub-block sums instead of outputs.
//
// The grid is sized to what the GPU holds at once and each workgroup walks
// row tiles (16 R rows each) tile = blockIdx.x, + gridDim.x, ...; the one-block
// lookahead runs across tile boundaries, so the next tile's first block is in
// flight while the current tile finishes and reduces.
template <class Fmt, int GPW, int NT, int R, bool ISUMS>
__global__ __launch_bounds__(512) void mmvq_mfma_kernel(const uint8_t *__restrict__ w,
                                                        const uint8_t *__restrict__ a,
                                                        float *y, const float *resid,
                                                        int32_t *__restrict__ isums, int64_t N,
                                                        int nb, int T, int lr_log2, int ntiles)
{
    // per wave: its staged activation block; after those, the cross-wave
    // butterfly exchange
    extern __shared__ uint32_t smem[];
    const int nw = blockDim.x >> 6;
    // the wave index is uniform across the wave; saying so keeps the block
    // loop, the activation offsets and the branches on scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int Lr = 1 << lr_log2;
    const int kg = lane >> 4;                   // decode lane: row lane % 16, K group kg
    const typename Fmt::Ctx ctx(kg);
    const int col = lane & 15, rg = lane >> 4;  // output lane: column col, rows 4rg..4rg+3
    const int nblk = nb * 8;
    const uint32_t col_bytes = (uint32_t)nblk * kQ81BlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * Fmt::kBlockBytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    uint32_t *stage = smem + wave * (NT * 16 * kStageCol);
    float *red = reinterpret_cast<float *>(smem + nw * (NT * 16 * kStageCol));
    const StageMap smap(col_bytes, lane);

    // byte offsets of this decode lane's rows in tile t (rows past N read row 0)
    auto tile_rows = [&](int t, uint32_t (&ro)[R]) {
#pragma unroll
        for (int rt = 0; rt < R; rt++) {
            const int64_t rowA = (int64_t)t * 16 * R + 16 * rt + (lane & 15);
            ro[rt] = (uint32_t)((rowA < N ? rowA : 0) * nb * Fmt::kBlockBytes);
        }
    };

    int tile = blockIdx.x;
    uint32_t row_off[R];
    tile_rows(tile, row_off);
    // one block of lookahead: while block B is decoded and multiplied, the
    // weights and activations of the wave's next block are in flight
    typename Fmt::Lane lb[R];
    StagePieces<NT> pieces;
    if (tile < ntiles && wave < nb) {
#pragma unroll
        for (int rt = 0; rt < R; rt++)
            lb[rt] = Fmt::load(rw, row_off[rt] + (uint32_t)wave * Fmt::kBlockBytes, kg);
        pieces.issue(ra, smap, col_bytes, wave);
        pieces.land(stage, smap);
        wave_lds_order();
    }

    for (; tile < ntiles; tile += gridDim.x) {
        const int64_t r0 = (int64_t)tile * 16 * R;
        const int next_tile = tile + gridDim.x;
        uint32_t next_off[R];
        tile_rows(next_tile, next_off);

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
                // the wave's next block: the group's next one, else the next
                // group's first, else the first block of the next tile
                const bool same_tile = B + Lr < nb || (gi + 1 < GPW && g + nw < nb);
                const int Bn = B + Lr < nb ? B + Lr : (same_tile ? g + nw : wave);
                const bool have_next = same_tile || next_tile < ntiles;
                // the weights are loaded by every lane (at Fmt::kIdle
                // when there is no next block), so that their data is first
                // waited for where it is decoded
                typename Fmt::Lane ln[R];
#pragma unroll
                for (int rt = 0; rt < R; rt++)
                    ln[rt] = Fmt::load(
                        rw,
                        have_next ? (same_tile ? row_off[rt] : next_off[rt]) +
                                        (uint32_t)Bn * Fmt::kBlockBytes
                                  : Fmt::kIdle,
                        kg);
                if (have_next)
                    pieces.issue(ra, smap, col_bytes, Bn);

                // one row tile at a time: its digit operands meet every
                // sub-block and column tile of the staged activations (re-read
                // from LDS per row tile, which keeps one tile's operands in
                // registers)
#pragma unroll
                for (int rt = 0; rt < R; rt++) {
                    const TileOperands op = Fmt::decode(lb[rt], ctx);
                    float dw[4];  // block scales of the four rows this output lane holds
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        dw[i] = __shfl(op.dw, 4 * rg + i, 64);
                    float s[NT][4];
#pragma unroll
                    for (int b = 0; b < 8; b++) {
#pragma unroll
                        for (int ct = 0; ct < NT; ct++) {
                            const uint32_t *cs = stage + (ct * 16 + col) * kStageCol + 9 * b;
                            const long Bq = Fmt::operand_at(cs, kg, b);
                            // -sum(q) of this lane's column on every row, then + sum(u q)
                            const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                                kAllMinusOne, Bq, (i32x4){0, 0, 0, 0}, 0, 0, 0);
                            const i32x4 C = __builtin_amdgcn_mfma_i32_16x16x32_i8(op.A[b], Bq,
                                                                                  neg_sum, 0, 0, 0);
                            if (ISUMS) {
                                const int c = ct * 16 + col;
#pragma unroll
                                for (int i = 0; i < 4; i++) {
                                    const int64_t row = r0 + 16 * rt + 4 * rg + i;
                                    if (c < T && row < N)
                                        isums[((int64_t)c * N + row) * nblk + 8 * B + b] = C[i];
                                }
                            } else {
                                // the staged kernels' fp32 order: s = sum_b da[b] * isum[b]
                                // from b = 0 up, then acc + dw * s
                                const float da = f16_bits_to_f32(cs[8] & 0xffffu);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    s[ct][i] = b == 0 ? da * (float)C[i]
                                                      : fmaf(da, (float)C[i], s[ct][i]);
                            }
                        }
                    }
                    if (!ISUMS) {
#pragma unroll
                        for (int ct = 0; ct < NT; ct++)
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                acc[gi][rt][ct][i] = fmaf(dw[i], s[ct][i], acc[gi][rt][ct][i]);
                    }
                }
                if (have_next) {
                    wave_lds_order();  // this block's operand reads come first
                    pieces.land(stage, smap);
                    wave_lds_order();
                }
#pragma unroll
                for (int rt = 0; rt < R; rt++)
                    lb[rt] = ln[rt];
            }
        }

        if (!ISUMS) {
            // butterfly over the Lr groups: first the levels that pair groups
            // held by this wave (group g = wave + nw * gi; the partner differs
            // in gi), then the levels across waves through LDS. Each side
            // forms mine + partner, so every group ends with the same value.
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
                __syncthreads();  // the previous level's (or tile's) reads are done
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
                                if (row < N) {
                                    const int64_t o = (int64_t)c * N + row;
                                    y[o] = epilogue(acc[0][rt][ct][i], resid, o);
                                }
                            }
                        }
                    }
            }
        }
#pragma unroll
        for (int rt = 0; rt < R; rt++)
            row_off[rt] = next_off[rt];
    }
}

template <class Fmt, int GPW, int NT, int R>
static void launch_mfma_r(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                          int32_t *isums,
                          int64_t N, int nb, int T, int lr, int nw, hipStream_t stream)
{
    const int64_t ntiles = (N + 16 * R - 1) / (16 * R);
    const size_t stage = (size_t)nw * NT * 16 * kStageCol * sizeof(uint32_t);
    const size_t exchange = (size_t)nw * 64 * R * NT * 4 * sizeof(float);
    const size_t lds = stage + exchange;
    const void *kt = reinterpret_cast<const void *>(&mmvq_mfma_kernel<Fmt, GPW, NT, R, true>);
    const void *kf = reinterpret_cast<const void *>(&mmvq_mfma_kernel<Fmt, GPW, NT, R, false>);
    allow_dynamic_lds(kt, lds);
    allow_dynamic_lds(kf, lds);
    // as many workgroups as are resident at once, each taking the same number
    // of tiles (give or take one)
    const int cap = resident_workgroups(isums ? kt : kf, 64 * nw, lds);
    const int64_t per = (ntiles + cap - 1) / cap;
    const dim3 grid((unsigned)((ntiles + per - 1) / per));
    if (isums)
        hipLaunchKernelGGL((mmvq_mfma_kernel<Fmt, GPW, NT, R, true>), grid, dim3(64 * nw), lds,
                           stream, w, a, nullptr, nullptr, isums, N, nb, T, lr, (int)ntiles);
    else
        hipLaunchKernelGGL((mmvq_mfma_kernel<Fmt, GPW, NT, R, false>), grid, dim3(64 * nw), lds,
                           stream, w, a, y, r, nullptr, N, nb, T, lr, (int)ntiles);
}

template <class Fmt, int GPW, int NT>
static void launch_mfma_gn(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                           int32_t *isums,
                           int64_t N, int nb, int T, int lr, int nw, hipStream_t stream)
{
    // R, the row tiles sharing each staged activation block: at most what
    // keeps the wave's accumulators (GPW * R * NT sets of four) within eight
    // sets and the digit operands within the register file; within that, the
    // most that still gives every compute unit two tiles.
    constexpr int Rcap = NT == 1 ? 2 : 1;
    constexpr int Racc = GPW * NT >= 8 ? 1 : 8 / (GPW * NT);
    constexpr int Rmax = Racc < Rcap ? Racc : Rcap;
    const int64_t want = 2 * (int64_t)compute_units();
    if (Rmax >= 2 && (N + 31) / 32 >= want)
        launch_mfma_r<Fmt, GPW, NT, (Rmax >= 2 ? 2 : 1)>(w, a, y, r, isums, N, nb, T, lr, nw,
                                                         stream);
    else
        launch_mfma_r<Fmt, GPW, NT, 1>(w, a, y, r, isums, N, nb, T, lr, nw, stream);
}

template <class Fmt, int NT>
static void launch_mfma_n(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                          int32_t *isums,
                          int64_t N, int nb, int T, int lr, hipStream_t stream)
{
    const int Lr = 1 << lr;
    const int nw = Lr < kMfmaMaxWaves ? Lr : kMfmaMaxWaves;
    switch (Lr / nw) {
    case 1: launch_mfma_gn<Fmt, 1, NT>(w, a, y, r, isums, N, nb, T, lr, nw, stream); break;
    case 2: launch_mfma_gn<Fmt, 2, NT>(w, a, y, r, isums, N, nb, T, lr, nw, stream); break;
    case 4: launch_mfma_gn<Fmt, 4, NT>(w, a, y, r, isums, N, nb, T, lr, nw, stream); break;
    default: launch_mfma_gn<Fmt, 8, NT>(w, a, y, r, isums, N, nb, T, lr, nw, stream); break;
    }
}

template <class Fmt>
static int launch_mfma_fmt(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                           int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (T <= 16)
        launch_mfma_n<Fmt, 1>(wp, ap, y, r, isums, N, nb, T, lr, stream);
    else
        launch_mfma_n<Fmt, 2>(wp, ap, y, r, isums, N, nb, T, lr, stream);
    return check_launch();
}

int launch_mmvq_mfma(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_mfma_fmt<Tq1Tile>(w, a, y, isums, N, K, T, stream, r);
}

int launch_mmvq_mfma_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                         int64_t K, int32_t T, hipStream_t stream)
{
    return launch_mfma_fmt<Tq2Tile>(w, a, y, isums, N, K, T, stream, nullptr);
}

}  // namespace bqm
