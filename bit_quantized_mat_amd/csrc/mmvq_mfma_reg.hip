// mmvq_mfma_reg.hip -- TQ1_0 (and TQ2_0) x Q8_1 product for 5 to 32
// activation columns on gfx950 matrix cores, with every wave's activation
// operands held in registers for the whole call.
//
// The arithmetic is that of the other matrix-core kernels (mfma_common.hpp):
// a 16-row tile's digit operands decoded in registers, one
// v_mfma_i32_16x16x32_i8 per 32-element sub-block and 16-column tile, the
// -sum q term from an all -1 operand, and the staged kernels' fp32 order, so a
// column's result is bitwise that of a one-column call (the exactness the
// multi-column kernel of "cuda: opt-in MMVQ activation reuse across output
// rows" keeps against single-column calls).
//
// What is different is where the activations live. A row's blocks are split
// into Lr lane groups (block B in group B mod Lr), and for rows of at most Lr
// blocks a group is one block. The workgroup has NW waves; wave w owns the
// groups w + NW gi (gi < GPW), hence the same GPW blocks of every row tile.
// So before its first tile each wave loads the B operands (8 bytes per lane
// and sub-block) and the sub-block scales of its own blocks and of every
// column tile straight into registers, and keeps them for all its tiles: the
// activations are read once per wave and never pass through LDS, and no
// workgroup-wide copy or barrier precedes the first tile. The workgroup walks
// row tiles; per tile every wave decodes its blocks (the next tile's weights
// in flight meanwhile), multiplies, scales, and the waves' partial sums are
// combined through LDS by the xor butterfly (one barrier per tile, the
// partial sums double-buffered).
//
// The weight format enters through a policy (Tq1Tile, Tq2Tile): how a lane
// loads and decodes its share of a block and which staged activation bytes
// make its B operand. Everything else is common to both formats.
//
// Pair-tile mode (PAIR, at most 8 columns): a work unit is 32 rows, two
// 16-row tiles on one v_mfma_i32_16x16x64_i8 per sub-block (the layout in
// mfma_common.hpp), so each fp32 conversion and fma of the epilogue serves a
// real column; a decode lane then takes half of a row's block instead of a
// quarter. The per-column fp32 order is unchanged, so the results are
// bitwise those of the 16-column form.
#include <type_traits>

#include "tq2_decode.hpp"

namespace bqm {

// One lane's activation operands for one block and 16-column tile: the B
// operand of each sub-block and the fp16 sub-block scales of its column,
// two per dword (sub-block 2p in the low half, 2p + 1 in the high half).
// PAIR: 16-byte B operands, zero in the lane groups of the other tile.
template <bool PAIR>
struct RegOperands {
    typename std::conditional<PAIR, i32x4, long>::type Bq[8];
    uint32_t da2[4];
};

// Read them from a staged 16-column tile (mfma_common.hpp): lane (col, kg).
// PAIR: D column col is activation column col % 8 against tile col / 8, and
// lane group kg carries half kg % 2 of tile kg / 2.
template <class Fmt, bool PAIR>
__device__ __forceinline__ RegOperands<PAIR> read_reg_operands(const uint32_t *__restrict__ tile,
                                                               int col, int kg)
{
    RegOperands<PAIR> o;
    uint32_t d[8];
    const int c = PAIR ? (col & 7) : col;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        if constexpr (PAIR)
            o.Bq[b] = (col >> 3) == (kg >> 1) ? Fmt::pair_operand(tile, c, kg & 1, b)
                                              : (i32x4){0, 0, 0, 0};
        else
            o.Bq[b] = Fmt::operand(tile, col, kg, b);
        d[b] = tile[c * kStageCol + 9 * b + 8];
    }
#pragma unroll
    for (int p = 0; p < 4; p++)
        o.da2[p] = __builtin_amdgcn_perm(d[2 * p + 1], d[2 * p], 0x05040100u);
    return o;
}

// Fmt: the weight format policy; NW: waves per workgroup (8 or 16); GPW:
// blocks per wave (Lr = NW GPW); NT: 16-column tiles; ISUMS: write the exact
// per-sub-block sums instead of outputs; PAIR: the pair-tile mode (NT = 1,
// T <= 8, work units of 32 rows). Rows hold at most Lr blocks.
template <class Fmt, int NW, int GPW, int NT, bool ISUMS, bool PAIR = false>
__global__ __launch_bounds__(64 * NW) void mmvq_mfma_reg_kernel(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ a,
                                                                float *y, const float *resid,
                                                                int32_t *__restrict__ isums,
                                                                int64_t N, int nb, int T,
                                                                int ntiles)
{
    // LDS: [2][NW][lane][NT 4] fp32 partial sums of the waves, then per wave
    // one staged 16-column tile of activations (used before the first tile)
    extern __shared__ float red[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int kg = lane >> 4;                   // decode lane: row lane % 16, K group kg
    const typename Fmt::Ctx ctx(kg);
    const int col = lane & 15, rg = lane >> 4;  // output lane: column col, rows 4rg..4rg+3
    const int nblk = nb * 8;
    const uint32_t col_bytes = (uint32_t)nblk * kQ81BlockBytes;
    const uint32_t row_bytes = (uint32_t)nb * Fmt::kBlockBytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);

    static_assert(!PAIR || NT == 1, "pair tiles take at most 8 columns");
    constexpr uint32_t kRows = PAIR ? 32u : 16u;  // rows per work unit
    typedef typename std::conditional<PAIR, typename Fmt::PairLane, typename Fmt::Lane>::type
        LaneT;
    auto load_lane = [&](uint32_t off) -> LaneT {
        if constexpr (PAIR)
            return Fmt::load_pair(rw, off, kg & 1);
        else
            return Fmt::load(rw, off, kg);
    };

    int tile = blockIdx.x;
    if (tile >= ntiles)
        return;  // uniform

    // this decode lane's row offset in tile t (rows past N read row 0). The
    // matrix is below 4 GiB with at least 5 blocks (270 bytes) per row, so
    // rows stay below 2^24, and a 24-bit product gives the byte offset
    auto row_offset = [&](int t) -> uint32_t {
        const uint32_t r = (uint32_t)t * kRows + (PAIR ? 16u * (uint32_t)(kg >> 1) : 0u) +
                           (uint32_t)(lane & 15);
        return r < (uint64_t)N ? __umul24(r, row_bytes) : 0u;
    };

    // the first tile's weights, then this wave's activation operands
    LaneT lb[GPW];
    uint32_t roff = row_offset(tile);
#pragma unroll
    for (int gi = 0; gi < GPW; gi++) {
        const int B = wave + NW * gi;
        lb[gi] = load_lane(B < nb ? roff + (uint32_t)B * Fmt::kBlockBytes : Fmt::kIdle);
    }
    // every (block, column tile) of this wave: its 16 columns' 288-byte runs
    // of Q8_1 blocks loaded as coalesced 8-byte pieces (all sets in flight
    // at once), landed in the wave's stage one set at a time, read back as
    // operands. Columns at or past T read zeros (or wrapped in-range bytes):
    // they only feed output columns that are never stored.
    constexpr int kSets = GPW * NT;
    uint32_t *stage = reinterpret_cast<uint32_t *>(red) + 2 * NW * 64 * NT * 4 +
                      wave * 16 * kStageCol;
    const StageMap smap(col_bytes, lane);
    u32x2 piece[kSets][9];
#pragma unroll
    for (int st = 0; st < kSets; st++) {
        const int gi = st / NT, ct = st % NT;
        const int B = wave + NW * gi < nb ? wave + NW * gi : 0;
        const uint32_t so = __builtin_amdgcn_readfirstlane(
            (uint32_t)B * (8 * kQ81BlockBytes) + (uint32_t)ct * 16 * col_bytes);
#pragma unroll
        for (int k = 0; k < 9; k++)
            piece[st][k] = __builtin_amdgcn_raw_buffer_load_b64(ra, smap.gofs[k], so, 0);
    }
    RegOperands<PAIR> opnd[GPW][NT];
#pragma unroll
    for (int st = 0; st < kSets; st++) {
        if (st > 0)
            wave_lds_order();  // the previous set's reads come first
#pragma unroll
        for (int k = 0; k < 9; k++)
            *reinterpret_cast<u32x2 *>(stage + smap.lofs[k]) = piece[st][k];
        wave_lds_order();
        opnd[st / NT][st % NT] = read_reg_operands<Fmt, PAIR>(stage, col, kg);
    }

    int parity = 0;
    for (;;) {
        const int64_t r0 = (int64_t)tile * kRows;
        const int next_tile = tile + gridDim.x;
        const bool have_next = next_tile < ntiles;
        const uint32_t next_roff = row_offset(next_tile);
        // the next tile's weights, in flight while this tile is decoded and
        // multiplied (every lane issues them, at Fmt::kIdle when there
        // is no next tile, so that their data is first waited for where it is
        // decoded)
        LaneT ln[GPW];
#pragma unroll
        for (int gi = 0; gi < GPW; gi++) {
            const int B = wave + NW * gi;
            ln[gi] = load_lane(have_next && B < nb ? next_roff + (uint32_t)B * Fmt::kBlockBytes
                                                   : Fmt::kIdle);
        }

        float acc[GPW][NT][4];
#pragma unroll
        for (int gi = 0; gi < GPW; gi++) {
            const int B = wave + NW * gi;
#pragma unroll
            for (int ct = 0; ct < NT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[gi][ct][i] = 0.0f;
            if (B < nb) {  // uniform: else this group holds no block
            typedef typename std::conditional<PAIR, PairOperands, TileOperands>::type OpsT;
            OpsT op;
            if constexpr (PAIR)
                op = Fmt::decode_pair(lb[gi], ctx, kg & 1);
            else
                op = Fmt::decode(lb[gi], ctx);
            // PAIR: the output lane's rows are in tile col / 8, whose block
            // scales sit in the decode lanes of its half 1
            const int dw_src = PAIR ? 4 * rg + 16 * (2 * (col >> 3) + 1) : 4 * rg;
            float dw[4];  // block scales of the four rows this output lane holds
#pragma unroll
            for (int i = 0; i < 4; i++)
                dw[i] = __shfl(op.dw, dw_src + i, 64);
            // the products of (column tile, sub-block) j + 1 are issued
            // before the work on those of j, so that work does not wait for
            // the matrix cores
            auto product = [&](int j) -> i32x4 {
                const RegOperands<PAIR> &o = opnd[gi][j >> 3];
                const int b = j & 7;
                // -sum(q) of this lane's column on every row, then + sum(u q)
                if constexpr (PAIR) {
                    const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        kAllMinusOne4, o.Bq[b], (i32x4){0, 0, 0, 0}, 0, 0, 0);
                    return __builtin_amdgcn_mfma_i32_16x16x64_i8(op.A[b], o.Bq[b], neg_sum, 0, 0,
                                                                 0);
                } else {
                    const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                        kAllMinusOne, o.Bq[b], (i32x4){0, 0, 0, 0}, 0, 0, 0);
                    return __builtin_amdgcn_mfma_i32_16x16x32_i8(op.A[b], o.Bq[b], neg_sum, 0, 0,
                                                                 0);
                }
            };
            i32x4 Cn = product(0);
            float s[4];
#pragma unroll
            for (int j = 0; j < 8 * NT; j++) {
                const int ct = j >> 3, b = j & 7;
                const i32x4 C = Cn;
                if (j + 1 < 8 * NT)
                    Cn = product(j + 1);
                __builtin_amdgcn_sched_barrier(0);
                if (ISUMS) {
                    const int c = PAIR ? (col & 7) : ct * 16 + col;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int64_t row = r0 + (PAIR ? 16 * (col >> 3) : 0) + 4 * rg + i;
                        if (c < T && row < N)
                            isums[((int64_t)c * N + row) * nblk + 8 * B + b] = C[i];
                    }
                } else {
                    // the staged kernels' fp32 order: s = sum_b da[b] * isum[b]
                    // from b = 0 up, then acc + dw * s
                    const float da =
                        f16_bits_to_f32(opnd[gi][ct].da2[b >> 1] >> (16 * (b & 1)));
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        s[i] = b == 0 ? da * (float)C[i] : fmaf(da, (float)C[i], s[i]);
                    if (b == 7) {
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[gi][ct][i] = fmaf(dw[i], s[i], acc[gi][ct][i]);
                    }
                }
            }
            }
        }

        if (!ISUMS) {
            // butterfly levels inside the wave (the partner group differs in gi)
#pragma unroll
            for (int m = GPW >> 1; m >= 1; m >>= 1) {
                float nxt[GPW][NT][4];
#pragma unroll
                for (int gi = 0; gi < GPW; gi++)
#pragma unroll
                    for (int ct = 0; ct < NT; ct++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            nxt[gi][ct][i] = acc[gi][ct][i] + acc[gi ^ m][ct][i];
#pragma unroll
                for (int gi = 0; gi < GPW; gi++)
#pragma unroll
                    for (int ct = 0; ct < NT; ct++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[gi][ct][i] = nxt[gi][ct][i];
            }
            // the levels across waves: every wave leaves its partial sums in
            // this tile's half of red, then every wave folds 16 of the tile's
            // outputs per pass, four lanes per output: lane j of a quad takes
            // waves j, j + 4, ..., applies the levels of 4 and up among its own
            // values, the quad the levels 2 and 1 by DPP, so that the quad's
            // lane 0 ends with what the xor butterfly gives wave 0 (level m
            // adds wave w + m's running value to wave w's). The other half
            // belongs to the next tile, so one barrier per tile suffices.
            constexpr int kPer = NT * 4;
            constexpr int kWavesPerLane = NW / 4;
            constexpr int kPasses = 4 * kPer / NW;
            static_assert(NW % 4 == 0 && (4 * kPer) % NW == 0, "fold layout");
            float *half = red + (size_t)parity * NW * 64 * kPer;
#pragma unroll
            for (int ct = 0; ct < NT; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    half[((size_t)wave * 64 + lane) * kPer + ct * 4 + i] = acc[0][ct][i];
            __syncthreads();
            const int j = lane & 3;
#pragma unroll
            for (int pass = 0; pass < kPasses; pass++) {
                // output o of the tile: lane slot o / kPer, value o % kPer
                const int o = (pass * NW + wave) * 16 + (lane >> 2);
                float x[kWavesPerLane];
#pragma unroll
                for (int q = 0; q < kWavesPerLane; q++)
                    x[q] = half[(size_t)(j + 4 * q) * 64 * kPer + o];
#pragma unroll
                for (int m = kWavesPerLane >> 1; m >= 1; m >>= 1)
#pragma unroll
                    for (int q = 0; q < m; q++)
                        x[q] = x[q] + x[q + m];
                float v = x[0];
                v = v + dpp_move<0x4e>(v);  // quad_perm [2, 3, 0, 1]: level 2
                v = v + dpp_move<0xb1>(v);  // quad_perm [1, 0, 3, 2]: level 1
                const int ls = o / kPer, k = o - (o / kPer) * kPer;
                const int oc = ls & 15, org = ls >> 4;
                const int ct = k >> 2, i = k & 3;
                const int c = PAIR ? (oc & 7) : ct * 16 + oc;
                const int64_t row = r0 + (PAIR ? 16 * (oc >> 3) : 0) + 4 * org + i;
                if (j == 0 && c < T && row < N) {
                    const int64_t oi = (int64_t)c * N + row;
                    y[oi] = epilogue(v, resid, oi);
                }
            }
        }
        if (!have_next)
            break;
        tile = next_tile;
        parity ^= 1;
#pragma unroll
        for (int gi = 0; gi < GPW; gi++)
            lb[gi] = ln[gi];
    }
}

// Waves and blocks per wave for a row of nb blocks: Lr = NW GPW lane groups
// (the smallest power of two not below nb), NW in {8, 16}, one block per
// wave. Rows of 17 to 32 blocks (two per wave) stay with the resident
// kernel: the second operand set's staging cost more than it saved
// (5120 x 6144, 5 columns: 10.1 against 9.6 us; 8 columns: 10.0 against
// 10.4 us), and 320 row tiles balance poorly over 256 workgroups either way.
static bool reg_config(int nb, int T, int &NW, int &GPW, int &NT)
{
    const int Lr = 1 << lanes_per_row_log2(nb);
    NT = T <= 16 ? 1 : 2;
    if (T < 1 || T > 32 || Lr < 8 || Lr > 16)
        return false;
    NW = Lr;
    GPW = 1;
    return true;
}

bool mfma_reg_supported(int64_t K, int32_t T)
{
    int NW, GPW, NT;
    return reg_config((int)(K / kTq1BlockElems), T, NW, GPW, NT);
}

template <class Fmt, int NW, int GPW, int NT, bool PAIR = false>
static int launch_reg(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                      int32_t *isums, int64_t N, int nb, int T, hipStream_t stream)
{
    const int64_t rows = PAIR ? 32 : 16;
    const int64_t ntiles = (N + rows - 1) / rows;
    const size_t lds = ((size_t)2 * NW * 64 * NT * 4 + (size_t)NW * 16 * kStageCol) * 4;
    const void *kt =
        reinterpret_cast<const void *>(&mmvq_mfma_reg_kernel<Fmt, NW, GPW, NT, true, PAIR>);
    const void *kf =
        reinterpret_cast<const void *>(&mmvq_mfma_reg_kernel<Fmt, NW, GPW, NT, false, PAIR>);
    allow_dynamic_lds(kt, lds);
    allow_dynamic_lds(kf, lds);
    // persistent: as many workgroups as the device holds at once, each
    // walking row tiles blockIdx.x, + gridDim.x, ...
    const int cap = resident_workgroups(isums ? kt : kf, 64 * NW, lds);
    const dim3 grid((unsigned)(ntiles < cap ? ntiles : cap));
    if (isums)
        hipLaunchKernelGGL((mmvq_mfma_reg_kernel<Fmt, NW, GPW, NT, true, PAIR>), grid,
                           dim3(64 * NW), lds, stream, w, a, nullptr, nullptr, isums, N, nb, T,
                           (int)ntiles);
    else
        hipLaunchKernelGGL((mmvq_mfma_reg_kernel<Fmt, NW, GPW, NT, false, PAIR>), grid,
                           dim3(64 * NW), lds, stream, w, a, y, r, nullptr, N, nb, T, (int)ntiles);
    return check_launch();
}

bool pair_tiles_pay(int64_t N)
{
    const int64_t cu = compute_units();
    const int64_t u32 = ((N + 31) / 32 + cu - 1) / cu, u16 = ((N + 15) / 16 + cu - 1) / cu;
    return 3 * u32 < 2 * u16;
}

// Pair tiles for calls of at most 8 columns when they pay (14336 x 4096:
// 11.3 -> 9.5 us at 5 columns, 11.2 -> 9.7 at 8; TQ2_0 10.0 -> 8.3 at 3; at
// 4096 rows, one unit per compute unit either way, 5.6 -> 6.4 us).
static bool use_pair(int64_t N, int T)
{
    return T <= 8 && pair_tiles_pay(N);
}

template <class Fmt>
static int launch_reg_fmt(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                          int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    const int nb = (int)(K / kTq1BlockElems);
    int NW, GPW, NT;
    if (!reg_config(nb, T, NW, GPW, NT))
        return BQM_ERR_SHAPE;
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (NT == 2)
        return NW == 8 ? launch_reg<Fmt, 8, 1, 2>(wp, ap, y, r, isums, N, nb, T, stream)
                       : launch_reg<Fmt, 16, 1, 2>(wp, ap, y, r, isums, N, nb, T, stream);
    if (use_pair(N, T))
        return NW == 8 ? launch_reg<Fmt, 8, 1, 1, true>(wp, ap, y, r, isums, N, nb, T, stream)
                       : launch_reg<Fmt, 16, 1, 1, true>(wp, ap, y, r, isums, N, nb, T, stream);
    return NW == 8 ? launch_reg<Fmt, 8, 1, 1>(wp, ap, y, r, isums, N, nb, T, stream)
                   : launch_reg<Fmt, 16, 1, 1>(wp, ap, y, r, isums, N, nb, T, stream);
}

int launch_mmvq_mfma_reg(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                         int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_reg_fmt<Tq1Tile>(w, a, y, isums, N, K, T, stream, r);
}

int launch_mmvq_mfma_reg_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                             int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_reg_fmt<Tq2Tile>(w, a, y, isums, N, K, T, stream, r);
}

}  // namespace bqm
