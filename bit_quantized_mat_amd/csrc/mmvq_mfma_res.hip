// mmvq_mfma_res.hip -- TQ1_0 (and TQ2_0) x Q8_1 product for many activation
// columns on gfx950, matrix cores, with every activation column resident in
// LDS.
//
// Same arithmetic as the streamed matrix-core kernel (mmvq_mfma.hip): digit
// operands decoded in registers, one v_mfma_i32_16x16x32_i8 per sub-block,
// -sum q from an all -1 operand, the staged kernels' fp32 order. What differs
// is where the activations live. The grid holds one workgroup per compute
// unit at most; each workgroup first copies all T Q8_1 columns into LDS, laid
// out as the matrix-core B operands (lane-contiguous 8-byte pieces, so every
// operand read is one conflict-free ds_read_b64) plus each column's fp16
// sub-block scales, and then walks its row tiles, streaming only weights.
// The activations are read from L2 once per workgroup instead of once per
// block and wave ("cuda: opt-in MMVQ activation reuse across output rows"
// reuses the Q8_1 fragments across rows for the same reason).
//
// Reduction order: a row's blocks are split into Lr lane groups (block B in
// group B mod Lr); each wave owns Lr / NW groups, accumulates each group's
// blocks in order and combines its own groups by the xor butterfly; the
// waves' partial sums then go through LDS, and every wave combines 16 of the
// tile's outputs per pass by the remaining butterfly levels (four lanes per
// output). The result is bitwise the staged kernel's.
//
// The weight format enters through a policy (Tq1Tile, Tq2Tile): a lane's
// share of a block, its decode, and which q bytes of a Q8_1 block make each
// lane's B operand (so the staged operand layout follows the format).
#include <type_traits>

#include "tq2_decode.hpp"

namespace bqm {

// LDS layout, in dwords (nb blocks per row, NT column tiles of 16):
//   bq   [ct][B][b][lane] x 2   B operand of `lane` for sub-block b of block B
//        pair tiles (at most 8 columns, mfma_common.hpp): [B][b] x kPairSlot,
//        each slot [h][c] x 4 (half h of column c's sub-block) then 4 zero
//        dwords, read by the lanes of the other tile's half
//   dah  [B][c] x 4             fp16 scales of column c's sub-blocks 8B..8B+7
//   red  [DB ? 2 : 1][NW][lane][R NT 4]  partial sums of the waves
// The partial sums are double-buffered (one barrier per tile) when LDS has
// room for both halves, else single (a second barrier per tile).
constexpr int kPairSlot = 68;
__host__ __device__ inline size_t res_bq_dwords(int NT, int nb, bool pair = false)
{
    return pair ? (size_t)nb * 8 * kPairSlot : (size_t)NT * nb * 8 * 128;
}
__host__ __device__ inline size_t res_dah_dwords(int NT, int nb) { return (size_t)nb * 16 * NT * 4; }
__host__ __device__ inline size_t res_red_dwords(int NW, int NT, int R, bool db)
{
    return (size_t)(db ? 2 : 1) * NW * 64 * R * NT * 4;
}
// id: room for the expert-routed mode's two 16 NT-entry column tables
inline size_t res_lds_bytes(int NW, int NT, int R, int nb, bool db, bool id = false,
                            bool pair = false)
{
    return (res_bq_dwords(NT, nb, pair) + res_dah_dwords(NT, nb) +
            res_red_dwords(NW, NT, R, db) + (id ? 32 * NT : 0)) * 4;
}

// Store one staged Q8_1 block (block j of column c, its 36 bytes in v0, v1,
// ds) as B operands in bq and its fp16 scale in dah.
template <class Fmt, int NT>
__device__ __forceinline__ void stage_block(uint32_t *__restrict__ bq, uint32_t *__restrict__ dah,
                                            int nb, int c, int j, const u32x4 &v0, const u32x4 &v1,
                                            uint32_t ds)
{
    const int ct = c >> 4, cc = c & 15;
    const int B = j >> 3, b = j & 7;
    const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t *dst = bq + ((size_t)(ct * nb + B) * 8 + b) * 128;
#pragma unroll
    for (int kg = 0; kg < 4; kg++)
        *reinterpret_cast<u32x2 *>(dst + 2 * (16 * kg + cc)) = Fmt::operand_dwords(q, kg, b);
    reinterpret_cast<uint16_t *>(dah + ((size_t)B * 16 * NT + c) * 4)[b] = (uint16_t)ds;
}

// Copy all T activation columns into bq / dah, one Q8_1 block per thread and
// step. Column c's Q8_1 row starts at byte c * nb * 8 * 36 of ra, or, for
// expert items (ID), at byte colbase[c] (an LDS table). With RUNS (plain
// products and column chunks) above 8 columns, lane l of a wave takes
// column 8 g + (l & 7) and blocks (l >> 3) + (blockDim / 8) i: each load of a
// wave reads 8 runs of 8 consecutive blocks (288 bytes each) instead of 64
// blocks of 64 different columns, and the 8 lanes of one block store 8
// consecutive operand slots. Otherwise (few columns, or an expert item's
// 5 to 16 gathered columns) consecutive threads take consecutive columns of
// one block, which keeps every lane busy when T is not a multiple of 8.
// Columns T .. 16 NT - 1 are left as they are: they only feed output columns
// that are never stored.
template <class Fmt, int NT, bool ID, bool RUNS>
__device__ __forceinline__ void stage_all_columns(uint32_t *__restrict__ bq,
                                                  uint32_t *__restrict__ dah,
                                                  __amdgpu_buffer_rsrc_t ra, int T, int nb,
                                                  const uint32_t *colbase)
{
    const int nblk = nb * 8;
    if (RUNS && T > 8) {
        const int cl = threadIdx.x & 7, jl = (int)threadIdx.x >> 3;
        const int jstep = (int)blockDim.x >> 3;
        for (int c0 = 0; c0 < T; c0 += 8) {
            const int c = c0 + cl;
            if (c >= T)
                continue;
            const uint32_t cbase = ID ? colbase[c] : (uint32_t)c * nblk * kQ81BlockBytes;
            for (int j = jl; j < nblk; j += jstep) {
                const uint32_t off = cbase + (uint32_t)j * kQ81BlockBytes;
                const u32x4 v0 = ld_b128(ra, off);
                const u32x4 v1 = ld_b128(ra, off + 16);
                stage_block<Fmt, NT>(bq, dah, nb, c, j, v0, v1, ld_b32(ra, off + 32));
            }
        }
        return;
    }
    const int items = T * nblk;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int j = it / T, c = it - j * T;
        const int B = j >> 3, b = j & 7;
        const uint32_t off = (ID ? colbase[c] : (uint32_t)c * nblk * kQ81BlockBytes) +
                             (uint32_t)j * kQ81BlockBytes;
        const u32x4 v0 = ld_b128(ra, off);
        const u32x4 v1 = ld_b128(ra, off + 16);
        const uint32_t ds = ld_b32(ra, off + 32);
        const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const int ct = c >> 4, cc = c & 15;
        uint32_t *dst = bq + ((size_t)(ct * nb + B) * 8 + b) * 128;
#pragma unroll
        for (int kg = 0; kg < 4; kg++)
            *reinterpret_cast<u32x2 *>(dst + 2 * (16 * kg + cc)) = Fmt::operand_dwords(q, kg, b);
        reinterpret_cast<uint16_t *>(dah + ((size_t)B * 16 * NT + c) * 4)[b] = (uint16_t)ds;
    }
}

// Pair tiles: the T <= 8 columns into the pair slots (and dah), one Q8_1
// block per thread and step, consecutive threads on consecutive columns of
// one block; then the slots' zero dwords.
template <class Fmt, bool ID>
__device__ __forceinline__ void stage_pair_columns(uint32_t *__restrict__ bq,
                                                   uint32_t *__restrict__ dah,
                                                   __amdgpu_buffer_rsrc_t ra, int T, int nb,
                                                   const uint32_t *colbase)
{
    const int nblk = nb * 8;
    const int items = T * nblk;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int j = it / T, c = it - j * T;
        const int B = j >> 3, b = j & 7;
        const uint32_t off = (ID ? colbase[c] : (uint32_t)c * nblk * kQ81BlockBytes) +
                             (uint32_t)j * kQ81BlockBytes;
        const u32x4 v0 = ld_b128(ra, off);
        const u32x4 v1 = ld_b128(ra, off + 16);
        const uint32_t ds = ld_b32(ra, off + 32);
        const uint32_t q[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t *slot = bq + (size_t)j * kPairSlot;
#pragma unroll
        for (int h = 0; h < 2; h++)
            *reinterpret_cast<u32x4 *>(slot + (h * 8 + c) * 4) = Fmt::pair_dwords(q, h, b);
        reinterpret_cast<uint16_t *>(dah + ((size_t)B * 16 + c) * 4)[b] = (uint16_t)ds;
    }
    for (int j = threadIdx.x; j < nblk; j += blockDim.x)
        *reinterpret_cast<u32x4 *>(bq + (size_t)j * kPairSlot + 64) = (u32x4){0, 0, 0, 0};
}

// Work items of the item mode. Expert-routed products: the routing table the
// routing pre-pass writes (mmvq_id.hip): item k of the wide list is
// routed[2 + 3 (max_items + k) ..] = (expert, first run slot, pairs), and run
// slot s holds pair index routed[2 + 6 max_items + s]; routed[1] counts the
// wide items. Many-column products (routed == nullptr): item k is columns
// 16 NT k .. 16 NT k + 16 NT - 1 of the one matrix's a_cols columns.
struct WideItems {
    const int32_t *routed;
    int max_items;
    int pairs_per_col;  // consecutive pairs that read one activation column
};

// Fmt: the weight format policy; NW: waves per workgroup; GPW: butterfly
// groups per wave (Lr / NW); NT:
// 16-column tiles (1 or 2); R: 16-row tiles per workgroup tile; DB: partial
// sums double-buffered; ISUMS: write the exact per-sub-block sums instead of
// outputs; ID: item mode, work items of up to 16 NT columns (an expert's
// matrix against its pairs' columns, outputs y[pair][row]; or a chunk of the
// columns of a many-column product); RUNS: columns copied in runs of blocks
// (stage_all_columns; plain products and column chunks, not expert items);
// `a_cols` is the number of columns a holds (T in the plain mode); PAIR:
// pair tiles (NT = R = 1, at most 8 columns, units of 32 rows).
template <class Fmt, int NW, int GPW, int NT, int R, bool DB, bool ISUMS, bool ID, bool RUNS,
          bool PAIR = false>
__global__ __launch_bounds__(64 * NW) void mmvq_mfma_res_kernel(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ a,
                                                                float *y, const float *resid,
                                                                int32_t *__restrict__ isums,
                                                                int64_t N, int nb, int T,
                                                                int ntiles, int a_cols,
                                                                WideItems items)
{
    static_assert(!PAIR || (NT == 1 && R == 1 && !RUNS), "pair tiles: one 8-column tile");
    extern __shared__ uint32_t smem[];
    uint32_t *bq = smem;
    uint32_t *dah = smem + res_bq_dwords(NT, nb, PAIR);
    float *red = reinterpret_cast<float *>(dah + res_dah_dwords(NT, nb));
    // ID: per-column tables after the partial sums (byte offset of the token's
    // Q8_1 row, pair index)
    uint32_t *colbase = reinterpret_cast<uint32_t *>(red) + res_red_dwords(NW, NT, R, DB);
    int *colpair = reinterpret_cast<int *>(colbase + 16 * NT);
    // the wave index is uniform across the wave; saying so keeps the block
    // loop and its branches on scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    constexpr int Lr = NW * GPW;
    const int kg = lane >> 4;                   // decode lane: row lane % 16, K group kg
    const typename Fmt::Ctx ctx(kg);
    const int col = lane & 15, rg = lane >> 4;  // output lane: column col, rows 4rg..4rg+3
    const int nblk = nb * 8;
    const uint64_t w_bytes = (uint64_t)N * nb * Fmt::kBlockBytes;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)a_cols * nblk * kQ81BlockBytes);
    constexpr int kRows = PAIR ? 32 : 16 * R;  // rows per unit
    typedef typename std::conditional<PAIR, typename Fmt::PairLane, typename Fmt::Lane>::type
        LaneT;
    // PAIR: this lane's dword offset in a pair slot (the zero dwords for a
    // lane group of the other tile)
    const int pair_off = (col >> 3) == (kg >> 1) ? ((kg & 1) * 8 + (col & 7)) * 4 : 64;

    // Work units: in the plain mode the row tiles, strided over the grid; in
    // the expert mode (wide item, row tile) pairs, item-major, workgroup i
    // taking the contiguous range [i U / G, (i + 1) U / G) of the U units, so
    // that it restages columns only when its range enters the next item.
    int64_t u, u_end;
    int ustride;
    constexpr int C = 16 * NT;  // columns of a chunk (item mode, no routing table)
    if (ID) {
        const int n_items = items.routed ? items.routed[1] : (a_cols + C - 1) / C;
        const int64_t units = (int64_t)n_items * ntiles;
        u = (int64_t)blockIdx.x * units / gridDim.x;
        u_end = (int64_t)(blockIdx.x + 1) * units / gridDim.x;
        ustride = 1;
    } else {
        u = blockIdx.x;
        u_end = ntiles;
        ustride = gridDim.x;
    }
    if (u >= u_end)
        return;  // uniform
    int item = ID ? (int)(u / ntiles) : 0;
    int tile = (int)(u - (int64_t)item * ntiles);
    // the item's matrix, column count and column tables (ID)
    auto take_item = [&](int k) {
        if (!items.routed) {
            const int c0 = k * C;
            T = a_cols - c0 < C ? a_cols - c0 : C;
            if ((int)threadIdx.x < T) {
                colpair[threadIdx.x] = c0 + threadIdx.x;
                colbase[threadIdx.x] = (uint32_t)(c0 + threadIdx.x) * nblk * kQ81BlockBytes;
            }
            return make_rsrc(w, w_bytes);
        }
        // the item's fields are the same for the whole workgroup: read into
        // scalar registers, so that the weights' buffer descriptor is too
        // (a descriptor in vector registers wraps every load in a loop over
        // the lanes' distinct values)
        const int32_t *it = items.routed + 2 + 3 * (items.max_items + k);
        const int expert = __builtin_amdgcn_readfirstlane(it[0]);
        const int first = __builtin_amdgcn_readfirstlane(it[1]);
        T = __builtin_amdgcn_readfirstlane(it[2]);
        if ((int)threadIdx.x < T) {
            const int pr = items.routed[2 + 6 * items.max_items + first + threadIdx.x];
            colpair[threadIdx.x] = pr;
            colbase[threadIdx.x] =
                (uint32_t)(pr / items.pairs_per_col) * (uint32_t)nblk * kQ81BlockBytes;
        }
        return make_rsrc(w + (uint64_t)expert * w_bytes, w_bytes);
    };
    __amdgpu_buffer_rsrc_t rw = ID ? take_item(item) : make_rsrc(w, w_bytes);
    auto load_lane = [&](uint32_t off) -> LaneT {
        if constexpr (PAIR)
            return Fmt::load_pair(rw, off, kg & 1);
        else
            return Fmt::load(rw, off, kg);
    };

    // byte offsets of this decode lane's rows in tile t (rows past N read row 0)
    auto tile_rows = [&](int t, uint32_t (&ro)[R]) {
#pragma unroll
        for (int rt = 0; rt < R; rt++) {
            const int64_t rowA = (int64_t)t * kRows + (PAIR ? 16 * (kg >> 1) : 16 * rt) +
                                 (lane & 15);
            ro[rt] = (uint32_t)((rowA < N ? rowA : 0) * nb * Fmt::kBlockBytes);
        }
    };

    uint32_t row_off[R];
    LaneT lb[R];
    // the first block's weights are in flight while the activations are staged
    auto start_item = [&]() {
        tile_rows(tile, row_off);
        if (wave < nb) {
#pragma unroll
            for (int rt = 0; rt < R; rt++)
                lb[rt] = load_lane(row_off[rt] + (uint32_t)wave * Fmt::kBlockBytes);
        }
        if (ID)
            __syncthreads();  // the column tables
        if constexpr (PAIR)
            stage_pair_columns<Fmt, ID>(bq, dah, ra, T, nb, colbase);
        else
            stage_all_columns<Fmt, NT, ID, RUNS>(bq, dah, ra, T, nb, colbase);
        __syncthreads();
    };
    start_item();

    int parity = 0;
    for (;;) {
        const int64_t r0 = (int64_t)tile * kRows;
        const int64_t un = u + ustride;
        const int item_n = ID ? (int)(un / ntiles) : 0;
        const int next_tile = (int)(un - (int64_t)item_n * ntiles);
        // the next unit works on the columns staged now
        const bool next_here = un < u_end && item_n == item;
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
            const int g = wave + NW * gi;
            for (int B = g; B < nb; B += Lr) {
                // one block of lookahead: the group's next block, else the next
                // group's first, else the first block of the next tile
                const bool same_tile = B + Lr < nb || (gi + 1 < GPW && g + NW < nb);
                const int Bn = B + Lr < nb ? B + Lr : (same_tile ? g + NW : wave);
                const bool have_next = same_tile || next_here;
                // issued by every lane (at Fmt::kIdle when there is no
                // next block), so that the compiler can count the loads in
                // flight and the data is first waited for where it is decoded
                LaneT ln[R];
#pragma unroll
                for (int rt = 0; rt < R; rt++)
                    ln[rt] = load_lane(have_next ? (same_tile ? row_off[rt] : next_off[rt]) +
                                                       (uint32_t)Bn * Fmt::kBlockBytes
                                                 : Fmt::kIdle);
#pragma unroll
                for (int rt = 0; rt < R; rt++) {
                    typedef typename std::conditional<PAIR, PairOperands, TileOperands>::type OpsT;
                    OpsT op;
                    if constexpr (PAIR)
                        op = Fmt::decode_pair(lb[rt], ctx, kg & 1);
                    else
                        op = Fmt::decode(lb[rt], ctx);
                    // PAIR: the output lane's rows are in tile col / 8, whose
                    // block scales sit in the decode lanes of its half 1
                    const int dw_src = PAIR ? 4 * rg + 16 * (2 * (col >> 3) + 1) : 4 * rg;
                    float dw[4];  // block scales of the four rows this output lane holds
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        dw[i] = __shfl(op.dw, dw_src + i, 64);
#pragma unroll
                    for (int ct = 0; ct < NT; ct++) {
                        // this output lane's column scales, sub-blocks 8B .. 8B+7
                        const u32x4 dv = *reinterpret_cast<const u32x4 *>(
                            dah + ((size_t)B * 16 * NT + ct * 16 + (PAIR ? col & 7 : col)) * 4);
                        const uint32_t *bqb = bq + (size_t)(ct * nb + B) * 8 * 128 + 2 * lane;
                        float s[4];
#pragma unroll
                        for (int b = 0; b < 8; b++) {
                            // -sum(q) of this lane's column on every row, then + sum(u q)
                            i32x4 C;
                            if constexpr (PAIR) {
                                const u32x4 bv = *reinterpret_cast<const u32x4 *>(
                                    bq + (size_t)(B * 8 + b) * kPairSlot + pair_off);
                                const i32x4 Bq = (i32x4){(int)bv.x, (int)bv.y, (int)bv.z,
                                                         (int)bv.w};
                                const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                    kAllMinusOne4, Bq, (i32x4){0, 0, 0, 0}, 0, 0, 0);
                                C = __builtin_amdgcn_mfma_i32_16x16x64_i8(op.A[b], Bq, neg_sum, 0,
                                                                          0, 0);
                            } else {
                                const u32x2 bv = *reinterpret_cast<const u32x2 *>(bqb + b * 128);
                                const long Bq = (long)(((uint64_t)bv.y << 32) | bv.x);
                                const i32x4 neg_sum = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                                    kAllMinusOne, Bq, (i32x4){0, 0, 0, 0}, 0, 0, 0);
                                C = __builtin_amdgcn_mfma_i32_16x16x32_i8(op.A[b], Bq, neg_sum, 0,
                                                                          0, 0);
                            }
                            if (ISUMS) {
                                const int c = PAIR ? (col & 7) : ct * 16 + col;
#pragma unroll
                                for (int i = 0; i < 4; i++) {
                                    const int64_t row = r0 + (PAIR ? 16 * (col >> 3) : 16 * rt) +
                                                        4 * rg + i;
                                    if (c < T && row < N)
                                        isums[((int64_t)c * N + row) * nblk + 8 * B + b] = C[i];
                                }
                            } else {
                                // the staged kernels' fp32 order: s = sum_b da[b] * isum[b]
                                // from b = 0 up, then acc + dw * s
                                const float da = f16_bits_to_f32(dv[b >> 1] >> (16 * (b & 1)));
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    s[i] = b == 0 ? da * (float)C[i] : fmaf(da, (float)C[i], s[i]);
                            }
                        }
                        if (!ISUMS) {
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                acc[gi][rt][ct][i] = fmaf(dw[i], s[i], acc[gi][rt][ct][i]);
                        }
                    }
                }
#pragma unroll
                for (int rt = 0; rt < R; rt++)
                    lb[rt] = ln[rt];
            }
        }

        if (!ISUMS) {
            // butterfly levels inside the wave (the partner group differs in gi)
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
            // the levels across waves: every wave leaves its partial sums in
            // this tile's half of red, and then (kAllWavesFold) every wave
            // folds 16 of the tile's outputs per pass, four lanes per output,
            // or wave 0 folds them all. Lane j of a
            // quad takes waves j, j + 4, ...: it applies the levels of 4 and
            // up among its own values, the quad the levels 2 and 1 by DPP, so
            // that the quad's lane 0 ends with what the xor butterfly gives
            // wave 0 (level m adds wave w + m's running value to wave w's). The
            // other half belongs to the next tile, so one barrier per tile
            // suffices.
            constexpr int kPer = R * NT * 4;
            // expert items fold in wave 0 alone (the spread fold measured
            // slower there: moe 128 x 1536 x 4096, T = 64, 82.9 against
            // 84.7 us; it gains 2 to 7% on plain products and column chunks)
            constexpr bool kAllWavesFold = !ID || RUNS;
            constexpr int kWavesPerLane = NW / 4;
            constexpr int kPasses = 4 * kPer / NW;
            static_assert(NW % 4 == 0 && (4 * kPer) % NW == 0, "fold layout");
            float *half = red + (size_t)(DB ? parity : 0) * NW * 64 * kPer;
#pragma unroll
            for (int rt = 0; rt < R; rt++)
#pragma unroll
                for (int ct = 0; ct < NT; ct++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        half[((size_t)wave * 64 + lane) * kPer + (rt * NT + ct) * 4 + i] =
                            acc[0][rt][ct][i];
            __syncthreads();
            if constexpr (kAllWavesFold) {
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
                    const int rt = k / (NT * 4), ct = (k >> 2) % NT, i = k & 3;
                    const int c = PAIR ? (oc & 7) : ct * 16 + oc;
                    const int64_t row = r0 + (PAIR ? 16 * (oc >> 3) : 16 * rt) + 4 * org + i;
                    if (j == 0 && c < T && row < N) {
                        const int64_t yc = ID ? colpair[c] : c;
                        const int64_t o = yc * N + row;
                        y[o] = ID ? v : epilogue(v, resid, o);  // expert items add nothing
                    }
                }
            } else {
                if (wave == 0) {
#pragma unroll
                    for (int rt = 0; rt < R; rt++)
#pragma unroll
                        for (int ct = 0; ct < NT; ct++)
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                const int k = (rt * NT + ct) * 4 + i;
                                float v[NW];
#pragma unroll
                                for (int u = 0; u < NW; u++)
                                    v[u] = half[((size_t)u * 64 + lane) * kPer + k];
#pragma unroll
                                for (int m = NW >> 1; m >= 1; m >>= 1)
#pragma unroll
                                    for (int u = 0; u < m; u++)
                                        v[u] = v[u] + v[u + m];
                                acc[0][rt][ct][i] = v[0];
                            }
#pragma unroll
                    for (int rt = 0; rt < R; rt++)
#pragma unroll
                        for (int ct = 0; ct < NT; ct++) {
                            const int c = PAIR ? (col & 7) : ct * 16 + col;
                            if (c < T) {
                                const int64_t yc = ID ? colpair[c] : c;
#pragma unroll
                                for (int i = 0; i < 4; i++) {
                                    const int64_t row = r0 + (PAIR ? 16 * (col >> 3) : 16 * rt) +
                                                        4 * rg + i;
                                    if (row < N) {
                                        const int64_t o = yc * N + row;
                                        y[o] = ID ? acc[0][rt][ct][i]
                                                  : epilogue(acc[0][rt][ct][i], resid, o);
                                    }
                                }
                            }
                        }
                }
            }
            if (!DB)
                __syncthreads();  // the partial sums have been read
        }
#pragma unroll
        for (int rt = 0; rt < R; rt++)
            row_off[rt] = next_off[rt];
        u = un;
        tile = next_tile;
        parity ^= 1;
        if (u >= u_end)
            break;
        if (ID && item_n != item) {
            __syncthreads();  // every wave is done with this item's LDS
            item = item_n;
            rw = take_item(item);
            start_item();
        }
    }
}

template <class Fmt, int NW, int GPW, int NT, bool DB, bool PAIR = false>
static int launch_res(const uint8_t *w, const uint8_t *a, float *y, const float *r,
                      int32_t *isums, int64_t N, int nb, int T, hipStream_t stream)
{
    constexpr int R = 1;
    constexpr bool RUNS = !PAIR;
    const int64_t rows = PAIR ? 32 : 16 * R;
    const int64_t ntiles = (N + rows - 1) / rows;
    const size_t lds = res_lds_bytes(NW, NT, R, nb, DB, false, PAIR);
    const void *kt = reinterpret_cast<const void *>(
        &mmvq_mfma_res_kernel<Fmt, NW, GPW, NT, R, DB, true, false, RUNS, PAIR>);
    const void *kf = reinterpret_cast<const void *>(
        &mmvq_mfma_res_kernel<Fmt, NW, GPW, NT, R, DB, false, false, RUNS, PAIR>);
    allow_dynamic_lds(kt, lds);
    allow_dynamic_lds(kf, lds);
    const int cap = resident_workgroups(isums ? kt : kf, 64 * NW, lds);
    const dim3 grid((unsigned)(ntiles < cap ? ntiles : cap));
    const WideItems none = {nullptr, 0, 1};
    if (isums)
        hipLaunchKernelGGL((mmvq_mfma_res_kernel<Fmt, NW, GPW, NT, R, DB, true, false, RUNS, PAIR>),
                           grid, dim3(64 * NW), lds, stream, w, a, nullptr, nullptr, isums, N, nb,
                           T, (int)ntiles, T, none);
    else
        hipLaunchKernelGGL((mmvq_mfma_res_kernel<Fmt, NW, GPW, NT, R, DB, false, false, RUNS, PAIR>),
                           grid, dim3(64 * NW), lds, stream, w, a, y, r, nullptr, N, nb, T,
                           (int)ntiles, T, none);
    return check_launch();
}

// Expert-routed mode: one 16-column tile (items of at most 16 pairs), 16
// waves, a persistent grid of the workgroups the device runs at once.
template <int GPW>
static int launch_res_id(const uint8_t *w, const uint8_t *a, float *y, int64_t N, int nb,
                         int a_cols, const int32_t *routed, int max_items, int max_wide,
                         int pairs_per_col, hipStream_t stream)
{
    constexpr int NW = 16, NT = 1, R = 1;
    constexpr bool DB = true;
    const int64_t ntiles = (N + 16 * R - 1) / (16 * R);
    const size_t lds = res_lds_bytes(NW, NT, R, nb, DB, true);
    const void *k =
        reinterpret_cast<const void *>(&mmvq_mfma_res_kernel<Tq1Tile, NW, GPW, NT, R, DB, false, true, false>);
    allow_dynamic_lds(k, lds);
    const int64_t cap = resident_workgroups(k, 64 * NW, lds);
    const int64_t most = (int64_t)max_wide * ntiles;  // units when every item is in use
    const dim3 grid((unsigned)(most < cap ? most : cap));
    const WideItems items = {routed, max_items, pairs_per_col};
    hipLaunchKernelGGL((mmvq_mfma_res_kernel<Tq1Tile, NW, GPW, NT, R, DB, false, true, false>), grid,
                       dim3(64 * NW), lds, stream, w, a, y, nullptr, nullptr, N, nb, 16,
                       (int)ntiles, a_cols, items);
    return check_launch();
}

// 16 waves for one column tile, 8 for two (their register budgets); the
// column tiles' partial sums double-buffered for one tile, single for two
static int res_waves(int NT) { return NT == 1 ? 16 : 8; }

// Many-column product: chunks of 32 columns on 8 waves where they fit LDS,
// else of 16 columns on 16 waves; 0 if neither fits.
static int mm_chunk_cols(int nb)
{
    const int Lr = 1 << lanes_per_row_log2(nb);
    if (Lr >= 8 && res_lds_bytes(8, 2, 1, nb, false, true) <= lds_budget())
        return 32;
    if (Lr >= 16 && res_lds_bytes(16, 1, 1, nb, true, true) <= lds_budget())
        return 16;
    return 0;
}

bool mm_chunked_supported(int64_t K) { return mm_chunk_cols((int)(K / kTq1BlockElems)) > 0; }

template <int NW, int GPW, int NT, bool DB>
static int launch_mm(const uint8_t *w, const uint8_t *a, float *y, int64_t N, int nb, int T,
                     hipStream_t stream)
{
    constexpr int R = 1;
    const int64_t ntiles = (N + 16 * R - 1) / (16 * R);
    const size_t lds = res_lds_bytes(NW, NT, R, nb, DB, true);
    const void *k =
        reinterpret_cast<const void *>(&mmvq_mfma_res_kernel<Tq1Tile, NW, GPW, NT, R, DB, false, true, true>);
    allow_dynamic_lds(k, lds);
    const int64_t cap = resident_workgroups(k, 64 * NW, lds);
    const int64_t units = (int64_t)((T + 16 * NT - 1) / (16 * NT)) * ntiles;
    const dim3 grid((unsigned)(units < cap ? units : cap));
    const WideItems chunks = {nullptr, 0, 1};
    hipLaunchKernelGGL((mmvq_mfma_res_kernel<Tq1Tile, NW, GPW, NT, R, DB, false, true, true>), grid,
                       dim3(64 * NW), lds, stream, w, a, y, nullptr, nullptr, N, nb, 16 * NT,
                       (int)ntiles, T, chunks);
    return check_launch();
}

int launch_mm_chunked(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
                      hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int Lr = 1 << lanes_per_row_log2(nb);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (mm_chunk_cols(nb) == 32) {
        switch (Lr) {
        case 8: return launch_mm<8, 1, 2, false>(wp, ap, y, N, nb, (int)T, stream);
        case 16: return launch_mm<8, 2, 2, false>(wp, ap, y, N, nb, (int)T, stream);
        case 32: return launch_mm<8, 4, 2, false>(wp, ap, y, N, nb, (int)T, stream);
        default: return launch_mm<8, 8, 2, false>(wp, ap, y, N, nb, (int)T, stream);
        }
    }
    switch (Lr) {
    case 16: return launch_mm<16, 1, 1, true>(wp, ap, y, N, nb, (int)T, stream);
    case 32: return launch_mm<16, 2, 1, true>(wp, ap, y, N, nb, (int)T, stream);
    default: return launch_mm<16, 4, 1, true>(wp, ap, y, N, nb, (int)T, stream);
    }
}

bool mfma_resident_id_supported(int64_t K)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int Lr = 1 << lanes_per_row_log2(nb);
    return Lr >= 16 && res_lds_bytes(16, 1, 1, nb, true, true) <= lds_budget();
}

int launch_mmvq_mfma_resident_id(const void *w, const void *a, float *y, int64_t N, int64_t K,
                                 int64_t a_cols, const int32_t *routed, int max_items,
                                 int max_wide, int pairs_per_col, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int Lr = 1 << lanes_per_row_log2(nb);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    switch (Lr) {
    case 16:
        return launch_res_id<1>(wp, ap, y, N, nb, (int)a_cols, routed, max_items, max_wide,
                                pairs_per_col, stream);
    case 32:
        return launch_res_id<2>(wp, ap, y, N, nb, (int)a_cols, routed, max_items, max_wide,
                                pairs_per_col, stream);
    default:
        return launch_res_id<4>(wp, ap, y, N, nb, (int)a_cols, routed, max_items, max_wide,
                                pairs_per_col, stream);
    }
}

bool mfma_resident_supported(int64_t K, int32_t T)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int Lr = 1 << lanes_per_row_log2(nb);
    const int NT = T <= 16 ? 1 : 2;
    const int NW = res_waves(NT);
    return Lr >= NW && res_lds_bytes(NW, NT, 1, nb, NT == 1) <= lds_budget();
}

template <class Fmt>
static int launch_resident_fmt(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                               int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    const int nb = (int)(K / kTq1BlockElems);
    const int Lr = 1 << lanes_per_row_log2(nb);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const uint8_t *ap = static_cast<const uint8_t *>(a);
    if (T <= 8 && pair_tiles_pay(N)) {
        switch (Lr) {
        case 16: return launch_res<Fmt, 16, 1, 1, true, true>(wp, ap, y, r, isums, N, nb, T, stream);
        case 32: return launch_res<Fmt, 16, 2, 1, true, true>(wp, ap, y, r, isums, N, nb, T, stream);
        default: return launch_res<Fmt, 16, 4, 1, true, true>(wp, ap, y, r, isums, N, nb, T, stream);
        }
    }
    if (T <= 16) {
        switch (Lr) {
        case 16: return launch_res<Fmt, 16, 1, 1, true>(wp, ap, y, r, isums, N, nb, T, stream);
        case 32: return launch_res<Fmt, 16, 2, 1, true>(wp, ap, y, r, isums, N, nb, T, stream);
        default: return launch_res<Fmt, 16, 4, 1, true>(wp, ap, y, r, isums, N, nb, T, stream);
        }
    }
    switch (Lr) {
    case 8: return launch_res<Fmt, 8, 1, 2, false>(wp, ap, y, r, isums, N, nb, T, stream);
    case 16: return launch_res<Fmt, 8, 2, 2, false>(wp, ap, y, r, isums, N, nb, T, stream);
    case 32: return launch_res<Fmt, 8, 4, 2, false>(wp, ap, y, r, isums, N, nb, T, stream);
    default: return launch_res<Fmt, 8, 8, 2, false>(wp, ap, y, r, isums, N, nb, T, stream);
    }
}

int launch_mmvq_mfma_resident(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                              int64_t K, int32_t T, hipStream_t stream, const float *r)
{
    return launch_resident_fmt<Tq1Tile>(w, a, y, isums, N, K, T, stream, r);
}

int launch_mmvq_mfma_resident_tq2(const void *w, const void *a, float *y, int32_t *isums,
                                  int64_t N, int64_t K, int32_t T, hipStream_t stream)
{
    return launch_resident_fmt<Tq2Tile>(w, a, y, isums, N, K, T, stream, nullptr);
}

}  // namespace bqm
