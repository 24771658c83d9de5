// mmvq_staged.hpp -- device building blocks of the staged TQ1_0 x Q8_1 kernels
// (activations staged in LDS, byte-major weight decode), shared by the plain
// and the expert-routed products.
#pragma once

#include <cstddef>
#include <type_traits>

#include "launch.hpp"
#include "q8_1.hpp"
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
constexpr int kStagedMaxCols = 8;

// Staging works in batches: a lane loads the tasks base + k * nthreads + tid
// (k < kStageAhead) of a column into registers, then writes them to LDS. A
// kernel issues the first batch before its weight loads: loads retire in issue
// order, so a batch issued after the weights would wait for them.
//   Q8_1 source: a task is one Q8_1 block (q dwords, d and s); lanes past
//   the last task issue their loads at kIdleLoadOffset.
//   fp32 source: a task is 16 of the 32 elements of a Q8_1 block; two lanes
//   quantize a block together (q8_1_block_by_2: the bytes the stand-alone
//   quantize kernel would write). Every lane takes part in the pair
//   exchanges: pairs past the end (whole pairs, the task count being even)
//   redo the last one and store nothing.
template <bool F32>
struct StageBatch;

template <>
struct StageBatch<false> {
    static constexpr int kAhead = 1;
    u32x4 v0[kAhead], v1[kAhead];
    uint32_t ds[kAhead];
};

template <>
struct StageBatch<true> {
    static constexpr int kAhead = 1;
    u32x4 v[kAhead][4];
};

// Tasks of one column of cb blocks starting at block B0: 8 per block (Q8_1)
// or 16 (fp32).
template <bool F32>
__device__ __forceinline__ int stage_tasks(int cb)
{
    return cb * (F32 ? 16 : 8);
}

template <bool F32>
__device__ __forceinline__ void stage_load(StageBatch<F32> &sb, __amdgpu_buffer_rsrc_t ra,
                                           uint32_t col_off, int B0, int cb, int base, int tid,
                                           int nthreads)
{
    constexpr int kAhead = StageBatch<F32>::kAhead;
    const int tasks = stage_tasks<F32>(cb);
#pragma unroll
    for (int k = 0; k < kAhead; k++) {
        const int i = base + k * nthreads + tid;
        if constexpr (F32) {
            const int ii = i < tasks ? i : tasks - 1;
            const int g = ii >> 1, h = ii & 1;  // Q8_1 block of the chunk, its half
            const int bi = g >> 3, c = g & 7;
            const uint32_t off = col_off + (uint32_t)(((B0 + bi) * kTq1BlockElems +
                                                       c * kQ81BlockElems + 16 * h) * 4);
#pragma unroll
            for (int u = 0; u < 4; u++)
                sb.v[k][u] = ld_b128(ra, off + 16 * u);
        } else {
            // lanes past the end load nothing real (no branch around the
            // loads, so the compiler can count them) and store nothing
            const uint32_t off = i < tasks ? col_off + (uint32_t)(B0 * 8 + i) * kQ81BlockBytes
                                           : kIdleLoadOffset;
            sb.v0[k] = ld_b128(ra, off);
            sb.v1[k] = ld_b128(ra, off + 16);
            sb.ds[k] = ld_b32(ra, off + 32);
        }
    }
}

template <bool F32>
__device__ __forceinline__ void stage_store(const StageBatch<F32> &sb, uint32_t *__restrict__ act,
                                            int cb, int base, int tid, int nthreads)
{
    constexpr int kAhead = StageBatch<F32>::kAhead;
    const int tasks = stage_tasks<F32>(cb);
#pragma unroll
    for (int k = 0; k < kAhead; k++) {
        const int i = base + k * nthreads + tid;
        if constexpr (F32) {
            float xs[16];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                xs[4 * u] = __uint_as_float(sb.v[k][u].x);
                xs[4 * u + 1] = __uint_as_float(sb.v[k][u].y);
                xs[4 * u + 2] = __uint_as_float(sb.v[k][u].z);
                xs[4 * u + 3] = __uint_as_float(sb.v[k][u].w);
            }
            const Q81Part p = q8_1_block_by_2(xs);
            if (i < tasks) {
                const int g = i >> 1, h = i & 1;
                const int bi = g >> 3, c = g & 7;
                uint32_t *dst = act + bi * kActStride;
#pragma unroll
                for (int u = 0; u < 4; u++)
                    dst[8 * (4 * h + u) + c] = p.q4[u];
                if (h == 0) {
                    dst[64 + c] = __float_as_uint(f16_bits_to_f32(f32_to_f16_bits(p.d)));
                    dst[72 + c] = (uint32_t)(-p.sum);
                }
            }
        } else {
            if (i < tasks) {
                const int bi = i >> 3, c = i & 7;
                uint32_t *dst = act + bi * kActStride;
                const uint32_t q[8] = {sb.v0[k].x, sb.v0[k].y, sb.v0[k].z, sb.v0[k].w,
                                       sb.v1[k].x, sb.v1[k].y, sb.v1[k].z, sb.v1[k].w};
                int sq = 0;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    dst[8 * j + c] = q[j];
                    sq = sdot4(0x01010101u, q[j], sq);
                }
                dst[64 + c] = __float_as_uint(f16_bits_to_f32(sb.ds[k] & 0xffffu));
                dst[72 + c] = (uint32_t)(-sq);
            }
        }
    }
}

// Stage one column (cb blocks from block B0) into act. If `first` is given,
// it holds the column's first batch, already loaded.
template <bool F32>
__device__ __forceinline__ void stage_column(uint32_t *__restrict__ act, __amdgpu_buffer_rsrc_t ra,
                                             uint32_t col_off, int B0, int cb, int tid,
                                             int nthreads, const StageBatch<F32> *first)
{
    const int step = StageBatch<F32>::kAhead * nthreads;
    const int tasks = stage_tasks<F32>(cb);
    int base = 0;
    if (first) {
        stage_store<F32>(*first, act, cb, 0, tid, nthreads);
        base = step;
    }
    for (; base < tasks; base += step) {
        StageBatch<F32> sb;
        stage_load<F32>(sb, ra, col_off, B0, cb, base, tid, nthreads);
        stage_store<F32>(sb, act, cb, base, tid, nthreads);
    }
}

// Integer sums of one block (raw weights) against one staged activation column,
// with the floor-pair products (cheapest when a decoded block meets one column).
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

// A block expanded to clean digits, for reuse across several columns.
struct DigitBlock {
    uint32_t lo[8][5];   // qs dword j < 8, digit c
    uint32_t hi[4][5];   // qs dword 8 + i, digit c
    uint32_t qh[4];      // qh dword, digit c
};

__device__ __forceinline__ void expand_block(const RawBlock &raw, DigitBlock &d)
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const QsDigits u = qs_digits(raw_dword(raw, j));
#pragma unroll
        for (int c = 0; c < 5; c++)
            d.lo[j][c] = u.U[c];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const QsDigits u = qs_digits(raw_dword(raw, 8 + i));
#pragma unroll
        for (int c = 0; c < 5; c++)
            d.hi[i][c] = u.U[c];
    }
    const QhDigits h = qh_digits(raw_dword(raw, 12));
#pragma unroll
    for (int c = 0; c < 4; c++)
        d.qh[c] = h.U[c];
}

// Integer sums of an expanded block against one staged activation column.
// Element map (see include/bqm.h): digit c of qs dword j < 8 is dword j of
// sub-block c; digits 0..4 of qs dword 8+i are dwords i, 4+i of sub-block 5,
// i, 4+i of sub-block 6 and i of sub-block 7; digit c of qh is dword 4+c of
// sub-block 7.
__device__ __forceinline__ void digit_sums_staged(const DigitBlock &d,
                                                  const uint32_t *__restrict__ ab, int (&isum)[8])
{
#pragma unroll
    for (int c = 0; c < 8; c++)
        isum[c] = (int)ab[72 + c];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint4 lo = *reinterpret_cast<const uint4 *>(ab + 8 * j);
        const uint32_t q4 = ab[8 * j + 4];
        isum[0] = sdot4(d.lo[j][0], lo.x, isum[0]);
        isum[1] = sdot4(d.lo[j][1], lo.y, isum[1]);
        isum[2] = sdot4(d.lo[j][2], lo.z, isum[2]);
        isum[3] = sdot4(d.lo[j][3], lo.w, isum[3]);
        isum[4] = sdot4(d.lo[j][4], q4, isum[4]);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint4 a = *reinterpret_cast<const uint4 *>(ab + 8 * i + 4);        // sb 4..7, dword i
        const uint4 b = *reinterpret_cast<const uint4 *>(ab + 8 * (4 + i) + 4);  // sb 4..7, dword 4+i
        isum[5] = sdot4(d.hi[i][0], a.y, isum[5]);
        isum[5] = sdot4(d.hi[i][1], b.y, isum[5]);
        isum[6] = sdot4(d.hi[i][2], a.z, isum[6]);
        isum[6] = sdot4(d.hi[i][3], b.z, isum[6]);
        isum[7] = sdot4(d.hi[i][4], a.w, isum[7]);
        isum[7] = sdot4(d.qh[i], b.w, isum[7]);
    }
}

// Exact sub-block sums of one block against NC staged columns (column t at
// ab0 + t * col_stride), one packed dword at a time: its clean digits meet
// every column before the next dword is expanded, so no expanded block stays
// live (about 60 registers where a whole DigitBlock takes 64 on its own).
template <int NC>
__device__ __forceinline__ void dword_sums_staged(const RawBlock &raw,
                                                  const uint32_t *__restrict__ ab0, int col_stride,
                                                  int (&isum)[NC][8])
{
#pragma unroll
    for (int t = 0; t < NC; t++)
#pragma unroll
        for (int c = 0; c < 8; c++)
            isum[t][c] = (int)ab0[t * col_stride + 72 + c];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const QsDigits u = qs_digits(raw_dword(raw, j));
#pragma unroll
        for (int t = 0; t < NC; t++) {
            const uint32_t *ab = ab0 + t * col_stride;
            const uint4 lo = *reinterpret_cast<const uint4 *>(ab + 8 * j);
            const uint32_t q4 = ab[8 * j + 4];
            isum[t][0] = sdot4(u.U[0], lo.x, isum[t][0]);
            isum[t][1] = sdot4(u.U[1], lo.y, isum[t][1]);
            isum[t][2] = sdot4(u.U[2], lo.z, isum[t][2]);
            isum[t][3] = sdot4(u.U[3], lo.w, isum[t][3]);
            isum[t][4] = sdot4(u.U[4], q4, isum[t][4]);
        }
    }
    const QhDigits qh = qh_digits(raw_dword(raw, 12));
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const QsDigits u = qs_digits(raw_dword(raw, 8 + i));
#pragma unroll
        for (int t = 0; t < NC; t++) {
            const uint32_t *ab = ab0 + t * col_stride;
            const uint4 a = *reinterpret_cast<const uint4 *>(ab + 8 * i + 4);
            const uint4 b = *reinterpret_cast<const uint4 *>(ab + 8 * (4 + i) + 4);
            isum[t][5] = sdot4(u.U[0], a.y, isum[t][5]);
            isum[t][5] = sdot4(u.U[1], b.y, isum[t][5]);
            isum[t][6] = sdot4(u.U[2], a.z, isum[t][6]);
            isum[t][6] = sdot4(u.U[3], b.z, isum[t][6]);
            isum[t][7] = sdot4(u.U[4], a.w, isum[t][7]);
            isum[t][7] = sdot4(qh.U[i], b.w, isum[t][7]);
        }
    }
}

// The rows of one workgroup against T <= TC activation columns. Column t's
// Q8_1 row (fp32 row when F32: quantized while staging) starts at byte
// col_off[t] of the activation buffer ra and its outputs go to out[t][row]
// through the residual epilogue (common.hpp): plus resid[t * N + row] when
// resid is given (one fp32 addition after the product's own result), or, when
// resid is tagged as gate products, silu(gate) times the product; resid may
// be the output buffer itself.
// With a `store` functor, the row's lane 0 hands store(t, value) each
// column's result instead of writing out[t][row] (out and resid unused).
// All nthreads threads of the workgroup (its whole size) must call this (it
// synchronizes); lanes whose row is out of range only help with staging.
template <int TC, bool ISUMS, bool F32 = false, class Store = std::nullptr_t>
__device__ __forceinline__ void staged_rows(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t (&col_off)[TC],
                                            float *const (&out)[TC], const float *resid,
                                            int32_t *__restrict__ isums,
                                            uint32_t *__restrict__ act, int64_t row, bool row_ok,
                                            int64_t N, int nb, int T, int lr_log2, int chunk,
                                            int nthreads = 256, Store store = nullptr)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int Lr = 1 << lr_log2;
    const int sub = lane & (Lr - 1);
    const int nblk = nb * 8;
    const uint32_t row_off = (uint32_t)((row_ok ? row : 0) * nb * kTq1BlockBytes);
    float acc[TC];
#pragma unroll
    for (int t = 0; t < TC; t++)
        acc[t] = 0.0f;

    // one pass over the blocks [B0, B0 + chunk) of the row
    auto pass = [&](int B0) {
        const int end = min(B0 + chunk, nb);
        const int cb = end - B0;
        const int first = B0 + sub;
        if (B0 > 0)
            __syncthreads();  // readers of the previous chunk are done
        // the first column's first staging batch, then this lane's first
        // weight block: the HBM latency of the weights overlaps the activation
        // copy, and the copy does not wait for the weights. The weight load is
        // issued by every lane (lanes without a block load at
        // kIdleLoadOffset), so the compiler knows how many loads follow the
        // batch and waits for the batch alone. Later blocks of the chunk are loaded into the same
        // registers at the top of their iteration.
        // Wavefront-scope fences (no instructions) keep the compiler from
        // moving the loads across each other: it would otherwise sink the
        // batch's loads towards their first use, below the weights'.
        StageBatch<F32> head;
        stage_load<F32>(head, ra, col_off[0], B0, cb, 0, tid, nthreads);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        RawBlock cur = load_raw_block(rw, row_ok && first < end
                                              ? row_off + (uint32_t)first * kTq1BlockBytes
                                              : kIdleLoadOffset);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // and no arithmetic on the batch (with its wait) moves up between
        // the weight loads
        __builtin_amdgcn_sched_barrier(0);
        stage_column<F32>(act, ra, col_off[0], B0, cb, tid, nthreads, &head);  // T >= 1
#pragma unroll
        for (int t = 1; t < TC; t++)
            if (t < T)
                stage_column<F32>(act + t * cb * kActStride, ra, col_off[t], B0, cb, tid, nthreads,
                                  nullptr);
        __syncthreads();
        // one block of the row against the staged columns, into ac[]
        auto block_terms = [&](const RawBlock &blk, float (&ac)[TC], int B) {
            const float dw = f16_bits_to_f32(raw_scale_bits(blk));
            DigitBlock d;
            if (TC > 2)
                expand_block(blk, d);
            // two columns (T == 2 exactly): one dword's digits at a time
            int isum2[2][8];
            if (TC == 2) {
                dword_sums_staged<2>(blk, act + (B - B0) * kActStride, cb * kActStride, isum2);
                // the exact sums pass through an empty asm statement
                // before their fp32 terms: without it the compiler
                // reshapes the products around the conversions and needs
                // over 250 registers
#pragma unroll
                for (int t = 0; t < 2; t++)
#pragma unroll
                    for (int b = 0; b < 8; b++)
                        asm volatile("" : "+v"(isum2[t][b]));
            }
#pragma unroll
            for (int t = 0; t < TC; t++) {
                if (t < T) {
                    const uint32_t *ab = act + (t * cb + (B - B0)) * kActStride;
                    int isum[8];
                    if (TC == 1)
                        block_sums_staged(blk, ab, isum);
                    else if (TC == 2)
#pragma unroll
                        for (int b = 0; b < 8; b++)
                            isum[b] = isum2[t][b];
                    else
                        digit_sums_staged(d, ab, isum);
                    if (ISUMS) {
                        int32_t *dst = isums + ((int64_t)t * N + row) * nblk + 8 * B;
#pragma unroll
                        for (int b = 0; b < 8; b++)
                            dst[b] = isum[b];
                    } else {
                        float da[8];
#pragma unroll
                        for (int b = 0; b < 8; b++)
                            da[b] = __uint_as_float(ab[64 + b]);
                        ac[t] = fmaf(dw, block_dot_f32(isum, da), ac[t]);
                    }
                }
            }
        };
        if (row_ok) {
            for (int B = first; B < end; B += Lr) {
                if (B != first)
                    cur = load_raw_block(rw, row_off + (uint32_t)B * kTq1BlockBytes);
                block_terms(cur, acc, B);
            }
        }
    };
    // rows that fit one pass take straight-line code: with no loop around
    // it, the compiler knows exactly which loads are in flight at each wait
    if (chunk >= nb) {
        pass(0);
    } else {
        for (int B0 = 0; B0 < nb; B0 += chunk)
            pass(B0);
    }
    if (!ISUMS) {
        // butterfly over the Lr lanes of the row (every lane of the wave takes part)
#pragma unroll
        for (int t = 0; t < TC; t++)
            acc[t] = row_sum(acc[t], lr_log2);
        if (row_ok && sub == 0) {
#pragma unroll
            for (int t = 0; t < TC; t++)
                if (t < T) {
                    if constexpr (std::is_same_v<Store, std::nullptr_t>)
                        // gate-up calls come here from three columns (TC 4, 8)
                        out[t][row] = epilogue<(TC > 2)>(acc[t], resid, (int64_t)t * N + row);
                    else
                        store(t, acc[t]);
                }
        }
    }
}

// Blocks staged per pass: all of a row's blocks if they fit (rows with fewer
// blocks than lanes leave the surplus lanes idle), else the largest multiple
// of the lanes per row, at most 128, whose T staged columns fit lds_budget
// bytes; 0 if not even one multiple fits.
inline int staged_chunk(int nb, int lr, int T, size_t lds_budget)
{
    const int Lr = 1 << lr;
    auto fits = [&](int c) { return (size_t)T * c * kActStride * 4 <= lds_budget; };
    if (nb <= Lr)
        return fits(nb) ? nb : 0;
    int chunk = (nb < kMaxChunkBlocks ? nb : kMaxChunkBlocks) / Lr * Lr;
    while (chunk >= Lr && !fits(chunk))
        chunk -= Lr;
    return chunk >= Lr ? chunk : 0;
}

}  // namespace bqm
