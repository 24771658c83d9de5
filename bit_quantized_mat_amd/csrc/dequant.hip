// dequant.hip -- TQ1_0 dequantization and row gather on gfx950.
//
// The two operations beside the mat-vec in "CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract" ("Current behavior": a
// TQ1_0 dequantize kernel; "Proposed approach": the Vulkan work covering
// dequant and get_rows): out[i][k] = fp32(d) * trit for source row rows[i]
// (or i), written as fp32, fp16 or bf16.
//
// Elements in order: for fp16 and bf16 half a wave per 256-element block,
// lane L writing elements 8L..8L+7 of its block; for fp32 a wave per block,
// lane L writing 4L..4L+3. Either way a lane stores 16 bytes and a wave's
// store is one contiguous 1 KiB run. Four consecutive elements are one digit
// level c of one packed dword (the element map in include/bqm.h puts four
// consecutive elements on four consecutive bytes), so the lane reads its
// dwords (from its block's LDS copy: a wave loads its blocks with one
// coalesced 16-byte load per lane) and extracts only that level: with
// X = v / 3^k in 8.8 fixed point
// per 16-bit lane (tq1_decode.hpp), floor(v / 3^c) is byte 1 of X * 3^(k - c),
// and the digit is floor(v / 3^c) - 3 floor(v / 3^(c+1)).
#include "launch.hpp"
#include "tq1_decode.hpp"

namespace bqm {

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    const uint32_t x = __float_as_uint(f);
    return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

// The three values an element can take, d * (u - 1) for digit u = 0, 1, 2,
// as 16-bit patterns (fp16 or bf16 of the fp32 products; -d is the negated
// pattern, and d * 0 is a zero with d's sign): a byte-permute table,
// t_lo = [-d | d * 0] (bytes 0..3), t_hi = [d | -] (bytes 4..7).
struct HalfTable {
    uint32_t lo, hi;
};

template <int DT>
__device__ __forceinline__ HalfTable half_table(float d, uint32_t d16)
{
    // fp16 output: d itself is an fp16 value, so its pattern is the scale's
    const uint32_t pd = DT == BQM_DTYPE_F16 ? d16 : f32_to_bf16_bits(d);
    const uint32_t nd = pd ^ 0x8000u, zd = pd & 0x8000u;
    return HalfTable{nd | (zd << 16), pd};
}

// Per-16-bit-lane constants of digit level c (0..4) of a qs dword, or (qh)
// of a qh dword. The lanes hold X1, v / 3^k in 8.8 fixed point (k = 4 for
// qs bytes, 3 for qh; tq1_decode.hpp), whose multiples X1 * 3^m have
// floor(v / 3^(k-m)) in byte 1. Below the top level, X = X1 * 3^(k-c-1) is
// 256 floor(v / 3^(c+1)) + f, and floor(v / 3^c) = 3 floor(v / 3^(c+1)) +
// floor(3 f / 256): the digit is floor(3 f / 256), byte 1 of 3 (X & 0xff).
// At the top level c = k the digit is byte 1 of X1 itself. So
// Y = ((X1 * m1) & mask) * m2 carries the digit in byte 1 of each 16-bit
// lane, with (m1, mask, m2) = (3^(k-c-1), 0xff, 3) below the top and
// (1, 0xffff, 1) at it. Computed once per lane: a lane's level is the same
// in every block.
struct LevelConsts {
    uint32_t m1, mask, m2;  // both 16-bit lanes carry each constant
};

__device__ __forceinline__ LevelConsts level_consts(int c, bool qh)
{
    const int p = (qh ? 3 : 4) - c - 1;
    if (p < 0)
        return LevelConsts{0x00010001u, 0xffffffffu, 0x00010001u};
    const uint32_t m = p == 0 ? 1u : p == 1 ? 3u : p == 2 ? 9u : 27u;
    return LevelConsts{m * 0x00010001u, kLaneMask, 3u * 0x00010001u};
}

// The digits of one level of the four bytes of w, in byte 1 of the 16-bit
// lanes of ye (source bytes 0 and 2) and yo (source bytes 1 and 3).
struct DigitLanes {
    uint32_t ye, yo;
};

__device__ __forceinline__ DigitLanes digit_lanes(uint32_t w, LevelConsts lc, bool qh)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);  // bytes 1, 3 -> lanes
    const uint32_t mul = qh ? kQhMul : kQsMul, add = qh ? kQhAdd : kQsAdd;
    const uint32_t shift = qh ? kQhShift : kQsShift;
    const uint32_t e1 = pk_shr(__umul24(e, mul) + add, shift);
    const uint32_t o1 = pk_shr(__umul24(o, mul) + add, shift);
    return DigitLanes{pk_mul_lanes(pk_mul_lanes(e1, lc.m1) & lc.mask, lc.m2),
                      pk_mul_lanes(pk_mul_lanes(o1, lc.m1) & lc.mask, lc.m2)};
}

// The 16-bit values of the four elements of `dl` from the table: a
// byte-permute selector per pair of elements, bytes (2u, 2u + 1) of the
// table for each element's digit u.
__device__ __forceinline__ u32x2 half_values(DigitLanes dl, HalfTable tab)
{
    const uint32_t p01 = __builtin_amdgcn_perm(dl.yo, dl.ye, 0x05050101u);  // u0 u0 u1 u1
    const uint32_t p23 = __builtin_amdgcn_perm(dl.yo, dl.ye, 0x07070303u);  // u2 u2 u3 u3
    const uint32_t s01 = (p01 << 1) + 0x01000100u, s23 = (p23 << 1) + 0x01000100u;
    return (u32x2){__builtin_amdgcn_perm(tab.hi, tab.lo, s01),
                   __builtin_amdgcn_perm(tab.hi, tab.lo, s23)};
}

// The four fp32 values d * (u - 1) of the elements of `dl`.
__device__ __forceinline__ u32x4 f32_values(DigitLanes dl, float d)
{
    const uint32_t u = __builtin_amdgcn_perm(dl.yo, dl.ye, 0x07030501u);  // u0 u1 u2 u3
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        v[k] = d * (float)((int)((u >> (8 * k)) & 0xffu) - 1);
    return (u32x4){__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3])};
}

// Blocks per wave: 32 from kDqHugeBlocks blocks and 16 from kDqLargeBlocks
// (a wave's loads are one or two instructions whatever the count, so fewer,
// longer waves: 14336 x 4096 to fp16 22.8 us at 32 against 23.3-24.3 at 16,
// to fp32 37.0 against 39.7; 4096 x 4096 to fp16 slower at 32, 9.7 against
// 9.0, too few waves), fewer on smaller calls, for more waves: 8 below
// kDqLargeBlocks, 4 below kDqMidBlocks, 2 below kDqSmallBlocks.
constexpr int64_t kDqHugeBlocks = 131072;
constexpr int64_t kDqLargeBlocks = 65536;
constexpr int64_t kDqMidBlocks = 16384;
constexpr int64_t kDqSmallBlocks = 4096;

// One wave per BPW consecutive blocks of the output (rows i of the result in
// order, or of w when rows is null). The loads: lane L < 4 BPW reads bytes
// [16 (L mod 4), +16) of block L / 4 counted from the dword holding its first
// byte (s = its offset mod 4, 0 or 2), one 16-byte load per lane for the
// whole wave; each lane realigns its 16 bytes to the block's first byte with
// the next lane's first dword, and the block's 64-byte LDS slot receives its
// 13 dwords of digits (qs, then qh), the scale's dword, and in the last two
// dwords (past the block) the values the output takes: the two dwords of a
// HalfTable, or fp32 d. The stores:
//   fp16 / bf16: step k (BPW / 2 steps) covers blocks 2k and 2k + 1, lane L
//     writing elements 8 (L mod 32) .. +7 of block 2k + L / 32: one digit
//     level of two consecutive qs dwords, or two levels of the qh dword;
//   fp32: step k covers block k, lane L writing elements 4L .. 4L + 3, one
//     digit level of one dword.
// Each lane stores 16 bytes per step and a wave's step is one contiguous
// 1 KiB run of the output, through a buffer resource over the wave's part of
// the output (stores past the last block fall outside it and are dropped:
// the whole offset is the lane's vector offset, which the range check
// covers).
template <int DT, int BPW, bool NT>
__global__ __launch_bounds__(256) void tq1_dequantize_kernel(const uint8_t *__restrict__ w,
                                                             const int32_t *__restrict__ rows,
                                                             void *__restrict__ out, int64_t N,
                                                             int nb, int64_t n_rows)
{
    constexpr bool kF32 = DT == BQM_DTYPE_F32;
    constexpr int kEsz = kF32 ? 4 : 2;
    __shared__ u32x4 slots[4][4 * BPW];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    const int64_t nblocks = n_rows * nb;
    const int64_t first = wave * BPW;
    if (first >= nblocks)
        return;  // whole waves
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
#pragma unroll
    for (int q = 0; q < (4 * BPW + 63) / 64; q++) {
        // chunk t of the wave's slots; blocks past the end, and chunks past
        // 4 BPW, load nothing (their slots are never stored)
        const int t = lane + 64 * q;
        const int64_t blk = first + (t >> 2);
        const bool in = t < 4 * BPW && blk < nblocks;
        // output block -> (result row i, block B); fewer than 2^27 blocks
        const uint32_t ub = in ? (uint32_t)blk : 0u;
        const uint32_t i = ub / (uint32_t)nb, B = ub - i * (uint32_t)nb;
        // (signed: a negative id must not turn into a large unsigned one)
        int64_t r = rows ? (int64_t)rows[i] : (int64_t)i;
        r = r < 0 ? 0 : (r >= N ? N - 1 : r);  // ids outside [0, N) stay inside w
        const uint32_t off = (uint32_t)((r * nb + B) * kTq1BlockBytes);
        const uint32_t sh = off & 3u;
        const u32x4 x = ld_b128(rw, in ? off - sh + 16u * (t & 3) : kIdleLoadOffset);
        // the next lane's first dword (row shift left by one lane; the last
        // lane of a row gets 0, and only feeds bytes past its block)
        const uint32_t nx = (uint32_t)__builtin_amdgcn_mov_dpp((int)x.x, 0x101, 0xf, 0xf, true);
        u32x4 a = {align_bytes(x.y, x.x, sh), align_bytes(x.z, x.y, sh),
                   align_bytes(x.w, x.z, sh), align_bytes(nx, x.w, sh)};
        if ((t & 3) == 3) {
            // block bytes 48..63: the qh dword, the scale, then the values
            const uint32_t d16 = a.y & 0xffffu;
            const float d = f16_bits_to_f32(d16);
            if constexpr (kF32) {
                a.w = __float_as_uint(d);
            } else {
                const HalfTable tab = half_table<DT>(d, d16);
                a.z = tab.lo;
                a.w = tab.hi;
            }
        }
        if (t < 4 * BPW)
            slots[wid][t] = a;
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t *slot0 = reinterpret_cast<const uint32_t *>(&slots[wid][0]);
    // the wave's part of the output
    const int64_t left = (nblocks - first) * kTq1BlockElems * kEsz;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(static_cast<uint8_t *>(out) + first * kTq1BlockElems * kEsz,
                  (uint64_t)(left < BPW * kTq1BlockElems * kEsz ? left : BPW * kTq1BlockElems * kEsz));
    constexpr int kAux = NT ? 2 : 0;  // nt: streamed past the caches
    if constexpr (kF32) {
        // elements 4L..4L+3: their dword and digit level
        const int e0 = 4 * lane;
        int j, c;
        if (e0 < 160) {
            j = lane & 7;
            c = e0 >> 5;
        } else if (e0 < 240) {
            j = 8 + (((e0 - 160) & 15) >> 2);
            c = (e0 - 160) >> 4;
        } else {
            j = 12;
            c = lane - 60;
        }
        const bool qh = j == 12;
        const LevelConsts lc = level_consts(c, qh);
#pragma unroll
        for (int k = 0; k < BPW; k++) {
            const uint32_t *sl = slot0 + 16 * k;
            const u32x4 v = f32_values(digit_lanes(sl[j], lc, qh), __uint_as_float(sl[15]));
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, 16 * lane + 1024 * k, 0, kAux);
        }
    } else {
        const int lp = lane & 31, half = lane >> 5;
        const int e0 = 8 * lp;
        int j, c;  // first dword and digit level of the lane's elements
        if (e0 < 160) {
            j = 2 * (lp & 3);
            c = lp >> 2;
        } else if (e0 < 240) {
            j = 8 + 2 * ((lp - 20) & 1);
            c = (lp - 20) >> 1;
        } else {
            j = 12;
            c = 2 * (lp - 30);
        }
        const bool qh = j == 12;
        // qs lanes: level c of dwords j and j + 1; qh lanes: levels c and
        // c + 1 of the qh dword
        const int ja = j, jb = qh ? j : j + 1;
        const LevelConsts la = level_consts(c, qh), lb = level_consts(qh ? c + 1 : c, qh);
        const uint32_t *sw = slot0 + 16 * half;
#pragma unroll
        for (int k = 0; k < BPW / 2; k++) {
            const uint32_t *sl = sw + 32 * k;
            const HalfTable tab = {sl[14], sl[15]};
            const u32x2 va = half_values(digit_lanes(sl[ja], la, qh), tab);
            const u32x2 vb = half_values(digit_lanes(sl[jb], lb, qh), tab);
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){va.x, va.y, vb.x, vb.y}, ro,
                                                   512 * half + 2 * e0 + 1024 * k, 0, kAux);
        }
    }
}

// Outputs below kDqStreamBytes are stored non-temporally (4096 x 4096 to
// fp16 9.0 -> 7.3 us, a 1024-row fp16 gather from 14336 x 4096 4.65 -> 4.0
// us; 14336 x 4096 to fp32 39.7 -> 46.8 us the other way).
constexpr int64_t kDqStreamBytes = 64ll << 20;

template <int DT, int BPW>
static void launch_dq(const uint8_t *w, const int32_t *rows, void *out, int64_t N, int nb,
                      int64_t n_rows, hipStream_t stream)
{
    const int64_t blocks = n_rows * nb;
    const int64_t waves = (blocks + BPW - 1) / BPW;
    const dim3 grid((unsigned)((waves + 3) / 4));
    const int64_t out_bytes = blocks * kTq1BlockElems * (DT == BQM_DTYPE_F32 ? 4 : 2);
    if (out_bytes < kDqStreamBytes)
        hipLaunchKernelGGL((tq1_dequantize_kernel<DT, BPW, true>), grid, dim3(256), 0, stream, w,
                           rows, out, N, nb, n_rows);
    else
        hipLaunchKernelGGL((tq1_dequantize_kernel<DT, BPW, false>), grid, dim3(256), 0, stream, w,
                           rows, out, N, nb, n_rows);
}

template <int DT>
static void launch_dq_sized(const uint8_t *w, const int32_t *rows, void *out, int64_t N, int nb,
                            int64_t n_rows, hipStream_t stream)
{
    const int64_t blocks = n_rows * nb;
    if (blocks >= kDqHugeBlocks)
        launch_dq<DT, 32>(w, rows, out, N, nb, n_rows, stream);
    else if (blocks >= kDqLargeBlocks)
        launch_dq<DT, 16>(w, rows, out, N, nb, n_rows, stream);
    else if (blocks >= kDqMidBlocks)
        launch_dq<DT, 8>(w, rows, out, N, nb, n_rows, stream);
    else if (blocks >= kDqSmallBlocks)
        launch_dq<DT, 4>(w, rows, out, N, nb, n_rows, stream);
    else
        launch_dq<DT, 2>(w, rows, out, N, nb, n_rows, stream);
}

int launch_tq1_dequantize(const void *w, const int32_t *rows, void *out, int64_t N, int64_t K,
                          int64_t n_rows, int dtype, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    if (dtype == BQM_DTYPE_F32)
        launch_dq_sized<BQM_DTYPE_F32>(wp, rows, out, N, nb, n_rows, stream);
    else if (dtype == BQM_DTYPE_F16)
        launch_dq_sized<BQM_DTYPE_F16>(wp, rows, out, N, nb, n_rows, stream);
    else
        launch_dq_sized<BQM_DTYPE_BF16>(wp, rows, out, N, nb, n_rows, stream);
    return check_launch();
}

}  // namespace bqm
