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

// A lane's 16-byte store; NT marks it non-temporal (streamed past the
// caches), which pays on outputs well inside the last-level cache.
template <bool NT>
__device__ __forceinline__ void store16(void *__restrict__ p, u32x4 v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, static_cast<u32x4 *>(p));
    else
        *static_cast<u32x4 *>(p) = v;
}

// Store the four values d * (u - 1) of the digit bytes of `u` at out + e
// (fp32).
template <bool NT>
__device__ __forceinline__ void store_run_f32(void *__restrict__ out, int64_t e, uint32_t u, float d)
{
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        v[k] = d * (float)((int)((u >> (8 * k)) & 0xffu) - 1);
    store16<NT>(static_cast<float *>(out) + e, (u32x4){__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                       __float_as_uint(v[2]), __float_as_uint(v[3])});
}

// The two dwords of 16-bit patterns for the four digit bytes of u.
__device__ __forceinline__ u32x2 half_patterns(uint32_t u, const HalfTable &tab)
{
    // selector bytes (2u, 2u + 1) pick the element's pattern from the table
    const uint32_t u2 = u + u;
    const uint32_t s01 = __builtin_amdgcn_perm(0u, u2, 0x0c010c00u) * 0x0101u + 0x01000100u;
    const uint32_t s23 = __builtin_amdgcn_perm(0u, u2, 0x0c030c02u) * 0x0101u + 0x01000100u;
    return (u32x2){__builtin_amdgcn_perm(tab.hi, tab.lo, s01), __builtin_amdgcn_perm(tab.hi, tab.lo, s23)};
}

// Store the eight 16-bit values d * (u - 1) of the digit bytes of ua
// (elements e..e+3) and ub (e+4..e+7) at out + e: 16 bytes per lane.
template <bool NT>
__device__ __forceinline__ void store_run8(void *__restrict__ out, int64_t e, uint32_t ua,
                                           uint32_t ub, const HalfTable &tab)
{
    const u32x2 a = half_patterns(ua, tab), b2 = half_patterns(ub, tab);
    store16<NT>(static_cast<uint16_t *>(out) + e, (u32x4){a.x, a.y, b2.x, b2.y});
}

// Per-16-bit-lane multipliers of digit level c (0..4) of a qs dword, or (qh)
// of a qh dword: X1 holds v / 3^k with k = 4 (qs) or 3 (qh), so
// floor(v / 3^c) is byte 1 of X1 * 3^(k-c), and floor(v / 3^(c+1)) of
// X1 * 3^(k-c-1) (a zero multiplier past the top digit). Computed once per
// lane: the level of a lane's elements is the same in every block.
struct LevelMuls {
    uint32_t cur, next;  // both 16-bit lanes carry the multiplier
};

__device__ __forceinline__ uint32_t pow3_lanes(int p)
{
    const uint32_t m = p < 0 ? 0u : p == 0 ? 1u : p == 1 ? 3u : p == 2 ? 9u : p == 3 ? 27u : 81u;
    return m * 0x00010001u;
}

__device__ __forceinline__ LevelMuls level_muls(int c, bool qh)
{
    const int k = qh ? 3 : 4;
    return LevelMuls{pow3_lanes(k - c), pow3_lanes(k - c - 1)};
}

// The digits of one level of the four bytes of w (a qs dword, or a qh dword
// when qh): floor(v / 3^c) - 3 floor(v / 3^(c+1)) per byte.
__device__ __forceinline__ uint32_t digit_level(uint32_t w, LevelMuls lm, bool qh)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);  // bytes 1, 3 -> lanes
    const uint32_t mul = qh ? kQhMul : kQsMul, add = qh ? kQhAdd : kQsAdd;
    const uint32_t shift = qh ? kQhShift : kQsShift;
    const uint32_t e1 = pk_shr(__umul24(e, mul) + add, shift);
    const uint32_t o1 = pk_shr(__umul24(o, mul) + add, shift);
    const uint32_t f_c = hi_bytes(pk_mul_lanes(o1, lm.cur), pk_mul_lanes(e1, lm.cur));
    const uint32_t f_n = hi_bytes(pk_mul_lanes(o1, lm.next), pk_mul_lanes(e1, lm.next));
    return f_c - mul3_bytes(f_n);
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
// whole wave, into that block's 64-byte LDS slot (its bytes at s .. s + 53;
// slot bytes 60..63 are past them in either case and carry s). The stores:
//   fp16 / bf16: step k (BPW / 2 steps) covers blocks 2k and 2k + 1, lane L
//     writing elements 8 (L mod 32) .. +7 of block 2k + L / 32: one digit
//     level of two consecutive qs dwords, or two levels of the qh dword;
//   fp32: step k covers block k, lane L writing elements 4L .. 4L + 3, one
//     digit level of one dword.
// Each lane stores 16 bytes per step and a wave's step is one contiguous
// 1 KiB run of the output.
template <int DT, int BPW, bool NT>
__global__ __launch_bounds__(256) void tq1_dequantize_kernel(const uint8_t *__restrict__ w,
                                                             const int32_t *__restrict__ rows,
                                                             void *__restrict__ out, int64_t N,
                                                             int nb, int64_t n_rows)
{
    constexpr bool kF32 = DT == BQM_DTYPE_F32;
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
        // 4 BPW, load nothing (their slots are never read)
        const int t = lane + 64 * q;
        const int64_t blk = first + (t >> 2);
        const bool in = t < 4 * BPW && blk < nblocks;
        // output block -> (result row i, block B); fewer than 2^27 blocks
        const uint32_t ub = in ? (uint32_t)blk : 0u;
        const uint32_t i = ub / (uint32_t)nb, B = ub - i * (uint32_t)nb;
        int64_t r = rows ? rows[i] : i;
        r = r < 0 ? 0 : (r >= N ? N - 1 : r);  // ids outside [0, N) stay inside w
        const uint32_t off = (uint32_t)((r * nb + B) * kTq1BlockBytes);
        const uint32_t sh = off & 3u;
        u32x4 x = ld_b128(rw, in ? off - sh + 16u * (t & 3) : kIdleLoadOffset);
        if ((t & 3) == 3)
            x.w = sh;
        if (t < 4 * BPW)
            slots[wid][t] = x;
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t *slot0 = reinterpret_cast<const uint32_t *>(&slots[wid][0]);
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
        const LevelMuls lm = level_muls(c, qh);
#pragma unroll
        for (int k = 0; k < BPW; k++) {
            const int64_t blk = first + k;
            if (blk < nblocks) {
                const uint32_t *sl = slot0 + 16 * k;
                const uint32_t sh = sl[15];
                const uint32_t dd = sl[13];
                const uint32_t d16 = sh ? (dd >> 16) : (dd & 0xffffu);
                const uint32_t u = digit_level(align_bytes(sl[j + 1], sl[j], sh), lm, qh);
                store_run_f32<NT>(out, blk * kTq1BlockElems + e0, u, f16_bits_to_f32(d16));
            }
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
        // dwords jj .. jj + 2 cover the lane's bytes (qh lanes: 11 .. 13, the
        // block's last dword at most)
        const int jj = qh ? 11 : j;
        const LevelMuls lma = level_muls(c, qh), lmb = level_muls(qh ? c + 1 : c, qh);
#pragma unroll
        for (int k = 0; k < BPW / 2; k++) {
            const int64_t blk = first + 2 * k + half;
            if (blk < nblocks) {
                const uint32_t *sl = slot0 + 16 * (2 * k + half);
                const uint32_t sh = sl[15];
                const uint32_t dd = sl[13];
                const uint32_t x0 = sl[jj], x1 = sl[jj + 1], x2 = sl[jj + 2];
                const uint32_t d16 = sh ? (dd >> 16) : (dd & 0xffffu);
                const float d = f16_bits_to_f32(d16);
                const uint32_t w0 = align_bytes(x1, x0, sh);
                const uint32_t w1 = align_bytes(x2, x1, sh);
                // qh (w1 is the qh dword): levels c and c + 1 of it; else
                // level c of the two dwords
                const uint32_t ua = digit_level(qh ? w1 : w0, lma, qh);
                const uint32_t ub = digit_level(w1, lmb, qh);
                store_run8<NT>(out, blk * kTq1BlockElems + e0, ua, ub, half_table<DT>(d, d16));
            }
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
