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
// consecutive elements on four consecutive bytes), so the lane loads its
// dwords and extracts only that level: with X = v / 3^k in 8.8 fixed point
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

// Store the four values d * (u - 1) of the digit bytes of `u` at out + e
// (fp32).
__device__ __forceinline__ void store_run_f32(void *__restrict__ out, int64_t e, uint32_t u, float d)
{
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        v[k] = d * (float)((int)((u >> (8 * k)) & 0xffu) - 1);
    *reinterpret_cast<float4 *>(static_cast<float *>(out) + e) = make_float4(v[0], v[1], v[2], v[3]);
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
__device__ __forceinline__ void store_run8(void *__restrict__ out, int64_t e, uint32_t ua,
                                           uint32_t ub, const HalfTable &tab)
{
    const u32x2 a = half_patterns(ua, tab), b2 = half_patterns(ub, tab);
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(out) + e) = (u32x4){a.x, a.y, b2.x, b2.y};
}

// Digit level c (0..4) of the four bytes of a qs dword, or (qh) of a qh dword.
__device__ __forceinline__ uint32_t digit_level(uint32_t w, int c, bool qh)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);  // bytes 1, 3 -> lanes
    const uint32_t mul = qh ? kQhMul : kQsMul, add = qh ? kQhAdd : kQsAdd;
    const uint32_t shift = qh ? kQhShift : kQsShift;
    const uint32_t e1 = pk_shr(__umul24(e, mul) + add, shift);
    const uint32_t o1 = pk_shr(__umul24(o, mul) + add, shift);
    // X1 holds v / 3^k with k = 4 (qs) or 3 (qh): floor(v / 3^c) is byte 1 of
    // X1 * 3^(k-c); floor(v / 3^(c+1)) of X1 * 3^(k-c-1) (0 past the top digit)
    const int k = qh ? 3 : 4;
    const unsigned short pw[6] = {1, 3, 9, 27, 81, 0};
    const unsigned short m_c = pw[k - c];
    const unsigned short m_n = c + 1 <= k ? pw[k - c - 1] : (unsigned short)0;
    const uint32_t f_c = hi_bytes(pk_mul(o1, m_c), pk_mul(e1, m_c));
    const uint32_t f_n = hi_bytes(pk_mul(o1, m_n), pk_mul(e1, m_n));
    return f_c - mul3_bytes(f_n);
}

// Blocks per wave, the loads of all of them issued before any decode: fp16
// and bf16 16 on large calls (more bytes per wave to cover its HBM round
// trip); fewer, for more waves, on smaller calls of every type: 8 below
// kDqLargeBlocks blocks (fp32: from kDqMidBlocks up), 4 below kDqMidBlocks,
// 2 below kDqSmallBlocks (fp16 row gathers from a 14336 x 4096 matrix: 64
// rows 3.54 -> 2.23 us, 256 rows 3.96 -> 2.63 us, 1024 rows 5.80 -> 4.91 us,
// 2048 rows 7.85 -> 7.08 us; at 3072 rows eight blocks per wave stay faster,
// 8.9 against 9.8 us).
constexpr int kDqBlocksPerWave = 8;
constexpr int64_t kDqLargeBlocks = 65536;
constexpr int64_t kDqMidBlocks = 40960;
constexpr int64_t kDqSmallBlocks = 8192;

// fp16 and bf16 output: lane L of a wave takes elements 8 (L mod 32) .. +7 of
// block 2 k + L / 32 of its step k, a 16-byte store; a wave's store covers two
// whole blocks (1 KiB). By the element map those eight elements are one digit
// level of two consecutive qs dwords, or two levels of the qh dword.
template <int DT, int BPW>
__global__ __launch_bounds__(256) void tq1_dequantize_kernel(const uint8_t *__restrict__ w,
                                                             const int32_t *__restrict__ rows,
                                                             void *__restrict__ out, int64_t N,
                                                             int nb, int64_t n_rows)
{
    const int lane = threadIdx.x & 63;
    // wave-uniform block coordinates (scalar registers)
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nblocks = n_rows * nb;
    const int64_t first = wave * BPW;
    if (first >= nblocks)
        return;  // whole waves
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
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    constexpr int kSteps = BPW / 2;
    u32x3 v[kSteps];
    uint32_t dd[kSteps], sh[kSteps];
    int64_t blk[kSteps];
    // (row, block) of this lane's first block, then stepped by two blocks
    int64_t i = first / nb;
    int B = (int)(first - i * nb) + half;
    while (B >= nb) {
        B -= nb;
        i++;
    }
#pragma unroll
    for (int k = 0; k < kSteps; k++) {
        // blocks past the end reload the last one (their stores are skipped)
        blk[k] = first + 2 * k + half;
        const bool in = blk[k] < nblocks;
        const int64_t ic = in ? i : n_rows - 1;
        const int Bc = in ? B : nb - 1;
        B += 2;
        while (B >= nb) {
            B -= nb;
            i++;
        }
        int64_t r = rows ? rows[ic] : ic;
        r = r < 0 ? 0 : (r >= N ? N - 1 : r);  // ids outside [0, N) stay inside w
        const uint32_t off = (uint32_t)((r * nb + Bc) * kTq1BlockBytes);
        sh[k] = off & 3u;
        const uint32_t base = off - sh[k];
        // cover dwords j .. j + 2 (qh lanes: 11 .. 13, never past the block's
        // last dword)
        v[k] = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 4 * (qh ? 11 : j), 0, 0);
        dd[k] = ld_b32(rw, base + 52);
    }
#pragma unroll
    for (int k = 0; k < kSteps; k++) {
        if (blk[k] < nblocks) {
            const uint32_t d16 = sh[k] ? (dd[k] >> 16) : (dd[k] & 0xffffu);
            const float d = f16_bits_to_f32(d16);
            const uint32_t w0 = align_bytes(v[k].y, v[k].x, sh[k]);
            const uint32_t w1 = align_bytes(v[k].z, v[k].y, sh[k]);
            // qh (w1 is the qh dword): levels c and c + 1 of it; else level c
            // of the two dwords
            const uint32_t ua = digit_level(qh ? w1 : w0, c, qh);
            const uint32_t ub = digit_level(w1, qh ? c + 1 : c, qh);
            store_run8(out, blk[k] * kTq1BlockElems + e0, ua, ub, half_table<DT>(d, d16));
        }
    }
}

// fp32 output: one wave per block, lane L writing elements 4L..4L+3 (one
// 16-byte store per lane, a wave's store 1 KiB of consecutive outputs).
template <int BPW>
__global__ __launch_bounds__(256) void tq1_dequantize_f32_kernel(const uint8_t *__restrict__ w,
                                                                 const int32_t *__restrict__ rows,
                                                                 void *__restrict__ out, int64_t N,
                                                                 int nb, int64_t n_rows)
{
    const int lane = threadIdx.x & 63;
    // wave-uniform block coordinates (scalar registers)
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nblocks = n_rows * nb;
    const int64_t first = wave * BPW;
    if (first >= nblocks)
        return;  // whole waves
    // this lane's elements 4L..4L+3 of every block: their dword and digit level
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
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint64_t)N * nb * kTq1BlockBytes);
    int64_t i = first / nb;
    int B = (int)(first - i * nb);
    u32x2 v[BPW];
    uint32_t dd[BPW], sh[BPW];
#pragma unroll
    for (int k = 0; k < BPW; k++) {
        // blocks past the end reload the last one (their stores are skipped)
        const int64_t ic = first + k < nblocks ? i : n_rows - 1;
        const int Bc = first + k < nblocks ? B : nb - 1;
        int64_t r = rows ? rows[ic] : ic;
        r = r < 0 ? 0 : (r >= N ? N - 1 : r);  // ids outside [0, N) stay inside w
        const uint32_t off = (uint32_t)((r * nb + Bc) * kTq1BlockBytes);
        sh[k] = off & 3u;
        const uint32_t base = off - sh[k];
        v[k] = ld_b64(rw, base + 4 * j);
        dd[k] = ld_b32(rw, base + 52);
        if (++B == nb) {
            B = 0;
            i++;
        }
    }
#pragma unroll
    for (int k = 0; k < BPW; k++) {
        if (first + k < nblocks) {
            const uint32_t d16 = sh[k] ? (dd[k] >> 16) : (dd[k] & 0xffffu);
            const float d = f16_bits_to_f32(d16);
            const uint32_t u = digit_level(align_bytes(v[k].y, v[k].x, sh[k]), c, j == 12);
            store_run_f32(out, (first + k) * kTq1BlockElems + e0, u, d);
        }
    }
}

template <int DT, int BPW>
static void launch_half(const uint8_t *w, const int32_t *rows, void *out, int64_t N, int nb,
                        int64_t n_rows, hipStream_t stream)
{
    const int64_t waves = (n_rows * nb + BPW - 1) / BPW;
    const dim3 grid((unsigned)((waves * 64 + 255) / 256));
    hipLaunchKernelGGL((tq1_dequantize_kernel<DT, BPW>), grid, dim3(256), 0, stream, w, rows, out,
                       N, nb, n_rows);
}

template <int BPW>
static void launch_f32(const uint8_t *w, const int32_t *rows, void *out, int64_t N, int nb,
                       int64_t n_rows, hipStream_t stream)
{
    const int64_t waves = (n_rows * nb + BPW - 1) / BPW;
    const dim3 grid((unsigned)((waves * 64 + 255) / 256));
    hipLaunchKernelGGL((tq1_dequantize_f32_kernel<BPW>), grid, dim3(256), 0, stream, w, rows, out,
                       N, nb, n_rows);
}

int launch_tq1_dequantize(const void *w, const int32_t *rows, void *out, int64_t N, int64_t K,
                          int64_t n_rows, int dtype, hipStream_t stream)
{
    const int nb = (int)(K / kTq1BlockElems);
    const uint8_t *wp = static_cast<const uint8_t *>(w);
    const int64_t blocks = n_rows * nb;
    if (dtype == BQM_DTYPE_F32) {
        if (blocks >= kDqMidBlocks)
            launch_f32<kDqBlocksPerWave>(wp, rows, out, N, nb, n_rows, stream);
        else if (blocks >= kDqSmallBlocks)
            launch_f32<4>(wp, rows, out, N, nb, n_rows, stream);
        else
            launch_f32<2>(wp, rows, out, N, nb, n_rows, stream);
    } else if (dtype == BQM_DTYPE_F16) {
        if (blocks >= kDqLargeBlocks)
            launch_half<BQM_DTYPE_F16, 16>(wp, rows, out, N, nb, n_rows, stream);
        else if (blocks >= kDqMidBlocks)
            launch_half<BQM_DTYPE_F16, 8>(wp, rows, out, N, nb, n_rows, stream);
        else if (blocks >= kDqSmallBlocks)
            launch_half<BQM_DTYPE_F16, 4>(wp, rows, out, N, nb, n_rows, stream);
        else
            launch_half<BQM_DTYPE_F16, 2>(wp, rows, out, N, nb, n_rows, stream);
    } else {
        if (blocks >= kDqLargeBlocks)
            launch_half<BQM_DTYPE_BF16, 16>(wp, rows, out, N, nb, n_rows, stream);
        else if (blocks >= kDqMidBlocks)
            launch_half<BQM_DTYPE_BF16, 8>(wp, rows, out, N, nb, n_rows, stream);
        else if (blocks >= kDqSmallBlocks)
            launch_half<BQM_DTYPE_BF16, 4>(wp, rows, out, N, nb, n_rows, stream);
        else
            launch_half<BQM_DTYPE_BF16, 2>(wp, rows, out, N, nb, n_rows, stream);
    }
    return check_launch();
}

}  // namespace bqm
