// tq1_decode.hpp -- byte-major TQ1_0 digit expansion for gfx950.
//
// Five base-3 trits live in each qs byte and four in each qh byte ("CUDA:
// TQ1_0 mat-vec is load-bound by the per-32-element chunk contract",
// "Current behavior"). A byte v = sum_c u_c 3^c cannot be split with shifts and
// masks; the same page ("Upstream state") describes expanding all digits of a
// loaded byte in place instead of re-reading it per digit. This header does
// that with multiply-shift steps on two bytes at once, in the two 16-bit lanes
// of a 32-bit register:
//
//   X1 = (101 v + 63) >> 5      (qs bytes; X1 / 256 lies in [v/81, (v+1)/81))
//   X1 = (19 v + 1) >> 1        (qh bytes; X1 / 256 lies in [v/27, (v+1)/27))
//   X(k+1) = 3 X(k)
//
// so byte 1 of each 16-bit lane of X(k) holds F = floor(v / 3^m) for the
// successive powers m (the integer part of the fixed-point value; byte 0 is
// its fraction), and the lowest digit is v - 3 floor(v / 3). The constants
// were found by exhaustive search over every byte value and are re-checked
// on the CPU by tests/test_decode_arith.py.
//
// A digit is u_m = F_m - 3 F_(m+1). Rather than forming it, the dot products
// keep two integer sums per Q8_1 sub-block: P = sum F_m q and N = sum F_(m+1) q,
// so the sub-block's unsigned-digit sum is P - 3 N; starting P at -sum(q)
// turns that into the trit sum, since trit = u - 1.
#pragma once

#include "common.hpp"

namespace bqm {

constexpr uint32_t kLaneMask = 0x00ff00ffu;   // byte 0 of each 16-bit lane
constexpr uint32_t kQsMul = 101u, kQsAdd = 63u * 0x00010001u, kQsShift = 5u;
constexpr uint32_t kQhMul = 19u, kQhAdd = 1u * 0x00010001u, kQhShift = 1u;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Per-16-bit-lane logical shift right (v_pk_lshrrev_b16).
__device__ __forceinline__ uint32_t pk_shr(uint32_t x, uint32_t s)
{
    u16x2 v = __builtin_bit_cast(u16x2, x);
    v = v >> (unsigned short)s;
    return __builtin_bit_cast(uint32_t, v);
}

// k * x on both 16-bit lanes (v_pk_mul_lo_u16; no lane ever exceeds 16 bits
// here). Written as a packed 16-bit product so that chains of them fold into
// one full-rate packed multiply rather than a quarter-rate 32-bit one.
__device__ __forceinline__ uint32_t pk_mul(uint32_t x, unsigned short k)
{
    u16x2 v = __builtin_bit_cast(u16x2, x);
    v = v * (u16x2)k;
    return __builtin_bit_cast(uint32_t, v);
}

// 3 * f for a dword of four floor bytes, each at most 80 (so 3 f per byte
// stays below 256 and no byte carries into the next). As two 16-bit lanes the
// product is exact too; the packed multiply keeps the compiler from choosing a
// quarter-rate 32-bit multiply where it would not use a shift-add.
__device__ __forceinline__ uint32_t mul3_bytes(uint32_t f) { return pk_mul(f, 3); }

// Bytes 1 and 3 of e (bytes 0, 2 of the source dword) and of o (bytes 1, 3)
// interleaved back into source byte order.
__device__ __forceinline__ uint32_t hi_bytes(uint32_t o, uint32_t e)
{
    return __builtin_amdgcn_perm(o, e, 0x07030501u);
}

// Floor quotients of the four bytes of a qs dword: F[m] holds
// floor(v / 3^(4-m)) per byte for m = 0..3 (i.e. F4, F3, F2, F1), and U0 the
// lowest digit, v - 3 floor(v / 3) per byte: every byte of that difference
// is a digit (>= 0), so the dword subtraction never borrows across bytes.
struct QsFloors {
    uint32_t F4, F3, F2, F1, U0;
};

__device__ __forceinline__ QsFloors qs_floors(uint32_t w)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);  // bytes 1, 3 -> lanes
    const uint32_t e1 = pk_shr(__umul24(e, kQsMul) + kQsAdd, kQsShift);
    const uint32_t o1 = pk_shr(__umul24(o, kQsMul) + kQsAdd, kQsShift);
    const uint32_t e2 = pk_mul(e1, 3), o2 = pk_mul(o1, 3);
    const uint32_t e3 = pk_mul(e1, 9), o3 = pk_mul(o1, 9);
    const uint32_t e4 = pk_mul(e1, 27), o4 = pk_mul(o1, 27);
    QsFloors f;
    f.F4 = hi_bytes(o1, e1);
    f.F3 = hi_bytes(o2, e2);
    f.F2 = hi_bytes(o3, e3);
    f.F1 = hi_bytes(o4, e4);
    f.U0 = w - mul3_bytes(f.F1);
    return f;
}

// Same for the qh dword (four digits per byte): F3, F2, F1 and U0.
struct QhFloors {
    uint32_t F3, F2, F1, U0;
};

__device__ __forceinline__ QhFloors qh_floors(uint32_t w)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);
    const uint32_t e1 = pk_shr(__umul24(e, kQhMul) + kQhAdd, kQhShift);
    const uint32_t o1 = pk_shr(__umul24(o, kQhMul) + kQhAdd, kQhShift);
    const uint32_t e2 = pk_mul(e1, 3), o2 = pk_mul(o1, 3);
    const uint32_t e3 = pk_mul(e1, 9), o3 = pk_mul(o1, 9);
    QhFloors f;
    f.F3 = hi_bytes(o1, e1);
    f.F2 = hi_bytes(o2, e2);
    f.F1 = hi_bytes(o3, e3);
    f.U0 = w - mul3_bytes(f.F1);
    return f;
}

// Integer sums of one 256-element block against one activation column:
// P[b], N[b] for the eight Q8_1 sub-blocks (N[0] and N[4] stay unused).
struct BlockSums {
    int P[8];
    int N[8];
};

// qs dword j < 8 (bytes 4j..4j+3): digit c of these bytes is element 4j..4j+3
// of sub-block c, so it meets activation dword j of sub-block c (qc).
__device__ __forceinline__ void dot_qs_lo(uint32_t w, uint32_t q0, uint32_t q1, uint32_t q2,
                                          uint32_t q3, uint32_t q4, BlockSums &s)
{
    const QsFloors f = qs_floors(w);
    s.P[4] = sdot4(f.F4, q4, s.P[4]);
    s.N[3] = sdot4(f.F4, q3, s.N[3]);
    s.P[3] = sdot4(f.F3, q3, s.P[3]);
    s.N[2] = sdot4(f.F3, q2, s.N[2]);
    s.P[2] = sdot4(f.F2, q2, s.P[2]);
    s.N[1] = sdot4(f.F2, q1, s.N[1]);
    s.P[1] = sdot4(f.F1, q1, s.P[1]);
    s.P[0] = sdot4(f.U0, q0, s.P[0]);
}

// qs dword 8+i (bytes 32+4i..): digits 0,1 are elements 4i.., 16+4i.. of
// sub-block 5, digits 2,3 the same of sub-block 6, digit 4 elements 4i.. of 7.
__device__ __forceinline__ void dot_qs_hi(uint32_t w, uint32_t q5a, uint32_t q5b, uint32_t q6a,
                                          uint32_t q6b, uint32_t q7a, BlockSums &s)
{
    const QsFloors f = qs_floors(w);
    s.P[5] = sdot4(f.U0, q5a, s.P[5]);
    s.P[5] = sdot4(f.F1, q5b, s.P[5]);
    s.N[5] = sdot4(f.F2, q5b, s.N[5]);
    s.P[6] = sdot4(f.F2, q6a, s.P[6]);
    s.N[6] = sdot4(f.F3, q6a, s.N[6]);
    s.P[6] = sdot4(f.F3, q6b, s.P[6]);
    s.N[6] = sdot4(f.F4, q6b, s.N[6]);
    s.P[7] = sdot4(f.F4, q7a, s.P[7]);
}

// qh dword: digit c of its bytes is elements 16+4c.. of sub-block 7 (q7_4c).
__device__ __forceinline__ void dot_qh(uint32_t w, uint32_t q74, uint32_t q75, uint32_t q76,
                                       uint32_t q77, BlockSums &s)
{
    const QhFloors f = qh_floors(w);
    s.P[7] = sdot4(f.F3, q77, s.P[7]);
    s.N[7] = sdot4(f.F3, q76, s.N[7]);
    s.P[7] = sdot4(f.F2, q76, s.P[7]);
    s.N[7] = sdot4(f.F2, q75, s.N[7]);
    s.P[7] = sdot4(f.F1, q75, s.P[7]);
    s.P[7] = sdot4(f.U0, q74, s.P[7]);
}

// Clean packed digits of a qs dword: U[c] holds digit c of each of its four
// bytes. u_c = F_c - 3 F_(c+1) per byte; the subtraction never borrows across
// bytes because every per-byte result is a digit (>= 0), and 3 F stays
// below 256. Worth its six extra operations once a decoded dword is spent on
// two or more activation columns (five products per column instead of eight).
// PK selects how 3 F is formed: a packed 16-bit multiply (full rate, but it
// ties up more registers in the compiler's schedule), or a plain 32-bit
// multiply-subtract.
template <bool PK>
__device__ __forceinline__ uint32_t minus3(uint32_t f, uint32_t f_next)
{
    return PK ? f - mul3_bytes(f_next) : f - 3u * f_next;
}

struct QsDigits {
    uint32_t U[5];
};

template <bool PK = false>
__device__ __forceinline__ QsDigits qs_digits(uint32_t w)
{
    const QsFloors f = qs_floors(w);
    QsDigits d;
    d.U[0] = f.U0;
    d.U[1] = minus3<PK>(f.F1, f.F2);
    d.U[2] = minus3<PK>(f.F2, f.F3);
    d.U[3] = minus3<PK>(f.F3, f.F4);
    d.U[4] = f.F4;
    return d;
}

struct QhDigits {
    uint32_t U[4];
};

template <bool PK = false>
__device__ __forceinline__ QhDigits qh_digits(uint32_t w)
{
    const QhFloors f = qh_floors(w);
    QhDigits d;
    d.U[0] = f.U0;
    d.U[1] = minus3<PK>(f.F1, f.F2);
    d.U[2] = minus3<PK>(f.F2, f.F3);
    d.U[3] = f.F3;
    return d;
}

// Digit c of each byte of a qh dword, for a digit index that differs from
// lane to lane. F_m = floor(v / 3^m) is byte 1 of X1 3^(3-m) in each 16-bit
// lane (X1 as in qh_floors: X1 / 256 lies in [v/27, (v+1)/27), so X1 3^(3-m)
// / 256 lies in [v/3^m, (v+1)/3^m), which holds no integer above
// floor(v/3^m); and X1 27 < 2^16). With the lane's multipliers 3^(3-c) and
// 3^(2-c) (0 for c = 3) on both 16-bit lanes, the digit is F_c - 3 F_(c+1).
struct QhLaneMuls {
    uint32_t cur, next;
};

__device__ __forceinline__ QhLaneMuls qh_lane_muls(int c)
{
    const uint32_t m = c == 0 ? 27u : c == 1 ? 9u : c == 2 ? 3u : 1u;
    const uint32_t n = m / 3u;  // 0 for c = 3
    return {m * 0x00010001u, n * 0x00010001u};
}

// x * y on each 16-bit lane (v_pk_mul_lo_u16; no lane exceeds 16 bits here).
__device__ __forceinline__ uint32_t pk_mul_lanes(uint32_t x, uint32_t y)
{
    const u16x2 a = __builtin_bit_cast(u16x2, x), b = __builtin_bit_cast(u16x2, y);
    return __builtin_bit_cast(uint32_t, (u16x2)(a * b));
}

__device__ __forceinline__ uint32_t qh_digit_lane(uint32_t w, QhLaneMuls m)
{
    const uint32_t e = w & kLaneMask;
    const uint32_t o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);
    const uint32_t e1 = pk_shr(__umul24(e, kQhMul) + kQhAdd, kQhShift);
    const uint32_t o1 = pk_shr(__umul24(o, kQhMul) + kQhAdd, kQhShift);
    const uint32_t fc = hi_bytes(pk_mul_lanes(o1, m.cur), pk_mul_lanes(e1, m.cur));
    const uint32_t fn = hi_bytes(pk_mul_lanes(o1, m.next), pk_mul_lanes(e1, m.next));
    return minus3<true>(fc, fn);
}

// Exact per-sub-block trit sums from the two running sums.
__device__ __forceinline__ void finish_isums(const BlockSums &s, int (&isum)[8])
{
    isum[0] = s.P[0];
    isum[1] = s.P[1] - 3 * s.N[1];
    isum[2] = s.P[2] - 3 * s.N[2];
    isum[3] = s.P[3] - 3 * s.N[3];
    isum[4] = s.P[4];
    isum[5] = s.P[5] - 3 * s.N[5];
    isum[6] = s.P[6] - 3 * s.N[6];
    isum[7] = s.P[7] - 3 * s.N[7];
}

// The fixed fp32 order every kernel of this library uses for one block:
// s = sum_b d_a[b] * isum[b] accumulated from b = 0 upward with fmaf, then
// acc + d_w * s. Keeping one order makes a column's result independent of how
// many columns a call carries.
__device__ __forceinline__ float block_dot_f32(const int (&isum)[8], const float (&da)[8])
{
    float s = da[0] * (float)isum[0];
#pragma unroll
    for (int b = 1; b < 8; b++)
        s = fmaf(da[b], (float)isum[b], s);
    return s;
}

// The 54-byte block as the 14 aligned dwords that cover it, plus the byte
// shift (0 or 2) of the block inside them: blocks of a row alternate between
// dword-aligned and 2 bytes past a dword boundary.
struct RawBlock {
    uint32_t r[14];
    uint32_t sh;
};

__device__ __forceinline__ RawBlock load_raw_block(__amdgpu_buffer_rsrc_t rw, uint32_t off)
{
    RawBlock b;
    const uint32_t base = off & ~3u;
    b.sh = off & 3u;
#pragma unroll
    for (int i = 0; i < 12; i += 4) {
        const u32x4 v = ld_b128(rw, base + 4 * i);
        b.r[i] = v.x;
        b.r[i + 1] = v.y;
        b.r[i + 2] = v.z;
        b.r[i + 3] = v.w;
    }
    const u32x2 t = ld_b64(rw, base + 48);
    b.r[12] = t.x;
    b.r[13] = t.y;
    return b;
}

// Dword i of the block (i < 13: qs[4i..4i+3] for i < 12, the qh dword at 12).
__device__ __forceinline__ uint32_t raw_dword(const RawBlock &b, int i)
{
    return align_bytes(b.r[i + 1], b.r[i], b.sh);
}

// fp16 bits of the block scale d.
__device__ __forceinline__ uint32_t raw_scale_bits(const RawBlock &b)
{
    return b.sh ? (b.r[13] >> 16) : (b.r[13] & 0xffffu);
}

}  // namespace bqm
