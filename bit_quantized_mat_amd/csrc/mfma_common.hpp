// mfma_common.hpp -- pieces shared by the matrix-core kernels: the per-lane
// share of a TQ1_0 block in the v_mfma_i32_16x16x32_i8 operand layout, its
// decode to digit operands, and the wave-level LDS ordering helper.
//
// Operand layout of v_mfma_i32_16x16x32_i8 (K = 32 = one Q8_1 sub-block):
//   A (weights): lane (r, kg) = (lane % 16, lane / 16) holds 8 digits of row r;
//   B (activations): lane (c, kg) holds the 8 matching q bytes of column c;
//   D: lane (c, rg) holds rows 4rg..4rg+3 of column c.
// The eight K positions of lane group kg are, per sub-block b:
//   b < 5: elements 8kg..8kg+7  (digit b of qs bytes 8kg..8kg+7),
//   b = 5: elements 4kg..4kg+3 and 16+4kg..16+4kg+3 (digits 0, 1 of qs dword
//          8+kg), b = 6 likewise with digits 2, 3, and b = 7: digit 4 of qs
//          dword 8+kg, then digit kg of the qh dword (elements 16+4kg..),
// so every lane decodes two qs dwords of the first 32 bytes, one of the next
// 16 and the qh dword, and the B operand of lane (c, kg) is q bytes
// 8kg..8kg+7 of the sub-block for b < 5, bytes 4kg..4kg+3 and 16+4kg..19+4kg
// for b >= 5.
//
// The A operand holds unsigned digits u (0, 1, 2), not trits: the trit sum is
// sum u q - sum q, and the -sum q term comes from the matrix core too, as a
// product with an all -1 operand that seeds the accumulator.
#pragma once

#include "launch.hpp"
#include "tq1_decode.hpp"

namespace bqm {

typedef int i32x4 __attribute__((ext_vector_type(4)));

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
// the 8-byte digit operand of sub-block b, dw the fp32 scale of the lane's row.
struct TileOperands {
    long A[8];
    float dw;
};

__device__ __forceinline__ TileOperands decode_lane_block(const LaneBlock &lb, int kg)
{
    const QsDigits lo0 = qs_digits<true>(lb.lo0);
    const QsDigits lo1 = qs_digits<true>(lb.lo1);
    const QsDigits hi = qs_digits<true>(lb.hi);
    const QhDigits qh = qh_digits<true>(lb.qh);
    const uint32_t qhk = kg == 0 ? qh.U[0] : kg == 1 ? qh.U[1] : kg == 2 ? qh.U[2] : qh.U[3];
    TileOperands t;
#pragma unroll
    for (int c = 0; c < 5; c++)
        t.A[c] = (long)(((uint64_t)lo1.U[c] << 32) | lo0.U[c]);
    t.A[5] = (long)(((uint64_t)hi.U[1] << 32) | hi.U[0]);
    t.A[6] = (long)(((uint64_t)hi.U[3] << 32) | hi.U[2]);
    t.A[7] = (long)(((uint64_t)qhk << 32) | hi.U[4]);
    t.dw = f16_bits_to_f32(lb.dbits);
    return t;
}

constexpr long kAllMinusOne = -1;    // eight int8 -1 bytes

// Orders this wave's LDS writes before its later LDS reads (a wave's LDS
// operations are executed in order; this only keeps the compiler from moving
// them).
__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace bqm
