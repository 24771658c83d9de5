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
// 2kg and 2kg+1, qs dword 8+kg, the qh dword and the fp16 scale, held as the
// aligned dwords that cover them plus the block's byte shift (odd blocks of a
// row start two bytes past a dword boundary). The realignment waits for
// decode_lane_block, so a block loaded ahead stays in flight until it is used.
struct LaneBlock {
    u32x3 l;      // qs dwords 2kg, 2kg+1
    u32x2 h;      // qs dword 8+kg
    u32x2 t;      // the qh dword and d
    uint32_t sh;  // byte shift, 0 or 2
};

__device__ __forceinline__ LaneBlock load_lane_block(__amdgpu_buffer_rsrc_t rw, uint32_t off, int kg)
{
    LaneBlock b;
    b.sh = off & 3u;
    const uint32_t base = off - b.sh;
    b.l = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 8 * kg, 0, 0);
    b.h = ld_b64(rw, base + 32 + 4 * kg);
    b.t = ld_b64(rw, base + 48);
    return b;
}

// Decoded weight operands of one lane for one 16-row tile and block: A[b] is
// the 8-byte digit operand of sub-block b, dw the fp32 scale of the lane's row.
struct TileOperands {
    long A[8];
    float dw;
};

// qm: the lane's multipliers for qh digit kg (qh_lane_muls(kg)).
__device__ __forceinline__ TileOperands decode_lane_block(const LaneBlock &lb, QhLaneMuls qm)
{
    const QsDigits lo0 = qs_digits<true>(align_bytes(lb.l.y, lb.l.x, lb.sh));
    const QsDigits lo1 = qs_digits<true>(align_bytes(lb.l.z, lb.l.y, lb.sh));
    const QsDigits hi = qs_digits<true>(align_bytes(lb.h.y, lb.h.x, lb.sh));
    const uint32_t qhk = qh_digit_lane(align_bytes(lb.t.y, lb.t.x, lb.sh), qm);
    TileOperands t;
#pragma unroll
    for (int c = 0; c < 5; c++)
        t.A[c] = (long)(((uint64_t)lo1.U[c] << 32) | lo0.U[c]);
    t.A[5] = (long)(((uint64_t)hi.U[1] << 32) | hi.U[0]);
    t.A[6] = (long)(((uint64_t)hi.U[3] << 32) | hi.U[2]);
    t.A[7] = (long)(((uint64_t)qhk << 32) | hi.U[4]);
    t.dw = f16_bits_to_f32(lb.sh ? (lb.t.y >> 16) : (lb.t.y & 0xffffu));
    return t;
}

constexpr long kAllMinusOne = -1;    // eight int8 -1 bytes

// Pair-tile form (at most 8 activation columns): two 16-row tiles share one
// v_mfma_i32_16x16x64_i8. Its 64-element K is four lane groups of 16 bytes
// (an A lane group pairs with the same B lane group; D as above: lane (j, rg)
// holds rows 4rg..4rg+3 of column j). Lane groups 0, 1 carry the first tile's
// rows and the columns' q bytes in D columns 0..7; groups 2, 3 the second
// tile's rows and the same columns' q bytes in D columns 8..15; a B lane of
// the other half holds zeros. So D column j < 8 is the sub-block sums of the
// first tile against column j, column 8 + j those of the second tile. Lane
// group g = 2 t + h holds half h of each sub-block of a row of tile t: 16 of
// its 32 elements (which 16 is the format's choice, matched on both sides).
struct PairOperands {
    i32x4 A[8];
    float dw;    // the row's block scale (valid in lanes of half 1)
};

constexpr i32x4 kAllMinusOne4 = {-1, -1, -1, -1};   // sixteen int8 -1 bytes

// Staging of one block of activations for a wave, through its own slice of
// LDS (coalesced 8-byte pieces in, B operands out).
constexpr int kStageCol = 74;        // dwords per staged column: 8 x 9 of Q8_1 data, 2 of padding

// Block B of activation columns 0 .. 16 NT - 1, in flight to this wave's
// stage: column c's eight Q8_1 blocks (288 bytes, 36 pieces of 8 bytes) go to
// dwords c * kStageCol .. c * kStageCol + 71. A 16-column tile is 576 pieces,
// nine per lane: piece i = lane + 64 k. The loads are issued one block ahead
// and written to LDS once the stage is free.
//
// Columns at or past T are not masked: their loads fall past the end of the
// activation buffer and read zeros, or (when the 32-bit offset wraps) some
// in-range bytes, and either way they only feed output columns that are never
// stored.
struct StageMap {
    uint32_t gofs[9];  // byte offset of piece k in block 0 of column tile 0
    uint32_t lofs[9];  // its dword offset in the stage

    __device__ __forceinline__ StageMap(uint32_t col_bytes, int lane)
    {
#pragma unroll
        for (int k = 0; k < 9; k++) {
            const int i = lane + 64 * k;
            const int c = i / 36, p = i - 36 * c;
            gofs[k] = (uint32_t)c * col_bytes + 8 * p;
            lofs[k] = c * kStageCol + 2 * p;
        }
    }
};

template <int NT>
struct StagePieces {
    u32x2 v[NT][9];

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t ra, const StageMap &m,
                                          uint32_t col_bytes, int B)
    {
#pragma unroll
        for (int ct = 0; ct < NT; ct++) {
            // wave-uniform part of the offset
            const uint32_t so = __builtin_amdgcn_readfirstlane(
                (uint32_t)B * (8 * kQ81BlockBytes) + (uint32_t)ct * 16 * col_bytes);
#pragma unroll
            for (int k = 0; k < 9; k++)
                v[ct][k] = __builtin_amdgcn_raw_buffer_load_b64(ra, m.gofs[k], so, 0);
        }
    }

    __device__ __forceinline__ void land(uint32_t *__restrict__ stage, const StageMap &m) const
    {
#pragma unroll
        for (int ct = 0; ct < NT; ct++)
#pragma unroll
            for (int k = 0; k < 9; k++)
                *reinterpret_cast<u32x2 *>(stage + ct * 16 * kStageCol + m.lofs[k]) = v[ct][k];
    }
};

// This lane's B operand of sub-block b from a staged 16-column tile (the
// layout above): column col, K group kg.
__device__ __forceinline__ long staged_operand(const uint32_t *__restrict__ tile, int col, int kg,
                                               int b)
{
    const uint32_t *cs = tile + col * kStageCol + 9 * b;
    const uint32_t q0 = b < 5 ? cs[2 * kg] : cs[kg];
    const uint32_t q1 = b < 5 ? cs[2 * kg + 1] : cs[4 + kg];
    return (long)(((uint64_t)q1 << 32) | q0);
}

// Weight format policy of the matrix-core kernels for TQ1_0 (the policy of
// TQ2_0 is in tq2_decode.hpp): a lane's share of a block, its decode to digit
// operands, and the staged activation bytes of its B operand.
struct Tq1Tile {
    static constexpr int kBlockBytes = kTq1BlockBytes;
    static constexpr uint32_t kIdle = kIdleLoadOffset;  // offset of a load without a block
    typedef LaneBlock Lane;
    struct Ctx {
        QhLaneMuls qm;
        __device__ __forceinline__ explicit Ctx(int kg) : qm(qh_lane_muls(kg)) {}
    };

    static __device__ __forceinline__ Lane load(__amdgpu_buffer_rsrc_t rw, uint32_t off, int kg)
    {
        return load_lane_block(rw, off, kg);
    }

    static __device__ __forceinline__ TileOperands decode(const Lane &lb, const Ctx &c)
    {
        return decode_lane_block(lb, c.qm);
    }

    static __device__ __forceinline__ long operand(const uint32_t *__restrict__ tile, int col,
                                                   int kg, int b)
    {
        return staged_operand(tile, col, kg, b);
    }

    // the same, given the staged sub-block's first dword
    // (tile + col * kStageCol + 9 b)
    static __device__ __forceinline__ long operand_at(const uint32_t *__restrict__ cs, int kg, int b)
    {
        const uint32_t q0 = b < 5 ? cs[2 * kg] : cs[kg];
        const uint32_t q1 = b < 5 ? cs[2 * kg + 1] : cs[4 + kg];
        return (long)(((uint64_t)q1 << 32) | q0);
    }

    // K group kg's B operand of sub-block b, from the eight q dwords of one
    // Q8_1 block (the layout above)
    static __device__ __forceinline__ u32x2 operand_dwords(const uint32_t (&q)[8], int kg, int b)
    {
        const uint32_t lo = b < 5 ? q[2 * kg] : q[kg];
        const uint32_t hi = b < 5 ? q[2 * kg + 1] : q[4 + kg];
        return (u32x2){lo, hi};
    }

    // Pair-tile form: half h of a row's block is elements 16h..16h+15 of
    // sub-blocks 0..4 (digit b of qs dwords 4h..4h+3) and elements 8h..8h+7,
    // 16+8h..16+8h+7 of sub-blocks 5..7 (digits of qs dwords 8+2h, 9+2h:
    // 0 and 1 for sub-block 5, 2 and 3 for 6; for 7 digit 4 and then qh
    // digits 2h, 2h+1). Loads: qs bytes 16h..16h+15 (five aligned dwords), qs
    // bytes 32+8h..39+8h (three), the qh dword and the scale (two).
    struct PairLane {
        u32x4 lo;
        uint32_t lo_x;
        u32x3 hi;
        u32x2 t;
        uint32_t sh;
    };

    static __device__ __forceinline__ PairLane load_pair(__amdgpu_buffer_rsrc_t rw, uint32_t off,
                                                         int h)
    {
        PairLane p;
        p.sh = off & 3u;
        const uint32_t base = off - p.sh;
        p.lo = ld_b128(rw, base + 16 * h);
        p.lo_x = ld_b32(rw, base + 16 * h + 16);
        p.hi = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 32 + 8 * h, 0, 0);
        p.t = ld_b64(rw, base + 48);
        return p;
    }

    static __device__ __forceinline__ PairOperands decode_pair(const PairLane &p, const Ctx &, int h)
    {
        const uint32_t w[4] = {align_bytes(p.lo.y, p.lo.x, p.sh), align_bytes(p.lo.z, p.lo.y, p.sh),
                               align_bytes(p.lo.w, p.lo.z, p.sh), align_bytes(p.lo_x, p.lo.w, p.sh)};
        QsDigits L[4];
#pragma unroll
        for (int d = 0; d < 4; d++)
            L[d] = qs_digits<true>(w[d]);
        const QsDigits H0 = qs_digits<true>(align_bytes(p.hi.y, p.hi.x, p.sh));
        const QsDigits H1 = qs_digits<true>(align_bytes(p.hi.z, p.hi.y, p.sh));
        const QhDigits Q = qh_digits<true>(align_bytes(p.t.y, p.t.x, p.sh));
        PairOperands o;
#pragma unroll
        for (int c = 0; c < 5; c++)
            o.A[c] = (i32x4){(int)L[0].U[c], (int)L[1].U[c], (int)L[2].U[c], (int)L[3].U[c]};
        o.A[5] = (i32x4){(int)H0.U[0], (int)H1.U[0], (int)H0.U[1], (int)H1.U[1]};
        o.A[6] = (i32x4){(int)H0.U[2], (int)H1.U[2], (int)H0.U[3], (int)H1.U[3]};
        o.A[7] = (i32x4){(int)H0.U[4], (int)H1.U[4], (int)(h ? Q.U[2] : Q.U[0]),
                         (int)(h ? Q.U[3] : Q.U[1])};
        o.dw = f16_bits_to_f32(p.sh ? (p.t.y >> 16) : (p.t.y & 0xffffu));
        return o;
    }

    // the matching q bytes of sub-block b from a staged tile
    // (tile + col * kStageCol + 9 b: the sub-block's eight q dwords)
    static __device__ __forceinline__ i32x4 pair_operand(const uint32_t *__restrict__ tile, int col,
                                                         int h, int b)
    {
        const uint32_t *cs = tile + col * kStageCol + 9 * b;
        return b < 5 ? (i32x4){(int)cs[4 * h], (int)cs[4 * h + 1], (int)cs[4 * h + 2], (int)cs[4 * h + 3]}
                     : (i32x4){(int)cs[2 * h], (int)cs[2 * h + 1], (int)cs[4 + 2 * h], (int)cs[5 + 2 * h]};
    }

    // the same from the eight q dwords of one Q8_1 block
    static __device__ __forceinline__ u32x4 pair_dwords(const uint32_t (&q)[8], int h, int b)
    {
        return b < 5 ? (u32x4){q[4 * h], q[4 * h + 1], q[4 * h + 2], q[4 * h + 3]}
                     : (u32x4){q[2 * h], q[2 * h + 1], q[4 + 2 * h], q[5 + 2 * h]};
    }
};

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
