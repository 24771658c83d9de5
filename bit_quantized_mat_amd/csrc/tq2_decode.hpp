// tq2_decode.hpp -- TQ2_0 blocks for gfx950: 2-bit digit fields.
//
// "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk contract",
// "Upstream state", names TQ2_0, the other ternary type, and prints no layout.
// The layout this library reads (include/bqm.h states it in full): 66-byte
// blocks of 256 elements, qs[64] then the fp16 scale d; element e holds the
// digit u = trit + 1 in field (e % 128) / 32 (bits 2f, 2f + 1) of byte
// 32 (e / 128) + e % 32. So 32-element sub-block b = 4h + f is field f of
// bytes 32h .. 32h + 31, and dword j of its q bytes meets qs dword 8h + j.
//
// Unlike base-3 bytes, the fields come apart with a mask. The dot products
// take each field in place, scaled: f0 = w & 0x03030303 is u, f1 = w &
// 0x0C0C0C0C is 4u, f2 = w & 0x30303030 is 16u and f3 = (w >> 1) & 0x60606060
// is 32u per byte (at most 64, so every byte stays a non-negative int8).
// A sub-block's sum of scaled products is an exact multiple of the scale and
// shifts back exactly.
#pragma once

#include "mfma_common.hpp"

namespace bqm {

constexpr int kTq2BlockBytes = 66;

// Byte offset of a block load a lane issues without a block (see
// kIdleLoadOffset): a TQ2_0 block load reaches 68 bytes past its offset, so
// this stays 64 bytes lower to keep every such load's end below 2^32.
constexpr uint32_t kTq2IdleOffset = kIdleLoadOffset - 64u;

// Scaled field f of the four bytes of a qs dword (see above).
__device__ __forceinline__ uint32_t tq2_field_scaled(uint32_t w, int f)
{
    return f == 0 ? (w & 0x03030303u)
         : f == 1 ? (w & 0x0C0C0C0Cu)
         : f == 2 ? (w & 0x30303030u)
                  : ((w >> 1) & 0x60606060u);
}

// log2 of field f's scale: 0, 2, 4, 5.
__device__ __forceinline__ constexpr int tq2_field_shift(int f) { return f == 3 ? 5 : 2 * f; }

// Field f of the four bytes, as plain digits.
__device__ __forceinline__ uint32_t tq2_field_digits(uint32_t w, int f)
{
    return (w >> (2 * f)) & 0x03030303u;
}

// The 66-byte block as the 17 aligned dwords that cover it, plus its byte
// shift (0 or 2): blocks of a row alternate between dword-aligned and 2 bytes
// past a dword boundary.
struct RawBlock2 {
    uint32_t r[17];
    uint32_t sh;
};

__device__ __forceinline__ RawBlock2 load_raw_block2(__amdgpu_buffer_rsrc_t rw, uint32_t off)
{
    RawBlock2 b;
    const uint32_t base = off & ~3u;
    b.sh = off & 3u;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        const u32x4 v = ld_b128(rw, base + 4 * i);
        b.r[i] = v.x;
        b.r[i + 1] = v.y;
        b.r[i + 2] = v.z;
        b.r[i + 3] = v.w;
    }
    b.r[16] = ld_b32(rw, base + 64);
    return b;
}

// qs dword i (bytes 4i .. 4i + 3), i < 16.
__device__ __forceinline__ uint32_t raw2_dword(const RawBlock2 &b, int i)
{
    return align_bytes(b.r[i + 1], b.r[i], b.sh);
}

// fp16 bits of the block scale d (bytes 64, 65).
__device__ __forceinline__ uint32_t raw2_scale_bits(const RawBlock2 &b)
{
    return b.sh ? (b.r[16] >> 16) : (b.r[16] & 0xffffu);
}

// Matrix-core operand form (mfma_common.hpp's layout of
// v_mfma_i32_16x16x32_i8, sub-block b in K): lane (r, kg) needs q-order
// bytes 8kg .. 8kg + 7 of every sub-block, i.e. qs bytes 8kg .. 8kg + 7 of
// each half (fields 0..3 give sub-blocks 4h .. 4h + 3), and the scale.
struct LaneBlock2 {
    u32x3 lo;     // aligned dwords covering qs bytes 8kg .. 8kg + 7
    u32x3 hi;     // the same 32 bytes on
    uint32_t t;   // the dword holding d
    uint32_t sh;  // byte shift, 0 or 2
};

// Weight format policies of the matrix-core kernels: how a lane loads its
// share of a block, decodes it to digit operands, and which activation bytes
// its B operand takes from a staged tile (mfma_common.hpp's kStageCol layout).
struct Tq2Tile {
    static constexpr int kBlockBytes = kTq2BlockBytes;
    static constexpr uint32_t kIdle = kTq2IdleOffset;
    typedef LaneBlock2 Lane;
    struct Ctx {
        __device__ __forceinline__ explicit Ctx(int) {}
    };

    static __device__ __forceinline__ Lane load(__amdgpu_buffer_rsrc_t rw, uint32_t off, int kg)
    {
        Lane b;
        b.sh = off & 3u;
        const uint32_t base = off - b.sh;
        b.lo = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 8 * kg, 0, 0);
        b.hi = __builtin_amdgcn_raw_buffer_load_b96(rw, base + 32 + 8 * kg, 0, 0);
        b.t = ld_b32(rw, base + 64);
        return b;
    }

    static __device__ __forceinline__ TileOperands decode(const Lane &lb, const Ctx &)
    {
        const uint32_t x[2][2] = {
            {align_bytes(lb.lo.y, lb.lo.x, lb.sh), align_bytes(lb.lo.z, lb.lo.y, lb.sh)},
            {align_bytes(lb.hi.y, lb.hi.x, lb.sh), align_bytes(lb.hi.z, lb.hi.y, lb.sh)}};
        TileOperands o;
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int f = 0; f < 4; f++)
                o.A[4 * h + f] = (long)(((uint64_t)tq2_field_digits(x[h][1], f) << 32) |
                                        tq2_field_digits(x[h][0], f));
        o.dw = f16_bits_to_f32(lb.sh ? (lb.t >> 16) : (lb.t & 0xffffu));
        return o;
    }

    // q bytes 8kg .. 8kg + 7 of sub-block b, column col
    static __device__ __forceinline__ long operand(const uint32_t *__restrict__ tile, int col,
                                                   int kg, int b)
    {
        const uint32_t *cs = tile + col * kStageCol + 9 * b + 2 * kg;
        return (long)(((uint64_t)cs[1] << 32) | cs[0]);
    }

    // the same, given the staged sub-block's first dword
    // (tile + col * kStageCol + 9 b)
    static __device__ __forceinline__ long operand_at(const uint32_t *__restrict__ cs, int kg, int)
    {
        return (long)(((uint64_t)cs[2 * kg + 1] << 32) | cs[2 * kg]);
    }

    // the same from the eight q dwords of one Q8_1 block
    static __device__ __forceinline__ u32x2 operand_dwords(const uint32_t (&q)[8], int kg, int)
    {
        return (u32x2){q[2 * kg], q[2 * kg + 1]};
    }

    // Pair-tile form (mfma_common.hpp): half h of a row's block is elements
    // 16h..16h+15 of every sub-block, i.e. fields 0..3 of qs bytes
    // 16h..16h+15 (sub-blocks 0..3) and of qs bytes 32+16h..47+16h
    // (sub-blocks 4..7). Loads: five aligned dwords from each; for h = 1 the
    // fifth of the second holds the scale.
    struct PairLane {
        u32x4 lo;
        uint32_t lo_x;
        u32x4 hi;
        uint32_t hi_x;
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
        p.hi = ld_b128(rw, base + 32 + 16 * h);
        p.hi_x = ld_b32(rw, base + 48 + 16 * h);
        return p;
    }

    static __device__ __forceinline__ PairOperands decode_pair(const PairLane &p, const Ctx &, int)
    {
        const uint32_t x[2][4] = {
            {align_bytes(p.lo.y, p.lo.x, p.sh), align_bytes(p.lo.z, p.lo.y, p.sh),
             align_bytes(p.lo.w, p.lo.z, p.sh), align_bytes(p.lo_x, p.lo.w, p.sh)},
            {align_bytes(p.hi.y, p.hi.x, p.sh), align_bytes(p.hi.z, p.hi.y, p.sh),
             align_bytes(p.hi.w, p.hi.z, p.sh), align_bytes(p.hi_x, p.hi.w, p.sh)}};
        PairOperands o;
#pragma unroll
        for (int q = 0; q < 2; q++)
#pragma unroll
            for (int f = 0; f < 4; f++)
                o.A[4 * q + f] = (i32x4){(int)tq2_field_digits(x[q][0], f),
                                         (int)tq2_field_digits(x[q][1], f),
                                         (int)tq2_field_digits(x[q][2], f),
                                         (int)tq2_field_digits(x[q][3], f)};
        // bytes 64, 65 of the block sit in hi_x of half 1
        o.dw = f16_bits_to_f32(p.sh ? (p.hi_x >> 16) : (p.hi_x & 0xffffu));
        return o;
    }

    static __device__ __forceinline__ i32x4 pair_operand(const uint32_t *__restrict__ tile, int col,
                                                         int h, int b)
    {
        const uint32_t *cs = tile + col * kStageCol + 9 * b + 4 * h;
        return (i32x4){(int)cs[0], (int)cs[1], (int)cs[2], (int)cs[3]};
    }

    static __device__ __forceinline__ u32x4 pair_dwords(const uint32_t (&q)[8], int h, int)
    {
        return (u32x4){q[4 * h], q[4 * h + 1], q[4 * h + 2], q[4 * h + 3]};
    }
};

}  // namespace bqm
