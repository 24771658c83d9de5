// q8_1.hpp -- Q8_1 quantization of one 32-element block by eight lanes.
//
// Q8_1 ("CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk
// contract", "Current behavior": the mat-vec consumes Q8_1 activations in
// 32-element chunks; byte layout and rounding rule in include/bqm.h):
//   amax = max |x_i|, d = amax / 127 (IEEE fp32 division), id = 1 / d (0 when
//   d = 0), q_i = round-half-away(x_i * id) clamped to +-127, and the fp16
//   sum field s = fp16(fp32(d * sum q)).
// Both the stand-alone quantize kernel and the fused quantize-and-multiply
// staging call this one routine, so their bytes agree by construction.
#pragma once

#include "common.hpp"

namespace bqm {

// Reductions over an aligned group of eight lanes with DPP lane moves (no
// LDS round trip): swap neighbours, swap pairs (quad permutes), then mirror
// the two quads of the half row. Every lane ends with the group's value.
constexpr int kDppQuadXor1 = 0xb1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4e;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfRowMirror = 0x141; // lane i <- lane 7 - i within 8

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ float group8_max(float v)
{
    v = fmaxf(v, __int_as_float(dpp_i32<kDppQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppHalfRowMirror>(__float_as_int(v))));
    return v;
}

__device__ __forceinline__ int group8_sum(int v)
{
    v += dpp_i32<kDppQuadXor1>(v);
    v += dpp_i32<kDppQuadXor2>(v);
    v += dpp_i32<kDppHalfRowMirror>(v);
    return v;
}

// The block held by eight consecutive lanes (an aligned group of 8 in the
// wave), lane j of the group holding elements 4j..4j+3. Every lane of the
// wave must call this (the reductions move values between lanes of a group).
struct Q81Part {
    uint32_t q4;  // this lane's four q bytes, element 4j in the low byte
    float d;      // the block's scale (fp32, before rounding to fp16)
    int sum;      // sum of the block's 32 q values
};

__device__ __forceinline__ Q81Part q8_1_block_by_8(float x0, float x1, float x2, float x3)
{
    const float amax =
        group8_max(fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
    Q81Part r;
    r.d = amax / 127.0f;
    const float id = r.d != 0.0f ? 1.0f / r.d : 0.0f;
    const float xs[4] = {x0, x1, x2, x3};
    uint32_t q4 = 0;
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int q = (int)roundf(xs[i] * id);
        q = q > 127 ? 127 : (q < -127 ? -127 : q);
        sum += q;
        q4 |= (uint32_t)(q & 0xff) << (8 * i);
    }
    r.q4 = q4;
    r.sum = group8_sum(sum);
    return r;
}

// The block's 32-bit d/s field: fp16(d) in the low half, fp16(d * sum) in the high.
__device__ __forceinline__ uint32_t q8_1_scale_field(const Q81Part &p)
{
    return f32_to_f16_bits(p.d) | (f32_to_f16_bits(p.d * (float)p.sum) << 16);
}

}  // namespace bqm
