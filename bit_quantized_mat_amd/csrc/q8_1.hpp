// q8_1.hpp -- Q8_1 quantization of one 32-element block by two lanes.
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

// A block is quantized by two neighbouring lanes (an aligned pair in the
// wave), lane h of the pair holding elements 16h..16h+15: per lane, one
// block-wide step (the two divisions) and one lane exchange per reduction,
// against sixteen elements of per-element work.
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1, 0, 3, 2]: swap neighbouring lanes

__device__ __forceinline__ int dpp_swap_pair(int v)
{
    return __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xf, 0xf, true);
}

struct Q81Part {
    uint32_t q4[4];  // this lane's sixteen q bytes, element 16h + 4k + i in byte i of q4[k]
    float d;         // the block's scale (fp32, before rounding to fp16)
    int sum;         // sum of the block's 32 q values
};

// Every lane of the wave must call this (the reductions move values between
// the lanes of a pair).
__device__ __forceinline__ Q81Part q8_1_block_by_2(const float (&x)[16])
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++)
        m = fmaxf(m, fabsf(x[i]));
    const float amax = fmaxf(m, __int_as_float(dpp_swap_pair(__float_as_int(m))));
    Q81Part r;
    r.d = amax / 127.0f;
    const float id = r.d != 0.0f ? 1.0f / r.d : 0.0f;
    int sum = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t q4 = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int q = (int)roundf(x[4 * k + i] * id);
            q = q > 127 ? 127 : (q < -127 ? -127 : q);
            sum += q;
            q4 |= (uint32_t)(q & 0xff) << (8 * i);
        }
        r.q4[k] = q4;
    }
    r.sum = sum + dpp_swap_pair(sum);
    return r;
}

// The block's 32-bit d/s field: fp16(d) in the low half, fp16(d * sum) in the high.
__device__ __forceinline__ uint32_t q8_1_scale_field(const Q81Part &p)
{
    return f32_to_f16_bits(p.d) | (f32_to_f16_bits(p.d * (float)p.sum) << 16);
}

}  // namespace bqm
