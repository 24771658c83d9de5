// common.hpp -- device helpers shared by the gfx950 kernels of this library.
//
// All global reads of packed weights and activations go through raw buffer
// resources: the descriptor carries the buffer's byte size, so a load whose
// dword starts past the end returns zero instead of touching memory outside
// the buffer. The descriptor size is rounded up to a whole dword; the at most
// three slack bytes that this admits lie in the same aligned dword (hence the
// same page) as the buffer's last byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqm {

constexpr int kTq1BlockElems = 256;
constexpr int kTq1BlockBytes = 54;
constexpr int kQ81BlockElems = 32;
constexpr int kQ81BlockBytes = 36;

// Fourth descriptor dword for raw (untyped, stride 0) buffers on gfx9-family GPUs.
constexpr int kRawBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes)
{
    uint32_t n = bytes >= 0xfffffffcull ? 0xfffffffcu : (uint32_t)((bytes + 3) & ~3ull);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             kRawBufferFlags);
}

// Byte offset for a load a lane issues only to keep the count of loads in
// flight the same on every lane: past the range of every resource below
// 0xffffffc0 bytes, so the hardware's range check returns zeros without a
// memory access (a larger resource reads in-range bytes there; either way
// the lane ignores the result and nothing faults).
constexpr uint32_t kIdleLoadOffset = 0xffffffc0u;

__device__ __forceinline__ uint32_t ld_b32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    _Float16 v;
    uint16_t b = (uint16_t)h;
    __builtin_memcpy(&v, &b, 2);
    return (float)v;
}

// fp32 -> fp16 bits, round to nearest even (the hardware conversion). The
// argument is first pinned in a register as an fp32 value: without that the
// backend folds a product feeding this conversion into one mixed-precision
// fma that rounds only once, straight to fp16, instead of to fp32 and then
// to fp16.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f)
{
    asm volatile("" : "+v"(f));
    _Float16 v = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &v, 2);
    return b;
}

// The residual argument of the product kernels, as their launchers pass it:
// nullptr; a residual r [T][N] (y = product + r); or, with bit 0 set, the
// gate products g [T][N] of a gate-up pair (y = silu(g) * product with
// silu(g) = g / (1 + exp(-g)), the gated unit's epilogue). r or g may be the
// output itself: each element is read and written by the same lane. The tag
// never crosses the C ABI, whose pointers are 4-byte aligned.
inline const float *gated_epilogue(const float *g)
{
    return reinterpret_cast<const float *>(reinterpret_cast<uintptr_t>(g) | 1u);
}

// silu(g) * v, kept out of line: only gate-up calls take it, and its exp
// inlined into every product kernel grew their code and slowed the plain
// calls of the larger ones
__device__ __attribute__((noinline)) float gated_value(float g, float v)
{
    return g / (1.0f + expf(-g)) * v;
}

// The stored value of output element o for product value v. GATED = false
// for kernel instances that gate-up calls never reach (they take the
// residual add only, and carry no call).
template <bool GATED = true>
__device__ __forceinline__ float epilogue(float v, const float *tagged, int64_t o)
{
    const uintptr_t p = reinterpret_cast<uintptr_t>(tagged);
    const float *r = reinterpret_cast<const float *>(p & ~(uintptr_t)1);
    if (!r)
        return v;
    const float e = r[o];
    if constexpr (!GATED)
        return v + e;
    else
        return (p & 1u) ? gated_value(e, v) : v + e;
}

// Bytes [s, s+4) of the 8-byte little-endian value hi:lo, s in {0, 2}.
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t s)
{
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// A DPP move of v (all lanes active): quad_perm, row rotation, ...
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum of v over the 1 << lr_log2 aligned lanes of a row (lr_log2 <= 6,
// uniform), bitwise the value the xor butterfly leaves in every lane of the
// row (levels m = Lr/2 down to 1, v = v + v of lane ^ m), with all lanes of
// the wave taking part. Levels of 16 lanes and more exchange through the LDS
// crossbar. Inside a 16-lane DPP row the levels 8, 4, 2, 1 are row rotations,
// a few cycles each: a rotation by m reads lane (k -+ m) mod 16, which is
// lane k ^ m itself for m = 8 and for smaller m differs from it by a sum of
// the larger levels' strides, so after those levels (a + b == b + a) it holds
// the same value. Rows of 8 lanes or fewer take the 4-lane level exactly and
// quad permutations below.
__device__ __forceinline__ float row_sum(float v, int lr_log2)
{
    if (lr_log2 >= 6)
        v += __shfl_xor(v, 32, 64);
    if (lr_log2 >= 5)
        v += __shfl_xor(v, 16, 64);
    if (lr_log2 >= 4) {
        v += dpp_move<0x128>(v);  // row_ror:8
        v += dpp_move<0x124>(v);  // row_ror:4
        v += dpp_move<0x122>(v);  // row_ror:2
        v += dpp_move<0x121>(v);  // row_ror:1
    } else {
        if (lr_log2 >= 3)
            v += __shfl_xor(v, 4, 64);
        if (lr_log2 >= 2)
            v += dpp_move<0x4e>(v);  // quad_perm [2, 3, 0, 1]
        if (lr_log2 >= 1)
            v += dpp_move<0xb1>(v);  // quad_perm [1, 0, 3, 2]
    }
    return v;
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

}  // namespace bqm
