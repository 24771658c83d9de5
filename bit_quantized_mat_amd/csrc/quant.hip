// quant.hip -- Q8_1 activation quantization and TQ1_0 weight packing (gfx950).
//
// Q8_1: 32-element blocks of int8 with an fp16 scale and an fp16 sum; the
// mat-vec consumes activations in this form ("CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract", "Current behavior").
// TQ1_0: five base-3 trits per byte in 256-element blocks (same section).
// Byte layouts and rounding rules are the ones declared in include/bqm.h.
#include "common.hpp"
#include "launch.hpp"

namespace bqm {

// One 32-lane half-wave per Q8_1 block: lane i owns element i.
// amax, the scale, and sum(q) are exact wave reductions; the scale and the
// reciprocal use IEEE division (the build keeps HIP's correctly rounded fp32
// divide), and q rounds half away from zero.
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float *__restrict__ x,
                                                            uint8_t *__restrict__ a,
                                                            int64_t nblocks)
{
    const int lane = threadIdx.x & 31;
    const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
    if (blk >= nblocks)
        return;  // whole half-waves exit together (nblocks counts 32-lane groups)
    const float v = x[blk * kQ81BlockElems + lane];
    float amax = fabsf(v);
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, m, 32));
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    int q = (int)roundf(v * id);
    q = q > 127 ? 127 : (q < -127 ? -127 : q);
    int sum = q;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1)
        sum += __shfl_xor(sum, m, 32);
    uint8_t *out = a + blk * kQ81BlockBytes;
    out[lane] = (uint8_t)(int8_t)q;
    if (lane == 0) {
        const uint32_t dh = f32_to_f16_bits(d);
        const uint32_t sh = f32_to_f16_bits(d * (float)sum);
        *reinterpret_cast<uint32_t *>(out + 32) = dh | (sh << 16);
    }
}

int launch_q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, hipStream_t stream)
{
    const int64_t nblocks = T * (K / kQ81BlockElems);
    const int64_t threads = nblocks * 32;
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x,
                       static_cast<uint8_t *>(a), nblocks);
    return check_launch();
}

// TQ1_0 packing: one thread per output byte. Byte p < 52 of block (n, B)
// gathers the trits of its digit slots (element map in include/bqm.h) and
// forms the plain base-3 value sum_c (trit + 1) * 3^c; bytes 52..53 copy the
// fp16 scale, little endian.
__device__ __forceinline__ int slot_element(int p, int c)
{
    if (p < 32)
        return 32 * c + p;
    if (p < 48)
        return 160 + 16 * c + (p - 32);
    return 240 + 4 * c + (p - 48);
}

__global__ __launch_bounds__(256) void tq1_pack_kernel(const int8_t *__restrict__ trits,
                                                       const uint16_t *__restrict__ d,
                                                       uint8_t *__restrict__ w, int64_t nb,
                                                       int64_t total_bytes)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_bytes)
        return;
    const int64_t g = i / kTq1BlockBytes;           // global block index n * nb + B
    const int p = (int)(i - g * kTq1BlockBytes);     // byte within the block
    uint32_t out;
    if (p < 52) {
        const int ndig = p < 48 ? 5 : 4;
        const int8_t *blk = trits + g * kTq1BlockElems;  // rows are K = nb * 256 long
        int v = 0, pw = 1;
        for (int c = 0; c < ndig; c++) {
            v += (blk[slot_element(p, c)] + 1) * pw;
            pw *= 3;
        }
        out = (uint32_t)v;
    } else {
        const uint32_t h = d[g];
        out = p == 52 ? (h & 0xffu) : (h >> 8);
    }
    w[i] = (uint8_t)out;
    (void)nb;
}

int launch_tq1_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
                    hipStream_t stream)
{
    const int64_t nb = K / kTq1BlockElems;
    const int64_t total = N * nb * kTq1BlockBytes;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(tq1_pack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, trits, d,
                       static_cast<uint8_t *>(w), nb, total);
    return check_launch();
}

}  // namespace bqm
