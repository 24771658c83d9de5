// quant.hip -- Q8_1 activation quantization and TQ1_0 weight packing (gfx950).
//
// Q8_1: 32-element blocks of int8 with an fp16 scale and an fp16 sum; the
// mat-vec consumes activations in this form ("CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract", "Current behavior").
// TQ1_0: five base-3 trits per byte in 256-element blocks (same section).
// Byte layouts and rounding rules are the ones declared in include/bqm.h.
#include "common.hpp"
#include "launch.hpp"
#include "q8_1.hpp"

namespace bqm {

// Two lanes per Q8_1 block, sixteen elements per lane (four 16-byte loads
// and four dwords of q bytes each); the arithmetic is q8_1_block_by_2.
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float *__restrict__ x,
                                                            uint8_t *__restrict__ a,
                                                            int64_t nblocks)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = t >> 1;
    const int h = (int)(t & 1);
    // pairs past the end compute on a copy of the last block and store nothing,
    // so that both lanes of every pair take part in the exchanges
    const int64_t src = blk < nblocks ? blk : nblocks - 1;
    // a buffer load needs only the dword alignment the entry point checks; the
    // descriptor covers this workgroup's 128 blocks
    const int64_t first = (int64_t)blockIdx.x * (blockDim.x >> 1);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(
        x + first * kQ81BlockElems, (uint64_t)(nblocks - first) * kQ81BlockElems * sizeof(float));
    const uint32_t off = (uint32_t)((src - first) * kQ81BlockElems + 16 * h) * 4;
    float xs[16];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const u32x4 v = ld_b128(rx, off + 16 * k);
        xs[4 * k] = __uint_as_float(v.x);
        xs[4 * k + 1] = __uint_as_float(v.y);
        xs[4 * k + 2] = __uint_as_float(v.z);
        xs[4 * k + 3] = __uint_as_float(v.w);
    }
    const Q81Part p = q8_1_block_by_2(xs);
    if (blk < nblocks) {
        uint32_t *out = reinterpret_cast<uint32_t *>(a + blk * kQ81BlockBytes);
        // blocks are 36 bytes apart: dword stores (the output is only
        // dword-aligned)
#pragma unroll
        for (int k = 0; k < 4; k++)
            out[4 * h + k] = p.q4[k];
        if (h == 0)
            out[8] = q8_1_scale_field(p);
    }
}

int launch_q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, hipStream_t stream)
{
    const int64_t nblocks = T * (K / kQ81BlockElems);
    const int64_t threads = nblocks * 2;
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
