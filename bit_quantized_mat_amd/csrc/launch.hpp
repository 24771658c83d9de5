// launch.hpp -- host-side launch helpers and the internal launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bqm.h"

namespace bqm {

// Status after enqueueing a kernel: BQM_ERR_LAUNCH if the runtime reports an error.
inline int check_launch()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BQM_OK : BQM_ERR_LAUNCH;
}

// Dynamic LDS: 64 KiB is always available; beyond that the launcher raises
// the kernel's limit up to what the device reports (160 KiB on gfx950).
constexpr size_t kLdsDefault = 64 * 1024;
constexpr size_t kLdsMax = 160 * 1024;

// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default (idempotent; the runtime keeps the attribute per function).
inline void allow_dynamic_lds(const void *kernel, size_t bytes)
{
    if (bytes > kLdsDefault)
        (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

int launch_q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, hipStream_t stream);
int launch_tq1_dequantize(const void *w, const int32_t *rows, void *out, int64_t N, int64_t K,
                          int64_t n_rows, int dtype, hipStream_t stream);
int launch_tq1_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
                    hipStream_t stream);
// Lanes that share one output row in the mat-vec kernels (log2): the smallest
// power of two, at most 64, not below the row's block count.
int lanes_per_row_log2(int64_t nb);
// Dynamic LDS bytes a workgroup may use on the current device.
size_t lds_budget();
// Compute units of the current device.
int compute_units();
// Workgroups of `kernel` (with this block size and dynamic LDS) that the
// current device runs at once.
int resident_workgroups(const void *kernel, int threads, size_t lds);
// Waves per workgroup of the staged kernels for N rows at 1 << lr lanes per
// row: 1, 4 or 8.
int staged_workgroup_waves(int64_t N, int lr);
// Staged kernel (one to eight columns, activations staged in LDS): whether it
// takes this shape, and its launcher.
bool staged_supported(int64_t K, int32_t T);
// r (every product launcher): when given, y = product + r, one fp32 addition
// after the product's own result (r [T][N], may be y itself); tagged by
// gated_epilogue (common.hpp), y = silu(r) * product instead (the up product
// of a gate-up pair, r the gate products).
int launch_mmvq_staged(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                       int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
// The staged kernel on fp32 activations, quantized to Q8_1 while staging.
int launch_mmvq_staged_f32(const void *w, const float *x, float *y, int64_t N, int64_t K,
                           int32_t T, hipStream_t stream, const float *r = nullptr);
// Gate-up pair with the SiLU-gated epilogue, y = silu(wg . a) * (wu . a), in
// one launch of the staged kernel's wave pairs: one or two columns (f32:
// fp32 columns, quantized while staging); BQM_ERR_SHAPE for other column
// counts or rows it cannot stage. (Wider calls run the gate product into y,
// then the up product with the gated epilogue reading y.)
constexpr int kGluMaxCols = 2;
int launch_mmvq_glu(const void *wg, const void *wu, const void *a, float *y, int64_t N, int64_t K,
                    int32_t T, bool f32, hipStream_t stream);
// Quad kernel (three to eight columns, whole-block decode per lane, sub-block
// sums on the matrix cores; rows of more than 8 blocks): whether it takes this
// shape, and its launchers (Q8_1 activations, and fp32 activations quantized
// while staging).
bool quad_supported(int64_t K, int32_t T);
int launch_mmvq_quad(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
int launch_mmvq_quad_f32(const void *w, const float *x, float *y, int64_t N, int64_t K,
                         int32_t T, hipStream_t stream, const float *r = nullptr);
// Matrix-core kernel: any shape, 1 to 32 columns; the dispatcher gives it
// every call of at least kMfmaMinCols columns, and the calls of fewer that
// neither the quad kernel nor the staged kernel takes or that are too small
// to give the staged kernel a second wave per SIMD.
constexpr int kMfmaMinCols = 5;

int launch_mmvq_mfma(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
// Matrix-core kernel with all activation columns resident in LDS: whether it
// takes this shape (the columns fit and a row has at least as many lane
// groups as the workgroup has waves), and its launcher.
bool mfma_resident_supported(int64_t K, int32_t T);
int launch_mmvq_mfma_resident(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                              int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
// Matrix-core kernel with each wave's activation operands in registers
// (rows of 5 to 16 blocks, up to 32 columns): whether it takes this shape,
// and its launcher.
bool mfma_reg_supported(int64_t K, int32_t T);
int launch_mmvq_mfma_reg(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                         int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
// Whether pair tiles (two 16-row tiles per 16 x 16 x 64 matrix product, at
// most 8 columns) pay for N rows: a 32-row unit costs about 1.5 of a 16-row
// one, so they do when the busiest compute unit has fewer than two thirds as
// many units.
bool pair_tiles_pay(int64_t N);
// The same kernel on TQ2_0 weights (same shapes).
int launch_mmvq_mfma_reg_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                             int64_t K, int32_t T, hipStream_t stream, const float *r = nullptr);
// The resident and streamed matrix-core kernels on TQ2_0 weights (same shapes
// as their TQ1_0 launchers).
int launch_mmvq_mfma_resident_tq2(const void *w, const void *a, float *y, int32_t *isums,
                                  int64_t N, int64_t K, int32_t T, hipStream_t stream);
int launch_mmvq_mfma_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                         int64_t K, int32_t T, hipStream_t stream);
// TQ2_0: packing, and the product's dispatch (any shape mmvq_tq2_0 accepts).
int launch_tq2_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
                    hipStream_t stream);
int launch_mmvq_tq2(const void *w, const void *a, float *y, int32_t *isums, int64_t N, int64_t K,
                    int32_t T, hipStream_t stream);
// Its expert-routed mode (wide work items of up to 16 pairs, written by the
// routing pre-pass): whether it takes rows of K elements, and its launcher.
bool mfma_resident_id_supported(int64_t K);
int launch_mmvq_mfma_resident_id(const void *w, const void *a, float *y, int64_t N, int64_t K,
                                 int64_t a_cols, const int32_t *routed, int max_items,
                                 int max_wide, int pairs_per_col, hipStream_t stream);
// Many-column product (any T): the resident kernel's item mode over chunks
// of 32 (or 16) columns; whether it takes rows of K elements, and its
// launcher.
bool mm_chunked_supported(int64_t K);
int launch_mm_chunked(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
                      hipStream_t stream);
int launch_mmvq(const void *w, const void *a, float *y, int32_t *isums, int64_t N, int64_t K,
                int32_t T, hipStream_t stream, const float *r = nullptr);
int launch_mm(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
              hipStream_t stream);
// K-streaming matrix-core kernel for many columns (any K and T): its grid
// size for a call, and its launcher.
int64_t mm_stream_workgroups(int64_t N, int64_t T);
int launch_mm_stream(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
                     hipStream_t stream);
// per_slot: a holds one Q8_1 column per (token, slot) pair instead of one
// per token.
int launch_mmvq_id(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                   int64_t N, int64_t K, int64_t T, int32_t n_used, bool per_slot,
                   void *workspace, hipStream_t stream);
size_t mmvq_id_workspace_bytes(int64_t E, int64_t T, int32_t n_used);
// Size of the device-resident scratch of mmvq_id_tq1_0_noalloc: at least the
// workspace of the largest call mmvq_id_tq1_0 accepts that uses one (4096
// experts, 65535 pairs: 729,344 bytes).
constexpr size_t kNoAllocScratchBytes = 768 * 1024;
// Device address of that scratch on the current device (looked up on the
// first call per device, then cached).
int noalloc_scratch(void **ptr);
int launch_mmvq_id_pairs(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                         int64_t N, int64_t K, int64_t T, int32_t n_used, int pairs_per_col,
                         hipStream_t stream);

}  // namespace bqm
