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

int launch_q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, hipStream_t stream);
int launch_tq1_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
                    hipStream_t stream);
// Lanes that share one output row in the mat-vec kernels (log2): the smallest
// power of two, at most 64, not below the row's block count.
int lanes_per_row_log2(int64_t nb);
// Dynamic LDS bytes a workgroup may use on the current device.
size_t lds_budget();
// Staged kernel (one to eight columns, activations staged in LDS): whether it
// takes this shape, and its launcher.
bool staged_supported(int64_t K, int32_t T);
int launch_mmvq_staged(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                       int64_t K, int32_t T, hipStream_t stream);
// Matrix-core kernel for 9 to 32 columns.
int launch_mmvq_mfma(const void *w, const void *a, float *y, int32_t *isums, int64_t N,
                     int64_t K, int32_t T, hipStream_t stream);
int launch_mmvq(const void *w, const void *a, float *y, int32_t *isums, int64_t N, int64_t K,
                int32_t T, hipStream_t stream);
int launch_mmvq_id(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                   int64_t N, int64_t K, int64_t T, int32_t n_used, void *workspace,
                   hipStream_t stream);
size_t mmvq_id_workspace_bytes(int64_t E, int64_t T, int32_t n_used);
int launch_mmvq_id_pairs(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                         int64_t N, int64_t K, int64_t T, int32_t n_used, hipStream_t stream);

}  // namespace bqm
