// bqm_api.hip -- the C ABI declared in include/bqm.h: argument validation on
// the host, one dispatch point per entry, launches on the caller's stream.
#include <string.h>

#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr uint64_t kMaxBufferBytes = 0xfffffffcull;  // 32-bit byte offsets inside one matrix

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// Device check, cached per device ordinal: gfx950 only.
int check_device()
{
    // 0 unknown, 1 ok, -1 not gfx950; atomics, so concurrent first calls
    // from several host threads each store the same value without a race
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return BQM_ERR_DEVICE;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c)
            return c > 0 ? BQM_OK : BQM_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    int ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
             strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64)
        cached[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? BQM_OK : BQM_ERR_DEVICE;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// block_bytes: 54 for TQ1_0, 66 for TQ2_0
int check_matrix(int64_t N, int64_t K, uint64_t block_bytes = 54)
{
    if (N < 1 || K < 256 || K % 256 != 0)
        return BQM_ERR_SHAPE;
    if ((uint64_t)N * (uint64_t)(K / 256) * block_bytes > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    return BQM_OK;
}

}  // namespace

extern "C" {

int tq1_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
             void *stream)
{
    if (!trits || !d || !w)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K))
        return rc;
    if (int rc = check_device())
        return rc;
    return bqm::launch_tq1_pack(trits, d, w, N, K, as_stream(stream));
}

int q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, void *stream)
{
    if (!x || !a)
        return BQM_ERR_NULL;
    if (T < 1 || K < 32 || K % 32 != 0 || (uint64_t)T * (uint64_t)K > (1ull << 40))
        return BQM_ERR_SHAPE;
    if (!aligned4(x) || !aligned4(a))
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return bqm::launch_q8_1_quantize(x, a, T, K, as_stream(stream));
}

// The residual must be the output itself or lie wholly outside it: each
// output element is read from r and written to y by the same lane, so only
// a partial overlap could mix elements.
static bool residual_ok(const float *r, const void *y, int64_t N, int32_t T)
{
    if ((const void *)r == y)
        return true;
    const uintptr_t rb = (uintptr_t)r, yb = (uintptr_t)y, n = (uintptr_t)N * (uintptr_t)T * 4u;
    return rb + n <= yb || yb + n <= rb;
}

// r: the residual of the add entry point (nullptr for the others);
// block_bytes: the weight format's block size.
static int mmvq_common(const void *w, const void *a, const void *out, int64_t N, int64_t K,
                       int32_t T, const float *r = nullptr, uint64_t block_bytes = 54)
{
    if (!w || !a || !out)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K, block_bytes))
        return rc;
    if (T < 1 || T > BQM_MMVQ_MAX_COLS)
        return BQM_ERR_SHAPE;
    if ((uint64_t)T * (uint64_t)(K / 32) * 36ull > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (r && !residual_ok(r, out, N, T))
        return BQM_ERR_SHAPE;
    if (!aligned4(w) || !aligned4(a) || !aligned4(out) || (r && !aligned4(r)))
        return BQM_ERR_ALIGN;
    return check_device();
}

int mmvq_tq1_0(const void *w, const void *a, float *y, int64_t N, int64_t K, int32_t T,
               void *stream)
{
    if (int rc = mmvq_common(w, a, y, N, K, T))
        return rc;
    return bqm::launch_mmvq(w, a, y, nullptr, N, K, T, as_stream(stream));
}

int mmvq_tq1_0_add(const void *w, const void *a, const float *r, float *y, int64_t N, int64_t K,
                   int32_t T, void *stream)
{
    if (!r)
        return BQM_ERR_NULL;
    if (int rc = mmvq_common(w, a, y, N, K, T, r))
        return rc;
    return bqm::launch_mmvq(w, a, y, nullptr, N, K, T, as_stream(stream), r);
}

int mm_tq1_0(const void *w, const void *a, float *y, int64_t N, int64_t K, int64_t T,
             void *stream)
{
    if (!w || !a || !y)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K))
        return rc;
    if (T < 1 || T > BQM_MM_MAX_COLS || (uint64_t)T * (uint64_t)(K / 32) * 36ull > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (!aligned4(w) || !aligned4(a) || !aligned4(y))
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return bqm::launch_mm(w, a, y, N, K, T, as_stream(stream));
}

// with_r: the residual-add entry point (r required).
static int mmvq_f32_call(const void *w, const float *x, const float *r, bool with_r, float *y,
                         int64_t N, int64_t K, int32_t T, void *stream)
{
    if (!w || !x || !y || (with_r && !r))
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K))
        return rc;
    if (T < 1 || T > BQM_MMVQ_F32_MAX_COLS || (uint64_t)T * (uint64_t)K * 4ull > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (with_r && !residual_ok(r, y, N, T))
        return BQM_ERR_SHAPE;
    if (!aligned4(w) || !aligned4(x) || !aligned4(y) || (with_r && !aligned4(r)))
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    // three to eight columns: the quad kernel where it takes the shape (it
    // stages, and so quantizes, each column once per 16 rows like the staged
    // kernel, with a quarter of the staged kernel's LDS reads)
    if (bqm::quad_supported(K, T))
        return bqm::launch_mmvq_quad_f32(w, x, y, N, K, T, as_stream(stream), r);
    if (!bqm::staged_supported(K, T))
        return BQM_ERR_SHAPE;
    return bqm::launch_mmvq_staged_f32(w, x, y, N, K, T, as_stream(stream), r);
}

int mmvq_tq1_0_f32(const void *w, const float *x, float *y, int64_t N, int64_t K, int32_t T,
                   void *stream)
{
    return mmvq_f32_call(w, x, nullptr, false, y, N, K, T, stream);
}

int mmvq_tq1_0_f32_add(const void *w, const float *x, const float *r, float *y, int64_t N,
                       int64_t K, int32_t T, void *stream)
{
    return mmvq_f32_call(w, x, r, true, y, N, K, T, stream);
}

// f32: the columns are fp32 (quantized inside the call, at most two), else
// Q8_1 blocks. Up to two columns one launch of the staged wave pairs; beyond,
// the gate product into y, then the up product with the gated epilogue
// reading y.
static int glu_call(const void *wg, const void *wu, const void *a, float *y, int64_t N,
                    int64_t K, int32_t T, bool f32, void *stream)
{
    if (!wg || !wu || !a || !y)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K))
        return rc;
    const uint64_t col_bytes = f32 ? (uint64_t)K * 4ull : (uint64_t)(K / 32) * 36ull;
    const int max_cols = f32 ? BQM_GLU_F32_MAX_COLS : BQM_GLU_MAX_COLS;
    if (T < 1 || T > max_cols || (uint64_t)T * col_bytes > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (!aligned4(wg) || !aligned4(wu) || !aligned4(a) || !aligned4(y))
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    const hipStream_t st = as_stream(stream);
    if (T <= bqm::kGluMaxCols)
        return bqm::launch_mmvq_glu(wg, wu, a, y, N, K, T, f32, st);
    if (int rc = bqm::launch_mmvq(wg, a, y, nullptr, N, K, T, st))
        return rc;
    return bqm::launch_mmvq(wu, a, y, nullptr, N, K, T, st, bqm::gated_epilogue(y));
}

int mmvq_tq1_0_glu(const void *w_gate, const void *w_up, const void *a, float *y, int64_t N,
                   int64_t K, int32_t T, void *stream)
{
    return glu_call(w_gate, w_up, a, y, N, K, T, false, stream);
}

int mmvq_tq1_0_f32_glu(const void *w_gate, const void *w_up, const float *x, float *y,
                       int64_t N, int64_t K, int32_t T, void *stream)
{
    return glu_call(w_gate, w_up, x, y, N, K, T, true, stream);
}

int mmvq_tq1_0_block_isums(const void *w, const void *a, int32_t *isums, int64_t N, int64_t K,
                           int32_t T, void *stream)
{
    if (int rc = mmvq_common(w, a, isums, N, K, T))
        return rc;
    return bqm::launch_mmvq(w, a, nullptr, isums, N, K, T, as_stream(stream));
}

int tq2_pack(const int8_t *trits, const uint16_t *d, void *w, int64_t N, int64_t K,
             void *stream)
{
    if (!trits || !d || !w)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K, 66))
        return rc;
    if (int rc = check_device())
        return rc;
    return bqm::launch_tq2_pack(trits, d, w, N, K, as_stream(stream));
}

int mmvq_tq2_0(const void *w, const void *a, float *y, int64_t N, int64_t K, int32_t T,
               void *stream)
{
    if (int rc = mmvq_common(w, a, y, N, K, T, nullptr, 66))
        return rc;
    return bqm::launch_mmvq_tq2(w, a, y, nullptr, N, K, T, as_stream(stream));
}

int mmvq_tq2_0_block_isums(const void *w, const void *a, int32_t *isums, int64_t N, int64_t K,
                           int32_t T, void *stream)
{
    if (int rc = mmvq_common(w, a, isums, N, K, T, nullptr, 66))
        return rc;
    return bqm::launch_mmvq_tq2(w, a, nullptr, isums, N, K, T, as_stream(stream));
}

int tq1_dequantize(const void *w, const int32_t *rows, void *out, int64_t N, int64_t K,
                   int64_t n_rows, int32_t out_dtype, void *stream)
{
    if (!w || !out)
        return BQM_ERR_NULL;
    if (int rc = check_matrix(N, K))
        return rc;
    if (n_rows < 1 || (!rows && n_rows > N) || n_rows * (K / 256) >= (1ll << 27) ||
        out_dtype < BQM_DTYPE_F32 || out_dtype > BQM_DTYPE_BF16)
        return BQM_ERR_SHAPE;
    // every dtype's kernel stores 16 bytes per lane
    if (!aligned4(w) || (rows && !aligned4(rows)) || ((uintptr_t)out & 15u))
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return bqm::launch_tq1_dequantize(w, rows, out, N, K, n_rows, out_dtype, as_stream(stream));
}

size_t mmvq_id_tq1_0_workspace_bytes(int64_t E, int64_t T, int32_t n_used)
{
    if (E < 1 || T < 1 || n_used < 1 || n_used > E || T * (int64_t)n_used > 65535)
        return 0;
    return bqm::mmvq_id_workspace_bytes(E, T, n_used);
}

// Both expert-routed products; per_slot: one activation column per
// (token, slot) pair instead of one per token.
static int mmvq_id_call(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                        int64_t N, int64_t K, int64_t T, int32_t n_used, bool per_slot,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    if (!w || !a || !ids || !y)
        return BQM_ERR_NULL;
    if (E < 1 || T < 1 || n_used < 1 || n_used > E || T * (int64_t)n_used > 65535)
        return BQM_ERR_SHAPE;
    if (int rc = check_matrix(N, K))
        return rc;
    const uint64_t a_cols = (uint64_t)T * (per_slot ? (uint64_t)n_used : 1ull);
    if (a_cols * (uint64_t)(K / 32) * 36ull > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (!aligned4(w) || !aligned4(a) || !aligned4(ids) || !aligned4(y))
        return BQM_ERR_ALIGN;
    const size_t need = bqm::mmvq_id_workspace_bytes(E, T, n_used);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return BQM_ERR_WORKSPACE;
    if (workspace && ((uintptr_t)workspace & 255u) != 0)
        return BQM_ERR_ALIGN;
    if (int rc = check_device())
        return rc;
    return bqm::launch_mmvq_id(w, a, ids, y, E, N, K, T, n_used, per_slot, workspace,
                               as_stream(stream));
}

int mmvq_id_tq1_0(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                  int64_t N, int64_t K, int64_t T, int32_t n_used, void *workspace,
                  size_t workspace_bytes, void *stream)
{
    return mmvq_id_call(w, a, ids, y, E, N, K, T, n_used, false, workspace, workspace_bytes,
                        stream);
}

int mmvq_id_tq1_0_noalloc(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                          int64_t N, int64_t K, int64_t T, int32_t n_used, void *stream)
{
    // the same checks as mmvq_id_tq1_0, except that the workspace is the
    // library's device scratch
    if (!w || !a || !ids || !y)
        return BQM_ERR_NULL;
    if (E < 1 || T < 1 || n_used < 1 || n_used > E || T * (int64_t)n_used > 65535)
        return BQM_ERR_SHAPE;
    if (int rc = check_matrix(N, K))
        return rc;
    if ((uint64_t)T * (uint64_t)(K / 32) * 36ull > kMaxBufferBytes)
        return BQM_ERR_SHAPE;
    if (!aligned4(w) || !aligned4(a) || !aligned4(ids) || !aligned4(y))
        return BQM_ERR_ALIGN;
    if (bqm::mmvq_id_workspace_bytes(E, T, n_used) > bqm::kNoAllocScratchBytes)
        return BQM_ERR_WORKSPACE;
    if (int rc = check_device())
        return rc;
    void *scratch = nullptr;
    if (int rc = bqm::noalloc_scratch(&scratch))
        return rc;
    return bqm::launch_mmvq_id(w, a, ids, y, E, N, K, T, n_used, false, scratch,
                               as_stream(stream));
}

int mmvq_id_tq1_0_slots(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                        int64_t N, int64_t K, int64_t T, int32_t n_used, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    return mmvq_id_call(w, a, ids, y, E, N, K, T, n_used, true, workspace, workspace_bytes,
                        stream);
}

const char *bqm_status_string(int status)
{
    switch (status) {
    case BQM_OK:
        return "ok";
    case BQM_ERR_NULL:
        return "a required pointer is NULL";
    case BQM_ERR_SHAPE:
        return "a size is out of range";
    case BQM_ERR_ALIGN:
        return "a buffer is misaligned";
    case BQM_ERR_WORKSPACE:
        return "workspace missing or too small";
    case BQM_ERR_LAUNCH:
        return "the HIP runtime reported a launch error";
    case BQM_ERR_DEVICE:
        return "the current device is not a gfx950 GPU";
    default:
        return "unknown status";
    }
}

int bqm_version(void) { return kVersion; }

}  // extern "C"
