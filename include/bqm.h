/*
 * bqm.h -- C ABI of the MI355X (gfx950) TQ1_0 x Q8_1 quantized mat-vec library.
 *
 * The operation: ternary weights stored in the TQ1_0 block format (five
 * base-3 trits per byte, 256-element blocks) multiplied against activations
 * quantized to Q8_1 (32-element int8 blocks), one or a few activation columns
 * at a time ("MMVQ"), plus the expert-routed variant used by mixture-of-experts
 * layers. Sources, cited by page title and section:
 *   - "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk
 *     contract": "Current behavior" (block format, digit-strided chunks, the
 *     Q8_1 activation blocks of the mat-vec path), "Proposed approach" (a
 *     dedicated byte-major kernel that consumes whole 256-element blocks),
 *     "Acceptance criteria" (plain and expert-routed mat-vec; experts at one
 *     activation per token, more than one block per row, fewer experts used
 *     than available).
 *   - "cuda: opt-in MMVQ activation reuse across output rows": exact
 *     multi-column mat-vec whose columns equal single-column calls.
 *
 * Formats (byte exact; every entry point reads or writes exactly these):
 *   TQ1_0 block, 54 bytes: qs[48] at 0, qh[4] at 48, fp16 scale d at 52
 *     (little endian). Byte value v = sum_c u_c * 3^c, digit u_c in {0,1,2},
 *     trit = u_c - 1. Element e of the block lives in
 *       e <  160: digit e/32         of qs[e % 32]
 *       e <  240: digit (e-160)/16   of qs[32 + (e-160) % 16]
 *       e >= 240: digit (e-240)/4    of qh[(e-240) % 4]
 *     and has value fp32(d) * trit. A weight matrix [N][K] is N rows of K/256
 *     blocks, rows contiguous: block (n, B) starts at byte (n*(K/256) + B)*54.
 *   Q8_1 block, 36 bytes: int8 q[32] at 0, fp16 d at 32, fp16 s at 34. An
 *     activation matrix [T][K] is T columns of K/32 blocks, columns contiguous.
 *     Quantization of 32 floats x: amax = max|x|, d = amax/127 (fp32),
 *     q = round-half-away(x * (1/d)) clamped to [-127, 127] (q = 0 if d = 0),
 *     stored d16 = fp16(d), s16 = fp16(d * sum(q)); fp16 rounding is to
 *     nearest even.
 *
 * Common contract:
 *   - All buffer pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronizes, and enqueues work only on
 *     `stream` (a hipStream_t; NULL = the null stream). Calls are
 *     asynchronous; outputs are fully overwritten.
 *   - Host state: the library keeps only caches of facts about devices and
 *     kernels, filled on first use and never invalidated: per device ordinal
 *     (up to 64), whether it is a gfx950 GPU, its compute-unit count and its
 *     per-workgroup LDS limit (arrays of atomics); and, per (kernel, block
 *     size, LDS size, device), how many workgroups the device holds at once
 *     (a table behind a mutex). Every thread that fills an entry computes the
 *     same value, so calls from several host threads at once are safe. The
 *     launchers also raise a kernel's dynamic-LDS limit through the runtime
 *     (hipFuncSetAttribute, idempotent). There is no other global state.
 *   - Inputs must not alias outputs.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and nothing is written.
 *   - Return value: BQM_OK (0) or a negative BQM_ERR_* code.
 *   - Contents the format rules out (trits outside {-1,0,1} given to tq1_pack,
 *     packed bytes qs > 242 or qh > 80, expert ids outside [0, E)) are not
 *     checked on the device; results for them are unspecified but every
 *     memory access stays inside the buffers described by the sizes given.
 */
#ifndef BQM_H
#define BQM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define BQM_API __attribute__((visibility("default")))
#else
#define BQM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BQM_OK = 0,
    BQM_ERR_NULL = -1,       /* a required pointer is NULL                     */
    BQM_ERR_SHAPE = -2,      /* a size is out of range (see each entry point)  */
    BQM_ERR_ALIGN = -3,      /* a buffer base is not 4-byte aligned            */
    BQM_ERR_WORKSPACE = -4,  /* workspace missing or too small                 */
    BQM_ERR_LAUNCH = -5,     /* the HIP runtime reported a launch error        */
    BQM_ERR_DEVICE = -6      /* the current device is not a gfx950 GPU         */
};

/* Element types of dequantized output. */
enum {
    BQM_DTYPE_F32 = 0,   /* IEEE binary32                                     */
    BQM_DTYPE_F16 = 1,   /* IEEE binary16 (exact here: +-d or 0)              */
    BQM_DTYPE_BF16 = 2   /* bfloat16, rounded to nearest even                 */
};

/* Largest number of activation columns mmvq_tq1_0 accepts. */
#define BQM_MMVQ_MAX_COLS 32

/* Pack ternary weights into TQ1_0 blocks: the inverse of the element map
 * above. "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk
 * contract", "Current behavior": five base-3 trits per qs byte, the qs bytes
 * read digit by digit in 32-element chunks, four trits per qh byte, one fp16
 * scale per 256-element block.
 *   trits [N][K] int8, values -1, 0, +1, row-major.
 *   d     [N][K/256] fp16 bit patterns (uint16), the block scales.
 *   w     [N][K/256] x 54 bytes, output.
 * Shapes: N >= 1, K >= 256, K % 256 == 0. Alignment: none required. */
BQM_API int tq1_pack(const int8_t *trits, const uint16_t *d, void *w,
             int64_t N, int64_t K, void *stream);

/* Quantize activations to Q8_1: the activation blocks the mat-vec consumes
 * ("CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk contract",
 * "Current behavior": the vec_dot reads Q8_1 blocks of 32 activations, each
 * with its own scale), with the scale rule and rounding stated above.
 *   x [T][K] fp32, row-major (column t of the product is row t of x).
 *   a [T][K/32] x 36 bytes, output.
 * Shapes: T >= 1, K >= 32, K % 32 == 0. Alignment: x 4 bytes, a 4 bytes. */
BQM_API int q8_1_quantize(const float *x, void *a, int64_t T, int64_t K, void *stream);

/* Quantized mat-vec / small-batch product ("CUDA: TQ1_0 mat-vec is
 * load-bound by the per-32-element chunk contract", "Current behavior" and
 * "Proposed approach": the blockwise product of TQ1_0 rows and Q8_1 columns,
 * computed by a kernel that reads each packed byte once; several columns per
 * call as in "cuda: opt-in MMVQ activation reuse across output rows", each
 * column's result bitwise that of a one-column call):
 *   y[t][n] = sum_{j < K/32} fp32(d_w[n][j/8]) * fp32(d_a[t][j]) * isum[t][n][j]
 *   isum[t][n][j] = sum_{i < 32} trit[n][32j+i] * q[t][32j+i]   (exact int32)
 *   w [N][K/256] TQ1_0 blocks; a [T][K/32] Q8_1 blocks; y [T][N] fp32 output.
 * Shapes: N >= 1, K >= 256, K % 256 == 0, 1 <= T <= BQM_MMVQ_MAX_COLS, and
 * the weight matrix is below 4 GiB. Alignment: w, a, y 4 bytes. fp32 results
 * differ from the exact sum by at most 1e-5 of sum |terms|; integer sums are
 * exact. */
BQM_API int mmvq_tq1_0(const void *w, const void *a, float *y,
               int64_t N, int64_t K, int32_t T, void *stream);

/* The product with a residual added in its epilogue (the linear-plus-add of a
 * residual block, one launch instead of two: "ops::linear q5: one
 * Capacity=32 K-split rung serves all T<=96", the linear_add route beside
 * the plain linear one):
 *   y[t][n] = mmvq_tq1_0(w, a)[t][n] + r[t][n]
 * computed as one fp32 addition after the product's own result, so y is
 * bitwise fp32(mmvq_tq1_0's output + r) and within 1e-5 of sum |terms| +
 * |r| of the exact value (the addition's rounding is one ulp of |y|).
 *   r [T][N] fp32, read once; it may be y itself (in-place accumulate) but
 *   must not otherwise overlap y (BQM_ERR_SHAPE).
 * Shapes, other arguments, alignment (r 4 bytes) and errors as mmvq_tq1_0. */
BQM_API int mmvq_tq1_0_add(const void *w, const void *a, const float *r, float *y,
                   int64_t N, int64_t K, int32_t T, void *stream);

/* Largest number of activation columns mm_tq1_0 accepts. */
#define BQM_MM_MAX_COLS 65536

/* Many-column product (prefill-sized batches; the step beside the decode
 * product: the pages' pp512 workload, "CUDA: TQ1_0 mat-vec is load-bound by
 * the per-32-element chunk contract", "Measured impact"): the same
 *   y[t][n] = sum_j fp32(d_w[n][j/8]) * fp32(d_a[t][j]) * isum[t][n][j]
 * as mmvq_tq1_0, for 1 <= T <= BQM_MM_MAX_COLS columns, the T columns of a
 * below 4 GiB. Up to 32 columns the call is mmvq_tq1_0. Beyond, the fp32 sums
 * of large calls run over K in order (folded every 64 blocks), so outputs
 * differ from the exact sum by at most about (73 + K/16384) * 2^-24 of
 * sum |terms| (below 1e-5 for K up to 2^20); smaller calls keep the plain
 * product's order. Either way the result is within that bound, and not
 * necessarily bitwise mmvq_tq1_0's. Other shapes, alignment, ownership and
 * errors as mmvq_tq1_0. */
BQM_API int mm_tq1_0(const void *w, const void *a, float *y,
             int64_t N, int64_t K, int64_t T, void *stream);

/* Largest number of activation columns mmvq_tq1_0_f32 accepts. */
#define BQM_MMVQ_F32_MAX_COLS 8

/* The same product on fp32 activations, quantized to Q8_1 inside the call:
 * the result is bitwise that of q8_1_quantize(x) followed by mmvq_tq1_0, with
 * one launch instead of two and no Q8_1 buffer (the quantized blocks live in
 * on-chip memory only). The decode step of a layer, where the two launches
 * would cost more than the product itself.
 *   w [N][K/256] TQ1_0 blocks; x [T][K] fp32, row-major; y [T][N] fp32 output.
 * Shapes: N >= 1, K >= 256, K % 256 == 0, 1 <= T <= BQM_MMVQ_F32_MAX_COLS,
 * the weight matrix and x each below 4 GiB, and the T quantized columns of
 * one staging pass fit the device's LDS (on a 160 KiB-LDS device, every shape
 * but T = 8 with K > 8192); otherwise BQM_ERR_SHAPE.
 * Alignment: w, x, y 4 bytes. */
BQM_API int mmvq_tq1_0_f32(const void *w, const float *x, float *y,
                   int64_t N, int64_t K, int32_t T, void *stream);

/* mmvq_tq1_0_f32 with a residual added in its epilogue: the decode step of
 * a residual block in one launch (quantize, multiply, add):
 *   y[t][n] = mmvq_tq1_0_f32(w, x)[t][n] + r[t][n]
 * bitwise fp32(mmvq_tq1_0_f32's output + r); r as for mmvq_tq1_0_add.
 * Shapes, other arguments, alignment and errors as mmvq_tq1_0_f32. */
BQM_API int mmvq_tq1_0_f32_add(const void *w, const float *x, const float *r, float *y,
                       int64_t N, int64_t K, int32_t T, void *stream);

/* Largest numbers of activation columns mmvq_tq1_0_glu and
 * mmvq_tq1_0_f32_glu accept. */
#define BQM_GLU_MAX_COLS 32
#define BQM_GLU_F32_MAX_COLS 2

/* Gate-up pair with a SiLU-gated epilogue in one launch (the fused mat-vec
 * path of "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk
 * contract", "Proposed approach": the fusion predicate beside the plain and
 * expert paths; the pages name the fusion, not its operation, and the one
 * used is the gated unit of a transformer feed-forward block):
 *   y[t][n] = silu(g[t][n]) * u[t][n],  silu(x) = x / (1 + exp(-x)),
 *   g = mmvq_tq1_0(w_gate, a), u = mmvq_tq1_0(w_up, a)
 * g and u are bitwise those two products' outputs; the epilogue is fp32
 * (exp accurate to a few ulp). Each matrix is read once: up to two columns in
 * one launch (the columns staged once for both matrices); from three, two
 * launches, the gate product into y and then the up product, whose epilogue
 * reads g back from y (no scratch memory).
 *   w_gate, w_up [N][K/256] TQ1_0 blocks each (same shape); a [T][K/32] Q8_1
 *   blocks; y [T][N] fp32 (must not overlap the inputs).
 * 1 <= T <= BQM_GLU_MAX_COLS. Other shapes, alignment and errors as
 * mmvq_tq1_0. */
BQM_API int mmvq_tq1_0_glu(const void *w_gate, const void *w_up, const void *a, float *y,
                           int64_t N, int64_t K, int32_t T, void *stream);

/* The same on fp32 activations quantized to Q8_1 inside the call (bitwise
 * q8_1_quantize followed by mmvq_tq1_0_glu): x [T][K] fp32, 4-byte aligned,
 * 1 <= T <= BQM_GLU_F32_MAX_COLS (the decode step; wider calls quantize once
 * and call mmvq_tq1_0_glu, which beats quantizing inside both products). */
BQM_API int mmvq_tq1_0_f32_glu(const void *w_gate, const void *w_up, const float *x, float *y,
                               int64_t N, int64_t K, int32_t T, void *stream);

/* Dequantize TQ1_0 rows (the dequantize and get_rows operations that sit
 * beside the mat-vec, "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element
 * chunk contract", "Current behavior" and "Proposed approach"):
 *   out[i][k] = fp32(d[r][k/256]) * trit[r][k], r = rows[i] (rows == NULL: r = i),
 *   computed as an fp32 product (a zero trit under a negative scale gives -0)
 *   and stored as out_dtype (BQM_DTYPE_*).
 *   w [N][K/256] TQ1_0 blocks; rows [n_rows] int32 (may be NULL, then
 *   n_rows <= N); out [n_rows][K] elements of out_dtype.
 * Shapes: N >= 1, K >= 256, K % 256 == 0, n_rows >= 1, n_rows * K / 256 < 2^27,
 * the weight matrix below 4 GiB. Row ids outside [0, N) are not checked;
 * they read a clamped row, never outside w.
 * Alignment: w and rows 4 bytes; out 16 bytes. */
BQM_API int tq1_dequantize(const void *w, const int32_t *rows, void *out,
                   int64_t N, int64_t K, int64_t n_rows, int32_t out_dtype, void *stream);

/* Expert-routed product (mixture of experts; MUL_MAT_ID of "CUDA: TQ1_0
 * mat-vec is load-bound by the per-32-element chunk contract", "Acceptance
 * criteria": one activation per token (ne11 = 1), more than one block per
 * row, fewer experts used than available; the per-expert grouping of tokens
 * is the ids compaction of "tools: add mmq-tune, an MMQ tile-width autotuning
 * harness", "Summary"):
 *   y[t][s][n] = mmvq(W[ids[t][s]], a[t])[n]   for t < T, s < n_used
 *   w   [E][N][K/256] TQ1_0 blocks (expert-major, each expert an N x K matrix).
 *   a   [T][K/32] Q8_1 blocks, one activation per token shared by its slots.
 *   ids [T][n_used] int32 expert ids in [0, E) (a repeated id is computed twice).
 *   y   [T][n_used][N] fp32 output.
 *   workspace: device scratch of at least mmvq_id_tq1_0_workspace_bytes(E, T,
 *   n_used) bytes, 256-byte aligned, owned by the caller; it may be reused
 *   between calls that are ordered on one stream (calls that overlap on two
 *   streams need one each). Up to 64 (token, slot) pairs are routed inside
 *   the product kernel and the size is 0: NULL is then accepted. More pairs
 *   (with E <= 4096) are routed by a pre-pass kernel that writes the work
 *   items to the workspace. Tokens that share an expert are multiplied
 *   together, so the expert's weights are read once per group of up to four
 *   of its tokens (64 pairs or fewer) or up to sixteen (more pairs, when the
 *   columns fit the device's LDS). Ids outside [0, E) are not checked:
 *   depending on the kernel the call takes, such a pair's outputs are left
 *   unwritten or computed from a clamped expert; no access leaves w.
 * Shapes: E >= 1, N >= 1, K >= 256, K % 256 == 0, T >= 1, 1 <= n_used <= E,
 * T * n_used <= 65535; one expert's matrix is below 4 GiB.
 * Alignment: w, a, y, ids 4 bytes; workspace 256 bytes. */
BQM_API int mmvq_id_tq1_0(const void *w, const void *a, const int32_t *ids, float *y,
                  int64_t E, int64_t N, int64_t K, int64_t T, int32_t n_used,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Expert-routed product with one activation per (token, slot) pair: the
 * down-projection shape of a mixture of experts, where each slot's input is
 * its own expert's earlier output (MUL_MAT_ID with ne11 = n_used, the other
 * MoE shape beside the ne11 = 1 one of "CUDA: TQ1_0 mat-vec is load-bound by
 * the per-32-element chunk contract", "Acceptance criteria"):
 *   y[t][s][n] = mmvq(W[ids[t][s]], a[t][s])[n]
 *   a [T][n_used][K/32] Q8_1 blocks, one column per pair; every other
 *   argument, the workspace (same size query), the shapes, the alignment and
 *   the error codes as mmvq_id_tq1_0, with the T * n_used columns of a below
 *   4 GiB. Pairs that share an expert are multiplied together. */
BQM_API int mmvq_id_tq1_0_slots(const void *w, const void *a, const int32_t *ids, float *y,
                        int64_t E, int64_t N, int64_t K, int64_t T, int32_t n_used,
                        void *workspace, size_t workspace_bytes, void *stream);

/* mmvq_id_tq1_0 without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation). The call itself allocates nothing: the
 * routing pre-pass writes its work items to a device array the library holds
 * (BQM_NOALLOC_SCRATCH_BYTES per GPU it runs on, kept until the process
 * ends; its device address is looked up on the first call per device).
 * Every shape mmvq_id_tq1_0 accepts fits that array (the largest workspace,
 * 4096 experts and 65535 pairs, is 729,344 bytes); a shape whose workspace
 * would not fit returns BQM_ERR_WORKSPACE before anything is enqueued.
 * Arguments, shapes, alignment, other errors and results (bitwise) as
 * mmvq_id_tq1_0. The array is shared by every call on one GPU and keeps the
 * last call's contents; the pre-pass writes every entry the product kernels
 * read, so nothing has to start at zero. Calls on one GPU that overlap in
 * time (on different streams, or from host threads whose streams are not
 * ordered) race on the array and must not be issued: order them on one
 * stream. */
#define BQM_NOALLOC_SCRATCH_BYTES (768 * 1024)
BQM_API int mmvq_id_tq1_0_noalloc(const void *w, const void *a, const int32_t *ids, float *y,
                          int64_t E, int64_t N, int64_t K, int64_t T, int32_t n_used,
                          void *stream);

/* Workspace size mmvq_id_tq1_0 and mmvq_id_tq1_0_slots need for these sizes
 * (may be 0). */
BQM_API size_t mmvq_id_tq1_0_workspace_bytes(int64_t E, int64_t T, int32_t n_used);

/* Test twin of mmvq_tq1_0: runs the same decode and integer inner loop and
 * writes the exact per-32-element sums isum[t][n][j] (int32 [T][N][K/32])
 * instead of the scaled outputs. Same shapes and alignment as mmvq_tq1_0. */
BQM_API int mmvq_tq1_0_block_isums(const void *w, const void *a, int32_t *isums,
                           int64_t N, int64_t K, int32_t T, void *stream);

/* ---- TQ2_0, the other ternary type ---------------------------------------
 * "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk contract",
 * "Upstream state", names TQ2_0 beside TQ1_0 but prints no layout. The layout
 * read here (the plainest one beside TQ1_0):
 *   TQ2_0 block, 66 bytes: qs[64] at 0, fp16 scale d at 64 (little endian).
 *     Each byte holds four 2-bit fields, field f in bits 2f and 2f+1, each the
 *     digit u = trit + 1 in {0,1,2} (3 is ruled out). Element e of the block
 *     lives in field (e % 128) / 32 of qs[32 * (e / 128) + e % 32], so
 *     32-element chunk c is field c % 4 of qs[32 * (c / 4) .. + 31]: TQ1_0's
 *     digit-major order for its first 128 elements, then again on the second
 *     32 bytes. Element value fp32(d) * trit; rows as for TQ1_0: block (n, B)
 *     starts at byte (n * (K/256) + B) * 66.
 * Fields holding 3 are not checked on the device (results unspecified, every
 * access stays in bounds, as for TQ1_0). */

/* Pack ternary weights into TQ2_0 blocks: the inverse of the element map
 * above.
 *   trits [N][K] int8, values -1, 0, +1, row-major.
 *   d     [N][K/256] fp16 bit patterns (uint16), the block scales.
 *   w     [N][K/256] x 66 bytes, output.
 * Shapes: N >= 1, K >= 256, K % 256 == 0, weight matrix below 4 GiB.
 * Alignment: none required. */
BQM_API int tq2_pack(const int8_t *trits, const uint16_t *d, void *w,
             int64_t N, int64_t K, void *stream);

/* The quantized product of mmvq_tq1_0 with TQ2_0 weights: the same
 * definition (y[t][n] = sum_j fp32(d_w[n][j/8]) * fp32(d_a[t][j]) *
 * isum[t][n][j], exact int32 sums), the same Q8_1 activations, the same fp32
 * order per block (so a TQ2_0 matrix and the TQ1_0 packing of the same trits
 * and scales give bitwise equal outputs), and a kernel that reads each packed
 * byte once ("Upstream state": every packed byte loaded once, all its digits
 * expanded in place).
 *   w [N][K/256] TQ2_0 blocks; a [T][K/32] Q8_1 blocks; y [T][N] fp32 output.
 * Shapes: N >= 1, K >= 256, K % 256 == 0, 1 <= T <= BQM_MMVQ_MAX_COLS, weight
 * matrix below 4 GiB. Alignment: w, a, y 4 bytes. Tolerance as mmvq_tq1_0. */
BQM_API int mmvq_tq2_0(const void *w, const void *a, float *y,
               int64_t N, int64_t K, int32_t T, void *stream);

/* Test twin of mmvq_tq2_0: the exact per-32-element sums isum[t][n][j]
 * (int32 [T][N][K/32]) instead of the outputs. Same shapes and alignment. */
BQM_API int mmvq_tq2_0_block_isums(const void *w, const void *a, int32_t *isums,
                           int64_t N, int64_t K, int32_t T, void *stream);

/* Human-readable text for a status code (static storage). */
BQM_API const char *bqm_status_string(int status);

/* Library version, as major * 10000 + minor * 100 + patch. */
BQM_API int bqm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BQM_H */
