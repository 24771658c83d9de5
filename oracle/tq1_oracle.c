/*
 * tq1_oracle.c -- TEST INFRASTRUCTURE ONLY. This is the plain, slow CPU
 * reference ("oracle") for the TQ1_0 x Q8_1 quantized mat-vec. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product library never links, calls or imports it, and the two share no code.
 *
 * Everything here follows the format and the product definition directly,
 * element by element, in the order the definition states it, with no blocking,
 * fusion or reordering. Sources (web pages; cited by title and section):
 *
 *  [P1] "CUDA: TQ1_0 mat-vec is load-bound by the per-32-element chunk
 *       contract", section "Current behavior": TQ1_0 stores five trits per
 *       byte in base 3; 32-element chunk c (c = 0..4) takes digit c of packed
 *       bytes qs[0..31]; the mat-vec consumes Q8_1-quantized activations
 *       (bq8_1) in 32-element chunks. Same section: the CPU reference walks a
 *       256-element block once and spends each packed byte on all its trits.
 *  [P1-acc] same page, section "Acceptance criteria": MUL_MAT_ID at ne11 = 1
 *       (one activation per token, broadcast over its expert slots).
 *
 * Readings where the pages are silent:
 *  - block = 54 bytes: qs[48] at 0, qh[4] at 48, fp16 d (little endian) at 52;
 *    byte value v = sum_c u_c * 3^c with digit u_c in {0,1,2} and trit
 *    t = u_c - 1 (digit 0 is the least significant);
 *  - elements 160..239 continue the digit-major stride over qs[32..47]
 *    (16 bytes per digit), elements 240..255 over qh[0..3] (4 per digit);
 *  - Q8_1 block = 36 bytes: int8 q[32] at 0, fp16 d at 32, fp16 s at 34;
 *    d = amax/127 (fp32), q = round-half-away(x * (1/d)) clamped to +-127,
 *    s = fp16(d * sum q); fp16 conversions round to nearest even.
 *
 *  [P1-up] same page, section "Upstream state": names a second ternary type,
 *       TQ2_0, and gives no layout for it. Reading used here (the plainest
 *       one beside TQ1_0): 256-element blocks, one 2-bit field per element
 *       holding the digit u = trit + 1 (the value 3 unused), four fields per
 *       byte, then the fp16 scale: qs[64] at 0, d at 64 (66 bytes). Element
 *       e lives in byte 32 * (e / 128) + e % 32, field (e % 128) / 32 (bits
 *       2f, 2f + 1): TQ1_0's digit-major order for its first 128 elements,
 *       repeated on the second 32 bytes, so 32-element chunk c is field c % 4
 *       of bytes 32 * (c / 4) .. + 31. Pinned by hand-worked blocks
 *       (tests/golden/tq2_blocks.txt) and by bitwise agreement with the TQ1_0
 *       product of the same trits.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TQ1_BLOCK_ELEMS 256
#define TQ1_BLOCK_BYTES 54
#define Q81_BLOCK_ELEMS 32
#define Q81_BLOCK_BYTES 36

#define TQ2_BLOCK_BYTES 66

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format definition.      */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> float (exact: every binary16 value is a binary32 value). */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expf = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    float v;
    if (expf == 0x1f) {
        v = man ? NAN : INFINITY;
    } else if (expf == 0) {
        v = ldexpf((float)man, -24); /* subnormal: man * 2^-24 */
    } else {
        v = ldexpf((float)(1024 + man), expf - 25); /* (1.man) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* float -> binary16 bits, round to nearest, ties to even. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    int expf = (int)((x >> 23) & 0xffu);
    uint32_t man = x & 0x7fffffu;
    if (expf == 0xff)
        return man ? (uint16_t)(sign | 0x7e00u) : (uint16_t)(sign | 0x7c00u);
    /* |f| = m * 2^E exactly */
    uint32_t m;
    int E;
    if (expf == 0) {
        m = man;
        E = -149;
    } else {
        m = man | 0x800000u;
        E = expf - 150;
    }
    if (m == 0)
        return sign;
    int bitlen = 0;
    for (uint32_t t = m; t; t >>= 1)
        bitlen++;
    int eh = bitlen - 1 + E;      /* floor(log2 |f|) */
    int q = eh - 10;              /* quantum of an 11-bit significand */
    if (q < -24)
        q = -24;                  /* binary16 subnormal quantum */
    uint64_t n;
    int r = q - E;                /* bits dropped */
    if (r <= 0) {
        n = (uint64_t)m << (-r);
    } else if (r > 40) {
        n = 0;                    /* far below half a quantum */
    } else {
        uint64_t mm = m;
        n = mm >> r;
        uint64_t rem = mm & ((1ull << r) - 1);
        uint64_t half = 1ull << (r - 1);
        if (rem > half || (rem == half && (n & 1)))
            n++;
    }
    if (n == 0)
        return sign;
    if (n == 2048) { /* rounding carried into the next binade */
        n = 1024;
        q++;
    }
    if (q == -24 && n < 1024)
        return (uint16_t)(sign | n); /* subnormal */
    int expfield = q + 25;
    if (expfield >= 31)
        return (uint16_t)(sign | 0x7c00u); /* overflow -> infinity */
    return (uint16_t)(sign | (expfield << 10) | (uint16_t)(n - 1024));
}

void oracle_f32_to_f16_array(const float *x, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        h[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *x, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        x[i] = oracle_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* TQ1_0 element map and base-3 digits [P1, "Current behavior"].            */
/* ------------------------------------------------------------------------ */

/* Element e of a block -> (packed byte index, base-3 digit index). */
void oracle_tq1_element_slot(int e, int *byte_index, int *digit)
{
    if (e < 160) {                 /* chunks 0..4: digit c of qs[0..31] */
        *byte_index = e % 32;
        *digit = e / 32;
    } else if (e < 240) {          /* digit-major over qs[32..47] */
        *byte_index = 32 + (e - 160) % 16;
        *digit = (e - 160) / 16;
    } else {                       /* digit-major over qh[0..3] */
        *byte_index = 48 + (e - 240) % 4;
        *digit = (e - 240) / 4;
    }
}

/* Inverse: (packed byte index, digit) -> element; -1 if the slot is unused. */
int oracle_tq1_slot_element(int byte_index, int digit)
{
    if (byte_index < 32)
        return digit < 5 ? 32 * digit + byte_index : -1;
    if (byte_index < 48)
        return digit < 5 ? 160 + 16 * digit + (byte_index - 32) : -1;
    if (byte_index < 52)
        return digit < 4 ? 240 + 4 * digit + (byte_index - 48) : -1;
    return -1;
}

static int pow3(int c)
{
    int p = 1;
    while (c-- > 0)
        p *= 3;
    return p;
}

/* Digit c of a plain base-3 byte value v: floor(v / 3^c) mod 3. */
int oracle_base3_digit(int v, int c)
{
    return (v / pow3(c)) % 3;
}

/* Pack trits[N][K] (values -1, 0, +1) and fp16 scales d[N][K/256] into
 * TQ1_0 blocks, rows contiguous. Returns 0, or -1 on a bad trit or shape. */
int oracle_tq1_pack(const int8_t *trits, const uint16_t *d, uint8_t *w,
                    int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t B = 0; B < nb; B++) {
            uint8_t *blk = w + (n * nb + B) * TQ1_BLOCK_BYTES;
            int value[52];
            for (int p = 0; p < 52; p++)
                value[p] = 0;
            for (int e = 0; e < TQ1_BLOCK_ELEMS; e++) {
                int t = trits[n * K + B * TQ1_BLOCK_ELEMS + e];
                if (t < -1 || t > 1)
                    return -1;
                int p, c;
                oracle_tq1_element_slot(e, &p, &c);
                value[p] += (t + 1) * pow3(c);
            }
            for (int p = 0; p < 52; p++)
                blk[p] = (uint8_t)value[p];
            uint16_t h = d[n * nb + B];
            blk[52] = (uint8_t)(h & 0xff);
            blk[53] = (uint8_t)(h >> 8);
        }
    }
    return 0;
}

/* Decode the trits of one row (K elements) and its block scales.
 * Returns -1 if a packed byte is outside the base-3 range (qs > 242, qh > 80). */
static int unpack_row(const uint8_t *row, int64_t K, int8_t *trits,
                      uint16_t *d)
{
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t B = 0; B < nb; B++) {
        const uint8_t *blk = row + B * TQ1_BLOCK_BYTES;
        for (int p = 0; p < 48; p++)
            if (blk[p] > 242)
                return -1;
        for (int p = 48; p < 52; p++)
            if (blk[p] > 80)
                return -1;
        for (int e = 0; e < TQ1_BLOCK_ELEMS; e++) {
            int p, c;
            oracle_tq1_element_slot(e, &p, &c);
            trits[B * TQ1_BLOCK_ELEMS + e] =
                (int8_t)(oracle_base3_digit(blk[p], c) - 1);
        }
        if (d)
            d[B] = (uint16_t)(blk[52] | (blk[53] << 8));
    }
    return 0;
}

int oracle_tq1_unpack(const uint8_t *w, int8_t *trits, uint16_t *d,
                      int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; n++)
        if (unpack_row(w + n * nb * TQ1_BLOCK_BYTES, K, trits + n * K,
                       d + n * nb))
            return -1;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Q8_1 activation quantization (32-element blocks, bq8_1 in [P1]).         */
/* ------------------------------------------------------------------------ */

int oracle_q8_1_quantize(const float *x, uint8_t *a, int64_t T, int64_t K)
{
    if (T < 0 || K <= 0 || K % Q81_BLOCK_ELEMS)
        return -1;
    int64_t nblk = K / Q81_BLOCK_ELEMS;
    for (int64_t t = 0; t < T; t++) {
        for (int64_t j = 0; j < nblk; j++) {
            const float *xb = x + t * K + j * Q81_BLOCK_ELEMS;
            uint8_t *blk = a + (t * nblk + j) * Q81_BLOCK_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
                float ax = fabsf(xb[i]);
                if (ax > amax)
                    amax = ax;
            }
            float dq = amax / 127.0f;
            float id = (dq != 0.0f) ? 1.0f / dq : 0.0f;
            int sum = 0;
            for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
                float r = roundf(xb[i] * id); /* ties away from zero */
                int q = (int)r;
                if (q > 127)
                    q = 127;
                if (q < -127)
                    q = -127;
                blk[i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            uint16_t dh = oracle_f32_to_f16(dq);
            uint16_t sh = oracle_f32_to_f16(dq * (float)sum);
            blk[32] = (uint8_t)(dh & 0xff);
            blk[33] = (uint8_t)(dh >> 8);
            blk[34] = (uint8_t)(sh & 0xff);
            blk[35] = (uint8_t)(sh >> 8);
        }
    }
    return 0;
}

static int8_t q81_value(const uint8_t *a, int64_t nblk, int64_t t, int64_t k)
{
    const uint8_t *blk = a + (t * nblk + k / Q81_BLOCK_ELEMS) * Q81_BLOCK_BYTES;
    return (int8_t)blk[k % Q81_BLOCK_ELEMS];
}

static uint16_t q81_scale(const uint8_t *a, int64_t nblk, int64_t t, int64_t j)
{
    const uint8_t *blk = a + (t * nblk + j) * Q81_BLOCK_BYTES;
    return (uint16_t)(blk[32] | (blk[33] << 8));
}

/* ------------------------------------------------------------------------ */
/* Per-32-element integer sums, two independent ways.                       */
/* isums[t][n][j] = sum_{i<32} trit[n][32j+i] * q[t][32j+i]                  */
/* ------------------------------------------------------------------------ */

/* (i) element loop over decoded trits: the plain definition. */
int oracle_block_isums_elem(const uint8_t *w, const uint8_t *a,
                            int32_t *isums, int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        int8_t *tr = (int8_t *)malloc((size_t)K);
        if (!tr || unpack_row(w + n * nb * TQ1_BLOCK_BYTES, K, tr, NULL)) {
            bad = 1;
            free(tr);
            continue;
        }
        for (int64_t t = 0; t < T; t++)
            for (int64_t j = 0; j < nblk; j++) {
                int32_t s = 0;
                for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
                    int64_t k = j * Q81_BLOCK_ELEMS + i;
                    s += (int32_t)tr[k] * (int32_t)q81_value(a, nblk, t, k);
                }
                isums[(t * N + n) * nblk + j] = s;
            }
        free(tr);
    }
    return bad ? -1 : 0;
}

/* (ii) byte-major walk, after the CPU block walk of [P1]: each packed byte
 * is read once and all of its digits u are spent in place against the
 * matching activation; since trit = u - 1, the sum is sum(u*q) - sum(q). */
int oracle_block_isums_bytes(const uint8_t *w, const uint8_t *a,
                             int32_t *isums, int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t t = 0; t < T; t++) {
            for (int64_t B = 0; B < nb; B++) {
                const uint8_t *blk = w + (n * nb + B) * TQ1_BLOCK_BYTES;
                int32_t su[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                for (int p = 0; p < 52; p++) {
                    int v = blk[p];
                    int ndig = p < 48 ? 5 : 4;
                    if (v >= pow3(ndig))
                        bad = 1;
                    for (int c = 0; c < ndig; c++) {
                        int u = v % 3;
                        v /= 3;
                        int e = oracle_tq1_slot_element(p, c);
                        int64_t k = B * TQ1_BLOCK_ELEMS + e;
                        su[e / 32] += u * (int32_t)q81_value(a, nblk, t, k);
                    }
                }
                for (int b = 0; b < 8; b++) {
                    int64_t j = B * 8 + b;
                    int32_t sq = 0;
                    for (int i = 0; i < Q81_BLOCK_ELEMS; i++)
                        sq += q81_value(a, nblk, t, j * Q81_BLOCK_ELEMS + i);
                    isums[(t * N + n) * nblk + j] = su[b] - sq;
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Mat-vec: y[t][n] = sum_j fp32(d_w[n][j/8]) * fp32(d_a[t][j]) * isum[t][n][j]
 * Each term is formed in fp64, where it is exact (11 x 11 x 12 significant
 * bits); terms are summed in fp64 in index order. Also returns the sum of
 * |term| that scales the comparison tolerance.                             */
/* ------------------------------------------------------------------------ */

static void row_dot(const uint8_t *row, const int8_t *tr, const uint8_t *a,
                    int64_t nblk, int64_t t, int64_t K, double *y,
                    double *aabs)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t j = 0; j < K / Q81_BLOCK_ELEMS; j++) {
        int64_t B = j / 8;
        const uint8_t *blk = row + B * TQ1_BLOCK_BYTES;
        double dw = (double)oracle_f16_to_f32((uint16_t)(blk[52] | (blk[53] << 8)));
        double da = (double)oracle_f16_to_f32(q81_scale(a, nblk, t, j));
        int32_t s = 0;
        for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
            int64_t k = j * Q81_BLOCK_ELEMS + i;
            s += (int32_t)tr[k] * (int32_t)q81_value(a, nblk, t, k);
        }
        double term = dw * da * (double)s;
        acc += term;
        acc_abs += fabs(term);
    }
    *y = acc;
    *aabs = acc_abs;
}

int oracle_mmvq(const uint8_t *w, const uint8_t *a, float *y, double *y64,
                double *abs64, int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        const uint8_t *row = w + n * nb * TQ1_BLOCK_BYTES;
        int8_t *tr = (int8_t *)malloc((size_t)K);
        if (!tr || unpack_row(row, K, tr, NULL)) {
            bad = 1;
            free(tr);
            continue;
        }
        for (int64_t t = 0; t < T; t++) {
            double v, va;
            row_dot(row, tr, a, nblk, t, K, &v, &va);
            if (y)
                y[t * N + n] = (float)v;
            if (y64)
                y64[t * N + n] = v;
            if (abs64)
                abs64[t * N + n] = va;
        }
        free(tr);
    }
    return bad ? -1 : 0;
}

/* Mat-vec with a residual: y[t][n] = (the mat-vec's exact value) + r[t][n].
 * The linear-plus-add of "ops::linear q5: one Capacity=32 K-split rung
 * serves all T<=96" (its linear_add route): the product as above, then the
 * residual added once, in fp64, to the fp64 sum of the terms. abs64 is
 * sum |term| + |r|, the scale of the comparison tolerance. r is [T][N]. */
int oracle_mmvq_add(const uint8_t *w, const uint8_t *a, const float *r, float *y,
                    double *y64, double *abs64, int64_t N, int64_t K, int64_t T)
{
    if (!r || !y64 || !abs64)
        return -1;
    if (oracle_mmvq(w, a, NULL, y64, abs64, N, K, T))
        return -1;
    for (int64_t t = 0; t < T; t++)
        for (int64_t n = 0; n < N; n++) {
            double rv = (double)r[t * N + n];
            y64[t * N + n] = y64[t * N + n] + rv;
            abs64[t * N + n] = abs64[t * N + n] + fabs(rv);
            if (y)
                y[t * N + n] = (float)y64[t * N + n];
        }
    return 0;
}

/* The gate-up pair with a gated-linear-unit epilogue: two mat-vecs of the
 * same activation columns, g by the gate matrix and u by the up matrix (each
 * exactly as oracle_mmvq), then y[t][n] = silu(g) * u with silu(x) =
 * x / (1 + exp(-x)), all in fp64. The fused mat-vec paths of "CUDA: TQ1_0
 * mat-vec is load-bound by the per-32-element chunk contract" ("Proposed
 * approach": the fusion predicate is a third gate beside the plain and
 * expert paths) are named there but not spelled out; the reading used here
 * is the SiLU-gated unit of a transformer feed-forward block (gate and up
 * projections of the same input). g64, u64 and their sum |term| scales
 * absg, absu are returned for the comparison tolerance. Arrays are [T][N]. */
int oracle_mmvq_glu(const uint8_t *wg, const uint8_t *wu, const uint8_t *a, float *y,
                    double *y64, double *g64, double *u64, double *absg, double *absu,
                    int64_t N, int64_t K, int64_t T)
{
    if (!y64 || !g64 || !u64 || !absg || !absu)
        return -1;
    if (oracle_mmvq(wg, a, NULL, g64, absg, N, K, T) || oracle_mmvq(wu, a, NULL, u64, absu, N, K, T))
        return -1;
    for (int64_t i = 0; i < T * N; i++) {
        double g = g64[i];
        double silu = g / (1.0 + exp(-g));
        y64[i] = silu * u64[i];
        if (y)
            y[i] = (float)y64[i];
    }
    return 0;
}

/* The expert-routed products: pair ts = t * n_used + s multiplies expert
 * ids[ts]'s matrix by activation column col(ts), where col(ts) = t when a
 * token's slots share its column and col(ts) = ts when every pair has its own.
 * Returns -1 on a bad shape, an id outside [0, E) or a bad packed byte. */
static int mmvq_id_pairs(const uint8_t *w, const uint8_t *a, const int32_t *ids,
                         float *y, double *y64, double *abs64, int64_t E, int64_t N,
                         int64_t K, int64_t T, int64_t n_used, int column_per_pair)
{
    if (E <= 0 || N < 0 || T < 0 || n_used <= 0 || n_used > E || K <= 0 ||
        K % TQ1_BLOCK_ELEMS)
        return -1;
    for (int64_t i = 0; i < T * n_used; i++)
        if (ids[i] < 0 || ids[i] >= E)
            return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int64_t expert_bytes = N * nb * TQ1_BLOCK_BYTES;
    int64_t total = T * n_used * N;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t idx = 0; idx < total; idx++) {
        int64_t n = idx % N;
        int64_t ts = idx / N;     /* t * n_used + s */
        int64_t col = column_per_pair ? ts : ts / n_used;
        const uint8_t *row = w + (int64_t)ids[ts] * expert_bytes +
                             n * nb * TQ1_BLOCK_BYTES;
        int8_t *tr = (int8_t *)malloc((size_t)K);
        if (!tr || unpack_row(row, K, tr, NULL)) {
            bad = 1;
            free(tr);
            continue;
        }
        double v, va;
        row_dot(row, tr, a, nblk, col, K, &v, &va);
        if (y)
            y[idx] = (float)v;
        if (y64)
            y64[idx] = v;
        if (abs64)
            abs64[idx] = va;
        free(tr);
    }
    return bad ? -1 : 0;
}

/* Expert-routed mat-vec: y[t][s][n] = mmvq(W[ids[t][s]], a[t])[n], with one
 * activation per token shared by its n_used slots ([P1-acc], ne11 = 1). */
int oracle_mmvq_id(const uint8_t *w, const uint8_t *a, const int32_t *ids,
                   float *y, double *y64, double *abs64, int64_t E, int64_t N,
                   int64_t K, int64_t T, int64_t n_used)
{
    return mmvq_id_pairs(w, a, ids, y, y64, abs64, E, N, K, T, n_used, 0);
}

/* The same with one activation per (token, slot) pair, a [T][n_used][K/32]
 * (the down-projection shape, ne11 = n_used):
 * y[t][s][n] = mmvq(W[ids[t][s]], a[t][s])[n]. */
int oracle_mmvq_id_slots(const uint8_t *w, const uint8_t *a, const int32_t *ids,
                         float *y, double *y64, double *abs64, int64_t E, int64_t N,
                         int64_t K, int64_t T, int64_t n_used)
{
    return mmvq_id_pairs(w, a, ids, y, y64, abs64, E, N, K, T, n_used, 1);
}

/* ------------------------------------------------------------------------ */
/* Dequantization and row gather (the dequantize and get_rows operations    */
/* [P1] "Current behavior" and "Proposed approach" list beside the mat-vec). */
/* ------------------------------------------------------------------------ */

/* float -> bfloat16 bits, round to nearest, ties to even (finite inputs):
 * bfloat16 is the upper half of the binary32 pattern; the lower half decides
 * the rounding. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t upper = x >> 16, lower = x & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/* out row i = dequantized source row (rows ? rows[i] : i): element k is
 * v = fp32(d) * trit (an fp32 product, so a zero trit under a negative scale
 * gives -0), stored as out_dtype 0 = fp32, 1 = fp16 bits, 2 = bf16 bits.
 * Returns -1 on a bad shape, a row id outside [0, N) or a bad packed byte. */
int oracle_tq1_dequantize_rows(const uint8_t *w, const int32_t *rows, void *out,
                               int64_t N, int64_t K, int64_t n_rows, int out_dtype)
{
    if (N <= 0 || n_rows < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS || out_dtype < 0 ||
        out_dtype > 2)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t i = 0; i < n_rows; i++)
        if (rows && (rows[i] < 0 || rows[i] >= N))
            return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t r = rows ? rows[i] : i;
        int8_t *tr = (int8_t *)malloc((size_t)K);
        uint16_t *dd = (uint16_t *)malloc((size_t)nb * sizeof(uint16_t));
        if (!tr || !dd || unpack_row(w + r * nb * TQ1_BLOCK_BYTES, K, tr, dd)) {
            bad = 1;
            free(tr);
            free(dd);
            continue;
        }
        for (int64_t k = 0; k < K; k++) {
            float v = oracle_f16_to_f32(dd[k / TQ1_BLOCK_ELEMS]) * (float)tr[k];
            if (out_dtype == 0)
                ((float *)out)[i * K + k] = v;
            else if (out_dtype == 1)
                ((uint16_t *)out)[i * K + k] = oracle_f32_to_f16(v);
            else
                ((uint16_t *)out)[i * K + k] = oracle_f32_to_bf16(v);
        }
        free(tr);
        free(dd);
    }
    return bad ? -1 : 0;
}

/* Thread control for the timed CPU baseline (OpenMP over output rows). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}


/* ------------------------------------------------------------------------ */
/* TQ2_0 (reading stated in the header): 2-bit digit fields.                */
/* ------------------------------------------------------------------------ */

/* Element e of a TQ2_0 block -> (byte index, 2-bit field index). */
void oracle_tq2_element_slot(int e, int *byte_index, int *field)
{
    *byte_index = 32 * (e / 128) + e % 32;
    *field = (e % 128) / 32;
}

int oracle_tq2_pack(const int8_t *trits, const uint16_t *d, uint8_t *w,
                    int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t B = 0; B < nb; B++) {
            uint8_t *blk = w + (n * nb + B) * TQ2_BLOCK_BYTES;
            int value[64];
            for (int p = 0; p < 64; p++)
                value[p] = 0;
            for (int e = 0; e < TQ1_BLOCK_ELEMS; e++) {
                int t = trits[n * K + B * TQ1_BLOCK_ELEMS + e];
                if (t < -1 || t > 1)
                    return -1;
                int p, f;
                oracle_tq2_element_slot(e, &p, &f);
                value[p] += (t + 1) << (2 * f);
            }
            for (int p = 0; p < 64; p++)
                blk[p] = (uint8_t)value[p];
            uint16_t h = d[n * nb + B];
            blk[64] = (uint8_t)(h & 0xff);
            blk[65] = (uint8_t)(h >> 8);
        }
    }
    return 0;
}

/* Trits and scales of one TQ2_0 row; -1 if a field holds 3. */
static int unpack2_row(const uint8_t *row, int64_t K, int8_t *trits, uint16_t *d)
{
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t B = 0; B < nb; B++) {
        const uint8_t *blk = row + B * TQ2_BLOCK_BYTES;
        for (int e = 0; e < TQ1_BLOCK_ELEMS; e++) {
            int p, f;
            oracle_tq2_element_slot(e, &p, &f);
            int u = (blk[p] >> (2 * f)) & 3;
            if (u == 3)
                return -1;
            trits[B * TQ1_BLOCK_ELEMS + e] = (int8_t)(u - 1);
        }
        if (d)
            d[B] = (uint16_t)(blk[64] | (blk[65] << 8));
    }
    return 0;
}

int oracle_tq2_unpack(const uint8_t *w, int8_t *trits, uint16_t *d, int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; n++)
        if (unpack2_row(w + n * nb * TQ2_BLOCK_BYTES, K, trits + n * K, d + n * nb))
            return -1;
    return 0;
}

/* Per-32-element integer sums of TQ2_0 rows: (i) element loop over decoded
 * trits; (ii) byte-major walk, each byte's four fields spent in place,
 * sum(u q) - sum(q). */
int oracle_tq2_block_isums_elem(const uint8_t *w, const uint8_t *a, int32_t *isums,
                                int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        int8_t *tr = (int8_t *)malloc((size_t)K);
        if (!tr || unpack2_row(w + n * nb * TQ2_BLOCK_BYTES, K, tr, NULL)) {
            bad = 1;
            free(tr);
            continue;
        }
        for (int64_t t = 0; t < T; t++)
            for (int64_t j = 0; j < nblk; j++) {
                int32_t s = 0;
                for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
                    int64_t k = j * Q81_BLOCK_ELEMS + i;
                    s += (int32_t)tr[k] * (int32_t)q81_value(a, nblk, t, k);
                }
                isums[(t * N + n) * nblk + j] = s;
            }
        free(tr);
    }
    return bad ? -1 : 0;
}

int oracle_tq2_block_isums_bytes(const uint8_t *w, const uint8_t *a, int32_t *isums,
                                 int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t t = 0; t < T; t++) {
            for (int64_t B = 0; B < nb; B++) {
                const uint8_t *blk = w + (n * nb + B) * TQ2_BLOCK_BYTES;
                int32_t su[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                for (int p = 0; p < 64; p++) {
                    for (int f = 0; f < 4; f++) {
                        int u = (blk[p] >> (2 * f)) & 3;
                        if (u == 3)
                            bad = 1;
                        int e = 128 * (p / 32) + 32 * f + p % 32;
                        su[e / 32] += u * (int32_t)q81_value(a, nblk, t,
                                                             B * TQ1_BLOCK_ELEMS + e);
                    }
                }
                for (int b = 0; b < 8; b++) {
                    int64_t j = B * 8 + b;
                    int32_t sumq = 0;
                    for (int i = 0; i < Q81_BLOCK_ELEMS; i++)
                        sumq += q81_value(a, nblk, t, j * Q81_BLOCK_ELEMS + i);
                    isums[(t * N + n) * nblk + j] = su[b] - sumq;
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* TQ2_0 mat-vec: the same definition as oracle_mmvq, every term
 * fp32(d_w) * fp32(d_a) * isum formed in fp64 (exact) and summed in index
 * order in fp64; also the sum of |term|. */
int oracle_tq2_mmvq(const uint8_t *w, const uint8_t *a, float *y, double *y64,
                    double *abs64, int64_t N, int64_t K, int64_t T)
{
    if (N < 0 || T < 0 || K <= 0 || K % TQ1_BLOCK_ELEMS)
        return -1;
    int64_t nb = K / TQ1_BLOCK_ELEMS, nblk = K / Q81_BLOCK_ELEMS;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        int8_t *tr = (int8_t *)malloc((size_t)K);
        uint16_t *dd = (uint16_t *)malloc((size_t)nb * sizeof(uint16_t));
        if (!tr || !dd || unpack2_row(w + n * nb * TQ2_BLOCK_BYTES, K, tr, dd)) {
            bad = 1;
            free(tr);
            free(dd);
            continue;
        }
        for (int64_t t = 0; t < T; t++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t j = 0; j < nblk; j++) {
                double dw = (double)oracle_f16_to_f32(dd[j / 8]);
                double da = (double)oracle_f16_to_f32(q81_scale(a, nblk, t, j));
                int32_t s = 0;
                for (int i = 0; i < Q81_BLOCK_ELEMS; i++) {
                    int64_t k = j * Q81_BLOCK_ELEMS + i;
                    s += (int32_t)tr[k] * (int32_t)q81_value(a, nblk, t, k);
                }
                double term = dw * da * (double)s;
                acc += term;
                acc_abs += fabs(term);
            }
            if (y)
                y[t * N + n] = (float)acc;
            if (y64)
                y64[t * N + n] = acc;
            if (abs64)
                abs64[t * N + n] = acc_abs;
        }
        free(tr);
        free(dd);
    }
    return bad ? -1 : 0;
}
