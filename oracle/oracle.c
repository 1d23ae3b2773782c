/*
 * Plain CPU oracle for the low-precision dense GEMM C = A.B.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or helper with the GPU path and must never be called
 * from it.
 *
 * What is computed (the pages define the operation only as "a GEMM" in FP16,
 * INT8 and INT4 -- the PTX-vs-WMMA summary page, the paragraphs on the three
 * precisions and on the s4 mma shape; the FP16 error procedure -- inputs from
 * N(0,1) rounded to fp16, compared against an fp64 accumulation over the same
 * rounded operands -- comes from the forum post on compiler-generated kernels,
 * paragraph on hybrid FP16/FP32 accumulation):
 *
 *   integer paths : C[i][j] = sum_k A[i][k] * B[k][j], summed exactly in
 *                   int64, then required to fit int32.
 *   int4          : same sum over signed 4-bit values, two per byte along k,
 *                   the low nibble holding the even k, two's complement.
 *   fp16          : ref[i][j] = sum_k a*b in fp64 over the exactly decoded
 *                   binary16 operands, and den[i][j] = sum_k |a|*|b| (the
 *                   normaliser of the relative-error metric).
 *   dequant       : s from the int8 path, then in binary32, left to right:
 *                   t = (float)s; t = t * rs[i]; t = t * cs[j].
 *   quantise      : per-row symmetric int8 quantisation of fp16 activations,
 *                   the step in front of a W8A8 projection (the pages leave
 *                   the rule open; this is the plainest reading): absmax =
 *                   max |x|, scale = absmax / 127 in binary32, q = the
 *                   nearest-even integer to x / scale computed in binary32,
 *                   clamped to [-127, 127]; an all-zero row gets scale 0 and
 *                   q = 0.
 *   fp64 emulation: the fp64 product through integer GEMMs (the day-12 page
 *                   of the FP64-emulation series: scale/exponent scan, then
 *                   integer products, then undo the scaling).  The pages
 *                   leave the scaling rule open; the plainest reading, with t
 *                   the target bits: each row of A (each column of B) is
 *                   multiplied by 2^(t - e), e the binary exponent of its
 *                   largest magnitude (max = f 2^e, 0.5 <= f < 1), and
 *                   rounded to the nearest integer (ties to even), so
 *                   |a'| <= 2^t.  X = A'.B' is summed exactly (128-bit
 *                   integers), converted to double with one rounding, and
 *                   scaled by 2^-(2t - eA[i] - eB[j]).  How the GPU obtains
 *                   X (residues modulo several moduli and the Chinese
 *                   remainder theorem) does not change the value, so this
 *                   oracle takes the direct product.
 *
 * Layouts: A is M x K row-major; B is stored K-contiguous (N rows of K);
 * C is M x N row-major.  Every entry point computes the output rows
 * [row_begin, row_end) and writes them to the first (row_end-row_begin)*N
 * elements of its output, so a caller can check sampled rows of a large
 * product without computing all of it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -std=c11 (no -ffast-math).
 * Rows are spread over OpenMP threads; each dot product runs sequentially
 * in increasing k.
 *
 * Return value: 0 on success; 1 if an integer result does not fit int32
 * (the input is outside the library's contract); 2 if an fp16 or fp64
 * operand is inf or NaN (outside the contract); 3 for a bad row range or a
 * target bit count outside [1, 53]; 4 if a working buffer cannot be
 * allocated.
 */
#include <stdint.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_INT32_RANGE 1
#define ORACLE_NONFINITE 2
#define ORACLE_BAD_RANGE 3
#define ORACLE_NO_MEMORY 4

static int bad_range(int64_t M, int64_t row_begin, int64_t row_end)
{
    return row_begin < 0 || row_end > M || row_begin > row_end;
}

/* int8 x int8 -> int32, exact. */
int oracle_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,
              int32_t *C, int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end))
        return ORACLE_BAD_RANGE;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];
            if (s < INT32_MIN || s > INT32_MAX) {
#pragma omp atomic write
                status = ORACLE_INT32_RANGE;
            }
            C[(i - row_begin) * N + j] = (int32_t)s;
        }
    }
    return status;
}

/* Value of the k-th signed 4-bit element of a packed row: byte k/2 holds
 * element k in its low nibble when k is even and in its high nibble when k
 * is odd; the nibble is two's complement, so 8..15 stand for -8..-1. */
static int64_t nibble_value(const uint8_t *row, int64_t k)
{
    uint8_t byte = row[k / 2];
    int64_t d = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return d >= 8 ? d - 16 : d;
}

/* packed int4 x packed int4 -> int32, exact.  A_packed is M x K/2 bytes,
 * B_packed is N x K/2 bytes; K must be even. */
int oracle_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A_packed,
              const uint8_t *B_packed, int32_t *C, int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end) || K % 2 != 0)
        return ORACLE_BAD_RANGE;
    const int64_t row_bytes = K / 2;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        const uint8_t *a = A_packed + i * row_bytes;
        for (int64_t j = 0; j < N; ++j) {
            const uint8_t *b = B_packed + j * row_bytes;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += nibble_value(a, k) * nibble_value(b, k);
            if (s < INT32_MIN || s > INT32_MAX) {
#pragma omp atomic write
                status = ORACLE_INT32_RANGE;
            }
            C[(i - row_begin) * N + j] = (int32_t)s;
        }
    }
    return status;
}

/* Exact value of an IEEE 754 binary16 bit pattern, as a double.
 * Layout: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 is zero or subnormal: f * 2^-24.  Otherwise (1024 + f) *
 * 2^(e - 25).  Exponent 31 is inf/NaN: *finite is set to 0. */
double oracle_f16_decode(uint16_t bits, int *finite)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1F;
    int f = bits & 0x3FF;
    double mag;
    if (e == 31) {
        *finite = 0;
        return 0.0;
    }
    *finite = 1;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* fp16 x fp16 summed in fp64: ref = sum a*b, den = sum |a|*|b|.
 * Each product of two binary16 values has at most 22 significant bits, so it
 * is exact in fp64; only the additions round. */
int oracle_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
               double *ref, double *den, int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end))
        return ORACLE_BAD_RANGE;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, d = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int fa, fb;
                double a = oracle_f16_decode(A[i * K + k], &fa);
                double b = oracle_f16_decode(B[j * K + k], &fb);
                if (!fa || !fb) {
#pragma omp atomic write
                    status = ORACLE_NONFINITE;
                }
                s += a * b;
                d += fabs(a) * fabs(b);
            }
            ref[(i - row_begin) * N + j] = s;
            den[(i - row_begin) * N + j] = d;
        }
    }
    return status;
}

/* int8 GEMM followed by the per-row x per-column fp32 dequantisation
 * "acc * row_scale * col_scale", read left to right, each step rounded to
 * binary32 (round to nearest even). */
int oracle_i8_dequant(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,
                      const float *row_scale, const float *col_scale, float *out,
                      int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end))
        return ORACLE_BAD_RANGE;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];
            if (s < INT32_MIN || s > INT32_MAX) {
#pragma omp atomic write
                status = ORACLE_INT32_RANGE;
            }
            volatile float t = (float)(int32_t)s;
            t = t * row_scale[i];
            t = t * col_scale[j];
            out[(i - row_begin) * N + j] = t;
        }
    }
    return status;
}

/* Per-row int8 quantisation of fp16 rows (see the header comment).
 * X: M x K binary16 bits; Q: (row_end-row_begin) x K int8; scale: one float
 * per computed row.  Division and rounding are binary32, round to nearest
 * even (SSE arithmetic, FLT_EVAL_METHOD == 0). */
int oracle_quantize_rows_f16(int64_t M, int64_t K, const uint16_t *X, int8_t *Q, float *scale,
                             int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end))
        return ORACLE_BAD_RANGE;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        double amax = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            int fin;
            double v = oracle_f16_decode(X[i * K + k], &fin);
            if (!fin) {
#pragma omp atomic write
                status = ORACLE_NONFINITE;
            }
            if (fabs(v) > amax)
                amax = fabs(v);
        }
        /* amax is a binary16 value, so the conversion is exact */
        volatile float s = (float)amax / 127.0f;
        scale[i - row_begin] = s;
        for (int64_t k = 0; k < K; ++k) {
            int fin;
            float v = (float)oracle_f16_decode(X[i * K + k], &fin);
            int8_t q = 0;
            if (s != 0.0f) {
                volatile float t = v / s;
                float r = rintf(t);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                q = (int8_t)r;
            }
            Q[(i - row_begin) * K + k] = q;
        }
    }
    return status;
}

/* Binary exponent of the largest magnitude of n doubles (frexp convention:
 * max = f 2^e with 0.5 <= f < 1); 0 for an all-zero row.  Sets *nonfinite
 * if a value is inf or NaN. */
static int row_exponent(const double *x, int64_t n, int *nonfinite)
{
    double amax = 0.0;
    for (int64_t k = 0; k < n; ++k) {
        if (!isfinite(x[k]))
            *nonfinite = 1;
        if (fabs(x[k]) > amax)
            amax = fabs(x[k]);
    }
    int e = 0;
    if (amax > 0.0)
        frexp(amax, &e);
    return e;
}

/* fp64 GEMM through scaled integers (see the header comment).  A: M x K
 * doubles, B_t: N x K doubles (B stored K-contiguous), C: (row_end-row_begin)
 * x N doubles; bits = t in [1, 53]. */
int oracle_f64_emu(int64_t M, int64_t N, int64_t K, const double *A, const double *B_t, int bits,
                   double *C, int64_t row_begin, int64_t row_end)
{
    if (bad_range(M, row_begin, row_end) || bits < 1 || bits > 53)
        return ORACLE_BAD_RANGE;
    int nonfinite = 0;
    /* scaled integers of B (every column is needed by every output row) */
    int64_t *Bi = (int64_t *)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(int64_t));
    int *eB = (int *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int));
    if (!Bi || !eB) {
        free(Bi);
        free(eB);
        return ORACLE_NO_MEMORY;
    }
    int no_memory = 0;
    for (int64_t j = 0; j < N; ++j) {
        eB[j] = row_exponent(B_t + j * K, K, &nonfinite);
        for (int64_t k = 0; k < K; ++k)
            Bi[j * K + k] = (int64_t)rint(ldexp(B_t[j * K + k], bits - eB[j]));
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = row_begin; i < row_end; ++i) {
        int nf = 0;
        const int eA = row_exponent(A + i * K, K, &nf);
        if (nf) {
#pragma omp atomic write
            nonfinite = 1;
        }
        int64_t *Ai = (int64_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof(int64_t));
        if (!Ai) {
#pragma omp atomic write
            no_memory = 1;
            continue;
        }
        for (int64_t k = 0; k < K; ++k)
            Ai[k] = (int64_t)rint(ldexp(A[i * K + k], bits - eA));
        for (int64_t j = 0; j < N; ++j) {
            __int128 x = 0;
            for (int64_t k = 0; k < K; ++k)
                x += (__int128)Ai[k] * (__int128)Bi[j * K + k];
            /* one rounding to double, then an exact power-of-two scaling */
            C[(i - row_begin) * N + j] = ldexp((double)x, -(2 * bits - eA - eB[j]));
        }
        free(Ai);
    }
    free(Bi);
    free(eB);
    if (no_memory)
        return ORACLE_NO_MEMORY;
    return nonfinite ? ORACLE_NONFINITE : ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
