/*
 * CPU oracle for the streamed AllGather + GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library.  It shares no code, header or
 * constant with the HIP library; the two never call one another.
 *
 * What it computes is the plain definition of the operation, not a
 * simulation of the pipeline:
 *
 *   A = the row blocks A_0 .. A_{n-1} stacked in shard (rank) order
 *       (PTO-ISA AllGather+GEMM README, "compute function": rank r owns
 *       rows [r*M/n, (r+1)*M/n); Triton-distributed AllGather GEMM
 *       tutorial, reference function: all_gather, concatenate on dim 0,
 *       then matmul)
 *   fp16 path:  C[i,j] = fp32_RNE( sum_k A[i,k] * B[k,j] )     (exact-ish)
 *       PTO-ISA README "spec" table: A M x K fp16, B K x N fp16, C M x N
 *       fp32.  The sum is carried in double.  Each product of two fp16
 *       values is exact in double (11 + 11 significand bits), so the only
 *       rounding inside the sum is that of the double additions, taken in
 *       k order; the result is then rounded once to fp32.
 *       The kernel is free to sum in any order, so the comparison uses an
 *       error bound; S[i,j] = sum_k |A[i,k] * B[k,j]| is emitted for it.
 *   bf16 path:  the same with bfloat16 A and B (a variant of the fp16
 *       path: same gather, same fp32 output, a different input format).
 *   fp8 path:   the same with OCP FP8 E4M3 A and B (the float8_e4m3fn
 *       inputs of the Ascend grouped-GEMM page's FP8 variant); a product
 *       of two such values (4 significant bits each) is exact in double.
 *   int8 path (catccos AllGatherMatmulDequant doc, section 2.2):
 *       v[i,j] = sum_k A[i,k] * B[k,j] + bias[j]     (exact, int64, must
 *                                                     fit in int32)
 *       D[i,j] = fp16_RNE( fp32(v[i,j]) * scale[j] )  with the int32 ->
 *       fp32 conversion and the fp32 product each rounded to nearest even;
 *       a single per-output-channel scale, no per-token scale.
 *
 * Loops are i-k-j over a row at a time, each output row computed by one
 * thread (OpenMP over rows), so an element's summation order is fixed and
 * the result does not depend on the thread count.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16, written from the format's definition:            */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.            */
/* ------------------------------------------------------------------ */

double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1.f) * 2^(e-15)     */
    }
    return sign ? -v : v;
}

/* fp32 -> fp16, round to nearest, ties to even; overflow gives +-inf. */
uint16_t oracle_float_to_half(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    int ef = (int)((u >> 23) & 0xff);
    uint32_t frac = u & 0x7fffffu;

    if (ef == 0xff)                                 /* inf or NaN */
        return (uint16_t)(sign | 0x7c00u | (frac ? 0x200u : 0u));

    /* value = sig * 2^(exp2), sig an integer */
    uint32_t sig;
    int exp2;
    if (ef == 0) { sig = frac; exp2 = -149; }
    else         { sig = frac | 0x800000u; exp2 = ef - 150; }
    if (sig == 0)
        return sign;

    /* Target: half value = q * 2^(eh - 25) for normals (q in [1024,2048)),
     * q * 2^-24 for subnormals.  Find the unbiased exponent of x. */
    int msb = 31 - __builtin_clz(sig);             /* sig in [2^msb, 2^(msb+1)) */
    int e_unb = exp2 + msb;                        /* x in [2^e_unb, 2^(e_unb+1)) */
    int q_exp = (e_unb >= -14) ? e_unb - 10 : -24; /* weight of the half ulp */
    int shift = q_exp - exp2;                      /* bits to drop from sig */
    uint64_t q;
    if (shift <= 0) {
        q = (uint64_t)sig << (-shift);
    } else if (shift > 40) {
        q = 0;                                     /* far below half the ulp */
    } else {
        uint64_t s64 = sig;
        q = s64 >> shift;
        uint64_t rem = s64 & ((1ull << shift) - 1);
        uint64_t halfway = 1ull << (shift - 1);
        if (rem > halfway || (rem == halfway && (q & 1)))
            q++;
    }
    if (e_unb >= -14) {
        /* normal: q in [1024, 2048]; 2048 carries into the exponent */
        int eh = e_unb + 15;
        uint32_t bits = ((uint32_t)eh << 10) + (uint32_t)(q - 1024);
        if (bits >= 0x7c00u)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | bits);
    }
    /* subnormal: q in [0, 1024]; 1024 is the smallest normal */
    return (uint16_t)(sign | (uint32_t)q);
}

/* Pointer to row i of the gathered A: shard i / S, local row i % S. */
static const void *gathered_row(const void *const *shards, int64_t S,
                                int64_t K, int64_t i, size_t elt)
{
    int64_t s = i / S;
    int64_t r = i % S;
    return (const char *)shards[s] + (size_t)(r * K) * elt;
}

static int check_shape(const void *const *shards, int n_shards, int64_t M,
                       int64_t K, int64_t N)
{
    if (!shards || n_shards < 1 || M < 0 || K < 0 || N < 0)
        return 1;
    if (M % n_shards)
        return 1;
    for (int s = 0; s < n_shards; s++)
        if (!shards[s] && M > 0 && K > 0)
            return 1;
    return 0;
}

/* ------------------------------------------------------------------ */
/* bfloat16, written from the format's definition: 1 sign bit, 8       */
/* exponent bits (bias 127), 7 fraction bits (the upper half of an     */
/* IEEE binary32).                                                      */
/* ------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);     /* (1.f) * 2^(e-127)     */
    }
    return sign ? -v : v;
}

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"), written from the format's definition: 1    */
/* sign bit, 4 exponent bits (bias 7), 3 fraction bits; no infinities; */
/* exponent 15 with fraction 7 is NaN, so the largest value is 448.    */
/* ------------------------------------------------------------------ */

double oracle_fp8e4m3_to_double(uint8_t h)
{
    int sign = (h >> 7) & 1;
    int e = (h >> 3) & 0xf;
    int f = h & 0x7;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -9);                  /* subnormal: f * 2^-9 */
    } else if (e == 15 && f == 7) {
        v = NAN;
    } else {
        v = ldexp((double)(8 + f), e - 10);        /* (1.f) * 2^(e-7)     */
    }
    return sign ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Float formats x the same format -> fp32 (fp16, bf16 and fp8 paths)   */
/* ------------------------------------------------------------------ */

/* element i of an array of the input format, as a double */
typedef double (*decode_fn)(const void *p, int64_t i);

static double dec_f16(const void *p, int64_t i)
{
    return oracle_half_to_double(((const uint16_t *)p)[i]);
}

static double dec_bf16(const void *p, int64_t i)
{
    return oracle_bf16_to_double(((const uint16_t *)p)[i]);
}

static double dec_fp8(const void *p, int64_t i)
{
    return oracle_fp8e4m3_to_double(((const uint8_t *)p)[i]);
}

/*
 * Rows `rows[0..n_rows)` of C = gather(shards) x B, the elements of both
 * (`elt` bytes each) decoded by `dec`.  C_rows: n_rows x N fp32; abs_rows
 * (may be NULL): n_rows x N double, the sum over k of |A[i,k] B[k,j]|.  A
 * product of two fp16 values (11 significant bits each), two bf16 values
 * (8 each) or two fp8 values (4 each) is exact in double.
 */
static int ag_gemm_float_rows(decode_fn dec, size_t elt, const void *const *shards,
                              int n_shards, const void *B, int64_t M,
                              int64_t K, int64_t N, const int64_t *rows,
                              int64_t n_rows, float *C_rows, double *abs_rows)
{
    if (check_shape(shards, n_shards, M, K, N))
        return 1;
    int64_t S = M / n_shards;
    for (int64_t t = 0; t < n_rows; t++)
        if (rows[t] < 0 || rows[t] >= M)
            return 1;

    double *Bd = (double *)malloc(sizeof(double) * (size_t)(K * N + 1));
    if (!Bd)
        return 2;
    for (int64_t x = 0; x < K * N; x++)
        Bd[x] = dec(B, x);

    int fail = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)(N + 1));
        double *mag = (double *)malloc(sizeof(double) * (size_t)(N + 1));
        if (!acc || !mag) {
#pragma omp atomic write
            fail = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_rows; t++) {
            if (!acc || !mag)
                continue;
            const void *a = gathered_row(shards, S, K, rows[t], elt);
            for (int64_t j = 0; j < N; j++) { acc[j] = 0.0; mag[j] = 0.0; }
            for (int64_t k = 0; k < K; k++) {
                double aik = dec(a, k);
                const double *b = Bd + k * N;
                for (int64_t j = 0; j < N; j++) {
                    double p = aik * b[j];          /* exact */
                    acc[j] += p;
                    mag[j] += fabs(p);
                }
            }
            for (int64_t j = 0; j < N; j++) {
                C_rows[t * N + j] = (float)acc[j];   /* one RNE rounding */
                if (abs_rows)
                    abs_rows[t * N + j] = mag[j];
            }
        }
        free(acc);
        free(mag);
    }
    free(Bd);
    return fail;
}

/* fp16 x fp16 -> fp32 (PTO-ISA README "spec" table). */
int oracle_ag_gemm_f16_rows(const uint16_t *const *shards, int n_shards,
                            const uint16_t *B, int64_t M, int64_t K, int64_t N,
                            const int64_t *rows, int64_t n_rows,
                            float *C_rows, double *abs_rows)
{
    return ag_gemm_float_rows(dec_f16, 2, (const void *const *)shards, n_shards, B,
                              M, K, N, rows, n_rows, C_rows, abs_rows);
}

/* bf16 x bf16 -> fp32: the same definition with bfloat16 inputs. */
int oracle_ag_gemm_bf16_rows(const uint16_t *const *shards, int n_shards,
                             const uint16_t *B, int64_t M, int64_t K, int64_t N,
                             const int64_t *rows, int64_t n_rows,
                             float *C_rows, double *abs_rows)
{
    return ag_gemm_float_rows(dec_bf16, 2, (const void *const *)shards, n_shards, B,
                              M, K, N, rows, n_rows, C_rows, abs_rows);
}

/* fp8 (E4M3) x fp8 -> fp32: the same definition with fp8 inputs. */
int oracle_ag_gemm_fp8_rows(const uint8_t *const *shards, int n_shards,
                            const uint8_t *B, int64_t M, int64_t K, int64_t N,
                            const int64_t *rows, int64_t n_rows,
                            float *C_rows, double *abs_rows)
{
    return ag_gemm_float_rows(dec_fp8, 1, (const void *const *)shards, n_shards, B,
                              M, K, N, rows, n_rows, C_rows, abs_rows);
}

/* Whole C (M x N fp32) and optionally the whole |.| sum (M x N double). */
int oracle_ag_gemm_f16(const uint16_t *const *shards, int n_shards,
                       const uint16_t *B, int64_t M, int64_t K, int64_t N,
                       float *C, double *abs_sum)
{
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 1));
    if (!rows)
        return 2;
    for (int64_t i = 0; i < M; i++)
        rows[i] = i;
    int rc = oracle_ag_gemm_f16_rows(shards, n_shards, B, M, K, N, rows, M,
                                     C, abs_sum);
    free(rows);
    return rc;
}

/* ------------------------------------------------------------------ */
/* int8 x int8 -> int32, + bias, x per-channel scale -> fp16            */
/* ------------------------------------------------------------------ */

/* fp32(v) * s, both steps rounded to nearest even in binary32. */
static uint16_t dequant_one(int32_t v, float s)
{
    volatile float f = (float)v;     /* int32 -> fp32, RNE */
    volatile float p = f * s;        /* fp32 multiply, RNE */
    return oracle_float_to_half(p);  /* fp32 -> fp16, RNE */
}

/*
 * Rows of the int8 path.  acc_rows (may be NULL): n_rows x N int32,
 * sum_k A*B + bias.  D_rows: n_rows x N fp16 bit patterns.
 * Returns 3 if some accumulator leaves the int32 range.
 */
int oracle_ag_gemm_i8_rows(const int8_t *const *shards, int n_shards,
                           const int8_t *B, const int32_t *bias,
                           const float *scale, int64_t M, int64_t K, int64_t N,
                           const int64_t *rows, int64_t n_rows,
                           int32_t *acc_rows, uint16_t *D_rows)
{
    if (check_shape((const void *const *)shards, n_shards, M, K, N))
        return 1;
    int64_t S = M / n_shards;
    for (int64_t t = 0; t < n_rows; t++)
        if (rows[t] < 0 || rows[t] >= M)
            return 1;

    int fail = 0;
#pragma omp parallel
    {
        int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
        if (!acc) {
#pragma omp atomic write
            fail = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_rows; t++) {
            if (!acc)
                continue;
            const int8_t *a = (const int8_t *)gathered_row(
                (const void *const *)shards, S, K, rows[t], 1);
            for (int64_t j = 0; j < N; j++)
                acc[j] = 0;
            for (int64_t k = 0; k < K; k++) {
                int64_t aik = a[k];
                const int8_t *b = B + k * N;
                for (int64_t j = 0; j < N; j++)
                    acc[j] += aik * (int64_t)b[j];
            }
            for (int64_t j = 0; j < N; j++) {
                int64_t v = acc[j] + (int64_t)bias[j];
                if (v > INT32_MAX || v < INT32_MIN) {
#pragma omp atomic write
                    fail = 3;
                    v = 0;
                }
                if (acc_rows)
                    acc_rows[t * N + j] = (int32_t)v;
                D_rows[t * N + j] = dequant_one((int32_t)v, scale[j]);
            }
        }
        free(acc);
    }
    return fail;
}

int oracle_ag_gemm_i8(const int8_t *const *shards, int n_shards,
                      const int8_t *B, const int32_t *bias, const float *scale,
                      int64_t M, int64_t K, int64_t N, int32_t *acc,
                      uint16_t *D)
{
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 1));
    if (!rows)
        return 2;
    for (int64_t i = 0; i < M; i++)
        rows[i] = i;
    int rc = oracle_ag_gemm_i8_rows(shards, n_shards, B, bias, scale, M, K, N,
                                    rows, M, acc, D);
    free(rows);
    return rc;
}

/* Array forms of the fp16 codecs, for exhaustive checks from Python. */
void oracle_half_to_double_n(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_half_to_double(h[i]);
}

void oracle_bf16_to_double_n(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_to_double(h[i]);
}

void oracle_fp8e4m3_to_double_n(const uint8_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_fp8e4m3_to_double(h[i]);
}

void oracle_float_to_half_n(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_float_to_half(x[i]);
}

void oracle_dequant_n(const int32_t *v, const float *s, uint16_t *out,
                      int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = dequant_one(v[i], s[i]);
}

/* Threads the parallel loops above use from now on (how the oracle's CPU
 * time is measured on one core or on all of them); returns the previous
 * count.  No effect on any result: every output element is summed by one
 * thread in a fixed order. */
int oracle_set_threads(int n)
{
    int old = omp_get_max_threads();
    if (n > 0) omp_set_num_threads(n);
    return old;
}
