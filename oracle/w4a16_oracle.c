/*
 * w4a16_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, obviously correct CPU reference for the group-wise INT4
 * weight-only GEMM (W4A16).  Only the tests, the smoke check and the bench's CPU
 * baseline leg load it; the product path never does.  It shares no source, header,
 * table or helper with the HIP library.
 *
 * What it computes (the pages' operation, made precise):
 *   "The Free Half of Speculative Decoding", third paragraph: the target model's
 *   weights are quantized to INT4 with AWQ; activations stay in 16-bit.
 *   "When Do Quantized Drafts Help Speculative Decoding?", sections "Current pilot
 *   setup" and "What is included": GPTQ INT4 drafts run through a W4A16 kernel; the
 *   verify pass runs the target over gamma+1 = 5 positions at batch 1.
 * The pages name the format (AWQ/GPTQ INT4, weight-only) but print neither the
 * dequantization rule nor the layout.  The plainest asymmetric group-wise reading is
 * used, with groups of 128 along K:
 *
 *   W[k,n] = (q[k,n] - z[g,n]) * s[g,n],      g = floor(k / 128)
 *   C[m,n] = sum_{k=0}^{K-1} A[m,k] * W[k,n]
 *
 *   A   bfloat16 [M,K] row-major
 *   Wq  uint32 [K/8,N] row-major; nibble j (bits 4j..4j+3) of Wq[kb,n] is q[8kb+j, n]
 *   s   IEEE binary16 [K/128,N]
 *   z   one byte per entry [K/128,N]; only the low nibble is used
 *
 * Precision: every term A*(q-z)*s is exact in binary64 (8 + 5 + 11 significant bits),
 * so the only rounding is the binary64 accumulation in plain k order.  The oracle
 * also returns sum_k |A[m,k]*W[k,n]| so a caller can state a per-element error bound.
 *
 * Build: plain C11, no -ffast-math, -ffp-contract=off; OpenMP over output columns
 * (each thread owns whole columns, so results do not depend on the thread count).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 128

/* bfloat16: sign bit 15, exponent bits 14..7 (bias 127), fraction bits 6..0. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0xFF) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -126 - 7); /* subnormal: 0.f * 2^-126 */
    } else {
        v = ldexp((double)(128 + f), e - 127 - 7); /* 1.f * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* IEEE binary16: sign bit 15, exponent bits 14..10 (bias 15), fraction bits 9..0. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: 0.f * 2^-14 */
    } else {
        v = ldexp((double)(1024 + f), e - 15 - 10);
    }
    return sign ? -v : v;
}

void oracle_decode_bf16_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}

void oracle_decode_f16_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}

/* The 4-bit code for row k, column n, read out of the packed words. */
static inline int oracle_code(const uint32_t *Wq, int64_t N, int64_t k, int64_t n)
{
    uint32_t w = Wq[(k / 8) * N + n];
    return (int)((w >> (4 * (k % 8))) & 0xFu);
}

/*
 * C[m, c] (and Cabs) for the output columns cols[0..ncols-1]; cols == NULL means all
 * N columns in order.  C and Cabs are [M, ncols] row-major binary64.
 * Returns 0, or -1 for a shape the format does not define.
 */
int oracle_w4a16_gemm(const uint16_t *A, const uint32_t *Wq, const uint16_t *S,
                      const uint8_t *Z, int64_t M, int64_t K, int64_t N,
                      const int64_t *cols, int64_t ncols, double *C, double *Cabs,
                      int nthreads)
{
    if (M < 1 || N < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP != 0) return -1;
    if (!cols) ncols = N;
    if (ncols < 1) return -1;
    for (int64_t c = 0; cols && c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;

    /* Activations decoded once, stored k-major so the M values of one k are adjacent. */
    double *Ak = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!Ak) return -2;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) Ak[k * M + m] = oracle_bf16_to_f64(A[m * K + k]);

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)M * 2);
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
        double *abs_acc = acc ? acc + M : NULL;
#pragma omp for schedule(static)
        for (int64_t c = 0; c < ncols; ++c) {
            if (!acc) continue;
            int64_t n = cols ? cols[c] : c;
            for (int64_t m = 0; m < M; ++m) { acc[m] = 0.0; abs_acc[m] = 0.0; }
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = k / ORACLE_GROUP;
                int zero = Z[g * N + n] & 0xF;
                double scale = oracle_f16_to_f64(S[g * N + n]);
                int d = oracle_code(Wq, N, k, n) - zero;
                double w = (double)d * scale;          /* exact: 5 x 11 bits */
                const double *a = Ak + k * M;
                for (int64_t m = 0; m < M; ++m) {
                    double t = a[m] * w;               /* exact: 8 x 16 bits */
                    acc[m] += t;
                    abs_acc[m] += fabs(t);
                }
            }
            for (int64_t m = 0; m < M; ++m) {
                C[m * ncols + c] = acc[m];
                if (Cabs) Cabs[m * ncols + c] = abs_acc[m];
            }
        }
        free(acc);
    }
    free(Ak);
    return failed ? -2 : 0;
}

/* Packing rule of the storage format: Wq[kb,n] = sum_j (q[8kb+j,n] & 0xF) << 4j. */
int oracle_w4_pack(const uint8_t *q, uint32_t *Wq, int64_t K, int64_t N)
{
    if (K < 8 || K % 8 != 0 || N < 1) return -1;
    for (int64_t kb = 0; kb < K / 8; ++kb)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t w = 0;
            for (int j = 0; j < 8; ++j)
                w |= (uint32_t)(q[(8 * kb + j) * N + n] & 0xF) << (4 * j);
            Wq[kb * N + n] = w;
        }
    return 0;
}

/* Inverse of the packing rule: q[k,n] = nibble (k mod 8) of Wq[k/8, n]. */
int oracle_w4_unpack(const uint32_t *Wq, uint8_t *q, int64_t K, int64_t N)
{
    if (K < 8 || K % 8 != 0 || N < 1) return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) q[k * N + n] = (uint8_t)oracle_code(Wq, N, k, n);
    return 0;
}
