/*
 * w4a16_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, obviously correct CPU reference for the group-wise INT4
 * weight-only GEMM (W4A16), its 8-bit variant (W8A16, further down), the 4-bit
 * activation variant (W4A4) with its activation quantizer, and the 4-bit weight quantizer.  Only the tests, the smoke check and the bench's CPU
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

/*
 * The 8-bit variant (W8A16).  "When Do Quantized Drafts Help Speculative Decoding?",
 * "Current pilot setup" and "Results": the pilot runs a GPTQ INT8 draft beside the GPTQ
 * INT4 one, through the same weight-only path.  The same group-wise asymmetric reading,
 * with 8-bit codes and 8-bit zero points:
 *
 *   W[k,n] = (q[k,n] - z[g,n]) * s[g,n],      q, z in 0..255,  g = floor(k / 128)
 *
 *   Wq8 uint32 [K/4,N] row-major; byte j (bits 8j..8j+7) of Wq8[kb,n] is q[4kb+j, n]
 *   s   IEEE binary16 [K/128,N]
 *   z   one byte per entry [K/128,N]; all eight bits are the zero point
 *
 * Every term A*(q-z)*s is exact in binary64 (8 + 9 + 11 significant bits); the sums run
 * in plain k order, as in the 4-bit GEMM above.
 */
static inline int oracle_byte_code(const uint32_t *Wq8, int64_t N, int64_t k, int64_t n)
{
    uint32_t word = Wq8[(k / 4) * N + n];
    return (int)((word >> (8 * (k % 4))) & 0xFFu);
}

int oracle_w8a16_gemm(const uint16_t *A, const uint32_t *Wq8, const uint16_t *S,
                      const uint8_t *Z, int64_t M, int64_t K, int64_t N,
                      const int64_t *cols, int64_t ncols, double *C, double *Cabs,
                      int nthreads)
{
    if (M < 1 || N < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP != 0) return -1;
    if (!cols) ncols = N;
    if (ncols < 1) return -1;
    for (int64_t c = 0; cols && c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;

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
        double *sum = (double *)malloc(sizeof(double) * (size_t)M * 2);
        if (!sum) {
#pragma omp atomic write
            failed = 1;
        }
        double *abs_sum = sum ? sum + M : NULL;
#pragma omp for schedule(static)
        for (int64_t c = 0; c < ncols; ++c) {
            if (!sum) continue;
            int64_t n = cols ? cols[c] : c;
            for (int64_t m = 0; m < M; ++m) { sum[m] = 0.0; abs_sum[m] = 0.0; }
            for (int64_t k = 0; k < K; ++k) {
                int64_t grp = k / ORACLE_GROUP;
                int zp = Z[grp * N + n];
                double sc = oracle_f16_to_f64(S[grp * N + n]);
                int diff = oracle_byte_code(Wq8, N, k, n) - zp;
                double wv = (double)diff * sc;          /* exact: 9 x 11 bits */
                const double *a = Ak + k * M;
                for (int64_t m = 0; m < M; ++m) {
                    double term = a[m] * wv;            /* exact: 8 x 20 bits */
                    sum[m] += term;
                    abs_sum[m] += fabs(term);
                }
            }
            for (int64_t m = 0; m < M; ++m) {
                C[m * ncols + c] = sum[m];
                if (Cabs) Cabs[m * ncols + c] = abs_sum[m];
            }
        }
        free(sum);
    }
    free(Ak);
    return failed ? -2 : 0;
}

/* Packing rule of the 8-bit format: Wq8[kb,n] = sum_j q[4kb+j,n] << 8j. */
int oracle_w8_pack(const uint8_t *q, uint32_t *Wq8, int64_t K, int64_t N)
{
    if (K < 4 || K % 4 != 0 || N < 1) return -1;
    for (int64_t kb = 0; kb < K / 4; ++kb)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t word = 0;
            for (int j = 0; j < 4; ++j)
                word |= (uint32_t)q[(4 * kb + j) * N + n] << (8 * j);
            Wq8[kb * N + n] = word;
        }
    return 0;
}

/* Inverse of the 8-bit packing rule: q[k,n] = byte (k mod 4) of Wq8[k/4, n]. */
int oracle_w8_unpack(const uint32_t *Wq8, uint8_t *q, int64_t K, int64_t N)
{
    if (K < 4 || K % 4 != 0 || N < 1) return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) q[k * N + n] = (uint8_t)oracle_byte_code(Wq8, N, k, n);
    return 0;
}

/*
 * The 4-bit-activation variant (W4A4).  "When Do Quantized Drafts Help Speculative
 * Decoding?", "What is open": QSPEC drafts with W4A4 and verifies with W4A16 on the same
 * 4-bit weights, and the unified W4A4 kernel was the missing piece.  The pages print no
 * activation format; the plainest reading keeps the weights in the W4A16 storage format
 * above and quantizes activations symmetrically to 4 bits per row and group of 128 along K:
 *
 *   amax     = max_{k in g} |A[m,k]|                       (binary32; exact from bfloat16)
 *   sa[m,g]  = amax / 7                                    (binary32, IEEE division)
 *   qa[m,k]  = clamp(rint(A[m,k] / sa[m,g]), -8, 7)        (rint ties to even; 0 if sa == 0)
 *   Aq       uint32 [M, K/8]; nibble j of Aq[m,kb] is qa[m, 8kb+j] + 8 (offset binary)
 *
 *   C[m,n]   = sum_g sa[m,g] * s[g,n] * sum_{k in g} qa[m,k] * (q[k,n] - z[g,n])
 *
 * Every term sa * s * qa * (q - z) is exact in binary64 (24 + 11 + 4 + 5 significant
 * bits); the sums run in plain k order, and Cabs sums their magnitudes.
 */
int oracle_a4_quantize(const uint16_t *A, uint32_t *Aq, float *As, int64_t M, int64_t K)
{
    if (M < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP != 0) return -1;
    memset(Aq, 0, (size_t)M * (size_t)(K / 8) * sizeof(uint32_t));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < K / ORACLE_GROUP; ++g) {
            float amax = 0.0f;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k)
                amax = fmaxf(amax, fabsf((float)oracle_bf16_to_f64(A[m * K + k])));
            const float sa = amax / 7.0f;
            As[m * (K / ORACLE_GROUP) + g] = sa;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k) {
                const float a = (float)oracle_bf16_to_f64(A[m * K + k]);
                const int qa = sa == 0.0f ? 0 : (int)fminf(fmaxf(rintf(a / sa), -8.0f), 7.0f);
                Aq[m * (K / 8) + k / 8] |= (uint32_t)(qa + 8) << (4 * (k % 8));
            }
        }
    return 0;
}

/* The signed 4-bit activation code of row m, column k. */
static inline int oracle_act_code(const uint32_t *Aq, int64_t K, int64_t m, int64_t k)
{
    return (int)((Aq[m * (K / 8) + k / 8] >> (4 * (k % 8))) & 0xFu) - 8;
}

int oracle_w4a4_gemm(const uint32_t *Aq, const float *As, const uint32_t *Wq, const uint16_t *S,
                     const uint8_t *Z, int64_t M, int64_t K, int64_t N,
                     const int64_t *cols, int64_t ncols, double *C, double *Cabs, int nthreads)
{
    if (M < 1 || N < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP != 0) return -1;
    if (!cols) ncols = N;
    if (ncols < 1) return -1;
    for (int64_t c = 0; cols && c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;
    const int64_t G = K / ORACLE_GROUP;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < ncols; ++c) {
        const int64_t n = cols ? cols[c] : c;
        for (int64_t m = 0; m < M; ++m) {
            double total = 0.0, magnitude = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t gk = k / ORACLE_GROUP;
                const double wdq = (double)(oracle_code(Wq, N, k, n) - (Z[gk * N + n] & 0xF)) *
                                   oracle_f16_to_f64(S[gk * N + n]);             /* exact: 5 x 11 bits */
                const double adq = (double)oracle_act_code(Aq, K, m, k) * (double)As[m * G + gk];  /* 4 x 24 */
                const double term = adq * wdq;                                      /* exact: 27 x 16 bits */
                total += term;
                magnitude += fabs(term);
            }
            C[m * ncols + c] = total;
            if (Cabs) Cabs[m * ncols + c] = magnitude;
        }
    }
    return 0;
}

/*
 * IEEE binary16 encoding of a binary32 value, rounding to nearest with ties to even (the
 * default rounding of IEEE 754), gradual underflow to subnormals, overflow to infinity.
 * Written from the format's definition: the value is scaled by a power of two (exact in
 * binary64) so that the 11 (or fewer, for subnormals) significant bits become an integer,
 * which rint() rounds in the default ties-to-even mode.
 */
uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5, 1): exponent e = e2 - 1 */
    int e = e2 - 1;
    if (e < -14) {          /* subnormal range: multiples of 2^-24 */
        double m = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m);  /* m = 1024 is the smallest normal */
    }
    double m = rint(ldexp(a, 10 - e));  /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

/*
 * The producer side of the storage format: a round-to-nearest min/max quantizer, one
 * (scale, zero) pair per group of 128 along K and per column, in the GPTQ style the pages
 * name for their INT4 drafts ("When Do Quantized Drafts Help Speculative Decoding?",
 * "Current pilot setup" and "What is open": GPTQ/AWQ INT4 weights).  The pages do not
 * print the rule; this is the plainest asymmetric reading, every step in binary32:
 *
 *   lo = min(0, min_k W),  hi = max(0, max_k W)          (the range holds 0, so z fits 0..15)
 *   s  = binary16((hi - lo) / 15)                         (ties to even)
 *   if s == 0 (all-zero group, or a range below binary16's resolution): s = binary16(2/15), z = 8
 *   else z = clamp(rint(-lo / s), 0, 15)
 *   q  = clamp(rint(W / s) + z, 0, 15)                    (s as stored, rint ties to even)
 *
 * W is binary16 [K, N] row-major; outputs are the storage format's Wq [K/8, N] (packed as
 * oracle_w4_pack), scales [K/128, N] binary16 bits and zeros [K/128, N] (0..15).
 * Non-finite inputs give unspecified codes (every operation stays defined).
 */
int oracle_w4_quantize(const uint16_t *W, uint32_t *Wq, uint16_t *S, uint8_t *Z, int64_t K, int64_t N)
{
    if (K < ORACLE_GROUP || K % ORACLE_GROUP != 0 || N < 1) return -1;
    memset(Wq, 0, (size_t)(K / 8) * (size_t)N * sizeof(uint32_t));
    for (int64_t g = 0; g < K / ORACLE_GROUP; ++g)
        for (int64_t n = 0; n < N; ++n) {
            float lo = 0.0f, hi = 0.0f;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k) {
                const float w = (float)oracle_f16_to_f64(W[k * N + n]);
                lo = fminf(lo, w);
                hi = fmaxf(hi, w);
            }
            uint16_t sb = oracle_f32_to_f16((hi - lo) / 15.0f);
            float s = (float)oracle_f16_to_f64(sb);
            int z;
            if (s == 0.0f) {
                sb = oracle_f32_to_f16(2.0f / 15.0f);
                s = (float)oracle_f16_to_f64(sb);
                z = 8;
            } else {
                z = (int)fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
            }
            S[g * N + n] = sb;
            Z[g * N + n] = (uint8_t)z;
            for (int64_t k = g * ORACLE_GROUP; k < (g + 1) * ORACLE_GROUP; ++k) {
                const float w = (float)oracle_f16_to_f64(W[k * N + n]);
                const int q = (int)fminf(fmaxf(rintf(w / s) + (float)z, 0.0f), 15.0f);
                Wq[(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));
            }
        }
    return 0;
}
