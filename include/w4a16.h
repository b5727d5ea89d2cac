/*
 * w4a16.h -- C ABI of the group-wise INT4 weight-only GEMM (W4A16) for AMD MI355X (gfx950).
 *
 * The operation.  "The Free Half of Speculative Decoding" (third paragraph) quantizes the
 * target model of a speculative decoder to INT4 with AWQ; "When Do Quantized Drafts Help
 * Speculative Decoding?" ("Current pilot setup", "What is included") runs GPTQ INT4 drafts
 * through a W4A16 kernel and verifies gamma+1 = 5 drafted positions per target forward.
 * Every linear layer of those forwards is the product computed here.  The pages do not
 * print the dequantization rule or the storage layout; this library uses the plainest
 * asymmetric group-wise reading, with groups of 128 along K:
 *
 *     W[k,n] = (q[k,n] - z[g,n]) * s[g,n],   g = floor(k / 128)
 *     C[m,n] = sum_k A[m,k] * W[k,n]
 *
 * Storage (all arrays dense, row-major, in device memory owned by the caller):
 *     A_bf16     [M, K]      bfloat16
 *     Wq         [K/8, N]    uint32; nibble j (bits 4j..4j+3) of Wq[kb,n] is q[8kb+j, n]
 *     scales_f16 [K/128, N]  IEEE binary16
 *     zeros_u4   [K/128, N]  one byte per entry, only the low nibble is read
 *     C          [M, N]      float32, overwritten
 *
 * Accuracy contract: every element satisfies
 *     |C - C_exact| <= 1e-4 * sum_k |A[m,k] * W[k,n]| + 1e-6.
 * The (q - z) factors and their products with A are exact; partial sums are float32.
 * M >= 64, and 17 <= M < 64 with K*N >= 2^25, run on the bfloat16 matrix cores with A
 * used as given.  Other shapes (the small-M and narrow-tile kernels) run on the
 * binary16 matrix cores with A rescaled by a power of two per (row, 128-wide group), so
 * that the group's largest |A| lands in [2^15, 2^16).  The contract above then holds for
 * every activation row whose magnitudes within each 128-wide group span at most 2^32
 * (largest |A| over smallest nonzero |A|): every such element is exact in binary16 after
 * scaling.  Beyond that span the contract is replaced by a documented bound: an element
 * whose binary exponent is more than 32 below that of its group's largest magnitude amax
 * is rounded to the binary16 subnormal grid, an absolute error of at most 2^-40 * amax, so
 *     |C - C_exact| <= 1e-4 * sum_k |A W| + 1e-6 + 2^-40 * sum_k' amax[m, g(k')] |W[k',n]|
 * with k' over those elements.  A group whose largest magnitude is below about 2^-100 can
 * lose bits in the float32 rescale; its whole contribution is then below 2^-90 and inside
 * the 1e-6 term.
 *
 * All entry points validate their arguments on the host before any HIP call and return a
 * status; launches are asynchronous on the given stream (NULL = the null stream), so device
 * faults surface at the caller's next synchronization.  No entry point synchronizes the
 * host in steady state.  Inputs must not alias C.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4_status {
    W4_OK = 0,
    W4_ERR_NULL = 1,      /* a required pointer is NULL                                    */
    W4_ERR_SHAPE = 2,     /* a size is out of range (see each entry point)                 */
    W4_ERR_ALIGN = 3,     /* a pointer is not aligned as required                           */
    W4_ERR_DEVICE = 4,    /* no HIP device, or the current device is not gfx950            */
    W4_ERR_HIP = 5,       /* a HIP runtime call or launch failed; see w4_last_error()      */
    W4_ERR_WORKSPACE = 6, /* the split-K workspace would have to grow while the stream is
                             being captured into a graph: run the same shape once before
                             capturing; or (w4a16_gemm_noalloc) the plan needs more scratch
                             than its fixed maximum                                        */
    W4_ERR_PLAN = 7       /* internal: the launch plan names no compiled kernel instance
                             (nothing was launched; C is not written)                      */
} w4_status;

/*
 * C = A . W for the group-wise INT4 format above (the verify and draft linear layers of
 * "When Do Quantized Drafts Help Speculative Decoding?", "Current pilot setup").
 *
 *   M >= 1 rows of A (tokens), K >= 128 with K % 128 == 0, N >= 1 columns.
 *   A_bf16, Wq and C must be 16-byte aligned (W4_ERR_ALIGN otherwise); scales_f16 2-byte.
 *   Any N is accepted; N % 4 == 0 with 8-byte aligned scales and 4-byte aligned zeros
 *   takes the vectorized load path.
 *   Split-K shapes use a library workspace (arrival counters and float32 partials) owned
 *   per (device, stream): it is allocated on first need (outside graph capture, so a graph
 *   must not capture the first call of a new split shape) and kept until the process ends.
 *   Calls issued on different streams each get their own workspace and may overlap.  A
 *   captured graph keeps the workspace of the stream it was captured on: replay it only
 *   where it cannot overlap other work that uses that same workspace (other calls or graphs
 *   issued on, or captured on, that stream); capture graphs that may run concurrently on
 *   distinct streams.  Overlapping users of one workspace race on its counters and give
 *   wrong results without an error.
 *   stream: a hipStream_t, or NULL.
 */
w4_status w4a16_gemm(const void *A_bf16, const uint32_t *Wq, const void *scales_f16,
                     const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N,
                     void *stream);

/*
 * w4a16_gemm for callers that cannot allocate device memory: code under HIP graph capture
 * (including a first call of a new split shape), tight serving loops, or harnesses that
 * forbid hipMalloc.  Same arguments, layouts, plan, kernels and results (bit for bit) as
 * w4a16_gemm, but the split-K scratch is a fixed array of 64 MiB per GPU inside the library
 * (its code object's zero-initialized data, held by every GPU the library is loaded on until
 * the process ends), not a workspace: the call makes no hipMalloc, hipFree or other
 * allocating call.  The first call on a device looks up that array's address and clears its
 * arrival counters with a kernel on `stream`.
 *   A shape whose plan needs more than 65536 arrival counters or more than 64 MiB - 256 KiB
 *   of partials (in practice large M with deep K splits, e.g. M * N * splits * 4 bytes
 *   beyond that) returns W4_ERR_WORKSPACE before anything is launched.
 *   Every call on one GPU shares that GPU's array: calls (and graphs holding calls) that
 *   overlap in time on one GPU race on its counters and partials and can return wrong C
 *   without an error.  Serialize them (for example, one stream).
 *   Other errors as for w4a16_gemm.
 */
w4_status w4a16_gemm_noalloc(const void *A_bf16, const uint32_t *Wq, const void *scales_f16,
                             const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N,
                             void *stream);

/*
 * C = A . W for the 8-bit variant of the format (W8A16): the GPTQ INT8 draft that "When
 * Do Quantized Drafts Help Speculative Decoding?" ("Current pilot setup", "Results") runs
 * beside the INT4 one.  Same group-wise rule, W[k,n] = (q[k,n] - z[g,n]) * s[g,n], with
 * 8-bit codes and zero points (0..255):
 *     Wq8        [K/4, N]    uint32; byte j (bits 8j..8j+7) of Wq8[kb,n] is q[4kb+j, n]
 *     scales_f16 [K/128, N]  IEEE binary16
 *     zeros_u8   [K/128, N]  one byte per entry, all 8 bits are the zero point
 *   A_bf16 and C, sizes, alignment, workspace, stream and errors as for w4a16_gemm; the
 *   packed codes must stay below 2 GiB (K/4 * N * 4 bytes).  Every M runs on the binary16
 *   matrix cores with the per-(row, group) power-of-two activation scaling described at
 *   the top of this file, in row blocks of 16, so the same accuracy contract holds.
 */
w4_status w8a16_gemm(const void *A_bf16, const uint32_t *Wq8, const void *scales_f16,
                     const uint8_t *zeros_u8, float *C, int64_t M, int64_t K, int64_t N,
                     void *stream);

/*
 * C = A . W with 4-bit activations on the 4-bit weights (W4A4): the draft side of QSPEC's
 * complementary scheme, which "When Do Quantized Drafts Help Speculative Decoding?" ("What
 * is open") describes as a W4A4 draft verified by W4A16 on the same weights.  The pages
 * print no activation format; this is the plainest reading, symmetric per row and group of
 * 128 along K (as produced by a4_quantize):
 *     Aq         [M, K/8]    uint32; nibble j of Aq[m,kb] is qa[m, 8kb+j] + 8, qa in -8..7
 *     A_scales   [M, K/128]  float32 sa
 *     Wq, scales_f16, zeros_u4: the 4-bit weight format of w4a16_gemm
 *     C[m,n] = sum_g sa[m,g] * s[g,n] * sum_{k in g} qa[m,k] * (q[k,n] - z[g,n])
 *   Aq and A_scales 4-byte aligned; Wq and C 16-byte aligned; scales_f16 2-byte.  Sizes,
 *   workspace, stream and errors as for w4a16_gemm.  Each group's inner sum is an exact
 *   integer; it is scaled by sa * s in float32, so every element is within
 *   1e-4 * sum_k |sa qa (q - z) s| + 1e-6 of the exact value.  Every M runs on the binary16
 *   matrix cores, in row blocks of 16; at 17..32 rows, in one block of 32 rows.
 */
w4_status w4a4_gemm(const uint32_t *Aq, const float *A_scales, const uint32_t *Wq, const void *scales_f16,
                    const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N, void *stream);

/*
 * The activation quantizer of w4a4_gemm: for each row m and group g of 128 along K,
 *     amax = max |A[m,k]|,  sa = amax / 7,  qa = clamp(rint(A / sa), -8, 7)  (0 if sa == 0)
 * every step in binary32 with IEEE division and rint ties to even, so the codes are
 * reproducible bit for bit.
 *   A_bf16:   [M, K] bfloat16, 16-byte aligned (not modified); inputs must be finite.
 *   Aq:       [M, K/8] uint32, 4-byte aligned, overwritten (nibble j = qa[8kb+j] + 8).
 *   A_scales: [M, K/128] float32, 4-byte aligned, overwritten.
 *   M >= 1, K >= 128, K % 128 == 0.  Asynchronous on `stream`; errors as for w4a16_gemm.
 */
w4_status a4_quantize(const void *A_bf16, uint32_t *Aq, float *A_scales, int64_t M, int64_t K, void *stream);

/*
 * Packs 8-bit codes into the 8-bit storage layout: Wq8[kb,n] = sum_j q[4kb+j,n] << 8j.
 *   q_u8: [K, N] bytes; Wq8: [K/4, N] uint32, overwritten.
 *   K >= 4 with K % 4 == 0, N >= 1; Wq8 must be 4-byte aligned.  Bit-exact.
 */
w4_status w8_pack(const uint8_t *q_u8, uint32_t *Wq8, int64_t K, int64_t N, void *stream);

/*
 * Packs 4-bit codes into the storage layout of the INT4 GPTQ weights that "When Do
 * Quantized Drafts Help Speculative Decoding?" ("Current pilot setup") runs its draft on
 * (the page names the format, not the bit order; this layout is the sequential reading,
 * eight codes per word along K): Wq[kb,n] = sum_j (q[8kb+j,n] & 0xF) << 4j.
 *   q_u4: [K, N] bytes (high nibbles ignored); Wq: [K/8, N] uint32, overwritten.
 *   K >= 8 with K % 8 == 0, N >= 1; Wq must be 4-byte aligned.  Bit-exact.
 */
w4_status w4_pack(const uint8_t *q_u4, uint32_t *Wq, int64_t K, int64_t N, void *stream);

/*
 * Round-to-nearest quantizer: produces the storage format from binary16 weights, one
 * (scale, zero) pair per column and group of 128 along K, in the GPTQ/AWQ style the pages
 * use for their INT4 drafts and target ("When Do Quantized Drafts Help Speculative
 * Decoding?", "Current pilot setup"; "The Free Half of Speculative Decoding", third
 * paragraph; neither prints the rule, so this is the plainest asymmetric reading).  Every
 * step is binary32 with IEEE division and rint ties to even:
 *     lo = min(0, min W), hi = max(0, max W)         over the group's 128 values
 *     s  = binary16((hi - lo) / 15)                  (ties to even)
 *     if s == 0 (all-zero or too narrow a range):    s = binary16(2/15), z = 8
 *     else                                           z = clamp(rint(-lo / s), 0, 15)
 *     q  = clamp(rint(W / s) + z, 0, 15)             (s as stored)
 *   W_f16:      [K, N] binary16 row-major, 2-byte aligned (not modified)
 *   Wq:         [K/8, N] uint32, 4-byte aligned, overwritten with the packed codes (as w4_pack)
 *   scales_f16: [K/128, N] binary16, 2-byte aligned, overwritten
 *   zeros_u4:   [K/128, N] bytes, overwritten with 0..15
 *   K >= 128, K % 128 == 0, K/128 <= 65535, N >= 1.  Bit-exact and deterministic.  Inputs
 *   must be finite: codes for NaN or infinite weights are unspecified (the call completes).
 * Asynchronous on `stream`; validation errors as for w4a16_gemm.
 */
w4_status w4_quantize(const void *W_f16, uint32_t *Wq, void *scales_f16, uint8_t *zeros_u4, int64_t K, int64_t N,
                      void *stream);

/*
 * Streaming-read probe (a measurement aid, not part of the GEMM): reads `bytes` bytes at
 * `src` once, with the weight stream's load policy (16-byte non-temporal loads, several in
 * flight per lane), so that its rate is the achievable HBM read ceiling for a buffer of that
 * size.
 *   src: device, 16-byte aligned, 16 <= bytes < 2^31 and bytes % 16 == 0 (not modified).
 *   xor_out: device [blocks][4] uint32, 4-byte aligned, overwritten: entry [b][w] is the
 *     XOR of the 32-bit words read by wave w of block b (each 16-byte chunk is read by
 *     exactly one wave), so the XOR over all entries equals the XOR of every word of the
 *     buffer.
 *   blocks: workgroups of 256 lanes, 1..65535 (768 fills three per CU).
 * Asynchronous on `stream`; validation errors as for w4a16_gemm.
 */
w4_status w4_read_probe(const void *src, int64_t bytes, uint32_t *xor_out, int64_t blocks, void *stream);

/* How w4a16_gemm would run a shape (host only, no HIP call). */
typedef struct w4_plan {
    int kernel;             /* 1 = small-M wide (4 waves per workgroup, fp16 MFMA),
                               2 = small-M tall (12 waves, fp16 MFMA),
                               3 = large-M (M >= 64, or M >= 17 with K*N >= 2^25:
                                   8 waves, bf16 MFMA),
                               4, 5 = 8-bit codes (w8a16_gemm), wide and tall as 1, 2,
                               6, 7 = 4-bit activations (w4a4_gemm), wide and tall,
                               8 = narrow tiles (M <= 16 with at most 64 groups, the
                                   activations staged whole in at most 64 KiB of LDS, and at
                                   most 256 tiles: 8 waves, one 16-column tile over all of
                                   K per workgroup, fp16 MFMA, no K split)                    */
    int tile_m;             /* output rows per row block: 16 for kernels 1, 2, 4, 5, 8; 16
                               for kernels 6, 7, except 32 at 17..32 rows; 1 to 160 for
                               kernel 3, computed in row tiles of 32                         */
    int tile_n;             /* output columns per workgroup tile (64; 256 for kernel 3; 16
                               for kernel 8)                                                 */
    int m_blocks;           /* row blocks of tile_m                                          */
    int n_tiles;            /* column tiles of tile_n                                        */
    int splits;             /* K splits across workgroups (1 = no workspace)                */
    int groups_per_split;   /* 128-wide K groups handled by one workgroup of a split tile
                               (kernel 3: (tile, group) steps per workgroup)                 */
    int full_tiles;         /* kernels 1, 4, 6: tiles 0..full_tiles-1 (tile t is row block
                               t % m_blocks of column tile t / m_blocks) run
                               unsplit, one workgroup each, and only the other tiles are
                               split (a multiple of 256: whole rounds of CUs); 0 otherwise  */
    int64_t workgroups;     /* grid size: full_tiles + (m_blocks*n_tiles - full_tiles)*splits,
                               except kernel 3: ceil(m_blocks*n_tiles*group_stride /
                               groups_per_split)                                              */
    int64_t workspace_bytes;/* split-K workspace needed (0 when splits == 1)                 */
    int64_t group_stride;   /* kernel 3 (0 for the others): the (tile, group) steps are
                               numbered tile-major with this many numbers per tile (the
                               K/128 groups, then unused numbers), and workgroup w takes
                               steps w*groups_per_split .. +groups_per_split-1.  Equal to
                               splits*groups_per_split, each workgroup works in one tile (a
                               K split); equal to the group count, the steps are shared out
                               evenly and a workgroup may finish one tile and start the
                               next.  splits is then the most workgroups any tile has     */
} w4_plan;

w4_status w4a16_plan(int64_t M, int64_t K, int64_t N, w4_plan *out);

/* How w8a16_gemm would run a shape (host only, no HIP call). */
w4_status w8a16_plan(int64_t M, int64_t K, int64_t N, w4_plan *out);

/* How w4a4_gemm would run a shape (host only, no HIP call). */
w4_status w4a4_plan(int64_t M, int64_t K, int64_t N, w4_plan *out);

/* Static text for a status code. */
const char *w4_status_string(w4_status s);

/* Text describing the last failure on the calling thread ("" if none). */
const char *w4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
