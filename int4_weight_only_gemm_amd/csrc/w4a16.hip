// w4a16.hip -- group-wise INT4 weight-only GEMM (W4A16) and the 4-bit pack, for gfx950.
//
// The operation is the INT4 weight-only linear layer of a speculative decoder's draft and
// verify forwards ("The Free Half of Speculative Decoding", third paragraph: AWQ INT4
// target; "When Do Quantized Drafts Help Speculative Decoding?", "Current pilot setup":
// GPTQ INT4 draft, gamma = 4 so the target verifies 5 positions at batch 1).  With the
// group-wise asymmetric reading of that format (groups of 128 along K):
//     C[m,n] = sum_g s[g,n] * sum_{k in g} A[m,k] * (q[k,n] - z[g,n])
// which is how the kernels below evaluate it: the inner sums use exact (q - z) factors
// and float32 accumulation, the outer sum applies each group's scale once per output.
//
// Hardware mapping (MI355X, CDNA4), small M (M < 64; M >= 64, and large GEMMs from M = 17,
// run the bf16 matrix-core kernel further down):
//  * Weights are streamed once from HBM with 16-byte non-temporal loads; a lane's load
//    holds four adjacent columns of one packed row (8 codes each).
//  * (q - z) is built in registers as exact binary16 pairs: a code is OR-ed into the
//    mantissa of 1024.0 (or of 1024.0 + 16 q for the odd nibble of a byte) and the zero
//    point is removed with one packed fp16 add/fma.  That is 9 VALU ops per 8 weights.
//  * The products run on the matrix cores (v_mfma_f32_16x16x32_f16).  Each wave converts
//    the activations of the group it is about to compute from bfloat16 to binary16 in its
//    own LDS tile, row r scaled by 2^x[r] so that the row's largest magnitude in the group
//    lands in [2^15, 2^16); the scale is undone exactly when the group's float32 partial
//    is rescaled by s.  Every product a*(q-z) is then exact; bfloat16 values more than
//    2^33 below the largest magnitude of their row within the group are rounded to the
//    binary16 subnormal grid (absolute error below 2^-40 of that maximum per element).
//  * The same kernel, by template parameter, runs 8-bit codes (4 per word, full-byte zero
//    points) and 4-bit activations (offset-binary codes with a float32 scale per row and
//    group, unpacked like the weights), and holds one or two 16-row matrix-core tiles per
//    wave (two share every unpacked weight operand).
//  * Split-K across workgroups writes float32 partials to a workspace with device-coherent
//    stores; a per-tile arrival counter elects the last workgroup, which sums the partials
//    in split order, writes C and resets the counter.  One launch per GEMM, no memset, no
//    cache flush, bitwise reproducible.  A plan may run whole rounds of tiles unsplit and
//    split only the remaining tiles, to balance the CUs.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <type_traits>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "w4a16.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTileN = 64;                 // output columns per workgroup (16 lanes x 4 words)
constexpr int kTileM = 16;                 // output rows per M-block (one MFMA tile)
constexpr int kGroup = 128;                // quantization group along K
constexpr int kChunksPerRow = kGroup / 8;  // 16-byte activation chunks per group row
constexpr int kARowBytes = (kChunksPerRow + 1) * 16;  // +16 bytes of padding: conflict-free reads
constexpr int kCacheStream = 2;            // buffer-load cache policy: non-temporal (streamed once)
constexpr int kCacheCoherent = 16;         // buffer-op cache policy: device-coherent (sc1), as for
                                           // agent-scope atomics on this target
constexpr int kCUs = 256;

// Two shapes of the same kernel.  "Wide": 4 waves per workgroup, 3 workgroups resident per
// CU, for outputs wide enough to fill the GPU with column tiles.  "Tall": 12 waves per
// workgroup (one per CU) splitting K inside the workgroup, for narrow outputs, so that K is
// reduced in LDS instead of across workgroups.  Both keep 3 waves per SIMD.
struct Variant {
    int waves;   // waves per workgroup
    int per_cu;  // resident workgroups per CU
};
constexpr Variant kWide = {4, 3};
constexpr Variant kTall = {12, 1};
constexpr int kOccupancy = 3;  // waves per SIMD: at most 168 VGPRs per lane
// 32-row blocks (two row tiles per wave) need more registers: 2 waves per SIMD.
constexpr Variant kWide2 = {4, 2};
constexpr Variant kTall2 = {8, 1};
constexpr int kOccupancy2 = 2;  // at most 256 VGPRs per lane

struct SmallParams {
    const uint16_t *A;  // bfloat16 [M, K]; with 4-bit activations the packed codes [M, K/8]
    const uint32_t *Wq;
    const uint16_t *S;
    const uint8_t *Z;
    float *C;
    float *part;        // [split tiles][splits][16][64] float32 partials
    unsigned *count;    // [split tiles] arrival counters, zero between calls
    int64_t M, K, N;
    int groups, splits, gps, n_tiles, m_blocks;
    int full_tiles;     // tiles [0, full_tiles) are not split (dispatched after the split parts)
    const float *As;    // 4-bit activations only: float32 scales [M, K/128]
};

// The small-M kernel's arguments: the fields every wave needs before its first weight load
// come first, 14 dwords in all, which is what the hardware can preload into scalar registers
// at wave launch (the tile and row-block counts follow from N and M); the rest follows as a
// struct.
struct SmallTail {
    float *C;
    float *part;
    unsigned *count;
    const float *As;
};

// ------------------------------------------------------------------------------------
// Bit-level helpers

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Eight codes of one packed word -> eight exact binary16 values (q_j - z), in the order
// j = 0,4,1,5,2,6,3,7 (element e holds nibble (e >> 1) + 4 * (e & 1)).  This is the
// published magic-number integer-to-float conversion (Kim et al. 2022, "Who Says Elephants
// Can't Run?", for FasterTransformer's mixed-precision GEMMs; also used by Marlin): an
// integer placed in the low mantissa bits of a float whose exponent makes the mantissa unit
// 1, here binary16 1024.0, then that float's value subtracted in one float add.  Here the
// per-column zero point is folded into the subtrahend.
//   zlo = fp16 pair of -(1024 + z), zhi = fp16 pair of -(64 + z).
//   magic = 0x64006400 (binary16 1024.0 in both halves), held in a VGPR so that each
//   mask-and-insert is one v_and_or_b32 (VOP3 takes one SGPR/literal operand on gfx9).
__device__ __forceinline__ f16x8 unpack8(uint32_t w, uint32_t zlo, uint32_t zhi, uint32_t magic)
{
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    uint32_t w8 = w >> 8;
    f16x2 x0 = as_h2((w & 0x000F000Fu) | magic);   // 1024 + q0 | 1024 + q4
    f16x2 x1 = as_h2((w & 0x00F000F0u) | magic);   // 1024 + 16 q1 | 1024 + 16 q5
    f16x2 x2 = as_h2((w8 & 0x000F000Fu) | magic);  // 1024 + q2 | 1024 + q6
    f16x2 x3 = as_h2((w8 & 0x00F000F0u) | magic);  // 1024 + 16 q3 | 1024 + 16 q7
    f16x2 d0 = x0 + as_h2(zlo);
    f16x2 d1 = __builtin_elementwise_fma(x1, sixteenth, as_h2(zhi));
    f16x2 d2 = x2 + as_h2(zlo);
    f16x2 d3 = __builtin_elementwise_fma(x3, sixteenth, as_h2(zhi));
    u32x4 r = {as_u(d0), as_u(d1), as_u(d2), as_u(d3)};
    return __builtin_bit_cast(f16x8, r);
}

// Eight 8-bit codes (two packed words, k order 0..7) -> eight exact binary16 values
// (q_j - z), in k order.  v_perm_b32 places each code byte under the high byte 0x64 (taken
// from `magic`, 0x64646464), which reads as the binary16 value 1024 + q; one packed add of
// zneg = the binary16 pair of -(1024 + z) leaves q - z, exact for q, z in 0..255.
__device__ __forceinline__ f16x8 unpack8_w8(uint32_t w0, uint32_t w1, uint32_t zneg, uint32_t magic,
                                            uint32_t sel01, uint32_t sel23)
{
    const f16x2 zn = as_h2(zneg);
    const f16x2 d0 = as_h2(__builtin_amdgcn_perm(magic, w0, sel01)) + zn;  // q0 | q1
    const f16x2 d1 = as_h2(__builtin_amdgcn_perm(magic, w0, sel23)) + zn;  // q2 | q3
    const f16x2 d2 = as_h2(__builtin_amdgcn_perm(magic, w1, sel01)) + zn;  // q4 | q5
    const f16x2 d3 = as_h2(__builtin_amdgcn_perm(magic, w1, sel23)) + zn;  // q6 | q7
    u32x4 r = {as_u(d0), as_u(d1), as_u(d2), as_u(d3)};
    return __builtin_bit_cast(f16x8, r);
}

// Largest biased bfloat16 exponent among the 8 values of a chunk.
__device__ __forceinline__ int chunk_max_exp(u32x4 v)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t m = 0x7F807F80u;  // exponent fields of both halves
    const u16x2 a = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v[0] & m), __builtin_bit_cast(u16x2, v[1] & m));
    const u16x2 b = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v[2] & m), __builtin_bit_cast(u16x2, v[3] & m));
    const u16x2 c = __builtin_elementwise_max(a, b);
    return (int)(max(c.x, c.y) >> 7);
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), in every lane: rotations
// by 8, 4, 2 and 1 within the row, without LDS traffic.
__device__ __forceinline__ int row16_max(int e)
{
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x128, 0xF, 0xF, false));  // row_ror:8
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x124, 0xF, 0xF, false));  // row_ror:4
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x122, 0xF, 0xF, false));  // row_ror:2
    e = max(e, __builtin_amdgcn_update_dpp(0, e, 0x121, 0xF, 0xF, false));  // row_ror:1
    return e;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    f16x2 h = {(_Float16)a, (_Float16)b};
    return as_u(h);
}

// 8 bfloat16 values (k order 0..7) -> 8 binary16 values scaled by 2^x, in the element
// order of the weight operand: unpack8's (0,4,1,5,2,6,3,7) for 4-bit codes, k order for
// 8-bit codes.
template <int BITS>
__device__ __forceinline__ u32x4 convert_chunk(u32x4 v, int x)
{
    float e0 = ldexpf(__builtin_bit_cast(float, v[0] << 16), x);
    float e1 = ldexpf(__builtin_bit_cast(float, v[0] & 0xFFFF0000u), x);
    float e2 = ldexpf(__builtin_bit_cast(float, v[1] << 16), x);
    float e3 = ldexpf(__builtin_bit_cast(float, v[1] & 0xFFFF0000u), x);
    float e4 = ldexpf(__builtin_bit_cast(float, v[2] << 16), x);
    float e5 = ldexpf(__builtin_bit_cast(float, v[2] & 0xFFFF0000u), x);
    float e6 = ldexpf(__builtin_bit_cast(float, v[3] << 16), x);
    float e7 = ldexpf(__builtin_bit_cast(float, v[3] & 0xFFFF0000u), x);
    if constexpr (BITS == 8) {
        u32x4 r = {pack_h2(e0, e1), pack_h2(e2, e3), pack_h2(e4, e5), pack_h2(e6, e7)};
        return r;
    }
    u32x4 r = {pack_h2(e0, e4), pack_h2(e1, e5), pack_h2(e2, e6), pack_h2(e3, e7)};
    return r;
}

// Maps the hardware workgroup id to a logical id so that logically consecutive
// workgroups (the K splits of one tile) are dispatched to the same XCD: workgroup b runs
// on XCD b % 8.
__device__ __forceinline__ uint32_t xcd_local_id(uint32_t b, uint32_t n)
{
    uint32_t per = n / 8, rem = n % 8, x = b % 8, slot = b / 8;
    return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

// ------------------------------------------------------------------------------------
// A group of 128 k holds 16 packed rows of 4-bit codes or 32 of 8-bit codes.  One 16-byte
// load per lane covers 4 rows (lane quarter kq takes one), so a group takes BITS loads.
//   4-bit: load st holds row 4 st + kq: k = 32 st + 8 kq .. + 7, one word per column.
//   8-bit: loads 2 ks and 2 ks + 1 hold rows 8 ks + 2 kq and 8 ks + 2 kq + 1: the same
//          k = 32 ks + 8 kq .. + 7, two words per column.
// Either way a lane holds the 8 k of its matrix-core operand for k-step st (or ks).
template <int BITS>
__device__ __forceinline__ constexpr int load_row(int st)
{
    return BITS == 4 ? 4 * st : 8 * (st >> 1) + (st & 1);
}

// Register slot of one wave for one group: BITS loads of 4 packed rows each and the
// group's scales and zeros for the lane's 4 columns.
template <int BITS>
struct GroupRegs {
    u32x4 w[BITS];
    u32x2 s;      // 4 binary16 scales
    uint32_t z;   // 4 zero bytes
};

// Per-lane byte offsets that stay fixed for a whole workgroup.  All loads are buffer
// loads: a scalar resource (base, size) per array, this per-lane offset, and a
// wave-uniform scalar offset per group, so a group's loads cost no address VGPRs.
// Out-of-range columns read a clamped in-range address (those values are never stored)
// and no load sits behind a branch, so the compiler waits for exactly the slot it needs
// while later groups stay in flight.
template <bool VEC>
struct LaneOffsets {
    uint32_t w[VEC ? 1 : 4];  // packed words: row kq of the group, this lane's column(s)
    uint32_t s[VEC ? 1 : 4];  // scales
    uint32_t z[VEC ? 1 : 4];  // zeros
};

struct Resources {
    __amdgpu_buffer_rsrc_t W, S, Z, A, As;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

template <bool VEC, int BITS>
__device__ __forceinline__ void lane_offsets(const SmallParams &p, int n0, int lane, LaneOffsets<VEC> &o)
{
    const int c = lane & 15, kq = lane >> 4;
    const int64_t N = p.N;
    const int64_t col = n0 + 4 * c;
    const int64_t krow = kq * (BITS / 4);  // the lane's first packed row within a load
    if (VEC) {
        const int64_t colv = col < N - 4 ? col : N - 4;  // N % 4 == 0, so N >= 4
        o.w[0] = (uint32_t)((krow * N + colv) * 4);
        o.s[0] = (uint32_t)(colv * 2);
        o.z[0] = (uint32_t)colv;
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t ct = col + t < N ? col + t : N - 1;
            o.w[t] = (uint32_t)((krow * N + ct) * 4);
            o.s[t] = (uint32_t)(ct * 2);
            o.z[t] = (uint32_t)ct;
        }
    }
}

template <bool VEC, int BITS>
__device__ __forceinline__ void load_group(const SmallParams &p, const Resources &rs,
                                           const LaneOffsets<VEC> &o, int g, GroupRegs<BITS> &r)
{
    const uint32_t rowbytes = (uint32_t)p.N * 4;
#pragma unroll
    for (int st = 0; st < BITS; ++st) {
        const uint32_t so = ((uint32_t)g * (4 * BITS) + load_row<BITS>(st)) * rowbytes;
        if (VEC) {
            r.w[st] = __builtin_amdgcn_raw_buffer_load_b128(rs.W, o.w[0], so, kCacheStream);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) r.w[st][t] = __builtin_amdgcn_raw_buffer_load_b32(rs.W, o.w[t], so, kCacheStream);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // the group's scales and zeros follow its own words
    const uint32_t gso = (uint32_t)g * (uint32_t)p.N;
    if (VEC) {
        r.s = __builtin_amdgcn_raw_buffer_load_b64(rs.S, o.s[0], gso * 2, 0);
        r.z = __builtin_amdgcn_raw_buffer_load_b32(rs.Z, o.z[0], gso, 0);
    } else {
        uint32_t sv[4], zv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sv[t] = __builtin_amdgcn_raw_buffer_load_b16(rs.S, o.s[t], gso * 2, 0);
            zv[t] = __builtin_amdgcn_raw_buffer_load_b8(rs.Z, o.z[t], gso, 0);
        }
        r.s = u32x2{sv[0] | (sv[1] << 16), sv[2] | (sv[3] << 16)};
        r.z = zv[0] | (zv[1] << 8) | (zv[2] << 16) | (zv[3] << 24);
    }
}


// ------------------------------------------------------------------------------------
// The GEMM kernel.  Each wave walks its own groups (every WAVES-th group of the
// workgroup's K range).  For each group it converts that group's activations itself, with
// one power-of-two scale per (row, group), right before computing it: the activation
// chunks travel in the register ring with the group's weights, so the conversion overlaps
// the loads still in flight and there is no workgroup-wide staging phase.

// Activation chunks of rows 4i + lane/16, chunk lane%16 of the group: 8 bfloat16 values, or
// (4-bit activations) one word of 8 codes and the row's scale bits.
template <int AV, bool A4>
struct ActRegs {
    typename std::conditional<A4, u32x2, u32x4>::type a[AV];
};

// Per-wave LDS: the activation tile (RB row tiles of 16 rows) and one word per row (the
// power-of-two exponent, or the 4-bit activations' scale).
constexpr int pipe_wave_bytes(int rb) { return rb * (kTileM * kARowBytes + kTileM * 4); }
constexpr int pipe_exp_offset(int rb) { return rb * kTileM * kARowBytes; }

// T1: the last pass holds a single row (M = 4 AV - 3 in one 16-row block, AV >= 2).  That row's 128
// values are spread over all 64 lanes, two per lane: lane l takes values q and q + 4 of chunk
// l / 4 (q = l % 4), the two that convert_chunk packs into word q of the chunk, so the pass
// costs two values of conversion per lane instead of eight.
template <int AV, bool A4, bool T1>
__device__ __forceinline__ void load_act(const Resources &rs, const uint32_t (&aoff)[AV], const uint32_t (&asoff)[AV],
                                         int g, ActRegs<AV, A4> &r)
{
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        if constexpr (!A4 && T1) {
            if (i == AV - 1) {
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs.A, aoff[i], (uint32_t)g * (kGroup * 2), 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs.A, aoff[i] + 8, (uint32_t)g * (kGroup * 2), 0);
                r.a[i].x = lo | (hi << 16);
                continue;
            }
        }
        if constexpr (A4) {
            r.a[i].x = __builtin_amdgcn_raw_buffer_load_b32(rs.A, aoff[i], (uint32_t)g * (kGroup / 2), 0);
            r.a[i].y = __builtin_amdgcn_raw_buffer_load_b32(rs.As, asoff[i], (uint32_t)g * 4, 0);
        } else {
            r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.A, aoff[i], (uint32_t)g * (kGroup * 2), 0);
        }
    }
}

// Convert this wave's group of activations into its LDS tile: row r scaled by 2^x[r],
// x[r] = 142 - (largest biased exponent of row r in the group); exponents stored next to
// the tile.  The 16 chunks of a row sit in 16 consecutive lanes.  4-bit activations are
// unpacked instead (offset-binary codes, zero point 8, exact in binary16, in the weight
// operand's element order) and the row's float32 scale is stored in place of x[r].
template <int AV, int BITS, bool A4, int RB, bool T1>
__device__ __forceinline__ void stage_pipe(const ActRegs<AV, A4> &r, char *lds_wave, int mv, int lane)
{
    constexpr int kExpOffset = pipe_exp_offset(RB);
    asm volatile("" ::: "memory");  // the previous group's LDS reads stay before these writes
    const int kc = lane & 15;
    if constexpr (A4) {
        uint32_t magic, zlo = (0xE400u | 8u) * 0x00010001u, zhi = (0xD400u | (8u << 4)) * 0x00010001u;
        asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
        asm volatile("" : "+v"(zlo), "+v"(zhi));
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int row = 4 * i + (lane >> 4);
            const f16x8 v = unpack8(r.a[i].x, zlo, zhi, magic);
            if (row < mv) *(u32x4 *)(lds_wave + row * kARowBytes + kc * 16) = __builtin_bit_cast(u32x4, v);
            if (kc == 0) *(uint32_t *)(lds_wave + kExpOffset + 4 * row) = row < mv ? r.a[i].y : 0u;
        }
    } else {
        constexpr int kFull = T1 ? AV - 1 : AV;  // passes of four rows
#pragma unroll
        for (int i = 0; i < kFull; ++i) {
            const int row = 4 * i + (lane >> 4);
            const int e = row16_max(chunk_max_exp(r.a[i]));
            const int x = 142 - max(e, 1);
            if (row < mv) *(u32x4 *)(lds_wave + row * kARowBytes + kc * 16) = convert_chunk<BITS>(r.a[i], x);
            if (kc == 0) *(int *)(lds_wave + kExpOffset + 4 * row) = row < mv ? x : 0;
        }
        if constexpr (T1) {
            // the single-row pass: the row's largest exponent over all 64 lanes (DPP within
            // each 16-lane row, then the four rows' results), the same x and the same
            // per-value conversion as a full pass, one word per lane
            static_assert(BITS == 4, "the one-row pass follows the 4-bit operand order");
            const int row = 4 * (AV - 1);
            const uint32_t v = r.a[AV - 1].x;
            const int e16 = row16_max((int)max((v >> 7) & 0xFFu, (v >> 23) & 0xFFu));
            const int e = max(max(__builtin_amdgcn_readlane(e16, 0), __builtin_amdgcn_readlane(e16, 16)),
                              max(__builtin_amdgcn_readlane(e16, 32), __builtin_amdgcn_readlane(e16, 48)));
            const int x = 142 - max(e, 1);
            const float lo = ldexpf(__builtin_bit_cast(float, v << 16), x);
            const float hi = ldexpf(__builtin_bit_cast(float, v & 0xFFFF0000u), x);
            *(uint32_t *)(lds_wave + row * kARowBytes + (lane >> 2) * 16 + (lane & 3) * 4) = pack_h2(lo, hi);
            if (lane == 0) *(int *)(lds_wave + kExpOffset + 4 * row) = x;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's tile is complete
}

template <int AV, int BITS, bool A4, int RB>
__device__ __forceinline__ void compute_pipe(const GroupRegs<BITS> &r, const char *lds_wave, int mv, int lane,
                                             f32x4 (&acc)[RB][4])
{
    constexpr int kExpOffset = pipe_exp_offset(RB);
    const int c = lane & 15, kq = lane >> 4;
    // row tile rb of the block holds rows 16 rb .. 16 rb + 15; each unpacked weight operand
    // feeds the matrix-core step of every row tile
    f32x4 P[RB][4];
    if constexpr (BITS == 4) {
        uint32_t magic;
        asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
        uint32_t zlo[4], zhi[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t z = (r.z >> (8 * t)) & 0xFu;
            zlo[t] = (0xE400u | z) * 0x00010001u;         // -(1024 + z)
            zhi[t] = (0xD400u | (z << 4)) * 0x00010001u;  // -(64 + z)
            asm volatile("" : "+v"(zlo[t]), "+v"(zhi[t]));
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // rows mv.. of the tile are zero (cleared once, never staged)
            f16x8 a_op[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                a_op[rb] = __builtin_bit_cast(
                    f16x8, *(const u32x4 *)(lds_wave + (16 * rb + c) * kARowBytes + (4 * st + kq) * 16));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f16x8 b_op = unpack8(r.w[st][t], zlo[t], zhi[t], magic);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    // the first k-step starts from a literal zero accumulator (no register clearing)
                    const f32x4 c_in = st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[rb][t];
                    P[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op[rb], b_op, c_in, 0, 0, 0);
                }
            }
        }
    } else {
        uint32_t magic, sel01, sel23;
        asm("v_mov_b32 %0, 0x64646464" : "=v"(magic));
        asm("s_mov_b32 %0, 0x04010400" : "=s"(sel01));  // bytes: q0, 0x64, q1, 0x64
        asm("s_mov_b32 %0, 0x04030402" : "=s"(sel23));  // bytes: q2, 0x64, q3, 0x64
        uint32_t zneg[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t z = (r.z >> (8 * t)) & 0xFFu;
            zneg[t] = (0xE400u | z) * 0x00010001u;  // -(1024 + z)
            asm volatile("" : "+v"(zneg[t]));
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f16x8 a_op[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                a_op[rb] = __builtin_bit_cast(
                    f16x8, *(const u32x4 *)(lds_wave + (16 * rb + c) * kARowBytes + (4 * ks + kq) * 16));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f16x8 b_op = unpack8_w8(r.w[2 * ks][t], r.w[2 * ks + 1][t], zneg[t], magic, sel01, sel23);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const f32x4 c_in = ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[rb][t];
                    P[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op[rb], b_op, c_in, 0, 0, 0);
                }
            }
        }
    }
    if constexpr (A4) {
        // the group's partials are exact integers; each is scaled by its row's activation
        // scale times its column's weight scale
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f32x4 sa = *(const f32x4 *)(lds_wave + kExpOffset + 64 * rb + 16 * kq);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint16_t sb = (uint16_t)(r.s[t >> 1] >> (16 * (t & 1)));
                const float sv = (float)__builtin_bit_cast(_Float16, sb);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rb][t][i] = __builtin_fmaf(sv * sa[i], P[rb][t][i], acc[rb][t][i]);
            }
        }
    } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int4 xr = *(const int4 *)(lds_wave + kExpOffset + 64 * rb + 16 * kq);
            const int xs[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint16_t sb = (uint16_t)(r.s[t >> 1] >> (16 * (t & 1)));
                const float sv = (float)__builtin_bit_cast(_Float16, sb);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rb][t][i] = __builtin_fmaf(ldexpf(sv, -xs[i]), P[rb][t][i], acc[rb][t][i]);
            }
        }
    }
}

template <bool VEC, int WAVES, int AV, int OCC, int BITS, bool A4, int RB, bool T1>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void w4a16_kernel(const uint16_t *A, const uint32_t *Wq, const uint16_t *S, const uint8_t *Z, int M, int K, int N,
                  int splits, int groups_per_split, int full_tiles, SmallTail tail)
{
    constexpr int kRows = RB * kTileM;  // rows per block: one or two matrix-core row tiles
    constexpr int kExpOffset = pipe_exp_offset(RB);
    extern __shared__ __attribute__((aligned(16))) char lds[];  // per-wave tiles, then reduction
    __shared__ int s_last;
    SmallParams p;
    p.A = A;
    p.Wq = Wq;
    p.S = S;
    p.Z = Z;
    p.C = tail.C;
    p.part = tail.part;
    p.count = tail.count;
    p.As = tail.As;
    p.M = M;
    p.K = K;
    p.N = N;
    p.groups = K / kGroup;
    p.splits = splits;
    p.gps = groups_per_split;
    p.n_tiles = (N + kTileN - 1) / kTileN;
    p.m_blocks = (M + kRows - 1) / kRows;
    p.full_tiles = full_tiles;
    if constexpr (A4) asm volatile("" ::"s"(p.As));  // the one pointer needed early that is not preloaded

    // Tiles [0, full_tiles) run unsplit, one workgroup each; the other tiles are split
    // `splits` ways, and their parts are dispatched first: issued ahead of the whole tiles,
    // their loads are served first, so the parts and their handoff finish while the whole
    // tiles still stream (dispatched last, the parts were the last workgroups to finish:
    // 3584x37888 at M = 5 measured 18.24 -> 17.89 us, 1536x17920 at M = 1 7.39 -> 6.24 us).
    // The parts' range starts at workgroup 0, so the splits of one tile run on one XCD; the
    // whole tiles (independent of each other) follow, spread over the XCDs.
    const uint32_t nfull = (uint32_t)p.full_tiles;
    // the grid is nfull + nparts workgroups (computed here rather than read from the grid
    // size, a hidden argument the compiler fetches in a round trip of its own)
    const uint32_t nparts = ((uint32_t)p.m_blocks * (uint32_t)p.n_tiles - nfull) * (uint32_t)p.splits;
    uint32_t tile;
    int sp, gps;
    if (blockIdx.x >= nparts) {
        tile = xcd_local_id(blockIdx.x - nparts, nfull);
        sp = 0;
        gps = p.groups;
    } else {
        const uint32_t logical = xcd_local_id(blockIdx.x, nparts);
        tile = nfull + logical / (uint32_t)p.splits;
        sp = (int)(logical % (uint32_t)p.splits);
        gps = p.gps;
    }
    const bool split = tile >= nfull && p.splits > 1;
    // Row blocks of one column tile are consecutive tiles, so they run side by side on one
    // XCD and the second block's weight loads find the lines the first one brought in.
    const int mb = (int)(tile % (uint32_t)p.m_blocks);
    const int nt = (int)(tile / (uint32_t)p.m_blocks);
    const int n0 = nt * kTileN, m0 = mb * kRows;
    const int mv = (p.M - m0 < kRows) ? (int)(p.M - m0) : kRows;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
    const int c = lane & 15, kq = lane >> 4;

    const int g_begin = sp * gps;
    const int g_end = min(p.groups, g_begin + gps);
    const int g0 = g_begin + wave;
    const int n_my = g0 < g_end ? (g_end - g0 + WAVES - 1) / WAVES : 0;
    char *tile_lds = lds + wave * pipe_wave_bytes(RB);

    Resources rs;
    rs.W = __builtin_amdgcn_make_buffer_rsrc((void *)p.Wq, (short)0, (int)(p.K * BITS / 32 * p.N * 4), kRsrcWord3);
    rs.S = __builtin_amdgcn_make_buffer_rsrc((void *)p.S, (short)0, (int)(p.K / kGroup * p.N * 2), kRsrcWord3);
    rs.Z = __builtin_amdgcn_make_buffer_rsrc((void *)p.Z, (short)0, (int)(p.K / kGroup * p.N), kRsrcWord3);
    rs.A = __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)(A4 ? p.M * p.K / 2 : p.M * p.K * 2), kRsrcWord3);
    if constexpr (A4)
        rs.As = __builtin_amdgcn_make_buffer_rsrc((void *)p.As, (short)0, (int)(p.M * (p.K / kGroup) * 4), kRsrcWord3);
    LaneOffsets<VEC> lo;
    lane_offsets<VEC, BITS>(p, n0, lane, lo);
    uint32_t aoff[AV], asoff[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        int row = 4 * i + (lane >> 4);
        row = row < mv ? row : mv - 1;
        if constexpr (A4) {
            aoff[i] = (uint32_t)(((int64_t)(m0 + row) * (p.K / 8) + (lane & 15)) * 4);
            asoff[i] = (uint32_t)((int64_t)(m0 + row) * (p.K / kGroup) * 4);
        } else {
            aoff[i] = (uint32_t)(((int64_t)(m0 + row) * p.K + (lane & 15) * 8) * 2);
            asoff[i] = 0;
            if (T1 && i == AV - 1)  // the single-row pass: value 8 (l / 4) + l % 4 of row 4 (AV - 1)
                aoff[i] = (uint32_t)(((int64_t)(m0 + 4 * i) * p.K + (lane >> 2) * 8 + (lane & 3)) * 2);
        }
    }
    f32x4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Two register slots: group j+1 (its activations, then its weights) is in flight while
    // group j is converted and computed; unrolled by two with an exact tail, so every load is
    // issued once and none sits behind a branch.
    //
    // Issue priority by remaining work.  The SIMD favours older waves, so in a 12-wave
    // workgroup the four oldest waves finish their groups while the youngest four, their
    // loads long landed, wait to compute (per-wave timestamps on 18944x3584 at M = 5: first
    // group computed at ~2.7 us for waves 0-3, ~7 us for waves 8-11).  A wave with 3 or more
    // groups left takes priority 3, then 2 and 1 for its last two, so waves that end together
    // (at the workgroup's reduction) progress together.  Only for waves with long loops
    // (5 or more groups, the whole tiles of the wide shape) and the 12-wave shape: a split
    // part of a balanced plan must not yield to whole tiles, or its handoff ends last
    // (1536x17920 at M = 1: 6.26 -> 6.79 us with priority on every wave).  Measured: Qwen2.5-7B
    // M = 5 step 1.205 -> 1.192 ms, gamma sweep 4.365 -> 4.229 ms, 1.5B draft unchanged.
    const bool prio = n_my >= 5 || WAVES == 12;
    auto G = [&](int j) { return g0 + WAVES * j; };
    auto run_loop = [&]() {
        GroupRegs<BITS> w0, w1;
        ActRegs<AV, A4> a0, a1;
        auto load2 = [&](int j, GroupRegs<BITS> &w, ActRegs<AV, A4> &a) {
            load_act<AV, A4, T1>(rs, aoff, asoff, G(j), a);
            load_group<VEC, BITS>(p, rs, lo, G(j), w);
        };
        int left = n_my;
        auto run1 = [&](const GroupRegs<BITS> &w, const ActRegs<AV, A4> &a) {
            if (prio) {
                if (left >= 3) __builtin_amdgcn_s_setprio(3);
                else if (left == 2) __builtin_amdgcn_s_setprio(2);
                else __builtin_amdgcn_s_setprio(1);
            }
            --left;
            stage_pipe<AV, BITS, A4, RB, T1>(a, tile_lds, mv, lane);
            compute_pipe<AV, BITS, A4, RB>(w, tile_lds, mv, lane, acc);
        };
        load2(0, w0, a0);
        // the first group's loads go out before the wave's LDS set-up below (measured: qkv at
        // M = 5 7.39 -> 7.13 us, 1536x17920 at M = 1 6.34 -> 5.96 us)
        __builtin_amdgcn_sched_barrier(0);
        // rows mv.. of this wave's exponent table read as 0 (rows 4*AV.. are never staged, and
        // the single-row pass stages only its own row); rows mv.. of its activation tile are
        // never staged either: they read as 0 in the MFMAs
        if (lane >= mv && lane < kRows) *(int *)(tile_lds + kExpOffset + 4 * lane) = 0;
        for (int i = lane; i < (kRows - mv) * (kARowBytes / 16); i += kWave)
            *(u32x4 *)(tile_lds + mv * kARowBytes + i * 16) = u32x4{0u, 0u, 0u, 0u};
        int j = 0;
        for (; j + 2 < n_my; j += 2) {
            load2(j + 1, w1, a1);
            run1(w0, a0);
            load2(j + 2, w0, a0);
            run1(w1, a1);
        }
        if (j + 1 < n_my) {
            load2(j + 1, w1, a1);
            run1(w0, a0);
            run1(w1, a1);
        } else {
            run1(w0, a0);
        }
    };
    if (n_my > 0) run_loop();
    if (prio) __builtin_amdgcn_s_setprio(0);

    // Reduce the waves' accumulators through LDS in wave order (reproducible).
    __syncthreads();
    float *red = (float *)lds;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * kq + i;
            if (row < mv) {
                f32x4 v = {acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]};
                *(f32x4 *)(red + (wave * mv + row) * kTileN + 4 * c) = v;
            }
        }
    __syncthreads();
    // Each thread owns one 4-column quad of up to kPasses rows: 16 threads per row, so a
    // workgroup covers WAVES * 4 rows per pass.
    constexpr int kRowsPerPass = WAVES * 4;
    constexpr int kPasses = (kRows + kRowsPerPass - 1) / kRowsPerPass;
    const int row0 = threadIdx.x >> 4, quad = threadIdx.x & 15;
    f32x4 sum[kPasses];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int row = row0 + ps * kRowsPerPass;
        sum[ps] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < mv) {
            sum[ps] = *(const f32x4 *)(red + row * kTileN + 4 * quad);
#pragma unroll
            for (int w = 1; w < WAVES; ++w) sum[ps] += *(const f32x4 *)(red + (w * mv + row) * kTileN + 4 * quad);
        }
    }
    const int64_t col = n0 + 4 * quad;
    auto store_c = [&](int row, const f32x4 &v) {
        float *dst = p.C + (int64_t)(m0 + row) * p.N + col;
        if (VEC) {
            if (col < p.N) *(f32x4 *)dst = v;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (col + t < p.N) dst[t] = v[t];
        }
    };
    if (!split) {
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps)
            if (row0 + ps * kRowsPerPass < mv) store_c(row0 + ps * kRowsPerPass, sum[ps]);
        return;
    }
    // Split-K handoff.  Writer side: every split stores its partial tile with device-scope
    // stores (the ISA's sc1 scope bit: written through to the device coherence point, one
    // 16-byte store per lane and pass); each wave waits until its stores are complete, the
    // workgroup barrier then orders all of them before thread 0's increment of the tile's
    // arrival counter (agent scope).  Reader side: the workgroup whose increment returns
    // splits - 1 is the last arriver; it takes an agent-scope acquire fence (invalidating its
    // non-coherent cache lines, and no later load may be moved above it), its second barrier
    // orders that fence before all of its waves' loads of the partials (device-scope loads),
    // and it sums them in split order, writes C and resets the counter for the next call
    // (ordered by the kernel boundary).  A release fence at agent scope in every writer (an
    // L2 write-back per workgroup) measured 8% slower on the M = 5 verify step and adds
    // nothing for stores that already carry device scope.
    const uint32_t stile = tile - nfull;  // index among the split tiles
    const int64_t split_tiles = (int64_t)p.m_blocks * p.n_tiles - nfull;
    constexpr uint32_t kPartBytes = kRows * kTileN * 4;  // one split's partial tile
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)p.part, (short)0, (int)(split_tiles * p.splits * kPartBytes), kRsrcWord3);
    const uint32_t tile_part = (uint32_t)stile * (uint32_t)p.splits * kPartBytes;
    auto lane_part = [&](int row) { return tile_part + (uint32_t)(row * kTileN + 4 * quad) * 4; };
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int row = row0 + ps * kRowsPerPass;
        if (row < mv)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sum[ps]), prs,
                                                   lane_part(row) + (uint32_t)sp * kPartBytes, 0, kCacheCoherent);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(p.count + stile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(p.splits - 1));
        if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int row = row0 + ps * kRowsPerPass;
        if (row < mv) {
            // up to kBatch splits' partials in flight at once, summed in split order
            constexpr int kBatch = 8;
            f32x4 tot = {0.f, 0.f, 0.f, 0.f};
            for (int b = 0; b < p.splits; b += kBatch) {
                u32x4 v[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int s2 = b + i < p.splits ? b + i : p.splits - 1;  // clamped: no branch around loads
                    v[i] = __builtin_amdgcn_raw_buffer_load_b128(prs, lane_part(row) + (uint32_t)s2 * kPartBytes, 0,
                                                                 kCacheCoherent);
                }
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    if (b + i < p.splits) tot += __builtin_bit_cast(f32x4, v[i]);
            }
            store_c(row, tot);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.count + stile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------
// Narrow-tile kernel (M <= 16, activations small enough to stage whole in LDS): one
// workgroup per 16-column tile, over all of K, so narrow outputs fill the GPU without a
// K split across workgroups and without its handoff.
//  * Prologue: each wave issues the weight loads of all its groups (4-byte loads: lane
//    (c, kq) reads packed row 4 st + kq of column c, so 16 lanes read 64 contiguous bytes
//    per row), then the workgroup converts the whole activation block A[M, K] once into
//    LDS as binary16, each (row, group) scaled by its own power of two as in the small-M
//    kernel (one 16-lane DPP row per (row, group)), and stores the exponents beside it.
//  * Main loop: wave w computes groups w, w + WAVES, ...: per group four 16x16x32 f16
//    matrix-core steps with the lane's unpacked word as B operand and A from LDS (rows
//    M.. read a zero chunk), then the float32 rescale by ldexp(s, -x).
//  * The waves' partial sums are added through LDS in wave order and written to C.
// Neighbouring tiles run on one XCD, so the two halves of each 128-byte line of a packed
// row are read through the same L2.

constexpr int kNarrowN = 16;  // output columns per workgroup
constexpr int kNarrowMaxGroups = 8;  // groups per wave held in registers at once

struct NarrowParams {
    const uint16_t *A;
    const uint32_t *Wq;
    const uint16_t *S;
    const uint8_t *Z;
    float *C;
    int64_t M, K, N;
    int groups;
    int n_tiles;
};

// LDS layout of the narrow kernel: activation rows [groups][M][kARowBytes] (binary16, row
// pitch padded for conflict-free reads), one zero chunk, then the exponents [groups][16].
__host__ __device__ constexpr int narrow_zero_offset(int groups, int M) { return groups * M * kARowBytes; }
__host__ __device__ constexpr int narrow_exp_offset(int groups, int M) { return groups * M * kARowBytes + 16; }
__host__ __device__ constexpr int narrow_lds_bytes(int groups, int M, int waves)
{
    const int stage = narrow_exp_offset(groups, M) + groups * kTileM * 4;
    const int red = waves * M * kNarrowN * 4;
    return stage > red ? stage : red;
}

template <int BITS>
struct NarrowW {
    uint32_t w[BITS];  // the lane's column in packed rows: 4-bit 4 st + kq (st = 0..3);
                       // 8-bit 8 (st / 2) + 2 kq + st % 2 (st = 0..7)
    uint32_t s;        // binary16 scale (low half)
    uint32_t z;        // zero byte
};

template <int WAVES, int BITS>
__global__ __launch_bounds__(WAVES * kWave) void w4a16_narrow_kernel(const uint16_t *A, const uint32_t *Wq,
                                                                      const uint16_t *S, const uint8_t *Z, float *C,
                                                                      int M_, int K_, int N_, int groups)
{
    // 14 dwords of arguments, all preloaded into scalar registers at wave launch; the grid
    // (one workgroup per tile) is derived from N rather than read from a hidden argument
    extern __shared__ __attribute__((aligned(16))) char lds[];
    NarrowParams p;
    p.A = A;
    p.Wq = Wq;
    p.S = S;
    p.Z = Z;
    p.C = C;
    p.M = M_;
    p.K = K_;
    p.N = N_;
    p.groups = groups;
    p.n_tiles = (N_ + kNarrowN - 1) / kNarrowN;
    const int tile = (int)xcd_local_id(blockIdx.x, (uint32_t)p.n_tiles);
    const int n0 = tile * kNarrowN;
    const int M = (int)p.M, G = p.groups;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, kq = lane >> 4;
    const int64_t N = p.N;
    const int64_t nc = n0 + c < N ? n0 + c : N - 1;  // clamped column for loads

    Resources rs;
    rs.W = __builtin_amdgcn_make_buffer_rsrc((void *)p.Wq, (short)0, (int)(p.K * BITS / 32 * N * 4), kRsrcWord3);
    rs.S = __builtin_amdgcn_make_buffer_rsrc((void *)p.S, (short)0, (int)(p.K / kGroup * N * 2), kRsrcWord3);
    rs.Z = __builtin_amdgcn_make_buffer_rsrc((void *)p.Z, (short)0, (int)(p.K / kGroup * N), kRsrcWord3);
    rs.A = __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)(p.M * p.K * 2), kRsrcWord3);
    // packed rows of the lane's first word: kq (4-bit) or 2 kq (8-bit)
    const uint32_t woff = (uint32_t)(((int64_t)(BITS == 4 ? kq : 2 * kq) * N + nc) * 4);
    const uint32_t rowbytes = (uint32_t)N * 4;

    const int n_my = wave < G ? (G - wave + WAVES - 1) / WAVES : 0;
    auto load_w = [&](int g, NarrowW<BITS> &r) {
#pragma unroll
        for (int st = 0; st < BITS; ++st) {
            const int row = BITS == 4 ? g * 16 + 4 * st : g * 32 + 8 * (st >> 1) + (st & 1);
            r.w[st] = __builtin_amdgcn_raw_buffer_load_b32(rs.W, woff, (uint32_t)row * rowbytes, kCacheStream);
        }
        r.s = __builtin_amdgcn_raw_buffer_load_b16(rs.S, (uint32_t)(nc * 2), (uint32_t)g * (uint32_t)N * 2, 0);
        r.z = __builtin_amdgcn_raw_buffer_load_b8(rs.Z, (uint32_t)nc, (uint32_t)g * (uint32_t)N, 0);
    };

    // Stage A: pair q = g * M + m is (row m, group g); DPP row d of the workgroup takes
    // pairs d, d + 4 WAVES, ...  Lane kc of a DPP row holds values 8 kc .. 8 kc + 7.
    const int pairs = G * M;
    const int dpp_rows = 4 * WAVES;
    const int drow = threadIdx.x >> 4, kc = lane & 15;
    // q = g * M + m split without an integer division: q < 16 * 64 (the plan keeps M <= 16
    // and at most 64 groups), (q + 0.5) * inv_m in float32 is within 2^-22 of (q + 0.5) / M,
    // and that quotient's fraction is at least 1/(2M) >= 1/32 away from an integer, so the
    // truncation gives g exactly
    const float inv_m = 1.0f / (float)M;
    auto split_q = [&](int q, int &g, int &m) {
        g = (int)(((float)q + 0.5f) * inv_m);
        m = q - g * M;
    };
    auto stage_pass = [&](int q0, const u32x4 &v) {
        const int q = q0 + drow;
        const int e = row16_max(chunk_max_exp(v));
        const int x = 142 - max(e, 1);
        const u32x4 h = convert_chunk<BITS>(v, x);
        if (q < pairs) {
            *(u32x4 *)(lds + q * kARowBytes + kc * 16) = h;
            if (kc == 0) {
                int g, m;
                split_q(q, g, m);
                *(int *)(lds + narrow_exp_offset(G, M) + (g * kTileM + m) * 4) = x;
            }
        }
    };
    auto load_a = [&](int q0) {
        int q = q0 + drow;
        q = q < pairs ? q : pairs - 1;  // clamped: no branch around the load
        int g, m;
        split_q(q, g, m);
        return __builtin_amdgcn_raw_buffer_load_b128(rs.A, (uint32_t)(((int64_t)m * p.K + g * kGroup + kc * 8) * 2), 0, 0);
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int zero_off = narrow_zero_offset(G, M);
    const int a_lane = c < M ? c * kARowBytes + kq * 16 : -1;  // -1: a row past M
    auto compute = [&](int g, const NarrowW<BITS> &r) {
        const int gbase = g * M * kARowBytes;
        f32x4 P;
        if constexpr (BITS == 4) {
            uint32_t magic;
            asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
            const uint32_t z = r.z & 0xFu;
            uint32_t zlo = (0xE400u | z) * 0x00010001u, zhi = (0xD400u | (z << 4)) * 0x00010001u;
            asm volatile("" : "+v"(zlo), "+v"(zhi));
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int ao = a_lane >= 0 ? gbase + a_lane + st * 64 : zero_off;
                const f16x8 a_op = __builtin_bit_cast(f16x8, *(const u32x4 *)(lds + ao));
                const f16x8 b_op = unpack8(r.w[st], zlo, zhi, magic);
                P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op, b_op, st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P, 0, 0, 0);
            }
        } else {
            uint32_t magic, sel01, sel23;
            asm("v_mov_b32 %0, 0x64646464" : "=v"(magic));
            asm("s_mov_b32 %0, 0x04010400" : "=s"(sel01));  // bytes: q0, 0x64, q1, 0x64
            asm("s_mov_b32 %0, 0x04030402" : "=s"(sel23));  // bytes: q2, 0x64, q3, 0x64
            uint32_t zneg = (0xE400u | (r.z & 0xFFu)) * 0x00010001u;  // -(1024 + z)
            asm volatile("" : "+v"(zneg));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int ao = a_lane >= 0 ? gbase + a_lane + ks * 64 : zero_off;
                const f16x8 a_op = __builtin_bit_cast(f16x8, *(const u32x4 *)(lds + ao));
                const f16x8 b_op = unpack8_w8(r.w[2 * ks], r.w[2 * ks + 1], zneg, magic, sel01, sel23);
                P = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op, b_op, ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P, 0, 0, 0);
            }
        }
        const int4 xr = *(const int4 *)(lds + narrow_exp_offset(G, M) + (g * kTileM + 4 * kq) * 4);
        const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)r.s);
        acc[0] = __builtin_fmaf(ldexpf(sv, -xr.x), P[0], acc[0]);
        acc[1] = __builtin_fmaf(ldexpf(sv, -xr.y), P[1], acc[1]);
        acc[2] = __builtin_fmaf(ldexpf(sv, -xr.z), P[2], acc[2]);
        acc[3] = __builtin_fmaf(ldexpf(sv, -xr.w), P[3], acc[3]);
    };

    // Every weight load of the wave's first kNarrowMaxGroups groups first (the plan keeps a
    // wave's groups within that), then the activation staging while they are in flight, then
    // the groups; any further groups are loaded and computed one at a time.
    auto run = [&](auto kconst) {
        constexpr int KG = decltype(kconst)::value;
        NarrowW<BITS> wr[KG > 0 ? KG : 1];
        // the first passes' activation loads come before the weights: loads complete in
        // issue order, so the staging below then overlaps the weight stream
        constexpr int kPre = 5;
        u32x4 va[kPre];
#pragma unroll
        for (int b = 0; b < kPre; ++b) va[b] = load_a(b * dpp_rows);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KG; ++u) {
            load_w(wave + WAVES * u, wr[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // exponents of rows M.. are 0 (their activation rows read the zero chunk); zero chunk.
        // Written after the loads are issued (1536x2048 at M = 1: 3.53 -> 3.47 us).
        for (int i = threadIdx.x; i < G * kTileM; i += WAVES * kWave)
            if (i % kTileM >= M) *(int *)(lds + narrow_exp_offset(G, M) + 4 * i) = 0;
        if (threadIdx.x == 0) *(u32x4 *)(lds + narrow_zero_offset(G, M)) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < kPre; ++b)
            if (b * dpp_rows < pairs) stage_pass(b * dpp_rows, va[b]);
        // any further passes (large M * K): batches of 4, the loads of a batch together
        for (int q0 = kPre * dpp_rows; q0 < pairs; q0 += 4 * dpp_rows) {
            u32x4 v[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) v[b] = load_a(q0 + b * dpp_rows);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (q0 + b * dpp_rows < pairs) stage_pass(q0 + b * dpp_rows, v[b]);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < KG; ++u) compute(wave + WAVES * u, wr[u]);
    };
    switch (n_my) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 4: run(std::integral_constant<int, 4>{}); break;
    case 5: run(std::integral_constant<int, 5>{}); break;
    case 6: run(std::integral_constant<int, 6>{}); break;
    case 7: run(std::integral_constant<int, 7>{}); break;
    default: run(std::integral_constant<int, kNarrowMaxGroups>{}); break;
    }
    for (int u = kNarrowMaxGroups; u < n_my; ++u) {
        NarrowW<BITS> r;
        load_w(wave + WAVES * u, r);
        compute(wave + WAVES * u, r);
    }

    // Reduce the waves' sums in wave order (reproducible) and write C.
    __syncthreads();
    float *red = (float *)lds;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * kq + i;
        if (row < M) red[(wave * M + row) * kNarrowN + c] = acc[i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < M * kNarrowN; e += WAVES * kWave) {
        const int row = e / kNarrowN, col = e % kNarrowN;
        float sum = red[row * kNarrowN + col];
        for (int w = 1; w < WAVES; ++w) sum += red[(w * M + row) * kNarrowN + col];
        if (n0 + col < N) p.C[(int64_t)row * N + n0 + col] = sum;
    }
}

// ------------------------------------------------------------------------------------
// Large-M kernel (batched verify: M >= 64, and large GEMMs from M = 17): a dense
// contraction on the bfloat16 matrix cores (v_mfma_f32_32x32x16_bf16).  A workgroup owns
// a row block of up to RT*32 rows and 256 columns; each of its 8 waves owns 32 columns,
// one per lane pair (lane l holds column l % 32 and k-half l / 32 of every B operand), so
// every weight is loaded and dequantized once per workgroup and reused by all RT row tiles.
//
// (q - z) is formed exactly in bfloat16: the codes of a word are biased into bytes
// (0x80 | q) so that subtracting z cannot borrow across bytes, the bias is removed with
// one xor, and each signed byte is converted int -> float -> bfloat16, all exact for
// |q - z| <= 15.  Products on the matrix cores are then exact, and each group's float32
// partial is rescaled by the fp16 scale once per output.
//
// Software pipeline per wave: weights are loaded two groups ahead; while group g's MFMAs
// run, the next group's words are dequantized and the previous row tile's partials are
// rescaled, so the VALU work interleaves with matrix-core work instead of forming a phase
// of its own.  The activations of a group (rows x 128 bfloat16) are staged in LDS by the
// whole workgroup, double-buffered, one barrier per group.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLWaves = 8;
constexpr int kLTileN = kLWaves * 32;  // 256 columns per workgroup
constexpr int kLMaxRT = 5;             // 32 to 160 rows per workgroup (row tiles of 32)
constexpr int kLargeSharedMaxRT = 2;   // most row tiles of a workgroup that may hold two tiles' steps
constexpr int kLThreads = kLWaves * kWave;

struct LargeParams {
    const uint16_t *A;
    const uint32_t *Wq;
    const uint16_t *S;
    const uint8_t *Z;
    float *C;
    float *part;        // [splits][stride] float32 partial products (split-K only)
    int64_t stride;     // floats per split slice: M * N rounded up to a multiple of 4
    int64_t M, K, N;
    int groups, splits, gps, n_tiles, m_blocks;
    int block_rows;     // rows per row block (<= RT * 32)
};

// The large-M kernel's arguments: the 14 dwords every wave needs before its first load
// (preloaded into scalar registers at wave launch; the tile count follows from N), then the
// output side as a struct.
struct LargeTail {
    float *C;
    float *part;
    int64_t stride;
};

__device__ __forceinline__ uint32_t pack_bf2(float a, float b)
{
    bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight codes of one packed word -> eight exact bfloat16 values (q_j - z), j = 0..7 in k
// order.  zz holds z in each of its four bytes.
__device__ __forceinline__ bf16x8 unpack8_bf16(uint32_t w, uint32_t zz)
{
    const uint32_t ev = (((w & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;         // q0 q2 q4 q6
    const uint32_t od = ((((w >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;  // q1 q3 q5 q7
    const float d0 = (float)(int8_t)ev, d2 = (float)(int8_t)(ev >> 8);
    const float d4 = (float)(int8_t)(ev >> 16), d6 = (float)(int8_t)(ev >> 24);
    const float d1 = (float)(int8_t)od, d3 = (float)(int8_t)(od >> 8);
    const float d5 = (float)(int8_t)(od >> 16), d7 = (float)(int8_t)(od >> 24);
    const u32x4 r = {pack_bf2(d0, d1), pack_bf2(d2, d3), pack_bf2(d4, d5), pack_bf2(d6, d7)};
    return __builtin_bit_cast(bf16x8, r);
}

// unpack8_bf16 in five pieces of 3-4 VALU operations each, so that a word's dequantization
// can be spread over five matrix-core steps (piece 4 completes r).  Interleaved this way the
// VALU work overlaps the matrix cores far better than in bursts of ~19 operations.
struct Unpack8 {
    uint32_t ev, od, t;
    float d0;
    u32x4 r;
};
// Each piece's results are pinned where the piece stands: without that, the compiler sinks
// the arithmetic to the first use and the pieces bunch up again.
__device__ __forceinline__ void unpack8_piece(int piece, Unpack8 &u, uint32_t w, uint32_t zz)
{
    switch (piece) {
    case 0:
        u.ev = (((w & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;  // q0 q2 q4 q6
        u.t = w >> 4;
        asm volatile("" : "+v"(u.ev), "+v"(u.t));
        break;
    case 1:
        u.od = (((u.t & 0x0F0F0F0Fu) | 0x80808080u) - zz) ^ 0x80808080u;  // q1 q3 q5 q7
        u.d0 = (float)(int8_t)u.ev;
        asm volatile("" : "+v"(u.od), "+v"(u.d0));
        break;
    case 2:
        u.r[0] = pack_bf2(u.d0, (float)(int8_t)u.od);
        u.r[1] = pack_bf2((float)(int8_t)(u.ev >> 8), (float)(int8_t)(u.od >> 8));
        asm volatile("" : "+v"(u.r[0]), "+v"(u.r[1]));
        break;
    case 3:
        u.r[2] = pack_bf2((float)(int8_t)(u.ev >> 16), (float)(int8_t)(u.od >> 16));
        asm volatile("" : "+v"(u.r[2]));
        break;
    default:
        u.r[3] = pack_bf2((float)(int8_t)(u.ev >> 24), (float)(int8_t)(u.od >> 24));
        asm volatile("" : "+v"(u.r[3]));
        break;
    }
}

// Order of a large-M workgroup's RT * 8 MFMA steps per group: row tiles in segments of one
// or two (RT = 2: {0,1}; 3: {0} {1,2}; 4: {0,1} {2,3}; 1 and 5: one tile per segment, five
// need the registers a second chain would take); within a segment of two the tiles
// alternate per k-step.
template <int RT> __host__ __device__ constexpr int large_segments() { return RT == 2 ? 1 : RT == 3 || RT == 4 ? 2 : RT; }
template <int RT> __host__ __device__ constexpr int large_seg_first(int sg)
{
    return RT == 2 ? 0 : RT == 3 ? (sg == 0 ? 0 : 1) : RT == 4 ? 2 * sg : sg;
}
template <int RT> __host__ __device__ constexpr int large_seg_count(int sg)
{
    return RT == 2 ? 2 : RT == 3 ? (sg == 0 ? 1 : 2) : RT == 4 ? 2 : 1;
}
template <int RT> __host__ __device__ constexpr int large_step_rt(int n)
{
    if (RT == 2) return n & 1;
    if (RT == 3) return n < 8 ? 0 : 1 + ((n - 8) & 1);
    if (RT == 4) return 2 * (n / 16) + (n & 1);
    return n >> 3;
}
template <int RT> __host__ __device__ constexpr int large_step_ks(int n)
{
    if (RT == 2) return n >> 1;
    if (RT == 3) return n < 8 ? n : (n - 8) >> 1;
    if (RT == 4) return (n % 16) >> 1;
    return n & 7;
}

// One group's packed words for the lane's column: word ks holds k = 16 ks + 8 h .. + 7.
struct LargeW {
    uint32_t w[8];
    uint32_t s;   // binary16 scale (low half)
    uint32_t z;   // zero byte
};

// SH: plans with shared steps (a workgroup may hold two tiles' steps; blocks of up to
// kLargeSharedMaxRT row tiles).  Without it a workgroup holds one segment, and the kernel has
// the register use and schedule of one without the segment loop.
template <int RT, bool SH>
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w4a16_mfma_kernel(const uint16_t *A, const uint32_t *Wq, const uint16_t *S, const uint8_t *Z, int M_, int K_,
                       int N_, int groups_per_split, int group_stride, int block_rows, LargeTail tail)
{
    static_assert(!SH || RT <= kLargeSharedMaxRT, "shared steps: blocks of up to two row tiles");
    constexpr int kRows = RT * 32;
    constexpr int kBuf = kRows * kARowBytes;
    constexpr int kAChunks = kRows * kChunksPerRow / kLThreads;  // == RT: one per row tile
    static_assert(kRows * kChunksPerRow % kLThreads == 0, "staging must tile the block");
    constexpr int kSteps = RT * 8;  // MFMAs per group per wave
    __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];
    LargeParams p;
    p.A = A;
    p.Wq = Wq;
    p.S = S;
    p.Z = Z;
    p.C = tail.C;
    p.part = tail.part;
    p.stride = tail.stride;
    p.M = M_;
    p.K = K_;
    p.N = N_;
    p.groups = K_ / kGroup;
    p.splits = 0;  // not used by the kernel
    p.gps = groups_per_split;
    p.n_tiles = (N_ + kLTileN - 1) / kLTileN;
    p.m_blocks = SH ? (M_ + block_rows - 1) / block_rows : 0;  // (not needed otherwise)
    p.block_rows = block_rows;

    const int64_t N = p.N;

    Resources rs;
    rs.W = __builtin_amdgcn_make_buffer_rsrc((void *)p.Wq, (short)0, (int)(p.K / 8 * N * 4), kRsrcWord3);
    rs.S = __builtin_amdgcn_make_buffer_rsrc((void *)p.S, (short)0, (int)(p.K / kGroup * N * 2), kRsrcWord3);
    rs.Z = __builtin_amdgcn_make_buffer_rsrc((void *)p.Z, (short)0, (int)(p.K / kGroup * N), kRsrcWord3);
    rs.A = __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)(p.M * p.K * 2), kRsrcWord3);
    const uint32_t rowbytes = (uint32_t)N * 4;

    // Work assignment.  The (tile, group) steps are numbered tile-major, tile t (row block
    // t / n_tiles, column tile t % n_tiles) owning steps t * group_stride .. + groups - 1
    // (group_stride >= groups; numbers past a tile's groups are skipped).  Workgroup w takes
    // steps w * groups_per_split .. + groups_per_split - 1: with group_stride = splits *
    // groups_per_split that is one tile's split, with group_stride = groups the workgroups
    // share out all the steps evenly and one may finish a tile and go on to the next.  Each
    // piece of a tile (a segment) is accumulated on its own; a segment covering the whole
    // tile goes to C, any other to the partial-product slice numbered by the workgroup's
    // place among the tile's workgroups (w - floor(t * group_stride / groups_per_split)).
    // Without shared steps (group_stride = splits * gps, checked on the host) a workgroup's
    // steps lie in one tile, so neither the step count nor the end of the range is needed
    // (one division less on the way to the first loads).
    constexpr bool kShared = SH;
    const uint32_t total = kShared ? (uint32_t)p.m_blocks * (uint32_t)p.n_tiles * (uint32_t)group_stride : 0u;
    uint32_t u = blockIdx.x * (uint32_t)p.gps;
    const uint32_t u_end = u + (uint32_t)p.gps < total ? u + (uint32_t)p.gps : total;
    for (;;) {
        // (uniform values: the divisions run on the vector unit, so their results are moved
        // back to scalar registers)
        const uint32_t tile = __builtin_amdgcn_readfirstlane(u / (uint32_t)group_stride);
        const int g_begin = (int)(u - tile * (uint32_t)group_stride);
        int g_stop = g_begin + p.gps;
        if constexpr (kShared)
            g_stop = g_begin + (int)(u_end - u) < group_stride ? g_begin + (int)(u_end - u) : group_stride;
        const int g_end = min(p.groups, g_stop);
        const int slot = __builtin_amdgcn_readfirstlane(blockIdx.x - tile * (uint32_t)group_stride / (uint32_t)p.gps);
        const int nt = __builtin_amdgcn_readfirstlane(tile % (uint32_t)p.n_tiles);
        const int mb = __builtin_amdgcn_readfirstlane(tile / (uint32_t)p.n_tiles);
        // Lane constants are derived anew in each segment: hoisted out of this loop they
        // would stay live through the group loop and cost it registers.
        uint32_t tid = threadIdx.x;
        if constexpr (kShared) asm volatile("" : "+v"(tid));
        const int lane = (int)(tid & 63);
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int c = lane & 31, h = lane >> 5;
        const int64_t m0 = (int64_t)mb * p.block_rows;
        const int64_t m_end = m0 + p.block_rows < p.M ? m0 + p.block_rows : p.M;
        const int64_t col = (int64_t)nt * kLTileN + wave * 32 + c;
        const int64_t colc = col < N ? col : N - 1;
        const uint32_t woff = (uint32_t)((h * N + colc) * 4);
        const uint32_t soff = (uint32_t)(colc * 2), zoff = (uint32_t)colc;

        // Activation staging: chunk id = thread + 512 j is (row id / 16, 16-byte chunk id % 16)
        // of the group; rows outside the block read row m_end - 1 (never stored).
        uint32_t aoff[kAChunks];
        int alds[kAChunks];
#pragma unroll
        for (int j = 0; j < kAChunks; ++j) {
            const int id = (int)tid + kLThreads * j;
            const int row = id >> 4, kc = id & 15;
            const int64_t srow = m0 + row < m_end ? m0 + row : m_end - 1;
            aoff[j] = (uint32_t)((srow * p.K + kc * 8) * 2);
            alds[j] = row * kARowBytes + kc * 16;
        }
        auto load_a = [&](int g, u32x4 (&ar)[kAChunks]) {
#pragma unroll
            for (int j = 0; j < kAChunks; ++j) ar[j] = __builtin_amdgcn_raw_buffer_load_b128(rs.A, aoff[j], (uint32_t)g * (kGroup * 2), 0);
        };
        auto store_a = [&](int buf, const u32x4 (&ar)[kAChunks]) {
#pragma unroll
            for (int j = 0; j < kAChunks; ++j) *(u32x4 *)(lds + buf * kBuf + alds[j]) = ar[j];
        };
        auto load_w = [&](int g, LargeW &r) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                r.w[ks] = __builtin_amdgcn_raw_buffer_load_b32(rs.W, woff, ((uint32_t)g * 16 + 2 * ks) * rowbytes, kCacheStream);
            r.s = __builtin_amdgcn_raw_buffer_load_b16(rs.S, soff, (uint32_t)g * (uint32_t)N * 2, 0);
            r.z = __builtin_amdgcn_raw_buffer_load_b8(rs.Z, zoff, (uint32_t)g * (uint32_t)N, 0);
        };
        auto scale_of = [](const LargeW &r) { return (float)__builtin_bit_cast(_Float16, (uint16_t)r.s); };

        f32x16 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rt][v] = 0.f;

        // A operand of (row tile rt, k-step ks): row rt*32 + c, k = 16 ks + 8 h .. + 7
        const int a_lane = c * kARowBytes + h * 16;

        // Two register sets for packed weights (X, Y) and two for dequantized operands (B0, B1)
        // alternate between consecutive groups (the loop is unrolled by two), so no register
        // set is ever copied: a copy would make the compiler wait for in-flight loads early.
        u32x4 ar[kAChunks];
        LargeW wx, wy;
        bf16x8 B0[8], B1[8];
        float sc0, sc1;

        // One group: MFMAs on Bc (group g), dequantize Wn (group g + 1) into Bn, load group
        // g + 2's weights into Wl and group g + 1's activations into ar.
        auto group_step = [&](int g, LargeW &Wn, LargeW &Wl, const bf16x8 (&Bc)[8], bf16x8 (&Bn)[8],
                              float sc, float &scn) {
            const int buf = (g - g_begin) & 1;
            const int gn1 = g + 1 < g_end ? g + 1 : g;  // clamped: the tail reloads, no branch
            const int gn2 = g + 2 < g_end ? g + 2 : gn1;
            load_a(gn1, ar);
            load_w(gn2, Wl);
            __builtin_amdgcn_sched_barrier(0);
            // Pin this group's dequantization inside this group: without it the compiler may
            // hoist it into the previous group, where it would wait for loads just issued.
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(Wn.w[ks]));
            asm volatile("" : "+v"(Wn.z), "+v"(Wn.s));

            const char *abase = lds + buf * kBuf + a_lane;
            const uint32_t zzn = (Wn.z & 0xFu) * 0x01010101u;
            constexpr int kAhead = 2;  // A operands read two MFMA steps ahead
            bf16x8 ring[kAhead + 1];
            auto a_at = [&](int n) {
                return *(const bf16x8 *)(abase + large_step_rt<RT>(n) * 32 * kARowBytes + large_step_ks<RT>(n) * 32);
            };
#pragma unroll
            for (int i = 0; i < kAhead; ++i) ring[i] = a_at(i);
            // MFMA step n runs (row tile, k-step) = (large_step_rt, large_step_ks): the row tiles
            // go in segments of one or two, and a segment of two interleaves its tiles' chains
            // per k-step (two independent accumulation chains hide each other's MFMA latency).
            // After each MFMA an even share of the VALU work: word n / RT's dequantization in
            // pieces over RT steps, and, from the segment's second step on, the rescale of the
            // previous segment's row tiles.  A scheduling barrier after each step keeps this
            // order.  Row tile rt accumulates in chain rt % 2 and is rescaled from Q[rt % 2].
            Unpack8 u;
            f32x16 P[2], Q[2];
#pragma unroll
            for (int sg = 0; sg < large_segments<RT>(); ++sg) {
                const int r0 = large_seg_first<RT>(sg), cnt = large_seg_count<RT>(sg);
                const int base = 8 * r0, len = 8 * cnt;
                const int pr0 = sg > 0 ? large_seg_first<RT>(sg - 1) : 0;
                const int pending = sg > 0 ? 16 * large_seg_count<RT>(sg - 1) : 0;
#pragma unroll
                for (int i = 0; i < len; ++i) {
                    const int n = base + i;
                    const int rt = large_step_rt<RT>(n), ks = large_step_ks<RT>(n);
                    if (n + kAhead < kSteps) ring[(n + kAhead) % (kAhead + 1)] = a_at(n + kAhead);
                    const bf16x8 a = ring[n % (kAhead + 1)];
                    f32x16 &Pc = P[rt & 1];
                    if (ks == 0) {
                        const f32x16 zero = {};
                        Pc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Bc[ks], zero, 0, 0, 0);
                    } else {
                        Pc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Bc[ks], Pc, 0, 0, 0);
                    }
                    const int word = n / RT, l = n % RT;
#pragma unroll
                    for (int pc = l * 5 / RT; pc < (l + 1) * 5 / RT; ++pc) unpack8_piece(pc, u, Wn.w[word], zzn);
                    if (l == RT - 1) Bn[word] = __builtin_bit_cast(bf16x8, u.r);
                    // the previous segment's partials, spread over steps 1 .. len - 1
                    if (pending > 0 && i > 0) {
                        const int f0 = (i - 1) * pending / (len - 1), f1 = i * pending / (len - 1);
#pragma unroll
                        for (int f = f0; f < f1; ++f) {
                            const int tr = pr0 + f / 16, v = f % 16;
                            acc[tr][v] = __builtin_fmaf(sc, Q[tr & 1][v], acc[tr][v]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int c = 0; c < cnt; ++c) {
                    Q[(r0 + c) & 1] = P[(r0 + c) & 1];
                    // stage one chunk of the next group's activations per row tile, so the LDS
                    // writes spread over the group instead of queueing behind its reads at the end
                    *(u32x4 *)(lds + (buf ^ 1) * kBuf + alds[r0 + c]) = ar[r0 + c];
                }
            }
            scn = scale_of(Wn);
            // ... and keep it from sinking into the next group: the operands are complete here.
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(Bn[ks]));
            // The barrier comes as soon as this wave's LDS traffic for the group is done; the
            // last row tile's rescale (which waits for its MFMAs) follows it.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            {
                constexpr int last = large_segments<RT>() - 1;
                const int r0 = large_seg_first<RT>(last), cnt = large_seg_count<RT>(last);
#pragma unroll
                for (int c = 0; c < cnt; ++c)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[r0 + c][v] = __builtin_fmaf(sc, Q[(r0 + c) & 1][v], acc[r0 + c][v]);
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        load_a(g_begin, ar);
        load_w(g_begin, wy);
        load_w(g_begin + 1 < g_end ? g_begin + 1 : g_begin, wx);
        {
            const uint32_t zz = (wy.z & 0xFu) * 0x01010101u;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) B0[ks] = unpack8_bf16(wy.w[ks], zz);
            sc0 = scale_of(wy);
        }
        store_a(0, ar);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int g = g_begin; g < g_end; g += 2) {
            group_step(g, wx, wy, B0, B1, sc0, sc1);
            if (g + 1 >= g_end) break;
            group_step(g + 1, wy, wx, B1, B0, sc1, sc0);
        }

        // Lane holds column col and rows rt*32 + 8 (v / 4) + 4 h + v % 4 of the block.  A
        // segment of the whole tile writes C; any other writes its partial product to its slice
        // of the [M, N] partials, and a second launch (w4a16_split_reduce where every tile is
        // split alike, else w4a16_tile_reduce) adds each tile's slices in workgroup order (the
        // kernel boundary orders the two).
        if (g_begin == 0 && g_end == p.groups) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = m0 + rt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (row < m_end && col < N) p.C[row * N + col] = acc[rt][v];
                }
        } else {
            // partial products are read once, by the reduction launch: non-temporal stores
            // (and loads there) keep them from displacing cached lines (Qwen2.5-7B M=40 step
            // 2.162 -> 2.128 ms with the stores; with the loads as well M=160 4.505 -> 4.357,
            // M=80 3.028 -> 2.946, M=40 2.129 -> 2.114)
            float *out = p.part + (int64_t)slot * p.stride;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = m0 + rt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    const float e = acc[rt][v];
                    if (row < m_end && col < N) __builtin_nontemporal_store(e, out + row * N + col);
                }
        }
        // without shared steps the workgroup holds one segment
        if constexpr (!kShared) break;
        u += (uint32_t)(g_stop - g_begin);
        if (u >= u_end) break;
    }
}

// Sums the split-K partial products in split order: C[i] = sum_s part[s * stride + i],
// four consecutive elements per thread (slices are 16-byte aligned: stride % 4 == 0); the
// last total % 4 elements are done by the first threads of workgroup 0.
__global__ __launch_bounds__(256) void w4a16_split_reduce(const float *__restrict__ part, float *__restrict__ C,
                                                          int64_t total, int64_t stride, int splits)
{
    const int64_t n4 = total / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        f32x4 acc = __builtin_nontemporal_load((const f32x4 *)(part + 4 * i));
        // unrolled so that the loads run ahead of the (ordered) additions: 17 slices at M=40
        // 5.5 -> 4.4 us; with the non-temporal loads also for few slices (M=80 step 2.957 ->
        // 2.890 ms, M=160 4.248 -> 4.227)
#pragma unroll 4
        for (int s2 = 1; s2 < splits; ++s2) acc += __builtin_nontemporal_load((const f32x4 *)(part + (int64_t)s2 * stride + 4 * i));
        *(f32x4 *)(C + 4 * i) = acc;
    }
    if (blockIdx.x == 0 && threadIdx.x < total - 4 * n4) {
        const int64_t e = 4 * n4 + threadIdx.x;
        float acc = part[e];
        for (int s2 = 1; s2 < splits; ++s2) acc += part[(int64_t)s2 * stride + e];
        C[e] = acc;
    }
}

// Adds each output tile's partial products in workgroup order.  Tile t (row block
// t / n_tiles, column tile t % n_tiles) owns the steps a = t * group_stride .. a + groups - 1
// of the large-M kernel's numbering, so workgroups floor(a / gps) .. floor((a + groups - 1)
// / gps) wrote its partials, to slices 0, 1, ... in that order:
//   C[r, c] = part[0][r, c] + part[1][r, c] + ... (left to right).
// Every tile has at least two slices here (the plan launches this only when no workgroup
// holds a whole tile).  One thread per four columns of a row, rows blockIdx.y + i gridDim.y;
// N % 4 == 0 takes 16-byte accesses (C and every slice are 16-byte aligned: stride % 4 == 0).
// Step numbers stay below 2^31 (checked on the host).
__global__ __launch_bounds__(256) void w4a16_tile_reduce(const float *__restrict__ part, float *__restrict__ C, int M,
                                                         int N, int64_t stride, int block_rows, int n_tiles,
                                                         int groups, int group_stride, int gps)
{
    const int c0 = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 4;
    if (c0 >= N) return;
    // a wave's 256 columns are one column tile, so the tile arithmetic is scalar
    const uint32_t nt = __builtin_amdgcn_readfirstlane((uint32_t)c0 / kLTileN);
    for (int row = (int)blockIdx.y; row < M; row += (int)gridDim.y) {
        const int64_t e = (int64_t)row * N + c0;
        f32x4 v0 = {}, v1 = {};
        if ((N & 3) == 0) {  // the two slices every tile has, loaded before the tile arithmetic
            v0 = __builtin_nontemporal_load((const f32x4 *)(part + e));
            v1 = __builtin_nontemporal_load((const f32x4 *)(part + stride + e));
        }
        const uint32_t t = (uint32_t)(row / block_rows) * (uint32_t)n_tiles + nt;
        const uint32_t a = t * (uint32_t)group_stride;
        const int nseg = (int)((a + (uint32_t)groups - 1) / (uint32_t)gps - a / (uint32_t)gps) + 1;
        if ((N & 3) == 0) {
            f32x4 acc = v0 + v1;
#pragma unroll 4
            for (int k = 2; k < nseg; ++k) acc += __builtin_nontemporal_load((const f32x4 *)(part + k * stride + e));
            *(f32x4 *)(C + e) = acc;
        } else {
            for (int j = 0; j < 4 && c0 + j < N; ++j) {
                float acc = part[e + j];
                for (int k = 1; k < nseg; ++k) acc += part[k * stride + e + j];
                C[e + j] = acc;
            }
        }
    }
}

// 4-bit activation quantizer: one (row, 128-wide group) per 16 lanes (a DPP row), each lane
// holding 8 consecutive values (one 16-byte load) and producing their packed word.
//   amax = max |A| over the group (the largest magnitude bit pattern: the order of
//          non-negative floats is that of their bits), sa = amax / 7 (IEEE division),
//   qa = clamp(rint(A / sa), -8, 7) (IEEE division, ties to even), 0 when sa == 0,
//   nibble j of the word = qa[8 kc + j] + 8.
__global__ __launch_bounds__(256) void a4_quantize_kernel(const uint16_t *__restrict__ A, uint32_t *__restrict__ Aq,
                                                          float *__restrict__ As, int64_t units, int groups)
{
    const int64_t unit = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int kc = threadIdx.x & 15;
    const bool live = unit < units;  // the whole DPP row shares `unit`, so rows are live or dead as one
    const int64_t u = live ? unit : units - 1;
    const u32x4 v = *(const u32x4 *)(A + u * kGroup + kc * 8);  // row-major [M, K]: unit = m * groups + g
    int mag = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        mag = max(mag, (int)(v[j] & 0x7FFFu));
        mag = max(mag, (int)((v[j] >> 16) & 0x7FFFu));
    }
    mag = row16_max(mag);
    const float amax = __builtin_bit_cast(float, (uint32_t)mag << 16);
    const float sa = amax / 7.0f;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t bits = (j & 1) ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16);
        const float a = __builtin_bit_cast(float, bits);
        const int qa = sa == 0.0f ? 0 : (int)fminf(fmaxf(rintf(a / sa), -8.0f), 7.0f);
        word |= (uint32_t)(qa + 8) << (4 * j);
    }
    if (live) {
        Aq[u * 16 + kc] = word;
        if (kc == 0) As[u] = sa;
    }
}

// 8-bit codes: Wq8[kb,n] = sum_j q[4kb+j,n] << 8j, one word per thread.
__global__ __launch_bounds__(256) void w8_pack_kernel(const uint8_t *__restrict__ q,
                                                      uint32_t *__restrict__ Wq8, int64_t KB, int64_t N)
{
    const int64_t total = KB * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t kb = idx / N, n = idx - kb * N;
        const uint8_t *src = q + (kb * 4) * N + n;
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= (uint32_t)src[j * N] << (8 * j);
        Wq8[idx] = w;
    }
}

__global__ __launch_bounds__(256) void w4_pack_kernel(const uint8_t *__restrict__ q,
                                                      uint32_t *__restrict__ Wq, int64_t KB, int64_t N)
{
    const int64_t total = KB * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t kb = idx / N, n = idx - kb * N;
        const uint8_t *src = q + (kb * 8) * N + n;
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) w |= (uint32_t)(src[j * N] & 0xFu) << (4 * j);
        Wq[idx] = w;
    }
}

// Round-to-nearest quantizer: the producer of the storage format.  For each column and
// group of 128 along K (the GPTQ/AWQ-style INT4 format the pages use for their drafts and
// targets, "When Do Quantized Drafts Help Speculative Decoding?", "Current pilot setup";
// "The Free Half of Speculative Decoding", third paragraph), every step in binary32:
//   lo = min(0, min W), hi = max(0, max W)     (the range holds 0, so z fits 0..15)
//   s  = binary16((hi - lo) / 15), ties to even; an all-zero or too-narrow range (s = 0)
//        takes s = binary16(2/15), z = 8
//   z  = clamp(rint(-lo / s), 0, 15),  q = clamp(rint(W / s) + z, 0, 15)   (s as stored)
// with IEEE division and rint ties to even, so the codes are reproducible bit for bit (the
// kernel divides by multiplying with the reciprocal where that provably gives the same
// integer, see quant_rint_div).
// Each thread owns two adjacent columns of one group and holds both columns' 128 rows in
// registers (one 4-byte load per row on the vector path), so every weight is read once;
// the codes are packed 8 rows to a word as they are produced.
__device__ __forceinline__ void quant_params(float lo, float hi, uint16_t &sbits, float &s, float &z)
{
    _Float16 sh = (_Float16)((hi - lo) / 15.0f);
    s = (float)sh;
    if (s == 0.0f) {
        sh = (_Float16)(2.0f / 15.0f);
        s = (float)sh;
        z = 8.0f;
    } else {
        z = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
    }
    sbits = __builtin_bit_cast(uint16_t, sh);
}

// rint(w / s) with IEEE division, computed as rint(w * r), r = 1/s correctly rounded: for
// |w / s| < 16 the product is within 2^-19 of the exact quotient and the correctly rounded
// quotient within 2^-20, so both round to the same integer unless the quotient lies within
// 2^-16 of a half-integer; those rare elements take the IEEE division (a branch that waves
// skip when none of their lanes needs it).  |w / s| <= 15 up to rounding here, since the
// grid spans the group's range.
__device__ __forceinline__ float quant_rint_div(float w, float s, float r)
{
    const float u = w * r;
    float q = rintf(u);
    if (__builtin_expect(fabsf(u - (floorf(u) + 0.5f)) < 0x1p-16f, 0)) q = rintf(w / s);
    return q;
}

__device__ __forceinline__ uint32_t quant_code(float w, float s, float r, float z)
{
    return (uint32_t)fminf(fmaxf(quant_rint_div(w, s, r) + z, 0.0f), 15.0f);
}

template <bool VEC>
__global__ __launch_bounds__(256) void w4_quantize_kernel(const uint16_t *__restrict__ W, uint32_t *__restrict__ Wq,
                                                          uint16_t *__restrict__ S, uint8_t *__restrict__ Z,
                                                          int64_t N)
{
    // A workgroup takes 256 columns of one group: lane l of wave w holds the column pair
    // c0, c0 + 1 (c0 = 2 (128 blockIdx.x + 32 w + l % 32)) over the group's rows
    // 64 (l / 32) .. + 63.  Each half finds its range, the halves swap theirs across the wave,
    // and both then derive the same parameters; each codes its own 64 rows.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t c0 = ((int64_t)blockIdx.x * 128 + wave * 32 + (lane & 31)) * 2;
    const bool active = c0 < N;  // both halves of a pair share c0, so they agree
    const bool two = c0 + 1 < N;
    const int64_t g = blockIdx.y;
    const uint16_t *src = W + (g * kGroup + 64 * half) * N + c0;
    uint32_t v[64];  // row k of the half: column c0 in the low half, c0 + 1 in the high half
#pragma unroll
    for (int k = 0; k < 64; ++k) {
        if (!active) {
            v[k] = 0;
        } else if (VEC) {
            v[k] = *(const uint32_t *)(src + k * N);
        } else {
            const uint32_t a = src[k * N], b = src[k * N + (two ? 1 : 0)];  // last column: read twice
            v[k] = a | (b << 16);
        }
    }
    float lo0 = 0.0f, hi0 = 0.0f, lo1 = 0.0f, hi1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k) {
        const f16x2 h = as_h2(v[k]);
        lo0 = fminf(lo0, (float)h.x);
        hi0 = fmaxf(hi0, (float)h.x);
        lo1 = fminf(lo1, (float)h.y);
        hi1 = fmaxf(hi1, (float)h.y);
    }
    // the other half's range (lane l ^ 32); min and max do not depend on the order
    lo0 = fminf(lo0, __shfl_xor(lo0, 32));
    hi0 = fmaxf(hi0, __shfl_xor(hi0, 32));
    lo1 = fminf(lo1, __shfl_xor(lo1, 32));
    hi1 = fmaxf(hi1, __shfl_xor(hi1, 32));
    if (!active) return;
    uint16_t sb0, sb1;
    float s0, z0, s1, z1;
    quant_params(lo0, hi0, sb0, s0, z0);
    quant_params(lo1, hi1, sb1, s1, z1);
    const float r0 = 1.0f / s0, r1 = 1.0f / s1;
    // the codes convert the packed halves again: keeping 128 converted values from the
    // range pass alive would double the registers
#pragma unroll
    for (int k = 0; k < 64; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const f16x2 h = as_h2(v[8 * kb + j]);
            w0 |= quant_code((float)h.x, s0, r0, z0) << (4 * j);
            w1 |= quant_code((float)h.y, s1, r1, z1) << (4 * j);
        }
        uint32_t *dst = Wq + (g * (kGroup / 8) + 8 * half + kb) * N + c0;
        if (VEC) {
            *(u32x2 *)dst = u32x2{w0, w1};
        } else {
            dst[0] = w0;
            if (two) dst[1] = w1;
        }
    }
    if (half != 0) return;
    if (VEC) {
        *(uint32_t *)(S + g * N + c0) = (uint32_t)sb0 | ((uint32_t)sb1 << 16);
        *(uint16_t *)(Z + g * N + c0) = (uint16_t)((uint32_t)z0 | ((uint32_t)z1 << 8));
    } else {
        S[g * N + c0] = sb0;
        Z[g * N + c0] = (uint8_t)z0;
        if (two) {
            S[g * N + c0 + 1] = sb1;
            Z[g * N + c0 + 1] = (uint8_t)z1;
        }
    }
}

// Streaming-read probe: the achievable HBM read rate for a buffer of a given size, as a
// ceiling for the weight stream.  Each lane keeps four 16-byte non-temporal buffer loads in
// flight (the weight stream's load policy) over a grid-stride loop and XORs what it reads;
// each wave writes the XOR of the 32-bit words it read, so a caller can check that every
// chunk was read once.  Loads past the end read the last chunk again (no branch around a load) and are
// dropped from the XOR.
__global__ __launch_bounds__(256) void w4_read_probe_kernel(const void *src, uint32_t n16, uint32_t *__restrict__ out)
{
    constexpr int kUnroll = 4;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)(n16 * 16), kRsrcWord3);
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint32_t stride = gridDim.x * 256 * kUnroll;
    for (uint32_t base = blockIdx.x * 256 * kUnroll + threadIdx.x; base < n16; base += stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t i = base + u * 256;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i < n16 ? i : n16 - 1) * 16, 0, kCacheStream);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (base + u * 256 < n16) acc ^= v[u];
    }
    // XOR of the lane's words, then across the wave (cross-lane shuffles, no barrier); lane 0
    // writes the wave's value
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

// ------------------------------------------------------------------------------------
// Host side

thread_local std::string g_last_error;

void set_error(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

w4_status hip_fail(const char *what, hipError_t e)
{
    set_error("%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return W4_ERR_HIP;
}

std::mutex g_mutex;
std::map<int, int> g_device_ok;  // device -> 1 gfx950, 0 other

w4_status check_device(int *dev_out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_error("hipGetDevice: %s", hipGetErrorString(e));
        return W4_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_device_ok.find(dev);
    if (it == g_device_ok.end()) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            set_error("hipGetDeviceProperties: %s", hipGetErrorString(e));
            return W4_ERR_DEVICE;
        }
        const int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_device_ok.emplace(dev, ok).first;
        if (!ok) set_error("device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    }
    if (!it->second) {
        set_error("device %d is not gfx950", dev);
        return W4_ERR_DEVICE;
    }
    *dev_out = dev;
    return W4_OK;
}

struct Workspace {
    char *ptr = nullptr;
    size_t counters = 0;     // capacity of the counter region, in counters
    size_t part_bytes = 0;   // capacity of the partial region
};
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;
std::vector<char *> g_retired;  // superseded buffers stay valid for graphs captured earlier

// Workspace layout, fixed for the life of a buffer: [counters][partials], the partial
// region starting at counters * 4 rounded up to 256 bytes.  Counters are zero whenever no
// call is in flight: the buffer is zeroed when allocated and every call resets the
// counters it used.
w4_status get_workspace(int dev, hipStream_t stream, size_t tiles, size_t part_bytes,
                        unsigned **count, float **part)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    Workspace &ws = g_workspaces[{dev, stream}];
    if (ws.counters < tiles || ws.part_bytes < part_bytes) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return hip_fail("hipStreamIsCapturing", e);
        if (cs != hipStreamCaptureStatusNone) {
            set_error("split-K workspace must grow (%zu counters, %zu bytes) while the stream is "
                      "capturing; run this shape once before capture", tiles, part_bytes);
            return W4_ERR_WORKSPACE;
        }
        const size_t mib = (size_t)1 << 20;
        size_t nc = ws.counters > tiles ? ws.counters : tiles;
        nc = ((nc < 4096 ? 4096 : nc) + 1023) & ~(size_t)1023;
        size_t pb = ws.part_bytes > part_bytes ? ws.part_bytes : part_bytes;
        pb = ((pb < mib ? mib : pb) + mib - 1) & ~(mib - 1);
        const size_t bytes = nc * 4 + pb;
        char *fresh = nullptr;
        e = hipMalloc((void **)&fresh, bytes);
        if (e != hipSuccess) return hip_fail("hipMalloc(workspace)", e);
        e = hipMemsetAsync(fresh, 0, bytes, stream);
        if (e != hipSuccess) return hip_fail("hipMemsetAsync(workspace)", e);
        if (ws.ptr) g_retired.push_back(ws.ptr);
        ws.ptr = fresh;
        ws.counters = nc;
        ws.part_bytes = pb;
    }
    *count = (unsigned *)ws.ptr;
    *part = (float *)(ws.ptr + ws.counters * 4);
    return W4_OK;
}

// Scratch for the entry point that allocates nothing (w4a16_gemm_noalloc): a file-scope
// device array with the workspace's layout, [arrival counters][partials], fixed for the life
// of the process.  In host code `scratch` is only a stand-in for the symbol: its device
// address differs per GPU and is looked up once per device (hipGetSymbolAddress, with that
// device current) and used in its place everywhere.  The counters must be zero between calls:
// they are zero when the code object is loaded, every call's last arrivers reset the ones it
// used, and the set-up clears them once more with a fill kernel (no memset node, so a set-up
// that happens under stream capture is replayed safely).
constexpr size_t kScratchCounters = 1 << 16;                  // arrival counters, 256 KiB
constexpr size_t kScratchCounterBytes = kScratchCounters * 4;
constexpr size_t kScratchBytes = (size_t)64 << 20;           // 64 MiB per GPU in all
constexpr size_t kScratchPartBytes = kScratchBytes - kScratchCounterBytes;
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void w4_fill_zero_kernel(uint32_t *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
char *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per GPU, set once

// Set-up on the entry point's first call on a device (with that device current): look up the
// array's device address and clear its counters on the caller's stream.
w4_status setup_scratch(int dev, hipStream_t stream)
{
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("w4a16_gemm_noalloc: device %d is beyond the %d this library tracks", dev, kMaxDevices);
        return W4_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev]) return W4_OK;
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!ptr) {
        set_error("hipGetSymbolAddress(scratch) returned a null address on device %d", dev);
        return W4_ERR_HIP;
    }
    hipLaunchKernelGGL(w4_fill_zero_kernel, dim3(256), dim3(256), 0, stream, (uint32_t *)ptr,
                       (int64_t)kScratchCounters);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("scratch set-up launch", e);
    g_scratch_ptr[dev] = (char *)ptr;
    return W4_OK;
}

// The scratch regions for one call's plan, or an error when the plan needs more than the
// array holds (nothing is launched then).
w4_status get_scratch(int dev, size_t tiles, size_t part_bytes, unsigned **count, float **part)
{
    if (tiles > kScratchCounters || part_bytes > kScratchPartBytes) {
        set_error("w4a16_gemm_noalloc: the plan needs %zu arrival counters and %zu partial bytes; the fixed "
                  "scratch holds %zu counters and %zu bytes", tiles, part_bytes, kScratchCounters, kScratchPartBytes);
        return W4_ERR_WORKSPACE;
    }
    *count = (unsigned *)g_scratch_ptr[dev];
    *part = (float *)(g_scratch_ptr[dev] + kScratchCounterBytes);
    return W4_OK;
}

w4_status validate_gemm_shape(int64_t M, int64_t K, int64_t N, int bits = 4, bool a4 = false)
{
    if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) {
        set_error("shape M=%lld K=%lld N=%lld: need M>=1, N>=1, K>=128, K%%128==0",
                  (long long)M, (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    // the kernels address each array with 32-bit byte offsets
    if (K * bits / 32 * N * 4 >= ((int64_t)1 << 31) || M * K * (a4 ? 1 : 4) / 2 >= ((int64_t)1 << 31)) {
        set_error("shape M=%lld K=%lld N=%lld: packed weights or activations exceed 2 GiB",
                  (long long)M, (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    const int64_t lim = (int64_t)1 << 40;
    if (M > lim / K || K > lim / N || M > lim / N || M > (int64_t)1 << 30 || N > (int64_t)1 << 30) {
        set_error("shape M=%lld K=%lld N=%lld is too large", (long long)M, (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    return W4_OK;
}

// Small-M launch plan.  Every workgroup of a launch must be resident at once (a second,
// partly filled round would double the time).  Each candidate (workgroup shape x split
// count) is scored with a cost model in microseconds, fitted to measured launches:
//   launch and first bytes + max(streaming time, per-wave compute) + split-K handoff
// where the per-wave compute is the groups a wave walks in turn times the time of one group
// at the CU's wave count, the streaming rate is limited by the bytes the waves keep in
// flight over the loaded latency (and by the achievable rate), and the handoff grows with
// the number of partial tiles the last workgroup sums.  A CU streams at most kGBsPerCU, so a
// plan on few CUs is bounded by the bytes each of them pulls (8-bit weights at M=1 on 72 CUs:
// 10.4 us measured, against 9.2 on 96 CUs and 7.9 on 144).  At (nearly) equal cost the
// shape with more waves in flight wins.
constexpr double kUsLaunch = 3.5;        // dispatch + first bytes from HBM
constexpr double kUsLatency = 1.0;       // loaded latency seen by the in-flight bytes
constexpr double kGBsPeak = 4500.0;      // achievable streaming rate of one launch
constexpr double kGBsPerCU = 42.5;       // achievable streaming rate of one CU
constexpr double kUsHandoff = 1.0;       // split-K: partial stores, arrival count
constexpr double kUsPerSplit = 0.4;      // ... and reading back one partial tile
constexpr double kUsPerGroup = 0.5;      // one group per wave, per wave resident on its SIMD
constexpr double kRowsFactor = 0.3;      // extra group cost per 4 rows beyond the first 4
constexpr int group_bytes(int bits) { return 4 * bits * 4 * kTileN; }  // packed weights of one wave-group
constexpr int kMinPartGroups = 4;        // balanced wide plan: groups per split part, at least

struct Choice {
    const Variant *v;
    int splits;
    double us;
};

Choice score(const Variant &v, int64_t base, int groups, int splits, int av, int64_t K, int64_t N, int bits,
             bool simd_sum = false)
{
    Choice c = {&v, splits, 1e30};
    const int gps = (groups + splits - 1) / splits;
    const int64_t wgs = base * splits;
    if (wgs > (int64_t)v.per_cu * kCUs) return c;
    const int64_t wg_per_cu = (wgs + kCUs - 1) / kCUs;  // on the busiest CU
    const double waves_per_simd = (double)v.waves * wg_per_cu / 4;
    const double t_group = kUsPerGroup * waves_per_simd * (1.0 + kRowsFactor * (av - 1));
    const int per_wave = (gps + v.waves - 1) / v.waves;
    double compute = per_wave * t_group;
    if (simd_sum) {
        // the busiest SIMD runs waves s, s + 4, ... of each workgroup and wave w holds
        // ceil((gps - w) / waves) groups: uneven counts cost that SIMD their sum, not
        // per_wave on each of its waves (which over-charges the 12-wave shape)
        int simd_groups = 0;
        for (int w = 0; w < v.waves; w += 4) simd_groups += gps > w ? (gps - w + v.waves - 1) / v.waves : 0;
        compute = simd_groups * (t_group / (v.waves / 4));
    }
    const int active_waves_per_wg = gps < v.waves ? gps : v.waves;
    const double inflight = (double)wgs * active_waves_per_wg * (per_wave < 2 ? per_wave : 2) * group_bytes(bits);
    double rate = inflight / (kUsLatency * 1e-6) / 1e9;  // GB/s
    if (rate > kGBsPeak) rate = kGBsPeak;
    const double bytes = (double)K * N * (bits / 8.0 + 3.0 / kGroup);
    const double busy_cus = (double)(wgs < kCUs ? wgs : kCUs);
    double stream = bytes / (rate * 1e3);  // us
    const double per_cu = bytes / busy_cus / (kGBsPerCU * 1e3);
    stream = stream > per_cu ? stream : per_cu;
    c.us = kUsLaunch + (stream > compute ? stream : compute) +
           (splits > 1 ? kUsHandoff + kUsPerSplit * splits : 0.0);
    return c;
}

// Large-M plan.  Candidates: row blocks of up to 160 rows (each weight dequantized once)
// or more, smaller row blocks (more tiles for narrow outputs, each weight dequantized once
// per block), times every K split.  The score is a small cost model in microseconds:
//   rounds of resident workgroups x groups per split x time per group
//   + split-K reduction (a second launch reading every split's partial product)
// where the time per group is the larger of the matrix-core time and the VALU time
// (dequantization, rescale and MFMA issue) of one workgroup, at a sustained efficiency.
constexpr double kLargeClockGHz = 2.4;
constexpr double kLargeEff = 0.44;         // sustained fraction of the issue-limited rate (measured)
constexpr double kUsLargeReduce = 2.5;     // second launch (split reduction) and its ramp
constexpr double kLargeReduceGBs = 4000.0; // split reduction: partial reads + C writes
// Evenly shared steps (a workgroup may end one tile and start the next): the second tile
// costs another ramp and another partial write, 2.6 us at 40 rows (per-workgroup
// timestamps: 1.3 us ramp, 1.3 us write).  They pay where whole-tile splits need extra
// rounds of workgroups: Qwen2.5-7B gate_up at M=40, 5 splits in 3 rounds of 6 groups
// against 17 shared steps in one round, 44.3 -> 37.5 us.  From three row tiles on they
// measured slower than the splits (M=80 gate_up 47.4 -> 49.3 us, M=160 qkv 34.4 -> 41.5,
// gate_up 50.7 -> 55.8): with more CUs busy each group's matrix-core work slows (M=160
// gate_up: 2.45 us per group on 172 CUs, 2.79 on 251), and the partials grow with the rows.
constexpr double kUsLargeSegment = 2.6;
// Which kernel: from M = 64 on, every shape runs on the bf16 kernel (the small-M kernel
// would dequantize each weight once per 16-row block).  From M = 17 (more than one 16-row
// block) the bf16 kernel also wins on large GEMMs, where its one dequantization per weight
// outweighs the padded rows; on narrow outputs it needs deep K splits and their reduction,
// and the small-M kernel stays faster (measured at M = 17..63 on the 7B layer shapes: K*N
// of 68M and 136M favour the bf16 kernel by up to 40% or tie, K*N of 13M and 17M favour
// the small-M kernel by 20-35%).
constexpr int kLargeMinM = 64;
constexpr int kLargeMidM = 17;
constexpr int64_t kLargeMidWeights = (int64_t)1 << 25;  // K*N at which 17 <= M < 64 goes large

bool large_path(int64_t M, int64_t K, int64_t N)
{
    return M >= kLargeMinM || (M >= kLargeMidM && K * N >= kLargeMidWeights);
}

double large_group_us(int rt)
{
    const double mfma = 2.0 * rt * 8 * 32;                     // cycles per SIMD, 2 waves
    const double valu = 2.0 * (160 + 16 * rt + 8 * rt) * 4;   // unpack + rescale + MFMA issue
    return (mfma > valu ? mfma : valu) / (kLargeClockGHz * 1e3) / kLargeEff;
}

// Large-M plan search over row blocks and split counts.  A split with fewer than
// min_gps groups is not a candidate; one-tile row blocks (32 rows) are candidates up to
// rt1_max_m rows.
struct LargeChoice {
    double us;
    int mb, splits, rows, gps, stride;  // splits: most partial slices any tile receives
};

// Most partial slices any tile receives when tile t owns steps t * stride .. + groups - 1
// and workgroup w takes steps w * gps .. + gps - 1.  t * stride mod gps repeats with a
// period that divides gps, so the first min(tiles, gps) tiles show every case.
int large_max_segments(int64_t tiles, int groups, int stride, int gps)
{
    int most = 1;
    for (int64_t t = 0; t < tiles && t < gps; ++t) {
        const int64_t a = t * stride;
        const int n = (int)((a + groups - 1) / gps - a / gps) + 1;
        most = n > most ? n : most;
    }
    return most;
}

LargeChoice search_large_plan(int64_t M, int64_t K, int64_t N, int min_gps, int64_t rt1_max_m)
{
    const int groups = (int)(K / kGroup);
    const int n_tiles = (int)((N + kLTileN - 1) / kLTileN);
    const int min_blocks = (int)((M + kLMaxRT * 32 - 1) / (kLMaxRT * 32));
    LargeChoice best = {1e30, min_blocks, 1, 0, groups, groups};
    for (int mbk = min_blocks; mbk <= 2 * min_blocks; ++mbk) {
        const int rows = (int)((M + mbk - 1) / mbk);
        const int rt = (rows + 31) / 32;
        if ((rt < 2 && M > rt1_max_m) || (int64_t)(mbk - 1) * rows >= M) continue;
        const int64_t base = (int64_t)mbk * n_tiles;
        const double tg = large_group_us(rt);
        // tiles split alike: sp workgroups per tile (stride sp * gps)
        for (int sp = 1; sp <= groups; ++sp) {
            const int gps = (groups + sp - 1) / sp;
            if ((groups + gps - 1) / gps != sp) continue;
            if (sp > 1 && gps < min_gps) continue;
            const int64_t rounds = (base * sp + kCUs - 1) / kCUs;
            double us = (double)rounds * gps * tg;
            if (sp > 1) us += kUsLargeReduce + (double)(sp + 1) * M * N * 4 / (kLargeReduceGBs * 1e3);
            if (us < best.us) best = {us, mbk, sp, rows, gps, sp * gps};
        }
        // the steps shared out evenly (stride = groups): only where gps does not divide the
        // groups (otherwise the same as a split above), and only for blocks of up to two row
        // tiles (see kLargeSharedMaxRT)
        for (int gps = min_gps > 1 ? min_gps : 1; gps < groups && rt <= kLargeSharedMaxRT; ++gps) {
            if (groups % gps == 0) continue;
            const int64_t wgs = (base * groups + gps - 1) / gps;
            const int64_t rounds = (wgs + kCUs - 1) / kCUs;
            const double slices = (double)(wgs + base - 1) / (double)base;  // mean per tile
            const double us = (double)rounds * gps * tg + kUsLargeSegment + kUsLargeReduce +
                              (slices + 1) * M * N * 4 / (kLargeReduceGBs * 1e3);
            if (us < best.us) best = {us, mbk, large_max_segments(base, groups, groups, gps), rows, gps, groups};
        }
    }
    return best;
}

void make_large_plan(int64_t M, int64_t K, int64_t N, w4_plan *pl)
{
    const int n_tiles = (int)((N + kLTileN - 1) / kLTileN);
    // First choice: splits of at least 4 groups, and one-tile row blocks up to 64 rows.
    // With fewer groups per workgroup its ramp and the partial tile it writes at the end
    // outweigh its share of the work: forced-plan sweeps of the Qwen2.5-7B qkv and o
    // projections at M = 64..96 ran 19-22% faster with 2 row blocks x 7 splits than with
    // the 1 x 14 the model alone picks (M=64 qkv: 19.5 -> 15.7 us).  The model's choice
    // stands where that plan would leave more than half of the CUs idle.
    auto workgroups = [&](const LargeChoice &c) {
        return ((int64_t)c.mb * n_tiles * c.stride + c.gps - 1) / c.gps;
    };
    LargeChoice c = search_large_plan(M, K, N, 4, 64);
    if (workgroups(c) < kCUs / 2) c = search_large_plan(M, K, N, 1, 32);
    pl->kernel = 3;
    pl->tile_m = c.rows;
    pl->tile_n = kLTileN;
    pl->m_blocks = c.mb;
    pl->n_tiles = n_tiles;
    pl->splits = c.splits;
    pl->groups_per_split = c.gps;
    pl->full_tiles = 0;
    pl->workgroups = workgroups(c);
    pl->workspace_bytes = c.splits > 1 ? c.splits * ((M * N + 3) / 4 * 4) * 4 : 0;
    pl->group_stride = c.stride;
}

// Kernel ids of the small-M shapes: 1 / 2 (4-bit codes, wide / tall), 4 / 5 (8-bit codes),
// 6 / 7 (4-bit codes and 4-bit activations).
int small_kernel_id(bool tall, int bits, bool a4)
{
    return (a4 ? 5 : bits == 8 ? 3 : 0) + (tall ? 2 : 1);
}

void make_small_plan(int64_t M, int64_t K, int64_t N, w4_plan *pl, int bits = 4, bool a4 = false)
{
    const int groups = (int)(K / kGroup);
    const int n_tiles = (int)((N + kTileN - 1) / kTileN);
    // Blocks of 16 rows.  With 4-bit activations at 17 to 32 rows, one block of 32: each wave
    // holds two matrix-core row tiles that share every unpacked weight operand (the
    // Llama-2-7B batch-32 draft step measured 1.94 -> 1.78 ms).  Not for bfloat16
    // activations, whose per-wave conversion doubles with the rows: there the same change
    // measured between 7% faster and 31% slower by shape, and beyond 32 rows a second block
    // mostly computes padding.
    const int rows = a4 && M > kTileM && M <= 2 * kTileM ? 2 * kTileM : kTileM;
    const int m_blocks = (int)((M + rows - 1) / rows);
    const int64_t base = (int64_t)n_tiles * m_blocks;
    Choice best = {&kWide, 1, 1e30};  // fallback (more tiles than resident slots): wide, no split
    const int av = (int)(((M < rows ? M : rows) + 3) / 4);
    const Variant &wide = rows > kTileM ? kWide2 : kWide, &tall = rows > kTileM ? kTall2 : kTall;
    best.v = &wide;
    // Near-ties go to the shape scored first: the 12-wave shape, which keeps more bytes in
    // flight, except for 8-bit codes with one activation chunk per lane (M <= 4).  There a
    // wide wave already has twice the bytes of a 4-bit group in flight, and the wide shape
    // measured faster at every split count (8960x1536 at M=1: 8.60 against 9.41 us at 4
    // splits, 7.39 against 7.76 at 6; qkv-sized 1536x2048: 5.24 against 5.59 us).
    const bool wide_first = bits == 8 && av == 1;
    // Several 16-row blocks of bfloat16 activations (M = 17..63): the per-SIMD group sum.
    // With it the 12-wave shape takes qkv- and o-sized outputs at the same split count, as
    // measured 4-15% faster (M = 24: 3584x4608 10.45 -> 9.35 us, 3584x3584 9.27 -> 8.75,
    // 8960x1536 9.29 -> 8.88; M = 40: 3584x4608 10.48 -> 9.38, 3584x3584 10.37 -> 9.20,
    // 4096x4096 11.67 -> 9.95; M = 56: 3584x3584 10.48 -> 9.31).  At one block the plans
    // keep the original estimate, which their forced-plan sweeps confirmed.
    const bool simd_sum = m_blocks > 1 && bits == 4 && !a4;
    for (const Variant *v : {wide_first ? &wide : &tall, wide_first ? &tall : &wide}) {
        for (int sp = 1; sp <= groups; ++sp) {
            const int gps = (groups + sp - 1) / sp;
            if ((groups + gps - 1) / gps != sp) continue;
            const Choice c = score(*v, base, groups, sp, av, K, N, bits, simd_sum);
            if (c.us < best.us * 0.98) best = c;
        }
    }
    // A tall plan whose workgroups hold fewer groups than waves leaves waves idle; the wide
    // shape with the same split count is then ~3% faster when the model scores them alike
    // (measured on qkv and o at M = 5: 7.72 -> 7.48 us and 7.53 -> 7.30 us).  With a single
    // 16-row block the same holds at exactly one group per wave (Qwen2.5-1.5B draft at M=1:
    // qkv, o, down 4.52 -> 4.49, 4.70 -> 4.57, 7.36 -> 7.16 us; 8-bit qkv and o 5.69 -> 5.36
    // and 5.70 -> 5.35 us); with more rows per workgroup the tall shape keeps it (measured
    // 1-3% faster on 16-row blocks at M = 24..60, 12-14% on 32-row blocks).
    const int best_gps = (groups + best.splits - 1) / best.splits;
    if (best.v == &tall && (best_gps < tall.waves || (best_gps == tall.waves && m_blocks == 1 && rows == kTileM))) {
        const Choice w = score(wide, base, groups, best.splits, av, K, N, bits, simd_sum);
        if (w.us <= best.us * 1.02) best = w;
    }
    // Balanced wide plan.  When the plain wide plan wins and its tiles fill r whole rounds of
    // CUs (r workgroups on every CU) plus a remainder, the busiest CUs hold r + 1 whole
    // tiles.  Instead, r*256 tiles run unsplit (r per CU) and the remaining tiles are split
    // over the slots still free, so that a CU holds r whole tiles and at most one split
    // part.  The parts are dispatched first and finish early, keeping their handoff off the
    // critical path; each keeps at least kMinPartGroups groups, below which the handoff and
    // the extra launch width cost more than the balance gains (measured).
    int64_t full = 0;
    const int r = (int)(base / kCUs);
    if (best.v == &wide && best.splits == 1 && r >= 1 && r < wide.per_cu && base % kCUs != 0) {
        const int64_t rem = base - (int64_t)r * kCUs;
        int64_t sp = (int64_t)kCUs * (wide.per_cu - r) / rem;
        sp = sp < groups / kMinPartGroups ? sp : groups / kMinPartGroups;
        if (sp >= 2) {
            const int g = (int)((groups + sp - 1) / sp);
            best.splits = (groups + g - 1) / g;
            full = (int64_t)r * kCUs;
        }
    }
    const int gps = (groups + best.splits - 1) / best.splits;
    const int splits = (groups + gps - 1) / gps;
    const int64_t split_tiles = splits > 1 ? base - full : 0;
    pl->kernel = small_kernel_id(best.v == &tall, bits, a4);
    pl->tile_m = rows;
    pl->tile_n = kTileN;
    pl->m_blocks = m_blocks;
    pl->n_tiles = n_tiles;
    pl->splits = splits;
    pl->groups_per_split = gps;
    pl->full_tiles = (int)full;
    pl->group_stride = 0;
    pl->workgroups = full + (base - full) * splits;
    pl->workspace_bytes = split_tiles * 4 + split_tiles * splits * rows * kTileN * 4;
}

// Narrow-tile kernel: eligible when the rows fit one 16-row block, the staged activations
// leave room for two workgroups per CU, and no wave holds more than kNarrowMaxGroups
// groups at once.
// (8 waves measured fastest: 12 and 16 waves per workgroup were 2-30% slower on every
// planned shape.)
constexpr int kNarrowWaves = 8;
constexpr int kNarrowMaxLds = 64 * 1024;

bool narrow_eligible(int64_t M, int64_t K, int64_t N)
{
    const int64_t groups = K / kGroup;
    const int64_t tiles = (N + kNarrowN - 1) / kNarrowN;
    return M <= kTileM && groups <= (int64_t)kNarrowMaxGroups * kNarrowWaves &&
           narrow_lds_bytes((int)groups, (int)M, kNarrowWaves) <= kNarrowMaxLds && tiles <= kCUs;
}

void make_narrow_plan(int64_t M, int64_t K, int64_t N, w4_plan *pl)
{
    pl->kernel = 8;
    pl->tile_m = kTileM;
    pl->tile_n = kNarrowN;
    pl->m_blocks = 1;
    pl->n_tiles = (int)((N + kNarrowN - 1) / kNarrowN);
    pl->splits = 1;
    pl->groups_per_split = (int)(K / kGroup);
    pl->full_tiles = 0;
    pl->group_stride = 0;
    pl->workgroups = pl->n_tiles;
    pl->workspace_bytes = 0;
}

// Shapes chosen by large_path run on the bf16 matrix-core kernel; narrow outputs whose
// activations fit in LDS on the narrow-tile kernel; everything else on the small-M kernel
// (row blocks of 16).
void make_plan(int64_t M, int64_t K, int64_t N, w4_plan *pl)
{
    if (large_path(M, K, N))
        make_large_plan(M, K, N, pl);
    else if (narrow_eligible(M, K, N))
        make_narrow_plan(M, K, N, pl);
    else
        make_small_plan(M, K, N, pl);
}

// 8-bit codes: narrow outputs on the narrow-tile kernel as for 4-bit codes (the same rule:
// the tile count, the groups per wave and the staged activations do not depend on the code
// width), everything else on the small-M kernel.
void make_plan8(int64_t M, int64_t K, int64_t N, w4_plan *pl)
{
    if (narrow_eligible(M, K, N))
        make_narrow_plan(M, K, N, pl);
    else
        make_small_plan(M, K, N, pl, 8);
}

size_t plan_lds_bytes(int64_t M, const w4_plan &pl)
{
    const int rows = M < pl.tile_m ? (int)M : pl.tile_m;
    const bool tall = pl.kernel == 2 || pl.kernel == 5 || pl.kernel == 7;
    const Variant &v = pl.tile_m > kTileM ? (tall ? kTall2 : kWide2) : (tall ? kTall : kWide);
    const size_t tiles = (size_t)v.waves * pipe_wave_bytes(pl.tile_m / kTileM);
    const size_t red = (size_t)v.waves * rows * kTileN * 4;
    return tiles > red ? tiles : red;
}

// The small-M instances compiled below: 16-row blocks (one activation chunk row per 4 rows,
// av = 1..4) for every code width and activation type, and 32-row blocks (av = 5..8) for
// 4-bit activations only.  A plan outside this set is an internal error, reported as
// W4_ERR_PLAN before anything is launched.
bool small_instance_exists(int rb, int av, int bits, bool a4)
{
    if (rb == 1) return av >= 1 && av <= 4 && (bits == 4 || (bits == 8 && !a4));
    return rb == 2 && a4 && bits == 4 && av >= 5 && av <= 8;
}

// Whether a plan names a compiled kernel: every large-M row-tile count (1..5) is compiled;
// small-M plans are checked against the instance table above.
bool plan_has_instance(int64_t M, const w4_plan &pl, int bits, bool a4)
{
    if (pl.kernel == 3) return !a4 && bits == 4 && pl.tile_m >= 1 && pl.tile_m <= kLMaxRT * 32;
    if (pl.kernel == 8) return !a4 && (bits == 4 || bits == 8) && M <= kTileM && pl.tile_n == kNarrowN;
    if (pl.tile_m % kTileM != 0) return false;
    const int rows = M < pl.tile_m ? (int)M : pl.tile_m;
    return small_instance_exists(pl.tile_m / kTileM, (rows + 3) / 4, bits, a4);
}

w4_status check_plan(const char *name, int64_t M, const w4_plan &pl, int bits, bool a4)
{
    if (plan_has_instance(M, pl, bits, a4)) return W4_OK;
    set_error("%s: internal error: plan (kernel %d, %d-row blocks) for M=%lld has no compiled instance", name,
              pl.kernel, pl.tile_m, (long long)M);
    return W4_ERR_PLAN;
}

// Small-M launches: one instantiation per (vectorized loads, waves, activation chunks per
// lane, code width); every shape keeps 3 waves per SIMD.  t1: the last activation pass holds
// a single row (4-bit codes with bfloat16 activations, one 16-row block of 5, 9 or 13 rows),
// which has instances of its own.
template <int BITS, bool A4>
bool launch_small(bool tall, int rb, int av, bool vec, bool t1, dim3 grid, size_t lds, hipStream_t s,
                  const SmallParams &p)
{
    const SmallTail tail = {p.C, p.part, p.count, p.As};
#define W4_ARGS p.A, p.Wq, p.S, p.Z, (int)p.M, (int)p.K, (int)p.N, p.splits, p.gps, p.full_tiles, tail
#define W4_LAUNCH(V, WV, AVV, OCCV, RBV) \
    hipLaunchKernelGGL((w4a16_kernel<V, WV, AVV, OCCV, BITS, A4, RBV, false>), grid, dim3(WV * kWave), lds, s, W4_ARGS)
#define W4_LAUNCH_T1(V, WV, AVV) \
    hipLaunchKernelGGL((w4a16_kernel<V, WV, AVV, kOccupancy, BITS, A4, 1, true>), grid, dim3(WV * kWave), lds, s, W4_ARGS)
#define W4_LAUNCH_16T1(V, WV) \
    switch (av) { case 2: W4_LAUNCH_T1(V, WV, 2); break; case 3: W4_LAUNCH_T1(V, WV, 3); break; \
                  default: W4_LAUNCH_T1(V, WV, 4); break; }
#define W4_LAUNCH_16(V, WV) \
    switch (av) { case 1: W4_LAUNCH(V, WV, 1, kOccupancy, 1); break; case 2: W4_LAUNCH(V, WV, 2, kOccupancy, 1); break; \
                  case 3: W4_LAUNCH(V, WV, 3, kOccupancy, 1); break; default: W4_LAUNCH(V, WV, 4, kOccupancy, 1); break; }
#define W4_LAUNCH_32(V, WV) \
    switch (av) { case 5: W4_LAUNCH(V, WV, 5, kOccupancy2, 2); break; case 6: W4_LAUNCH(V, WV, 6, kOccupancy2, 2); break; \
                  case 7: W4_LAUNCH(V, WV, 7, kOccupancy2, 2); break; default: W4_LAUNCH(V, WV, 8, kOccupancy2, 2); break; }
    if (!small_instance_exists(rb, av, BITS, A4)) return false;
    if (t1) {
        if constexpr (BITS == 4 && !A4) {
            if (rb != 1 || av < 2) return false;
            if (tall) { if (vec) { W4_LAUNCH_16T1(true, kTall.waves) } else { W4_LAUNCH_16T1(false, kTall.waves) } }
            else { if (vec) { W4_LAUNCH_16T1(true, kWide.waves) } else { W4_LAUNCH_16T1(false, kWide.waves) } }
            return true;
        }
        return false;
    }
    if (rb == 1) {
        if (tall) { if (vec) { W4_LAUNCH_16(true, kTall.waves) } else { W4_LAUNCH_16(false, kTall.waves) } }
        else { if (vec) { W4_LAUNCH_16(true, kWide.waves) } else { W4_LAUNCH_16(false, kWide.waves) } }
    } else if constexpr (A4) {  // 32-row blocks are planned for 4-bit activations only
        if (tall) { if (vec) { W4_LAUNCH_32(true, kTall2.waves) } else { W4_LAUNCH_32(false, kTall2.waves) } }
        else { if (vec) { W4_LAUNCH_32(true, kWide2.waves) } else { W4_LAUNCH_32(false, kWide2.waves) } }
    }
    return true;
#undef W4_LAUNCH_32
#undef W4_LAUNCH_16
#undef W4_LAUNCH_16T1
#undef W4_LAUNCH_T1
#undef W4_LAUNCH
#undef W4_ARGS
}

// The GEMM for every variant (code width, activation type): host validation, plan,
// workspace, launches.  With 4-bit activations, A_bf16 is the packed codes and As their
// scales.
w4_status run_gemm(int bits, bool a4, const char *name, const void *A_bf16, const float *As, const uint32_t *Wq,
                   const void *scales_f16, const uint8_t *zeros, float *C, int64_t M, int64_t K, int64_t N,
                   void *stream, bool noalloc = false)
{
    if (!A_bf16 || (a4 && !As) || !Wq || !scales_f16 || !zeros || !C) {
        set_error("%s: a required pointer is NULL", name);
        return W4_ERR_NULL;
    }
    w4_status st = validate_gemm_shape(M, K, N, bits, a4);
    if (st != W4_OK) return st;
    if (a4 ? (!aligned(A_bf16, 4) || !aligned(As, 4)) : !aligned(A_bf16, 16)) {
        set_error(a4 ? "%s: Aq and A_scales must be 4-byte aligned" : "%s: A must be 16-byte aligned", name);
        return W4_ERR_ALIGN;
    }
    if (!aligned(Wq, 16) || !aligned(C, 16) || !aligned(scales_f16, 2)) {
        set_error("%s: Wq and C must be 16-byte aligned and scales 2-byte aligned", name);
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    st = check_device(&dev);
    if (st != W4_OK) return st;

    w4_plan pl;
    if (a4)
        make_small_plan(M, K, N, &pl, bits, a4);
    else if (bits == 8)
        make_plan8(M, K, N, &pl);
    else
        make_plan(M, K, N, &pl);
    st = check_plan(name, M, pl, bits, a4);
    if (st != W4_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (noalloc) {
        st = setup_scratch(dev, s);
        if (st != W4_OK) return st;
    }
    unsigned *count = nullptr;
    float *part = nullptr;
    if (pl.workspace_bytes > 0) {
        // small-M: [tile counters][partial tiles]; large-M: [split slices] only
        const int64_t tiles = pl.kernel == 3 ? 0 : (int64_t)pl.n_tiles * pl.m_blocks - pl.full_tiles;
        st = noalloc ? get_scratch(dev, (size_t)tiles, (size_t)(pl.workspace_bytes - tiles * 4), &count, &part)
                     : get_workspace(dev, s, (size_t)tiles, (size_t)(pl.workspace_bytes - tiles * 4), &count, &part);
        if (st != W4_OK) return st;
    }
    const dim3 grid((unsigned)pl.workgroups);
    if (pl.kernel == 8) {
        NarrowParams q;
        q.A = (const uint16_t *)A_bf16;
        q.Wq = Wq;
        q.S = (const uint16_t *)scales_f16;
        q.Z = zeros;
        q.C = C;
        q.M = M;
        q.K = K;
        q.N = N;
        q.groups = (int)(K / kGroup);
        q.n_tiles = pl.n_tiles;
        const size_t lds = (size_t)narrow_lds_bytes(q.groups, (int)M, kNarrowWaves);
        if (bits == 8)
            hipLaunchKernelGGL((w4a16_narrow_kernel<kNarrowWaves, 8>), grid, dim3(kNarrowWaves * kWave), lds, s, q.A,
                               q.Wq, q.S, q.Z, q.C, (int)q.M, (int)q.K, (int)q.N, q.groups);
        else
            hipLaunchKernelGGL((w4a16_narrow_kernel<kNarrowWaves, 4>), grid, dim3(kNarrowWaves * kWave), lds, s, q.A,
                               q.Wq, q.S, q.Z, q.C, (int)q.M, (int)q.K, (int)q.N, q.groups);
    } else if (pl.kernel == 3) {
        LargeParams q;
        q.A = (const uint16_t *)A_bf16;
        q.Wq = Wq;
        q.S = (const uint16_t *)scales_f16;
        q.Z = zeros;
        q.C = C;
        q.part = part;
        q.stride = (M * N + 3) / 4 * 4;
        q.M = M;
        q.K = K;
        q.N = N;
        q.groups = (int)(K / kGroup);
        q.splits = pl.splits;
        q.gps = pl.groups_per_split;
        q.n_tiles = pl.n_tiles;
        q.m_blocks = pl.m_blocks;
        q.block_rows = pl.tile_m;
        const int64_t gstride = pl.group_stride;
        // The kernel derives the tile and row-block counts from N, M and the block rows, and
        // numbers the (tile, group) steps in 32 bits; the reduction relies on every tile
        // having two or more workgroups whenever it runs.
        const int64_t steps = (int64_t)q.m_blocks * q.n_tiles * gstride;
        if (q.n_tiles != (N + kLTileN - 1) / kLTileN || q.m_blocks != (M + q.block_rows - 1) / q.block_rows ||
            gstride < q.groups || q.gps < 1 || steps + q.gps >= ((int64_t)1 << 31) ||
            pl.workgroups != (steps + q.gps - 1) / q.gps ||
            (pl.splits > 1) != (q.gps < q.groups) ||
            (gstride != (int64_t)pl.splits * q.gps && (q.block_rows + 31) / 32 > kLargeSharedMaxRT) ||
            pl.splits != large_max_segments((int64_t)q.m_blocks * q.n_tiles, q.groups, (int)gstride, q.gps)) {
            set_error("%s: internal error: inconsistent large-M plan", name);
            return W4_ERR_PLAN;
        }
        const LargeTail tail = {q.C, q.part, q.stride};
#define W4_LAUNCH_L(RTV, SHV)                                                                                     \
    hipLaunchKernelGGL((w4a16_mfma_kernel<RTV, SHV>), grid, dim3(kLThreads), 0, s, q.A, q.Wq, q.S, q.Z, (int)q.M,      \
                       (int)q.K, (int)q.N, q.gps, (int)gstride, q.block_rows, tail)
        const bool shared = gstride != (int64_t)pl.splits * q.gps;  // (then 1 or 2 row tiles, checked above)
        switch ((pl.tile_m + 31) / 32) {
        case 1: if (shared) { W4_LAUNCH_L(1, true); } else { W4_LAUNCH_L(1, false); } break;
        case 2: if (shared) { W4_LAUNCH_L(2, true); } else { W4_LAUNCH_L(2, false); } break;
        case 3: W4_LAUNCH_L(3, false); break;
        case 4: W4_LAUNCH_L(4, false); break;
        default: W4_LAUNCH_L(5, false); break;
        }
#undef W4_LAUNCH_L
        if (pl.splits > 1) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(name, e);
            if (gstride == (int64_t)pl.splits * q.gps) {  // every tile split alike
                const int64_t n4 = M * N / 4;
                int64_t blocks = (n4 + 255) / 256;
                blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
                hipLaunchKernelGGL(w4a16_split_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, C, M * N,
                                   q.stride, pl.splits);
            } else {
                const dim3 rgrid((unsigned)((N + 1023) / 1024), (unsigned)(M < 65535 ? M : 65535));
                hipLaunchKernelGGL(w4a16_tile_reduce, rgrid, dim3(256), 0, s, part, C, (int)M, (int)N, q.stride,
                                   q.block_rows, q.n_tiles, q.groups, (int)gstride, q.gps);
            }
        }
    } else {
        SmallParams p;
        p.A = (const uint16_t *)A_bf16;
        p.As = As;
        p.Wq = Wq;
        p.S = (const uint16_t *)scales_f16;
        p.Z = zeros;
        p.C = C;
        p.part = part;
        p.count = count;
        p.M = M;
        p.K = K;
        p.N = N;
        p.groups = (int)(K / kGroup);
        p.splits = pl.splits;
        p.gps = pl.groups_per_split;
        p.n_tiles = pl.n_tiles;
        p.m_blocks = pl.m_blocks;
        p.full_tiles = pl.full_tiles;
        // the kernel derives its tile and row-block counts from N, M and its rows per block
        if (pl.n_tiles != (N + kTileN - 1) / kTileN || pl.m_blocks != (M + pl.tile_m - 1) / pl.tile_m) {
            set_error("%s: internal error: plan tiles (%d x %d) do not follow from the shape", name, pl.m_blocks,
                      pl.n_tiles);
            return W4_ERR_PLAN;
        }
        // the kernel derives its split-part count from these fields instead of the grid size
        if (pl.workgroups != (int64_t)pl.full_tiles + ((int64_t)pl.m_blocks * pl.n_tiles - pl.full_tiles) * pl.splits) {
            set_error("%s: internal error: plan grid (%lld workgroups) does not match its tiles", name,
                      (long long)pl.workgroups);
            return W4_ERR_PLAN;
        }
        const bool vec = (N % 4 == 0) && aligned(scales_f16, 8) && aligned(zeros, 4);
        const size_t lds = plan_lds_bytes(M, pl);
        const int rb = pl.tile_m / kTileM;
        const int rows = M < pl.tile_m ? (int)M : pl.tile_m;
        const int av = (rows + 3) / 4;
        const bool tall = pl.kernel == 2 || pl.kernel == 5 || pl.kernel == 7;
        // one 16-row block whose last activation pass holds a single row, after at least one
        // full pass: at M = 5 the single-row pass measured 1.4% faster on the Qwen2.5-7B verify
        // step (down 12.87 -> 12.69 us); at M = 1, where it is the only pass, no faster
        const bool t1 = !a4 && bits == 4 && pl.tile_m == kTileM && pl.m_blocks == 1 && rows % 4 == 1 && rows > 1;
        const bool launched = a4 ? launch_small<4, true>(tall, rb, av, vec, false, grid, lds, s, p)
                              : bits == 8 ? launch_small<8, false>(tall, rb, av, vec, false, grid, lds, s, p)
                                          : launch_small<4, false>(tall, rb, av, vec, t1, grid, lds, s, p);
        if (!launched) {
            set_error("%s: internal error: plan (kernel %d, %d-row blocks, %d chunk rows) has no compiled "
                      "instance", name, pl.kernel, pl.tile_m, av);
            return W4_ERR_PLAN;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(name, e);
    return W4_OK;
}

}  // namespace

extern "C" {

const char *w4_status_string(w4_status s)
{
    switch (s) {
    case W4_OK: return "ok";
    case W4_ERR_NULL: return "null pointer argument";
    case W4_ERR_SHAPE: return "invalid shape";
    case W4_ERR_ALIGN: return "misaligned pointer";
    case W4_ERR_DEVICE: return "no gfx950 device";
    case W4_ERR_HIP: return "HIP runtime error";
    case W4_ERR_WORKSPACE: return "workspace cannot grow during stream capture";
    case W4_ERR_PLAN: return "internal error: no kernel instance for the launch plan";
    }
    return "unknown status";
}

const char *w4_last_error(void) { return g_last_error.c_str(); }

w4_status w4a16_plan(int64_t M, int64_t K, int64_t N, w4_plan *out)
{
    if (!out) {
        set_error("w4a16_plan: out is NULL");
        return W4_ERR_NULL;
    }
    w4_status st = validate_gemm_shape(M, K, N);
    if (st != W4_OK) return st;
    make_plan(M, K, N, out);
    return check_plan("w4a16_plan", M, *out, 4, false);
}

w4_status w4a16_gemm(const void *A_bf16, const uint32_t *Wq, const void *scales_f16,
                     const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N,
                     void *stream)
{
    return run_gemm(4, false, "w4a16_gemm", A_bf16, nullptr, Wq, scales_f16, zeros_u4, C, M, K, N, stream);
}

w4_status w4a16_gemm_noalloc(const void *A_bf16, const uint32_t *Wq, const void *scales_f16,
                             const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N, void *stream)
{
    return run_gemm(4, false, "w4a16_gemm_noalloc", A_bf16, nullptr, Wq, scales_f16, zeros_u4, C, M, K, N, stream,
                    true);
}

w4_status w8a16_gemm(const void *A_bf16, const uint32_t *Wq8, const void *scales_f16,
                     const uint8_t *zeros_u8, float *C, int64_t M, int64_t K, int64_t N,
                     void *stream)
{
    return run_gemm(8, false, "w8a16_gemm", A_bf16, nullptr, Wq8, scales_f16, zeros_u8, C, M, K, N, stream);
}

w4_status w4a4_gemm(const uint32_t *Aq, const float *A_scales, const uint32_t *Wq, const void *scales_f16,
                    const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N, void *stream)
{
    return run_gemm(4, true, "w4a4_gemm", Aq, A_scales, Wq, scales_f16, zeros_u4, C, M, K, N, stream);
}

w4_status w4a4_plan(int64_t M, int64_t K, int64_t N, w4_plan *out)
{
    if (!out) {
        set_error("w4a4_plan: out is NULL");
        return W4_ERR_NULL;
    }
    w4_status st = validate_gemm_shape(M, K, N, 4, true);
    if (st != W4_OK) return st;
    make_small_plan(M, K, N, out, 4, true);
    return check_plan("w4a4_plan", M, *out, 4, true);
}

w4_status a4_quantize(const void *A_bf16, uint32_t *Aq, float *A_scales, int64_t M, int64_t K, void *stream)
{
    if (!A_bf16 || !Aq || !A_scales) {
        set_error("a4_quantize: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    if (M < 1 || K < kGroup || K % kGroup != 0 || M * K * 2 >= ((int64_t)1 << 40)) {
        set_error("a4_quantize: shape M=%lld K=%lld: need M>=1, K>=128, K%%128==0", (long long)M, (long long)K);
        return W4_ERR_SHAPE;
    }
    if (!aligned(A_bf16, 16) || !aligned(Aq, 4) || !aligned(A_scales, 4)) {
        set_error("a4_quantize: A must be 16-byte aligned, Aq and A_scales 4-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    w4_status st = check_device(&dev);
    if (st != W4_OK) return st;
    const int64_t units = M * (K / kGroup);
    const int64_t blocks = (units + 15) / 16;
    if (blocks > 0x7FFFFFFF) {
        set_error("a4_quantize: shape M=%lld K=%lld is too large", (long long)M, (long long)K);
        return W4_ERR_SHAPE;
    }
    hipLaunchKernelGGL(a4_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t *)A_bf16, Aq, A_scales, units, (int)(K / kGroup));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("a4_quantize launch", e);
    return W4_OK;
}

w4_status w8a16_plan(int64_t M, int64_t K, int64_t N, w4_plan *out)
{
    if (!out) {
        set_error("w8a16_plan: out is NULL");
        return W4_ERR_NULL;
    }
    w4_status st = validate_gemm_shape(M, K, N, 8);
    if (st != W4_OK) return st;
    make_plan8(M, K, N, out);
    return check_plan("w8a16_plan", M, *out, 8, false);
}

w4_status w4_quantize(const void *W_f16, uint32_t *Wq, void *scales_f16, uint8_t *zeros_u4, int64_t K, int64_t N,
                      void *stream)
{
    if (!W_f16 || !Wq || !scales_f16 || !zeros_u4) {
        set_error("w4_quantize: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    if (K < kGroup || K % kGroup != 0 || N < 1 || K / kGroup > 65535 || K > ((int64_t)1 << 40) / N) {
        set_error("w4_quantize: shape K=%lld N=%lld: need K>=128, K%%128==0, K/128<=65535, N>=1",
                  (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    if (!aligned(W_f16, 2) || !aligned(Wq, 4) || !aligned(scales_f16, 2)) {
        set_error("w4_quantize: W and scales must be 2-byte aligned and Wq 4-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    w4_status st = check_device(&dev);
    if (st != W4_OK) return st;
    const bool vec = N % 2 == 0 && aligned(W_f16, 4) && aligned(Wq, 8) && aligned(scales_f16, 4) && aligned(zeros_u4, 2);
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / kGroup));
    if (vec)
        hipLaunchKernelGGL(w4_quantize_kernel<true>, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t *)W_f16,
                           Wq, (uint16_t *)scales_f16, zeros_u4, N);
    else
        hipLaunchKernelGGL(w4_quantize_kernel<false>, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t *)W_f16,
                           Wq, (uint16_t *)scales_f16, zeros_u4, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("w4_quantize launch", e);
    return W4_OK;
}

w4_status w4_read_probe(const void *src, int64_t bytes, uint32_t *xor_out, int64_t blocks, void *stream)
{
    if (!src || !xor_out) {
        set_error("w4_read_probe: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    if (bytes < 16 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31) || blocks < 1 || blocks > 65535) {
        set_error("w4_read_probe: bytes=%lld blocks=%lld: need 16<=bytes<2^31, bytes%%16==0, 1<=blocks<=65535",
                  (long long)bytes, (long long)blocks);
        return W4_ERR_SHAPE;
    }
    if (!aligned(src, 16) || !aligned(xor_out, 4)) {
        set_error("w4_read_probe: src must be 16-byte aligned and xor_out 4-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    w4_status st = check_device(&dev);
    if (st != W4_OK) return st;
    hipLaunchKernelGGL(w4_read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       src, (uint32_t)(bytes / 16), xor_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("w4_read_probe launch", e);
    return W4_OK;
}

w4_status w4_pack(const uint8_t *q_u4, uint32_t *Wq, int64_t K, int64_t N, void *stream)
{
    if (!q_u4 || !Wq) {
        set_error("w4_pack: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    if (K < 8 || K % 8 != 0 || N < 1 || K > ((int64_t)1 << 40) / N) {
        set_error("w4_pack: shape K=%lld N=%lld: need K>=8, K%%8==0, N>=1", (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    if (!aligned(Wq, 4)) {
        set_error("w4_pack: Wq must be 4-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    w4_status st = check_device(&dev);
    if (st != W4_OK) return st;
    const int64_t total = (K / 8) * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       q_u4, Wq, K / 8, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("w4_pack launch", e);
    return W4_OK;
}

w4_status w8_pack(const uint8_t *q_u8, uint32_t *Wq8, int64_t K, int64_t N, void *stream)
{
    if (!q_u8 || !Wq8) {
        set_error("w8_pack: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    if (K < 4 || K % 4 != 0 || N < 1 || K > ((int64_t)1 << 40) / N) {
        set_error("w8_pack: shape K=%lld N=%lld: need K>=4, K%%4==0, N>=1", (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    if (!aligned(Wq8, 4)) {
        set_error("w8_pack: Wq8 must be 4-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    w4_status st = check_device(&dev);
    if (st != W4_OK) return st;
    const int64_t total = (K / 4) * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(w8_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       q_u8, Wq8, K / 4, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("w8_pack launch", e);
    return W4_OK;
}

}  // extern "C"
