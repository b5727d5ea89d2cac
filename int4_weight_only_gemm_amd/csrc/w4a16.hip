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
// Hardware mapping (MI355X, CDNA4):
//  * Weights are streamed once from HBM with 16-byte non-temporal loads; a lane's load
//    holds four adjacent columns of one packed row (8 codes each).
//  * (q - z) is built in registers as exact binary16 pairs: a code is OR-ed into the
//    mantissa of 1024.0 (or of 1024.0 + 16 q for the odd nibble of a byte) and the zero
//    point is removed with one packed fp16 add/fma.  That is 9 VALU ops per 8 weights.
//  * The products run on the matrix cores (v_mfma_f32_16x16x32_f16).  The activation tile
//    is converted from bfloat16 to binary16 in LDS with a power-of-two scale per row and
//    128-wide group, chosen so that row's largest magnitude in the group lands in
//    [2^15, 2^16); the scale is undone exactly when the group's float32 partial is
//    rescaled by s.  Every product a*(q-z) is then exact; bfloat16 values more than 2^29
//    below the largest magnitude of their row within the group may be flushed (error
//    below 2^-29 of that maximum per element).
//  * Split-K across workgroups writes float32 partials to a workspace with device-coherent
//    stores; a per-tile arrival counter elects the last workgroup, which sums the partials
//    in split order, writes C and resets the counter.  One launch per GEMM, no memset, no
//    cache flush, bitwise reproducible.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
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
constexpr int kWaves = 4;                  // waves per workgroup; each takes its own groups
constexpr int kThreads = kWave * kWaves;
constexpr int kTileN = 64;                 // output columns per workgroup (16 lanes x 4 words)
constexpr int kTileM = 16;                 // output rows per M-block (one MFMA tile)
constexpr int kGroup = 128;                // quantization group along K
constexpr int kChunksPerRow = kGroup / 8;  // 16-byte activation chunks per group row
constexpr int kARowBytes = (kChunksPerRow + 1) * 16;  // +16 bytes of padding: conflict-free reads
constexpr int kMaxChunksPerThread = 12;     // activation slice <= 12 x 256 chunks (51 KiB of LDS)
constexpr int kMaxSliceRowGroups = kMaxChunksPerThread * kThreads / kChunksPerRow;  // rows x groups
constexpr int kRedBytes = kWaves * kTileM * kTileN * 4;
constexpr int kTargetWorkgroups = 768;  // 256 CUs x 3 resident workgroups (3 waves per SIMD)
constexpr int kCacheStream = 2;         // buffer-load cache policy: non-temporal (streamed once)

struct SmallParams {
    const uint16_t *A;
    const uint32_t *Wq;
    const uint16_t *S;
    const uint8_t *Z;
    float *C;
    float *part;        // [m_blocks * n_tiles][splits][16][64] float32 partials
    unsigned *count;    // [m_blocks * n_tiles] arrival counters, zero between calls
    int64_t M, K, N;
    int groups, splits, gps, n_tiles, m_blocks;
};

// ------------------------------------------------------------------------------------
// Bit-level helpers

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Eight codes of one packed word -> eight exact binary16 values (q_j - z), in the order
// j = 0,4,1,5,2,6,3,7 (element e holds nibble (e >> 1) + 4 * (e & 1)).
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

// Largest biased bfloat16 exponent among the 8 values of a chunk.
__device__ __forceinline__ int chunk_max_exp(u32x4 v)
{
    int e = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t u = v[i];
        int lo = (int)((u >> 7) & 0xFFu), hi = (int)((u >> 23) & 0xFFu);
        e = max(e, max(lo, hi));
    }
    return e;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    f16x2 h = {(_Float16)a, (_Float16)b};
    return as_u(h);
}

// 8 bfloat16 values (k order 0..7) -> 8 binary16 values scaled by 2^x, in the same
// element order as unpack8 (0,4,1,5,2,6,3,7).
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
// Register slot of one wave for one group: 4 packed rows (one 16-byte load per lane each)
// and the group's scales and zeros for the lane's 4 columns.
struct GroupRegs {
    u32x4 w[4];
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
    __amdgpu_buffer_rsrc_t W, S, Z, A;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

template <bool VEC>
__device__ __forceinline__ void lane_offsets(const SmallParams &p, int n0, int lane, LaneOffsets<VEC> &o)
{
    const int c = lane & 15, kq = lane >> 4;
    const int64_t N = p.N;
    const int64_t col = n0 + 4 * c;
    if (VEC) {
        const int64_t colv = col < N - 4 ? col : N - 4;  // N % 4 == 0, so N >= 4
        o.w[0] = (uint32_t)((kq * N + colv) * 4);
        o.s[0] = (uint32_t)(colv * 2);
        o.z[0] = (uint32_t)colv;
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t ct = col + t < N ? col + t : N - 1;
            o.w[t] = (uint32_t)((kq * N + ct) * 4);
            o.s[t] = (uint32_t)(ct * 2);
            o.z[t] = (uint32_t)ct;
        }
    }
}

template <bool VEC>
__device__ __forceinline__ void load_group(const SmallParams &p, const Resources &rs,
                                           const LaneOffsets<VEC> &o, int g, GroupRegs &r)
{
    const uint32_t rowbytes = (uint32_t)p.N * 4;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const uint32_t so = ((uint32_t)g * 16 + 4 * st) * rowbytes;
        if (VEC) {
            r.w[st] = __builtin_amdgcn_raw_buffer_load_b128(rs.W, o.w[0], so, kCacheStream);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) r.w[st][t] = __builtin_amdgcn_raw_buffer_load_b32(rs.W, o.w[t], so, kCacheStream);
        }
    }
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

// One group of one wave: 4 MFMA steps per column subtile into the group partial P, then
// acc += s * P (the activation tile is in LDS, scaled per row by 2^x).
__device__ __forceinline__ void compute_group(const GroupRegs &r, const char *lds_group, int mv, int lane,
                                              f32x4 (&acc)[4])
{
    const int c = lane & 15, kq = lane >> 4;
    uint32_t magic;
    asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    uint32_t zlo[4], zhi[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t z = (r.z >> (8 * t)) & 0xFu;
        zlo[t] = (0xE400u | z) * 0x00010001u;         // -(1024 + z)
        zhi[t] = (0xD400u | (z << 4)) * 0x00010001u;  // -(64 + z)
        // keep them in registers for the whole group instead of re-deriving per word
        asm volatile("" : "+v"(zlo[t]), "+v"(zhi[t]));
    }
    f32x4 P[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) P[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f16x8 a_op = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
        if (c < mv) a_op = __builtin_bit_cast(f16x8, *(const u32x4 *)(lds_group + c * kARowBytes + (4 * st + kq) * 16));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f16x8 b_op = unpack8(r.w[st][t], zlo[t], zhi[t], magic);
            P[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op, b_op, P[t], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint16_t sb = (uint16_t)(r.s[t >> 1] >> (16 * (t & 1)));
        const float sv = (float)__builtin_bit_cast(_Float16, sb);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(sv, P[t][i], acc[t][i]);
    }
}

// Workgroup-wide barrier for LDS only: waits for this wave's LDS operations, not for its
// global loads, so the weight loads already in flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Stage the workgroup's activation slice A[m0 .. m0+mv-1, 128 g_begin .. 128 g_end) into
// LDS as binary16, row r scaled by 2^x[r] with x[r] = 142 - (largest biased exponent of
// row r in the slice), which puts the row's largest magnitude in [2^15, 2^16).  Layout:
// group gl, row r, chunk kc (8 values) at gl*mv*272 + r*272 + kc*16; 16 bytes of padding
// per row keep the MFMA operand reads free of bank conflicts.  row_e ends up holding the
// row exponents (0 for rows >= mv).
__device__ __forceinline__ void stage_slice(const SmallParams &p, const Resources &rs, int m0, int mv,
                                            int g_begin, int ng, char *lds_a, int *row_e)
{
    const int tid = threadIdx.x;
    const int nch = mv * ng * kChunksPerRow;
    u32x4 v[kMaxChunksPerThread];
#pragma unroll
    for (int i = 0; i < kMaxChunksPerThread; ++i) {
        int ch = tid + kThreads * i;
        ch = ch < nch ? ch : nch - 1;  // branch-free: spare threads reload the last chunk
        const int kc = ch % kChunksPerRow, gr = ch / kChunksPerRow;
        const int r = gr % mv, gl = gr / mv;
        const uint32_t off = (uint32_t)(((int64_t)(m0 + r) * p.K + (int64_t)(g_begin + gl) * kGroup + kc * 8) * 2);
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.A, off, 0, 0);
    }
    if (tid < kTileM) row_e[tid] = 1;  // smallest normal exponent: all-zero rows stay at 2^0 scale
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kMaxChunksPerThread; ++i) {
        const int ch = tid + kThreads * i;
        if (ch < nch) atomicMax(row_e + (ch / kChunksPerRow) % mv, chunk_max_exp(v[i]));
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kMaxChunksPerThread; ++i) {
        const int ch = tid + kThreads * i;
        if (ch < nch) {
            const int gr = ch / kChunksPerRow;
            const int x = 142 - row_e[gr % mv];
            *(u32x4 *)(lds_a + gr * kARowBytes + (ch % kChunksPerRow) * 16) = convert_chunk(v[i], x);
        }
    }
    lds_barrier();
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void w4a16_small_m_kernel(SmallParams p)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];  // activation slice, then reduction
    __shared__ int row_e[kTileM];
    __shared__ int s_last;

    const uint32_t logical = xcd_local_id(blockIdx.x, gridDim.x);
    const int sp = (int)(logical % (uint32_t)p.splits);
    const uint32_t tile = logical / (uint32_t)p.splits;
    const int nt = (int)(tile % (uint32_t)p.n_tiles);
    const int mb = (int)(tile / (uint32_t)p.n_tiles);
    const int n0 = nt * kTileN, m0 = mb * kTileM;
    const int mv = (p.M - m0 < kTileM) ? (int)(p.M - m0) : kTileM;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
    const int c = lane & 15, kq = lane >> 4;

    // This workgroup's groups are [g_begin, g_end); wave w takes g_begin + w, + 4, ...
    const int g_begin = sp * p.gps;
    const int g_end = min(p.groups, g_begin + p.gps);
    const int g0 = g_begin + wave;
    const int n_my = g0 < g_end ? (g_end - g0 + kWaves - 1) / kWaves : 0;

    Resources rs;
    rs.W = __builtin_amdgcn_make_buffer_rsrc((void *)p.Wq, (short)0, (int)(p.K / 8 * p.N * 4), kRsrcWord3);
    rs.S = __builtin_amdgcn_make_buffer_rsrc((void *)p.S, (short)0, (int)(p.K / kGroup * p.N * 2), kRsrcWord3);
    rs.Z = __builtin_amdgcn_make_buffer_rsrc((void *)p.Z, (short)0, (int)(p.K / kGroup * p.N), kRsrcWord3);
    rs.A = __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)(p.M * p.K * 2), kRsrcWord3);
    LaneOffsets<VEC> lo;
    lane_offsets<VEC>(p, n0, lane, lo);

    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The first group's weights are requested before the activation slice is staged, so
    // their latency overlaps the staging.
    GroupRegs r0, r1, r2;
    auto G = [&](int j) { return g0 + kWaves * j; };
    if (n_my > 0) load_group<VEC>(p, rs, lo, G(0), r0);
    stage_slice(p, rs, m0, mv, g_begin, g_end - g_begin, lds, row_e);
    if (n_my > 1) load_group<VEC>(p, rs, lo, G(1), r1);

    // Three register slots: while group j is computed, groups j+1 and j+2 are in flight.
    // The steady-state loop issues only loads that exist; the last 1-4 groups are peeled.
    if (n_my > 0) {
        auto run = [&](const GroupRegs &r, int j) {
            compute_group(r, lds + (wave + kWaves * j) * mv * kARowBytes, mv, lane, acc);
        };
        int j = 0;
        for (; j + 4 < n_my; j += 3) {
            load_group<VEC>(p, rs, lo, G(j + 2), r2);
            run(r0, j);
            load_group<VEC>(p, rs, lo, G(j + 3), r0);
            run(r1, j + 1);
            load_group<VEC>(p, rs, lo, G(j + 4), r1);
            run(r2, j + 2);
        }
        const int rem = n_my - j;  // 1..4 groups left; r0 (and r1) already loaded
        if (rem >= 3) load_group<VEC>(p, rs, lo, G(j + 2), r2);
        run(r0, j);
        if (rem == 4) load_group<VEC>(p, rs, lo, G(j + 3), r0);
        if (rem >= 2) run(r1, j + 1);
        if (rem >= 3) run(r2, j + 2);
        if (rem == 4) run(r0, j + 3);
    }

    // Undo the activation scale: output rows 4 kq + i were computed from A * 2^x[row].
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * kq + i;
        const int x = 142 - row_e[row < kTileM ? row : 0];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][i] = ldexpf(acc[t][i], -x);
    }

    // Reduce the 4 waves' accumulators through LDS (fixed order -> reproducible).
    __syncthreads();
    float *red = (float *)lds;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 v = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
        *(f32x4 *)(red + (wave * kTileM + 4 * kq + i) * kTileN + 4 * c) = v;
    }
    __syncthreads();
    const int row = threadIdx.x >> 4, quad = threadIdx.x & 15;
    f32x4 sum = *(const f32x4 *)(red + (0 * kTileM + row) * kTileN + 4 * quad);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += *(const f32x4 *)(red + (w * kTileM + row) * kTileN + 4 * quad);

    const int64_t col = n0 + 4 * quad;
    auto store_c = [&](const f32x4 &v) {
        if (row >= mv) return;
        float *dst = p.C + (int64_t)(m0 + row) * p.N + col;
        if (VEC) {
            if (col < p.N) *(f32x4 *)dst = v;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (col + t < p.N) dst[t] = v[t];
        }
    };

    if (p.splits == 1) {
        store_c(sum);
        return;
    }

    // Split-K handoff.  Partials are written with device-coherent (write-through) stores
    // and read back with device-coherent loads, so no L2 writeback or invalidate is
    // needed: every thread waits for its stores to complete, the barrier orders that
    // before thread 0 counts the arrival, and the workgroup that arrives last sums the
    // partials in split order.
    float *tile_part = p.part + (int64_t)tile * p.splits * (kTileM * kTileN);
    if (row < mv) {
        float *dst = tile_part + (int64_t)sp * (kTileM * kTileN) + row * kTileN + 4 * quad;
#pragma unroll
        for (int t = 0; t < 4; ++t) __hip_atomic_store(dst + t, sum[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(p.count + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(p.splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    asm volatile("" ::: "memory");
    if (row < mv) {
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        for (int sp2 = 0; sp2 < p.splits; ++sp2) {
            const float *src = tile_part + (int64_t)sp2 * (kTileM * kTileN) + row * kTileN + 4 * quad;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                tot[t] += __hip_atomic_load(src + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        store_c(tot);
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

w4_status validate_gemm_shape(int64_t M, int64_t K, int64_t N)
{
    if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) {
        set_error("shape M=%lld K=%lld N=%lld: need M>=1, N>=1, K>=128, K%%128==0",
                  (long long)M, (long long)K, (long long)N);
        return W4_ERR_SHAPE;
    }
    // the kernels address each array with 32-bit byte offsets
    if (K / 8 * N * 4 >= ((int64_t)1 << 31) || M * K * 2 >= ((int64_t)1 << 31)) {
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

void make_plan(int64_t M, int64_t K, int64_t N, w4_plan *pl)
{
    const int groups = (int)(K / kGroup);
    const int n_tiles = (int)((N + kTileN - 1) / kTileN);
    const int m_blocks = (int)((M + kTileM - 1) / kTileM);
    const int rows = M < kTileM ? (int)M : kTileM;
    const int64_t base = (int64_t)n_tiles * m_blocks;
    // enough workgroups to fill the GPU, at least one group per wave ...
    int splits = (int)((kTargetWorkgroups + base - 1) / base);
    const int max_splits = groups / kWaves > 1 ? groups / kWaves : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    // ... and an activation slice (rows x groups) that fits the LDS budget
    const int max_gps = kMaxSliceRowGroups / rows;
    const int min_splits = (groups + max_gps - 1) / max_gps;
    if (splits < min_splits) splits = min_splits;
    const int gps = (groups + splits - 1) / splits;
    splits = (groups + gps - 1) / gps;
    pl->kernel = 1;
    pl->m_blocks = m_blocks;
    pl->n_tiles = n_tiles;
    pl->splits = splits;
    pl->groups_per_split = gps;
    pl->workgroups = base * splits;
    pl->workspace_bytes = splits > 1 ? base * 4 + base * splits * kTileM * kTileN * 4 : 0;
}

size_t slice_lds_bytes(int64_t M, const w4_plan &pl)
{
    const int rows = M < kTileM ? (int)M : kTileM;
    const size_t slice = (size_t)rows * pl.groups_per_split * kARowBytes;
    return slice > (size_t)kRedBytes ? slice : (size_t)kRedBytes;
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
    return W4_OK;
}

w4_status w4a16_gemm(const void *A_bf16, const uint32_t *Wq, const void *scales_f16,
                     const uint8_t *zeros_u4, float *C, int64_t M, int64_t K, int64_t N,
                     void *stream)
{
    if (!A_bf16 || !Wq || !scales_f16 || !zeros_u4 || !C) {
        set_error("w4a16_gemm: a required pointer is NULL");
        return W4_ERR_NULL;
    }
    w4_status st = validate_gemm_shape(M, K, N);
    if (st != W4_OK) return st;
    if (!aligned(A_bf16, 16) || !aligned(Wq, 16) || !aligned(C, 16) || !aligned(scales_f16, 2)) {
        set_error("w4a16_gemm: A, Wq and C must be 16-byte aligned and scales 2-byte aligned");
        return W4_ERR_ALIGN;
    }
    int dev = -1;
    st = check_device(&dev);
    if (st != W4_OK) return st;

    w4_plan pl;
    make_plan(M, K, N, &pl);
    SmallParams p;
    p.A = (const uint16_t *)A_bf16;
    p.Wq = Wq;
    p.S = (const uint16_t *)scales_f16;
    p.Z = zeros_u4;
    p.C = C;
    p.part = nullptr;
    p.count = nullptr;
    p.M = M;
    p.K = K;
    p.N = N;
    p.groups = (int)(K / kGroup);
    p.splits = pl.splits;
    p.gps = pl.groups_per_split;
    p.n_tiles = pl.n_tiles;
    p.m_blocks = pl.m_blocks;
    hipStream_t s = (hipStream_t)stream;
    if (pl.splits > 1) {
        const int64_t tiles = (int64_t)pl.n_tiles * pl.m_blocks;
        st = get_workspace(dev, s, (size_t)tiles, (size_t)tiles * pl.splits * kTileM * kTileN * 4,
                           &p.count, &p.part);
        if (st != W4_OK) return st;
    }
    const bool vec = (N % 4 == 0) && aligned(scales_f16, 8) && aligned(zeros_u4, 4);
    const size_t lds = slice_lds_bytes(M, pl);
    if (vec)
        hipLaunchKernelGGL(w4a16_small_m_kernel<true>, dim3((unsigned)pl.workgroups), dim3(kThreads), lds, s, p);
    else
        hipLaunchKernelGGL(w4a16_small_m_kernel<false>, dim3((unsigned)pl.workgroups), dim3(kThreads), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("w4a16_gemm launch", e);
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

}  // extern "C"
