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
//    is converted from bfloat16 to binary16 in LDS with a power-of-two scale per 128-wide
//    group, chosen so the group's largest magnitude lands in [2^15, 2^16); the scale is
//    undone exactly when the group's float32 partial is rescaled by s.  Every product
//    a*(q-z) is then exact; bfloat16 values more than 2^29 below their group's maximum
//    may be flushed (error below 2^-29 of that maximum per element).
//  * Split-K across workgroups writes float32 partials to a workspace; a per-tile arrival
//    counter elects the last workgroup, which sums the partials in split order, writes C
//    and resets the counter.  One launch per GEMM, no memset, bitwise reproducible.

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
constexpr int kLdsRowChunks = kChunksPerRow + 1;  // +1 chunk of padding: conflict-free reads
constexpr int kLdsWaveBytes = kTileM * kLdsRowChunks * 16;
constexpr int kLdsBufBytes = kWaves * kLdsWaveBytes;
constexpr int kRedBytes = kWaves * kTileM * kTileN * 4;
constexpr int kLdsBytes = (2 * kLdsBufBytes > kRedBytes) ? 2 * kLdsBufBytes : kRedBytes;
constexpr int kTargetWorkgroups = 512;

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

__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
    return v;
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
// Per-group register set of one wave: 4 packed rows (one 16-byte load per lane each),
// the group's scales and zeros for the lane's 4 columns, and up to 4 activation chunks.
struct GroupRegs {
    u32x4 w[4];
    u32x2 s;      // 4 binary16 scales
    uint32_t z;   // 4 zero bytes
    u32x4 a[4];
};

template <bool VEC>
__device__ __forceinline__ void load_group(const SmallParams &p, int g, int n0, int m0, int mv,
                                           int lane, GroupRegs &r)
{
    const int c = lane & 15, kq = lane >> 4;
    const int64_t N = p.N;
    const int64_t col = n0 + 4 * c;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int64_t row = (int64_t)g * 16 + 4 * st + kq;
        const uint32_t *src = p.Wq + row * N + col;
        if (VEC) {
            r.w[st] = (col < N) ? __builtin_nontemporal_load((const u32x4 *)src) : u32x4{0, 0, 0, 0};
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                r.w[st][t] = (col + t < N) ? __builtin_nontemporal_load(src + t) : 0u;
        }
    }
    const int64_t gi = (int64_t)g * N + col;
    if (VEC) {
        r.s = (col < N) ? *(const u32x2 *)(p.S + gi) : u32x2{0, 0};
        r.z = (col < N) ? *(const uint32_t *)(p.Z + gi) : 0u;
    } else {
        uint32_t s01 = 0, s23 = 0, zz = 0;
        if (col + 0 < N) { s01 |= p.S[gi + 0]; zz |= (uint32_t)p.Z[gi + 0]; }
        if (col + 1 < N) { s01 |= (uint32_t)p.S[gi + 1] << 16; zz |= (uint32_t)p.Z[gi + 1] << 8; }
        if (col + 2 < N) { s23 |= p.S[gi + 2]; zz |= (uint32_t)p.Z[gi + 2] << 16; }
        if (col + 3 < N) { s23 |= (uint32_t)p.S[gi + 3] << 16; zz |= (uint32_t)p.Z[gi + 3] << 24; }
        r.s = u32x2{s01, s23};
        r.z = zz;
    }
    // activation chunks: chunk id ch = lane + 64 i -> row ch / 16, chunk ch % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ch = lane + 64 * i;
        const int rr = ch >> 4, kc = ch & 15;
        if (rr < mv) {
            const uint16_t *src = p.A + (int64_t)(m0 + rr) * p.K + (int64_t)g * kGroup + kc * 8;
            r.a[i] = *(const u32x4 *)src;
        } else {
            r.a[i] = u32x4{0, 0, 0, 0};
        }
    }
}

// One group of one wave: activation staging (already in LDS), 4 MFMA steps per column
// subtile, then acc += s * 2^-x * P.
__device__ __forceinline__ void compute_group(const GroupRegs &r, const char *lds_wave, int x,
                                              int mv, int lane, f32x4 (&acc)[4])
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
        f16x8 a_op;
        if (c < mv) {
            const u32x4 av = *(const u32x4 *)(lds_wave + (c * kLdsRowChunks + 4 * st + kq) * 16);
            a_op = __builtin_bit_cast(f16x8, av);
        } else {
            a_op = __builtin_bit_cast(f16x8, u32x4{0, 0, 0, 0});
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f16x8 b_op = unpack8(r.w[st][t], zlo[t], zhi[t], magic);
            P[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op, b_op, P[t], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint16_t sb = (uint16_t)(r.s[t >> 1] >> (16 * (t & 1)));
        const float sc = ldexpf((float)__builtin_bit_cast(_Float16, sb), -x);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(sc, P[t][i], acc[t][i]);
    }
}

// Stage the wave's group of activations into LDS as scaled binary16; return the scale
// exponent x (the group's values were multiplied by 2^x).
__device__ __forceinline__ int stage_activations(const GroupRegs &r, char *lds_wave, int mv, int lane)
{
    int e = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) e = max(e, chunk_max_exp(r.a[i]));
    e = wave_max(e);
    e = max(e, 1);            // all-zero / subnormal groups use the smallest normal exponent
    const int x = 142 - e;    // largest magnitude -> [2^15, 2^16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ch = lane + 64 * i;
        const int rr = ch >> 4, kc = ch & 15;
        if (rr < mv) *(u32x4 *)(lds_wave + (rr * kLdsRowChunks + kc) * 16) = convert_chunk(r.a[i], x);
    }
    return x;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void w4a16_small_m_kernel(SmallParams p)
{
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    __shared__ int s_last;

    const uint32_t logical = xcd_local_id(blockIdx.x, gridDim.x);
    const int sp = (int)(logical % (uint32_t)p.splits);
    const uint32_t tile = logical / (uint32_t)p.splits;
    const int nt = (int)(tile % (uint32_t)p.n_tiles);
    const int mb = (int)(tile / (uint32_t)p.n_tiles);
    const int n0 = nt * kTileN, m0 = mb * kTileM;
    const int mv = (p.M - m0 < kTileM) ? (int)(p.M - m0) : kTileM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, kq = lane >> 4;

    const int g_begin = sp * p.gps;
    const int g_end = min(p.groups, g_begin + p.gps);
    const int rounds = (g_end - g_begin + kWaves - 1) / kWaves;

    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Every wave runs the same number of rounds (barriers are workgroup-wide); a wave
    // whose group index falls past g_end skips the work of that round.
    GroupRegs ra, rb;
    int g = g_begin + wave;
    if (g < g_end) load_group<VEC>(p, g, n0, m0, mv, lane, ra);
    for (int rd = 0; rd < rounds; rd += 2) {
        {
            const int gn = g + kWaves;
            if (gn < g_end) load_group<VEC>(p, gn, n0, m0, mv, lane, rb);
            char *buf = lds + (rd & 1) * kLdsBufBytes + wave * kLdsWaveBytes;
            int x = 0;
            if (g < g_end) x = stage_activations(ra, buf, mv, lane);
            __syncthreads();
            if (g < g_end) compute_group(ra, buf, x, mv, lane, acc);
            g = gn;
        }
        if (rd + 1 < rounds) {
            const int gn = g + kWaves;
            if (gn < g_end) load_group<VEC>(p, gn, n0, m0, mv, lane, ra);
            char *buf = lds + ((rd + 1) & 1) * kLdsBufBytes + wave * kLdsWaveBytes;
            int x = 0;
            if (g < g_end) x = stage_activations(rb, buf, mv, lane);
            __syncthreads();
            if (g < g_end) compute_group(rb, buf, x, mv, lane, acc);
            g = gn;
        }
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

    float *tile_part = p.part + (int64_t)tile * p.splits * (kTileM * kTileN);
    if (row < mv) *(f32x4 *)(tile_part + (int64_t)sp * (kTileM * kTileN) + row * kTileN + 4 * quad) = sum;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(p.count + tile, 1u);
        s_last = (prev == (unsigned)(p.splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (row < mv) {
        f32x4 tot = *(const f32x4 *)(tile_part + row * kTileN + 4 * quad);
        for (int s = 1; s < p.splits; ++s)
            tot += *(const f32x4 *)(tile_part + (int64_t)s * (kTileM * kTileN) + row * kTileN + 4 * quad);
        store_c(tot);
    }
    if (threadIdx.x == 0) atomicExch(p.count + tile, 0u);
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
    size_t bytes = 0;
};
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;
std::vector<char *> g_retired;  // superseded buffers stay valid for graphs captured earlier

// Workspace layout: [counters, 256-byte aligned][partials]
w4_status get_workspace(int dev, hipStream_t stream, size_t counter_bytes, size_t part_bytes,
                        unsigned **count, float **part)
{
    const size_t cb = (counter_bytes + 255) & ~(size_t)255;
    const size_t need = cb + part_bytes;
    std::lock_guard<std::mutex> lock(g_mutex);
    Workspace &ws = g_workspaces[{dev, stream}];
    if (ws.bytes < need) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return hip_fail("hipStreamIsCapturing", e);
        if (cs != hipStreamCaptureStatusNone) {
            set_error("split-K workspace must grow to %zu bytes while the stream is capturing; "
                      "run this shape once before capture", need);
            return W4_ERR_WORKSPACE;
        }
        size_t bytes = need < ((size_t)1 << 20) ? ((size_t)1 << 20) : need;
        bytes = (bytes + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
        char *fresh = nullptr;
        e = hipMalloc((void **)&fresh, bytes);
        if (e != hipSuccess) return hip_fail("hipMalloc(workspace)", e);
        // Counters must start at zero; every call leaves them at zero again.
        e = hipMemsetAsync(fresh, 0, bytes, stream);
        if (e != hipSuccess) return hip_fail("hipMemsetAsync(workspace)", e);
        if (ws.ptr) g_retired.push_back(ws.ptr);
        ws.ptr = fresh;
        ws.bytes = bytes;
    }
    *count = (unsigned *)ws.ptr;
    *part = (float *)(ws.ptr + cb);
    return W4_OK;
}

w4_status validate_gemm_shape(int64_t M, int64_t K, int64_t N)
{
    if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) {
        set_error("shape M=%lld K=%lld N=%lld: need M>=1, N>=1, K>=128, K%%128==0",
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
    const int64_t base = (int64_t)n_tiles * m_blocks;
    int splits = (int)((kTargetWorkgroups + base - 1) / base);
    const int max_splits = groups / kWaves > 1 ? groups / kWaves : 1;  // >= 1 group per wave
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    const int gps = (groups + splits - 1) / splits;
    splits = (groups + gps - 1) / gps;
    pl->kernel = 1;
    pl->m_blocks = m_blocks;
    pl->n_tiles = n_tiles;
    pl->splits = splits;
    pl->groups_per_split = gps;
    pl->workgroups = base * splits;
    pl->workspace_bytes = splits > 1
        ? (int64_t)((base * 4 + 255) & ~(int64_t)255) + base * splits * kTileM * kTileN * 4
        : 0;
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
        st = get_workspace(dev, s, (size_t)tiles * 4,
                           (size_t)tiles * pl.splits * kTileM * kTileN * 4, &p.count, &p.part);
        if (st != W4_OK) return st;
    }
    const bool vec = (N % 4 == 0) && aligned(scales_f16, 8) && aligned(zeros_u4, 4);
    if (vec)
        hipLaunchKernelGGL(w4a16_small_m_kernel<true>, dim3((unsigned)pl.workgroups), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(w4a16_small_m_kernel<false>, dim3((unsigned)pl.workgroups), dim3(kThreads), 0, s, p);
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
