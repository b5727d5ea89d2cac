"""HIP path against the oracle, element by element, through the C-ABI (needs gfx950).

Tolerance (per element, float64): |C_gpu - C_oracle| <= 1e-4 * sum_k |A[m,k] W[k,n]| + 1e-6.
Packing is compared bit for bit. Cases that are exact in float32 (one-hot A, q = z, s = 0)
are compared bit for bit as well.
"""
import numpy as np
import pytest
import torch

import int4_weight_only_gemm_amd as w4
import oracle
import synth
from gpu_helpers import check, host_words, log, run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


# ------------------------------------------------------------------------------ packing
@pytest.mark.parametrize("K,N", [(8, 1), (16, 3), (128, 64), (384, 257), (1536, 1536), (1024, 4099)])
def test_pack_bit_exact(orc, K, N):
    log(f"pack K={K} N={N}")
    r = np.random.default_rng(K * 7 + N)
    q = r.integers(0, 256, size=(K, N), dtype=np.uint8)  # garbage high nibbles included
    q[0, 0], q[-1, -1] = 0x0F, 0xF0
    Wq = w4.pack(torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(Wq.cpu().numpy().view(np.uint32), orc.pack(q))


@pytest.mark.parametrize("nbytes,blocks", [(32, 768), (48, 1), ((1 << 20) + 48, 7), ((1 << 24) + 4096, 768)])
def test_read_probe_reads_every_chunk(nbytes, blocks):
    # the streaming-read probe's per-wave XORs combine to the XOR of every word of the buffer
    log(f"read probe bytes={nbytes} blocks={blocks}")
    host = np.random.default_rng(nbytes).integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = w4.read_probe(buf, blocks=blocks)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32).ravel())
    assert got == np.bitwise_xor.reduce(host)
    # a probe over all but the last chunk misses exactly that chunk's words
    out = w4.read_probe(buf[: nbytes // 4 - 4], blocks=blocks)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32).ravel())
    assert got == np.bitwise_xor.reduce(host[:-4])


# ---------------------------------------------------------------- quantizer (w4_quantize)
def _quant_weights(K, N, seed):
    """binary16 weights with per-column magnitudes and special groups: all-zero, one-signed,
    constant, binary16-subnormal ranges and values near the binary16 maximum."""
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-3, 2, N)
    W = (rng.standard_normal((K, N)) * mag).astype(np.float16)
    G = K // 128
    for n in range(min(N, 7)):
        g = n % G
        rows = slice(128 * g, 128 * g + 128)
        if n == 0:
            W[rows, n] = 0
        elif n == 1:
            W[rows, n] = np.abs(W[rows, n])
        elif n == 2:
            W[rows, n] = -np.abs(W[rows, n])
        elif n == 3:
            W[rows, n] = np.float16(0.3)
        elif n == 4:
            W[rows, n] = (rng.standard_normal(128) * 2.0 ** -22).astype(np.float16)
        elif n == 5:
            W[rows, n] = (rng.uniform(-1, 1, 128) * 65504).astype(np.float16)
        elif n == 6:
            W[rows, n] = (rng.standard_normal(128) * 2.0 ** -16).astype(np.float16)
    return W


@pytest.mark.parametrize("K,N", [(128, 1), (256, 7), (384, 64), (1024, 4099), (3584, 4608), (128, 66000)])
def test_quantize_bit_exact(orc, K, N):
    log(f"quantize K={K} N={N}")
    W = _quant_weights(K, N, seed=K + N)
    Wq, S, Z = w4.quantize(torch.from_numpy(W).cuda())
    rWq, rS, rZ = orc.quantize(W.view(np.uint16))
    assert np.array_equal(Wq.cpu().numpy().view(np.uint32), rWq), "packed codes differ"
    assert np.array_equal(S.cpu().numpy().view(np.uint16), rS), "scales differ"
    assert np.array_equal(Z.cpu().numpy(), rZ), "zeros differ"


def test_quantize_ties_and_near_ties(orc):
    # weights at and next to grid midpoints: the kernel's reciprocal shortcut must hand
    # these to the IEEE division and round ties to even, exactly as the oracle does
    rng = np.random.default_rng(61)
    cols = []
    for s, z in [(0.5, 6), (0.125, 0), (3 * 2.0 ** -6, 8), (1.25, 3), (2.0 ** -10, 15), (0.75, 9), (5.0, 7)]:
        mid = (np.arange(15) - z + 0.5) * s
        ulp = np.spacing(np.abs(mid).astype(np.float16)).astype(np.float64)
        near = np.r_[mid, mid + ulp, mid - ulp]
        g = np.r_[-z * s, (15 - z) * s, rng.choice(near, 126)]
        cols.append(g)
    W = np.stack(cols, 1).astype(np.float16)
    W = np.concatenate([W, W[::-1]], 0)  # two groups
    Wq, S, Z = w4.quantize(torch.from_numpy(W).cuda())
    rWq, rS, rZ = orc.quantize(W.view(np.uint16))
    assert np.array_equal(Wq.cpu().numpy().view(np.uint32), rWq), "codes differ at or near ties"
    assert np.array_equal(S.cpu().numpy().view(np.uint16), rS) and np.array_equal(Z.cpu().numpy(), rZ)


def test_quantize_scalar_path(orc):
    # odd N, and views whose addresses rule out the paired stores: the scalar path
    K, N = 256, 1001
    W = _quant_weights(K, N, seed=3)
    dev = torch.from_numpy(W).cuda()
    Wq, S, Z = w4.quantize(dev)
    rWq, rS, rZ = orc.quantize(W.view(np.uint16))
    assert np.array_equal(Wq.cpu().numpy().view(np.uint32), rWq)
    assert np.array_equal(S.cpu().numpy().view(np.uint16), rS) and np.array_equal(Z.cpu().numpy(), rZ)
    buf = torch.empty(K * 1000 + 1, dtype=torch.float16, device="cuda")
    Wv = buf[1:].view(K, 1000)  # 2-byte aligned only
    W2 = _quant_weights(K, 1000, seed=4)
    Wv.copy_(torch.from_numpy(W2))
    Wq2 = torch.empty((K // 8, 1000), dtype=torch.int32, device="cuda")
    Sb = torch.empty(2 * 1000 + 1, dtype=torch.float16, device="cuda")
    Zb = torch.empty(2 * 1000 + 1, dtype=torch.uint8, device="cuda")
    w4.quantize_raw(Wv.data_ptr(), Wq2.data_ptr(), Sb[1:].data_ptr(), Zb[1:].data_ptr(), K, 1000,
                    torch.cuda.current_stream().cuda_stream)
    rWq2, rS2, rZ2 = orc.quantize(W2.view(np.uint16))
    assert np.array_equal(Wq2.cpu().numpy().view(np.uint32), rWq2)
    assert np.array_equal(Sb[1:].cpu().numpy().view(np.uint16).reshape(2, 1000), rS2)
    assert np.array_equal(Zb[1:].cpu().numpy().reshape(2, 1000), rZ2)


def test_quantize_then_gemm(orc):
    # the producer feeds the consumer: quantize on the GPU, multiply on the GPU, and compare
    # with the oracle's GEMM over the oracle's quantization of the same weights
    M, K, N = 5, 3584, 4608
    W = _quant_weights(K, N, seed=11)
    Wq, S, Z = w4.quantize(torch.from_numpy(W).cuda())
    x = synth.generate_custom(M, K, N, seed=12)
    A = torch.from_numpy(x.A.view(np.int16)).cuda().view(torch.bfloat16)
    C = w4.gemm(A, Wq, S, Z).cpu().numpy()
    rWq, rS, rZ = orc.quantize(W.view(np.uint16))
    Cr, Cabs = orc.gemm(x.A, rWq, rS, rZ)
    check(C, Cr, Cabs, "quantize then gemm")


# ------------------------------------------------------------------- tiny-shape grid
GRID_M = [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17, 63, 64, 65, 160]
GRID_K = [128, 256, 384, 1152]
GRID_N = [1, 3, 7, 8, 63, 64, 65, 257]


@pytest.mark.parametrize("M", GRID_M)
def test_grid(orc, M):
    worst = 0.0
    for K in GRID_K:
        for N in GRID_N:
            log(f"grid M={M} K={K} N={N}")
            x = synth.generate_custom(M, K, N, seed=1)
            dev = to_dev(x)
            C = run(dev).cpu().numpy()
            Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
            worst = max(worst, check(C, Cr, Cabs, f"M={M} K={K} N={N}"))
    log(f"grid M={M}: worst error / bound = {worst:.3g}")


@pytest.mark.parametrize("M,K,N", [(5, 4096, 64), (1, 18944, 100), (7, 8192, 200), (16, 2048, 36),
                                   (3, 11008, 4096), (160, 1024, 130)])
def test_split_k_shapes(orc, M, K, N):
    p = w4.plan(M, K, N)
    log(f"split-K M={M} K={K} N={N} plan={p}")
    x = synth.generate_custom(M, K, N, seed=2)
    C = run(to_dev(x)).cpu().numpy()
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(3).integers(0, N, 64)])
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
    check(C[:, cols], Cr, Cabs, f"split M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(5, 1024, 19200), (20, 1024, 16640), (40, 2048, 8576), (3, 2048, 19198),
                                   (1, 3584, 37888)])
def test_balanced_wide_plan(orc, M, K, N):
    # whole rounds of unsplit tiles plus split remainder tiles: both kinds of workgroup, the
    # split tiles' counters and partials, row blocks crossing the boundary, ragged N
    p = w4.plan(M, K, N)
    log(f"balanced M={M} K={K} N={N} plan={p}")
    assert p["kernel"] == 1 and p["full_tiles"] > 0 and p["splits"] > 1
    x = synth.generate_custom(M, K, N, seed=21)
    dev = to_dev(x)
    C1 = run(dev)
    C2 = run(dev)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2), "balanced plan not reproducible"
    C = C1.cpu().numpy()
    if M * K * N <= 400_000_000:
        cols = None
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    else:  # full-size shape: both column ranges, the neighbourhood of their boundary
        # tile t covers row block t % m_blocks of column tile t / m_blocks
        edge = 64 * (p["full_tiles"] // p["m_blocks"])
        cols = np.unique(np.r_[0, edge - 1, edge, N - 1, np.random.default_rng(22).integers(0, N, 96)])
        cols = cols[(cols >= 0) & (cols < N)]
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
        C = C[:, cols]
    check(C, Cr, Cabs, f"balanced M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(17, 4096, 8192), (24, 18944, 3584), (32, 4096, 8193), (33, 4096, 8192),
                                   (37, 4096, 8193), (40, 4096, 8200), (63, 18944, 3584), (48, 3584, 37888)])
def test_mid_m_bf16_path(orc, M, K, N):
    # 17 <= M < 64 on large GEMMs runs the bf16 kernel: a row block of M rows in one or two
    # 32-row tiles (rows past M masked), ragged and odd N, deep K splits
    p = w4.plan(M, K, N)
    log(f"mid-M bf16 path M={M} K={K} N={N} plan={p}")
    assert p["kernel"] == 3
    x = synth.generate_custom(M, K, N, seed=41)
    C = run(to_dev(x)).cpu().numpy()
    cols = np.unique(np.r_[0, 255, 256, N - 257, N - 256, N - 1,
                           np.random.default_rng(42).integers(0, N, 96)]).astype(np.int64)
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
    check(C[:, cols], Cr, Cabs, f"mid-M M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,full", [(17, 1664, 33333, True), (17, 2048, 40003, True), (23, 1792, 33333, True),
                                        (40, 2688, 24576, True), (48, 3584, 37888, False), (64, 3584, 37888, False)])
def test_shared_steps(orc, M, K, N, full):
    # plans whose (tile, group) steps are shared out evenly: workgroups that end one tile and
    # start the next, tiles with 3-4 partial slices, the per-tile reduction (scalar path for
    # N % 4 != 0), one and two row tiles; every element, or the columns around the tile
    # edges plus a random sample
    p = w4.plan(M, K, N)
    log(f"shared steps M={M} K={K} N={N} plan={p}")
    G = K // 128
    assert p["kernel"] == 3 and p["group_stride"] == G and G % p["groups_per_split"] and p["splits"] >= 3
    x = synth.generate_custom(M, K, N, seed=43)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run(to_dev(x), out=out).cpu().numpy()
    if full:
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    else:
        edges = np.arange(256, N, 256)
        cols = np.unique(np.r_[0, N - 1, edges - 1, edges, np.random.default_rng(44).integers(0, N, 64)])
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
        C = C[:, cols]
    check(C, Cr, Cabs, f"shared steps M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(5, 65536, 65528), (64, 65536, 65528), (63, 1 << 24, 1), (8191, 131072, 8)])
def test_maximum_sizes(orc, M, K, N):
    # the largest arrays the kernels' 32-bit byte offsets address: packed weights
    # (K/8*N*4) or activations (M*K*2) just under 2 GiB, on both kernels; sampled rows and
    # columns (edges, row-block and tile boundaries) against the oracle
    assert K // 8 * N * 4 < 1 << 31 and M * K * 2 < 1 << 31
    p = w4.plan(M, K, N)
    log(f"maximum size M={M} K={K} N={N} plan={p}")
    x = synth.generate_custom(M, K, N, seed=31)
    dev = to_dev(x)
    C = run(dev).cpu().numpy()
    del dev
    rng = np.random.default_rng(32)
    rows = np.unique(np.r_[0, M - 1, [r for r in (15, 16, 159, 160, 4095) if r < M],
                           rng.integers(0, M, 4)]).astype(np.int64)
    cols = np.unique(np.r_[0, N - 1, [c for c in (63, 64, 255, 256) if c < N],
                           rng.integers(0, N, 24)]).astype(np.int64)
    Cr, Cabs = orc.gemm(x.A[rows], x.Wq, x.S, x.Z, cols=cols)
    check(C[np.ix_(rows, cols)], Cr, Cabs, f"max size M={M} K={K} N={N}")


# ------------------------------------------------------------- narrow-tile kernel
NARROW_SHAPES = [(1, 8192, 4095), (5, 3584, 3584), (8, 3584, 1000), (16, 1792, 300), (3, 128, 17),
                 (7, 640, 4096), (2, 8064, 33), (4, 1024, 1), (6, 2304, 257), (1, 1536, 2048)]


@pytest.mark.parametrize("M,K,N", NARROW_SHAPES)
def test_narrow_kernel_every_element(orc, M, K, N):
    # one 16-column tile per workgroup over all of K: 64 groups (eight per wave, the most a
    # wave holds), one group (seven idle waves), ragged N down to a single column, 16 rows,
    # 256 tiles; NaN-poisoned C, every element against the oracle
    p = w4.plan(M, K, N)
    log(f"narrow M={M} K={K} N={N} plan={p}")
    assert p["kernel"] == 8 and p["tile_n"] == 16 and p["splits"] == 1
    x = synth.generate_custom(M, K, N, seed=61)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run(to_dev(x), out=out).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    check(C, Cr, Cabs, f"narrow M={M} K={K} N={N}")


def test_narrow_kernel_one_hot_and_zero_bitwise(orc):
    # exact special cases on the narrow kernel: one-hot rows extract one dequantized row bit
    # for bit, and q == z gives exact zeros
    M, K, N = 5, 2048, 200
    assert w4.plan(M, K, N)["kernel"] == 8
    x = synth.generate_custom(M, K, N, seed=62)
    dev = to_dev(x)
    for (m0, k0, a0) in ((0, 0, 1.0), (M - 1, K - 1, -2.5), (2, 1037, 3.0e4), (3, 128, -0.0078125)):
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        Ab = synth.f32_to_bf16_bits(A)
        dev["A"] = torch.from_numpy(Ab.view(np.int16)).cuda().view(torch.bfloat16)
        log(f"narrow one-hot m={m0} k={k0} a={a0}")
        C = run(dev).cpu().numpy().astype(np.float64)
        Cr, _ = orc.gemm(Ab, x.Wq, x.S, x.Z)
        assert np.array_equal(C, Cr), f"one-hot ({m0},{k0}) differs"
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)
    C = run(to_dev(synth.GemmInputs(A=x.A, Wq=orc.pack(q), q=None, S=x.S, Z=x.Z))).cpu().numpy()
    assert np.all(C == 0.0)


# ----------------------------------------------------------------- exact special cases
@pytest.mark.parametrize("M,K,N", [(5, 384, 72), (16, 1152, 64), (1, 4096, 33)])
def test_one_hot_bitwise(orc, M, K, N):
    x = synth.generate_custom(M, K, N, seed=4)
    dev = to_dev(x)
    r = np.random.default_rng(5)
    for (m0, k0) in ((0, 0), (M - 1, K - 1), (M // 2, 131), (0, K // 2 + 5)):
        a0 = np.float32(r.choice([1.0, -2.5, 0.375, 96.0, -0.0078125, 3.0e4, 1.0e-3]))
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        Ab = synth.f32_to_bf16_bits(A)
        log(f"one-hot M={M} K={K} N={N} m0={m0} k0={k0} a0={a0}")
        dev["A"] = torch.from_numpy(Ab.view(np.int16)).cuda().view(torch.bfloat16)
        C = run(dev).cpu().numpy().astype(np.float64)
        Cr, _ = orc.gemm(Ab, x.Wq, x.S, x.Z)
        assert np.array_equal(C, Cr), f"one-hot ({m0},{k0}) differs"


def test_zero_cases_exact(orc):
    M, K, N = 7, 1152, 129
    x = synth.generate_custom(M, K, N, seed=6)
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)
    x_eq = synth.GemmInputs(A=x.A, Wq=orc.pack(q), q=None, S=x.S, Z=x.Z)
    log("zero case q == z")
    C = run(to_dev(x_eq)).cpu().numpy()
    assert np.all(C == 0.0)
    x_s0 = synth.GemmInputs(A=x.A, Wq=x.Wq, q=None, S=np.zeros_like(x.S), Z=x.Z)
    log("zero case s == 0")
    C = run(to_dev(x_s0)).cpu().numpy()
    assert np.all(C == 0.0)


def test_zero_high_nibble_ignored(orc):
    M, K, N = 5, 512, 96
    x = synth.generate_custom(M, K, N, seed=7)
    dev = to_dev(x)
    C1 = run(dev).cpu().numpy()
    dev["Z"] = dev["Z"] | 0xB0
    log("zero points with high nibbles set")
    C2 = run(dev).cpu().numpy()
    assert np.array_equal(C1, C2)


def test_identity_rowsum(orc):
    # q = z + 1, s = 1: every column is the row sum of A
    M, K, N = 5, 3584, 64
    r = np.random.default_rng(8)
    x = synth.generate_custom(M, K, N, seed=8)
    Z = r.integers(0, 15, size=x.Z.shape, dtype=np.uint8)
    q = np.repeat(Z + 1, 128, axis=0).astype(np.uint8)
    S = np.ones(x.S.shape, np.float16).view(np.uint16)
    xi = synth.GemmInputs(A=x.A, Wq=orc.pack(q), q=None, S=S, Z=Z)
    log("identity q = z + 1, s = 1")
    C = run(to_dev(xi)).cpu().numpy()
    Cr, Cabs = orc.gemm(xi.A, xi.Wq, xi.S, xi.Z)
    check(C, Cr, Cabs, "identity")
    assert np.all(C == C[:, :1])  # all columns identical


def test_activation_dynamic_range(orc):
    # rows of very large and very small bf16 magnitudes (beyond fp16 range) stay exact
    M, K, N = 6, 512, 64
    x = synth.generate_custom(M, K, N, seed=9)
    a = (x.A.astype(np.uint32) << 16).view(np.float32)
    scale = np.array([1e30, 1e-30, 7e4, 1e-6, 1.0, 3e-38], np.float32)[:, None]
    A = synth.f32_to_bf16_bits(a * scale)
    xs = synth.GemmInputs(A=A, Wq=x.Wq, q=None, S=x.S, Z=x.Z)
    log("activation dynamic range rows")
    C = run(to_dev(xs)).cpu().numpy()
    Cr, Cabs = orc.gemm(xs.A, xs.Wq, xs.S, xs.Z)
    check(C, Cr, Cabs, "dynamic range")


def test_error_well_inside_tolerance(orc):
    # exact (q - z) products and float32 partials keep the error under ~2e-5 of sum|A W|
    M, K, N = 5, 18944, 256
    x = synth.generate_custom(M, K, N, seed=10)
    log("error bound at K=18944")
    C = run(to_dev(x)).cpu().numpy().astype(np.float64)
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    rel = np.abs(C - Cr) / Cabs
    assert rel.max() < 2e-5, rel.max()


# ----------------------------------------------------------- workspace, poison, graphs
def test_poisoned_output_fully_written(orc):
    for (M, K, N) in ((5, 1536, 1536), (5, 18944, 192), (17, 256, 70)):
        x = synth.generate_custom(M, K, N, seed=11)
        dev = to_dev(x)
        out = torch.full((M, N), float("nan"), device="cuda")
        log(f"poisoned C M={M} K={K} N={N}")
        C = run(dev, out=out).cpu().numpy()
        assert np.all(np.isfinite(C))
        cols = np.arange(0, N, max(1, N // 50))
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
        check(C[:, cols], Cr, Cabs, "poisoned")


def test_back_to_back_shapes_reproducible(orc):
    # split-K shapes with different tile counts share one workspace and its counters
    shapes = [(5, 3584, 4608), (5, 18944, 3584), (1, 1536, 17920), (5, 3584, 4608)]
    devs = {}
    results = []
    for (M, K, N) in shapes:
        if (M, K, N) not in devs:
            devs[(M, K, N)] = (synth.generate_custom(M, K, N, seed=12),)
            devs[(M, K, N)] += (to_dev(devs[(M, K, N)][0]),)
        log(f"back-to-back M={M} K={K} N={N}")
        results.append(run(devs[(M, K, N)][1]))
    torch.cuda.synchronize()
    assert torch.equal(results[0], results[3]), "split-K result not reproducible"
    for (M, K, N), C in zip(shapes, results):
        x = devs[(M, K, N)][0]
        cols = np.arange(0, N, 61)
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
        check(C.cpu().numpy()[:, cols], Cr, Cabs, f"b2b {M}x{K}x{N}")


def test_concurrent_streams_and_threads():
    # split-K plans keep a workspace (partials and arrival counters) per stream: calls on
    # two streams, issued from two host threads with no synchronization between them, must
    # give the single-stream results bit for bit
    import threading
    shapes = [(5, 3584, 4608), (5, 18944, 3584), (5, 3584, 37888), (160, 4096, 4096)]
    xs = [to_dev(synth.generate_custom(M, K, N, seed=51)) for (M, K, N) in shapes]
    ref = [run(d).clone() for d in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(r) for r in ref] for _ in streams]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for rep in range(20):
                    for j in (range(len(xs)) if i == 0 else reversed(range(len(xs)))):
                        run(xs[j], out=outs[i][j])
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for j, r in enumerate(ref):
            assert torch.equal(outs[i][j], r), f"stream {i} shape {shapes[j]} differs"


def test_graph_replay_matches_eager():
    # tall split plans, and balanced wide plans (unsplit tiles plus split tiles)
    shapes = [(5, 3584, 4608), (5, 18944, 3584), (1, 1536, 17920), (5, 3584, 37888)]
    xs = [to_dev(synth.generate_custom(M, K, N, seed=13)) for (M, K, N) in shapes]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = [run(d).clone() for d in xs]  # also sizes the workspace for this stream
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    log("graph capture")
    with torch.cuda.graph(g, stream=s):
        for d, o in zip(xs, outs):
            run(d, out=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        del junk
        for e, o in zip(eager, outs):
            assert torch.equal(e, o), f"replay {rep} differs from eager"


def test_unaligned_scale_zero_views(orc):
    # scales/zeros views that are only 2-/1-byte aligned take the scalar load path
    M, K, N = 5, 512, 128
    x = synth.generate_custom(M, K, N, seed=14)
    dev = to_dev(x)
    G = K // 128
    s_big = torch.empty(G * N + 1, dtype=torch.float16, device="cuda")
    s_big[1:] = dev["S"].flatten()
    z_big = torch.empty(G * N + 1, dtype=torch.uint8, device="cuda")
    z_big[1:] = dev["Z"].flatten()
    dev["S"] = s_big[1:].view(G, N)
    dev["Z"] = z_big[1:].view(G, N)
    log("unaligned scale/zero views")
    C = run(dev).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    check(C, Cr, Cabs, "unaligned views")


def test_misaligned_pointer_rejected():
    M, K, N = 5, 128, 64
    A = torch.zeros(M * K + 8, dtype=torch.bfloat16, device="cuda")
    Wq = torch.zeros(K // 8, N, dtype=torch.int32, device="cuda")
    S = torch.zeros(K // 128, N, dtype=torch.float16, device="cuda")
    Z = torch.zeros(K // 128, N, dtype=torch.uint8, device="cuda")
    C = torch.zeros(M, N, dtype=torch.float32, device="cuda")
    with pytest.raises(w4.W4Error) as e:
        w4.gemm_raw(A.data_ptr() + 2, Wq.data_ptr(), S.data_ptr(), Z.data_ptr(), C.data_ptr(), M, K, N)
    assert e.value.code == 3


# ------------------------------------------ the workloads at full size, every element
def _full_check(orc, spec):
    """One GEMM of a workload at its full size, in the launch configuration the bench runs,
    compared with the oracle on every output element."""
    x = synth.generate(spec)
    dev = to_dev(x)
    if "q" in dev:
        dev["Wq"] = w4.pack(dev["q"])
    log(f"workload gemm {spec.name} M={spec.M} K={spec.K} N={spec.N} plan={w4.plan(spec.M, spec.K, spec.N)}")
    out = torch.full((spec.M, spec.N), float("nan"), device="cuda")
    C = run(dev, out=out).cpu().numpy()
    del dev
    Cr, Cabs = orc.gemm(x.A, host_words(x), x.S, x.Z)
    return check(C, Cr, Cabs, f"{spec.name} (every element)")


def test_workload_single_m5_full(orc):
    spec = synth.WORKLOADS["single-m5-k1536-n1536"].gemms[0]
    x = synth.generate(spec)
    dev = to_dev(x)
    dev["Wq"] = w4.pack(dev["q"])
    log("single M=5 K=N=1536, every element")
    C = run(dev).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, orc.pack(x.q), x.S, x.Z)
    check(C, Cr, Cabs, "single-m5")


@pytest.mark.parametrize("name", ["qwen2.5-1.5b-draft-m1", "qwen2.5-7b-verify-m5", "qwen2.5-7b-batched-verify-m40",
                                  "qwen2.5-7b-batched-verify-m80", "llama2-7b-batched-verify-m160"])
def test_workload_layer_every_element(orc, name):
    # one whole layer (every projection shape of the model: qkv, o, gate_up, down) and the
    # last GEMM of the pass, each on every output element
    wl = synth.WORKLOADS[name]
    worst = 0.0
    for spec in list(wl.gemms[:4]) + [wl.gemms[-1]]:
        worst = max(worst, _full_check(orc, spec))
    log(f"{name}: worst error / bound = {worst:.3g}")


@pytest.mark.parametrize("M", [3, 4, 5, 6, 7])
def test_workload_gamma_sweep_every_element(orc, M):
    # each gamma of the sweep: the first down and gate_up copies, every output element
    wl = synth.WORKLOADS["qwen2.5-7b-gamma-sweep"]
    specs = [g for g in wl.gemms if g.M == M][:2]
    assert {s.N for s in specs} == {3584, 37888}
    for spec in specs:
        _full_check(orc, spec)


def test_activation_span_at_the_exactness_edge(orc):
    # Rows whose magnitudes inside one 128-wide group span 2^30 (and, in one row, exactly
    # 2^32), where the group's largest element meets a zero weight (q = z) in half of the
    # columns: those columns' exact sums do not contain the large element at all, so a lost
    # small element would show against a bound built from the small ones alone.  The
    # small-M kernels scale each (row, group) by its largest magnitude; within a span of 2^32
    # every element stays exact, so the contract holds unchanged.
    M, K, N = 5, 512, 128
    x = synth.generate_custom(M, K, N, seed=91)
    r = np.random.default_rng(92)
    a = (1.0 + r.random((M, K))) * np.where(r.random((M, K)) < 0.5, -1.0, 1.0)  # |a| in [1, 2)
    big = {0: (0, 2.0 ** 30), 1: (1, 2.0 ** 30), 2: (3, -(2.0 ** 30)), 3: (0, 2.0 ** 31), 4: (2, 2.0 ** 32)}
    for m, (g, v) in big.items():
        k0 = 128 * g + 37 + m
        a[m, k0] = v
        if m == 4:  # exactly 2^32 above the smallest magnitude of the group
            a[m, 128 * g + 5] = 1.0
    A = synth.f32_to_bf16_bits(a.astype(np.float32))
    q = orc.unpack(x.Wq).astype(np.uint8)
    for m, (g, v) in big.items():
        k0 = 128 * g + 37 + m
        q[k0, : N // 2] = x.Z[g, : N // 2] & 0xF  # the large element meets a zero weight
    xe = synth.GemmInputs(A=A, Wq=orc.pack(q), q=None, S=x.S, Z=x.Z)
    log(f"exactness edge M={M} K={K} N={N} plan={w4.plan(M, K, N)}")
    C = run(to_dev(xe)).cpu().numpy()
    Cr, Cabs = orc.gemm(xe.A, xe.Wq, xe.S, xe.Z)
    check(C, Cr, Cabs, "span 2^30..2^32 with the large element on a zero weight")


def test_activation_span_beyond_the_edge(orc):
    # Beyond a span of 2^32 the header's extended bound applies: an element whose exponent is
    # more than 32 below its group's largest magnitude amax may be rounded to the binary16
    # subnormal grid, adding at most 2^-40 * amax * |W| per such element.  Groups here span
    # 2^40..2^60 with the large element on a zero weight in half of the columns.
    M, K, N = 4, 384, 96
    x = synth.generate_custom(M, K, N, seed=93)
    r = np.random.default_rng(94)
    a = r.standard_normal((M, K))
    spans = [40, 44, 50, 60]
    q = orc.unpack(x.Wq).astype(np.uint8)
    for m, e in enumerate(spans):
        g = m % (K // 128)
        k0 = 128 * g + 11
        a[m, k0] = 2.0 ** e
        q[k0, : N // 2] = x.Z[g, : N // 2] & 0xF
    A = synth.f32_to_bf16_bits(a.astype(np.float32))
    xe = synth.GemmInputs(A=A, Wq=orc.pack(q), q=None, S=x.S, Z=x.Z)
    log(f"beyond the exactness edge M={M} K={K} N={N}")
    C = run(to_dev(xe)).cpu().numpy().astype(np.float64)
    Cr, Cabs = orc.gemm(xe.A, xe.Wq, xe.S, xe.Z)
    # the extended bound: 2^-40 * amax[m, g] * |W[k, n]| summed over the elements of each
    # group whose binary exponent is more than 32 below that of the group's maximum
    av = orc.bf16_to_f64(xe.A)
    W = (orc.unpack(xe.Wq).astype(np.float64) - np.repeat(xe.Z & 0xF, 128, axis=0)) * \
        np.repeat(orc.f16_to_f64(xe.S), 128, axis=0)
    ext = np.zeros((M, N))
    for m in range(M):
        for g in range(K // 128):
            seg = av[m, 128 * g: 128 * g + 128]
            amax = np.abs(seg).max()
            if amax == 0:
                continue
            far = (seg != 0) & (np.floor(np.log2(np.abs(np.where(seg == 0, 1, seg)))) < np.floor(np.log2(amax)) - 32)
            ext[m] += 2.0 ** -40 * amax * np.abs(W[128 * g: 128 * g + 128][far]).sum(axis=0)
    err = np.abs(C - Cr)
    bound = 1e-4 * Cabs + 1e-6 + ext
    assert np.all(err <= bound), float((err / bound).max())
    assert ext.max() > 0  # the case really reaches beyond the exact span


# ------------------------------------------------------ large M (bf16 matrix-core kernel)
LARGE_SHAPES = [(128, 2), (256, 256), (384, 258), (1152, 520)]


@pytest.mark.parametrize("M", [64, 96, 100, 160, 161, 250, 320])
def test_large_m_grid(orc, M):
    worst = 0.0
    for K, N in LARGE_SHAPES:
        p = w4.plan(M, K, N)
        assert p["kernel"] == 3
        log(f"large grid M={M} K={K} N={N} plan={p}")
        x = synth.generate_custom(M, K, N, seed=21)
        C = run(to_dev(x)).cpu().numpy()
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
        worst = max(worst, check(C, Cr, Cabs, f"large M={M} K={K} N={N}"))
    log(f"large grid M={M}: worst error / bound = {worst:.3g}")


@pytest.mark.parametrize("M,K,N", [(160, 4096, 4096), (160, 11008, 4096), (64, 8192, 512), (200, 2048, 1030),
                                   (160, 4096, 12288), (64, 4096, 4096), (96, 3584, 3584), (64, 8960, 1536),
                                   (80, 2048, 8192), (64, 3584, 3590)])
def test_large_m_split_k(orc, M, K, N):
    p = w4.plan(M, K, N)
    log(f"large split-K M={M} K={K} N={N} plan={p}")
    x = synth.generate_custom(M, K, N, seed=22)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run(to_dev(x), out=out).cpu().numpy()
    assert np.all(np.isfinite(C))
    cols = np.unique(np.r_[0, 1, N - 2, N - 1, np.random.default_rng(23).integers(0, N, 40)])
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
    check(C[:, cols], Cr, Cabs, f"large split M={M} K={K} N={N}")


def test_large_m_one_hot_bitwise(orc):
    M, K, N = 160, 384, 256
    x = synth.generate_custom(M, K, N, seed=24)
    dev = to_dev(x)
    for (m0, k0, a0) in ((0, 0, 1.0), (M - 1, K - 1, -2.5), (77, 131, 3.0e4), (150, 200, -0.0078125)):
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        dev["A"] = torch.from_numpy(synth.f32_to_bf16_bits(A).view(np.int16)).cuda().view(torch.bfloat16)
        log(f"large one-hot m={m0} k={k0} a={a0}")
        C = run(dev).cpu().numpy()
        Cr, _ = orc.gemm(synth.f32_to_bf16_bits(A), x.Wq, x.S, x.Z)
        assert np.array_equal(C, Cr.astype(np.float32)), "one-hot row differs"


def test_large_m_zero_and_identity(orc):
    M, K, N = 160, 1152, 258
    x = synth.generate_custom(M, K, N, seed=25)
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)
    log("large zero case q == z")
    C = run(to_dev(synth.GemmInputs(A=x.A, Wq=orc.pack(q), q=None, S=x.S, Z=x.Z))).cpu().numpy()
    assert np.all(C == 0.0)
    Z = np.random.default_rng(26).integers(0, 15, size=x.Z.shape, dtype=np.uint8)
    q = np.repeat(Z + 1, 128, axis=0).astype(np.uint8)
    S = np.ones(x.S.shape, np.float16).view(np.uint16)
    xi = synth.GemmInputs(A=x.A, Wq=orc.pack(q), q=None, S=S, Z=Z)
    log("large identity q = z + 1, s = 1")
    C = run(to_dev(xi)).cpu().numpy()
    Cr, Cabs = orc.gemm(xi.A, xi.Wq, xi.S, xi.Z)
    check(C, Cr, Cabs, "large identity")
    assert np.all(C == C[:, :1])


def test_large_m_dynamic_range(orc):
    M, K, N = 64, 512, 64
    x = synth.generate_custom(M, K, N, seed=27)
    a = (x.A.astype(np.uint32) << 16).view(np.float32)
    scale = np.geomspace(1e30, 1e-30, M).astype(np.float32)[:, None]
    A = synth.f32_to_bf16_bits(a * scale)
    xs = synth.GemmInputs(A=A, Wq=x.Wq, q=None, S=x.S, Z=x.Z)
    log("large activation dynamic range")
    C = run(to_dev(xs)).cpu().numpy()
    Cr, Cabs = orc.gemm(xs.A, xs.Wq, xs.S, xs.Z)
    check(C, Cr, Cabs, "large dynamic range")


def test_large_m_unaligned_scale_view(orc):
    # the bf16 kernel reads each scale with a 2-byte load, so a scale view that is only
    # 2-byte aligned runs on it unchanged (the plan does not look at alignment)
    M, K, N = 96, 512, 128
    x = synth.generate_custom(M, K, N, seed=28)
    dev = to_dev(x)
    G = K // 128
    s_big = torch.empty(G * N + 1, dtype=torch.float16, device="cuda")
    s_big[1:] = dev["S"].flatten()
    dev["S"] = s_big[1:].view(G, N)
    assert w4.plan(M, K, N)["kernel"] == 3
    log("large unaligned scale view")
    C = run(dev).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z)
    check(C, Cr, Cabs, "large unaligned")


def test_large_m_graph_and_reproducible():
    # (the last two shapes share their (tile, group) steps out evenly)
    shapes = [(160, 4096, 4096), (160, 4096, 22016), (160, 11008, 4096), (40, 3584, 37888), (17, 2048, 40003)]
    xs = [to_dev(synth.generate_custom(M, K, N, seed=29)) for (M, K, N) in shapes]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = [run(d).clone() for d in xs]
        again = [run(d).clone() for d in xs]
    torch.cuda.synchronize()
    for e, a in zip(eager, again):
        assert torch.equal(e, a), "large split-K result not reproducible"
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    log("large graph capture")
    with torch.cuda.graph(g, stream=s):
        for d, o in zip(xs, outs):
            run(d, out=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"large graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e, o), f"replay {rep} differs from eager"


@pytest.mark.parametrize("M,K,N", [(65, 8192, 3), (97, 4096, 131), (161, 2048, 2049), (70, 8192, 1),
                                   (93, 8960, 1539)])
def test_large_m_split_odd_sizes(orc, M, K, N):
    # split-K plans whose M*N is not a multiple of 4 exercise the reduction's tail path
    p = w4.plan(M, K, N)
    assert p["kernel"] == 3 and p["splits"] > 1
    log(f"large split odd M={M} K={K} N={N} plan={p}")
    x = synth.generate_custom(M, K, N, seed=30)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run(to_dev(x), out=out).cpu().numpy()
    assert np.all(np.isfinite(C))
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(31).integers(0, N, 24)])
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
    check(C[:, cols], Cr, Cabs, f"large split odd M={M} K={K} N={N}")
