"""The 8-bit variant (w8a16_gemm, w8_pack) against the oracle through the C-ABI (needs gfx950).

Tolerance (per element, float64): |C_gpu - C_oracle| <= 1e-4 * sum_k |A[m,k] W[k,n]| + 1e-6.
Packing is compared bit for bit.  A one-hot A gives a single product a0 * (q - z) * s per
output, which the kernel forms exactly and rounds once: it must equal the oracle's value
rounded to float32.  q = z and s = 0 give exact zeros.
"""
import numpy as np
import pytest
import torch

import int4_weight_only_gemm_amd as w4
import oracle
import synth
from gpu_helpers import check, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run8(dev, out=None):
    return w4.gemm(dev["A"], dev["Wq"], dev["S"], dev["Z"], out=out, bits=8)


def gen8(M, K, N, seed):
    return synth.generate_custom(M, K, N, seed=seed, bits=8)


# ------------------------------------------------------------------------------ packing
@pytest.mark.parametrize("K,N", [(4, 1), (8, 3), (128, 64), (384, 257), (1536, 2048), (1024, 4099)])
def test_pack8_bit_exact(orc, K, N):
    log(f"pack8 K={K} N={N}")
    q = np.random.default_rng(K * 5 + N).integers(0, 256, size=(K, N), dtype=np.uint8)
    q[0, 0], q[-1, -1] = 0xFF, 0x80
    Wq8 = w4.pack(torch.from_numpy(q).cuda(), bits=8)
    torch.cuda.synchronize()
    assert np.array_equal(Wq8.cpu().numpy().view(np.uint32), orc.pack8(q))


# ------------------------------------------------------------------- tiny-shape grid
GRID_M = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 33, 64, 65]
GRID_K = [128, 256, 384, 1152]
GRID_N = [1, 3, 7, 8, 63, 64, 65, 257]


@pytest.mark.parametrize("M", GRID_M)
def test_grid8(orc, M):
    worst = 0.0
    for K in GRID_K:
        for N in GRID_N:
            log(f"w8 grid M={M} K={K} N={N}")
            x = gen8(M, K, N, seed=1)
            C = run8(to_dev(x)).cpu().numpy()
            Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
            worst = max(worst, check(C, Cr, Cabs, f"w8 M={M} K={K} N={N}"))
    log(f"w8 grid M={M}: worst error / bound = {worst:.3g}")


@pytest.mark.parametrize("M,K,N", [(5, 4096, 64), (1, 8960, 1536), (7, 8192, 200), (16, 2048, 36),
                                   (3, 11008, 4096), (1, 18944, 3584), (100, 1024, 130)])
def test_split_k_shapes8(orc, M, K, N):
    p = w4.plan(M, K, N, bits=8)
    log(f"w8 split-K M={M} K={K} N={N} plan={p}")
    x = gen8(M, K, N, seed=2)
    C = run8(to_dev(x)).cpu().numpy()
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(3).integers(0, N, 64)])
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols, bits=8)
    check(C[:, cols], Cr, Cabs, f"w8 split M={M} K={K} N={N}")


# ------------------------------------------------------------- narrow-tile kernel
NARROW8_SHAPES = [(1, 8192, 4095), (5, 3584, 3584), (8, 3584, 1000), (16, 1792, 300), (3, 128, 17),
                  (7, 640, 4096), (2, 8064, 33), (4, 1024, 1), (1, 1536, 2048)]


@pytest.mark.parametrize("M,K,N", NARROW8_SHAPES)
def test_narrow_kernel_every_element8(orc, M, K, N):
    # 8-bit codes on the narrow-tile kernel: 64 groups (eight per wave, the most a wave
    # holds), one group, ragged N down to a single column, 16 rows, 256 tiles; NaN-poisoned
    # C, every element against the oracle
    p = w4.plan(M, K, N, bits=8)
    log(f"w8 narrow M={M} K={K} N={N} plan={p}")
    assert p["kernel"] == 8 and p["tile_n"] == 16 and p["splits"] == 1
    x = gen8(M, K, N, seed=63)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run8(to_dev(x), out=out).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
    check(C, Cr, Cabs, f"w8 narrow M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(5, 9216, 65), (13, 8320, 7), (9, 128, 4160), (1, 16384, 3), (16, 8448, 130)])
def test_small_kernel_ragged8(orc, M, K, N):
    # rows in one 16-row block on the 8-bit small-M kernel (more than 64 groups, or more than
    # 256 narrow tiles): ragged N, every element
    p = w4.plan(M, K, N, bits=8)
    log(f"w8 small-M M={M} K={K} N={N} plan={p}")
    assert p["kernel"] in (4, 5)
    x = gen8(M, K, N, seed=64)
    out = torch.full((M, N), float("nan"), device="cuda")
    C = run8(to_dev(x), out=out).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
    check(C, Cr, Cabs, f"w8 small-M M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 1536, 17920), (5, 1024, 19200), (3, 2048, 19198)])
def test_balanced_wide_plan8(orc, M, K, N):
    p = w4.plan(M, K, N, bits=8)
    log(f"w8 balanced M={M} K={K} N={N} plan={p}")
    x = gen8(M, K, N, seed=21)
    dev = to_dev(x)
    C1 = run8(dev)
    C2 = run8(dev)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2), "w8 plan not reproducible"
    cols = np.unique(np.r_[0, N - 1, 64 * p["full_tiles"] - 1, 64 * p["full_tiles"],
                           np.random.default_rng(22).integers(0, N, 96)])
    cols = cols[(cols >= 0) & (cols < N)].astype(np.int64)
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols, bits=8)
    check(C1.cpu().numpy()[:, cols], Cr, Cabs, f"w8 balanced M={M} K={K} N={N}")


def test_maximum_size8(orc):
    # packed 8-bit codes just under 2 GiB (K/4 * N * 4 bytes), the largest array the kernel's
    # 32-bit byte offsets address; sampled columns at tile and edge positions
    M, K, N = 5, 65536, 32760
    assert K // 4 * N * 4 < 1 << 31
    p = w4.plan(M, K, N, bits=8)
    log(f"w8 maximum size M={M} K={K} N={N} plan={p}")
    x = gen8(M, K, N, seed=31)
    dev = to_dev(x)
    C = run8(dev).cpu().numpy()
    del dev
    cols = np.unique(np.r_[0, N - 1, 63, 64, 255, 256, np.random.default_rng(32).integers(0, N, 24)]).astype(np.int64)
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols, bits=8)
    check(C[:, cols], Cr, Cabs, f"w8 max size M={M} K={K} N={N}")


# ----------------------------------------------------------------- exact special cases
@pytest.mark.parametrize("M,K,N", [(5, 384, 72), (16, 1152, 64), (1, 4096, 33), (40, 256, 130)])
def test_one_hot_correctly_rounded8(orc, M, K, N):
    x = gen8(M, K, N, seed=4)
    dev = to_dev(x)
    r = np.random.default_rng(5)
    for (m0, k0) in ((0, 0), (M - 1, K - 1), (M // 2, 131), (0, K // 2 + 5)):
        a0 = np.float32(r.choice([1.0, -2.5, 0.375, 96.0, -0.0078125, 3.0e4, 1.0e-3]))
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        Ab = synth.f32_to_bf16_bits(A)
        log(f"w8 one-hot M={M} K={K} N={N} m0={m0} k0={k0} a0={a0}")
        dev["A"] = torch.from_numpy(Ab.view(np.int16)).cuda().view(torch.bfloat16)
        C = run8(dev).cpu().numpy()
        Cr, _ = orc.gemm(Ab, x.Wq, x.S, x.Z, bits=8)
        assert np.array_equal(C, Cr.astype(np.float32)), f"one-hot ({m0},{k0}) not the rounded exact product"


def test_zero_cases_exact8(orc):
    M, K, N = 7, 1152, 129
    x = gen8(M, K, N, seed=6)
    dev = to_dev(x)
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)  # q = z: every weight is zero
    dev["Wq"] = torch.from_numpy(orc.pack8(q).view(np.int32)).cuda()
    C = run8(dev).cpu().numpy()
    assert np.all(C == 0.0)
    dev = to_dev(x)
    dev["S"] = torch.zeros_like(dev["S"])
    C = run8(dev).cpu().numpy()
    assert np.all(C == 0.0)


def test_identity_rowsum8(orc):
    # q = z + 1 with zero points up to 254, s = 1: every column is the row sum of A
    M, K, N = 5, 2048, 96
    x = gen8(M, K, N, seed=7)
    Z = np.random.default_rng(8).integers(0, 255, size=x.Z.shape, dtype=np.uint8)
    Z[0, :4] = 254
    q = np.repeat(Z + 1, 128, axis=0).astype(np.uint8)
    S = np.full(x.S.shape, 0x3C00, np.uint16)  # binary16 1.0
    dev = to_dev(x)
    dev["Wq"] = torch.from_numpy(orc.pack8(q).view(np.int32)).cuda()
    dev["S"] = torch.from_numpy(S.view(np.int16)).cuda().view(torch.float16)
    dev["Z"] = torch.from_numpy(Z).cuda()
    C = run8(dev).cpu().numpy()
    Cr, Cabs = orc.gemm(x.A, orc.pack8(q), S, Z, bits=8)
    check(C, Cr, Cabs, "w8 identity")
    a = x.A.astype(np.uint32) << 16
    rs = a.view(np.float32).astype(np.float64).sum(axis=1)
    assert np.allclose(Cr, rs[:, None], rtol=0, atol=1e-9 * np.abs(a.view(np.float32)).sum())


def test_activation_dynamic_range8(orc):
    # rows and groups whose magnitudes differ by many binades: the per-(row, group)
    # power-of-two scaling keeps every product exact
    M, K, N = 6, 1024, 130
    x = gen8(M, K, N, seed=9)
    A = (x.A.astype(np.uint32) << 16).view(np.float32).copy()
    A[1] *= np.float32(2.0 ** 40)
    A[2] *= np.float32(2.0 ** -40)
    A[3, :128] *= np.float32(2.0 ** 20)
    A[4, 512:640] *= np.float32(2.0 ** -30)
    Ab = synth.f32_to_bf16_bits(A)
    dev = to_dev(x)
    dev["A"] = torch.from_numpy(Ab.view(np.int16)).cuda().view(torch.bfloat16)
    C = run8(dev).cpu().numpy()
    Cr, Cabs = orc.gemm(Ab, x.Wq, x.S, x.Z, bits=8)
    check(C, Cr, Cabs, "w8 dynamic range")


def test_poisoned_output_fully_written8(orc):
    M, K, N = 3, 2048, 1001
    x = gen8(M, K, N, seed=10)
    dev = to_dev(x)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    run8(dev, out=out)
    C = out.cpu().numpy()
    assert np.all(np.isfinite(C))
    Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
    check(C, Cr, Cabs, "w8 poisoned output")


def test_graph_replay_matches_eager8():
    # split-K shapes captured into a graph (workspace sized by the eager call first) replay
    # to the eager results bit for bit, with eager work and synchronizations in between
    shapes = [(1, 8960, 1536), (1, 1536, 17920), (5, 3584, 4608)]
    devs = [to_dev(gen8(M, K, N, seed=11 + i)) for i, (M, K, N) in enumerate(shapes)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = [run8(d) for d in devs]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for d, o in zip(devs, outs):
            run8(d, out=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        log(f"w8 graph replay {rep}")
        for e, o in zip(eager, outs):
            assert torch.equal(e, o), "replay differs from the eager call"
        with torch.cuda.stream(stream):
            run8(devs[0])  # eager work on the same stream between replays
        torch.cuda.synchronize()


def test_w8_matches_w4_on_4bit_codes(orc):
    # codes and zero points below 16 stored both ways give the same products; both paths
    # agree with the oracle, and the oracle's two functions agree exactly
    M, K, N = 5, 1536, 200
    x = synth.generate_custom(M, K, N, seed=12, q_as_bytes=True)
    dev = to_dev(x)
    Wq4 = w4.pack(dev["q"])
    Wq8 = w4.pack(dev["q"], bits=8)
    C4 = w4.gemm(dev["A"], Wq4, dev["S"], dev["Z"]).cpu().numpy()
    C8 = w4.gemm(dev["A"], Wq8, dev["S"], dev["Z"], bits=8).cpu().numpy()
    Cr4, Cabs = orc.gemm(x.A, orc.pack(x.q), x.S, x.Z)
    Cr8, _ = orc.gemm(x.A, orc.pack8(x.q), x.S, x.Z, bits=8)
    assert np.array_equal(Cr4, Cr8)
    check(C4, Cr4, Cabs, "w4 path")
    check(C8, Cr8, Cabs, "w8 path")


# ------------------------------------------- the 8-bit draft workload, every element
def test_workload_w8_draft_every_element(orc):
    # one whole layer (qkv, o, gate_up, down) and the last GEMM of the step, every element
    wl = synth.WORKLOADS["qwen2.5-1.5b-draft-m1-w8"]
    for spec in list(wl.gemms[:4]) + [wl.gemms[-1]]:
        x = synth.generate(spec)
        log(f"w8 workload gemm {spec.name} M={spec.M} K={spec.K} N={spec.N} plan={w4.plan(spec.M, spec.K, spec.N, bits=8)}")
        out = torch.full((spec.M, spec.N), float("nan"), device="cuda")
        C = run8(to_dev(x), out=out).cpu().numpy()
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
        check(C, Cr, Cabs, f"{spec.name} (every element)")
