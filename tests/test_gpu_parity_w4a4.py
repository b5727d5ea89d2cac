"""4-bit activations (a4_quantize, w4a4_gemm) against the oracle through the C-ABI (needs gfx950).

The activation quantizer decides integer codes in floating point, so it must match the
oracle bit for bit (codes and scales).  The product is compared per element within
|C_gpu - C_oracle| <= 1e-4 * sum_k |sa qa (q - z) s| + 1e-6; with power-of-two activation
scales a one-hot activation gives a single exactly scaled product, rounded once, which must
equal the oracle's value rounded to float32.
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


def dev_a4(Aq, As):
    return (torch.from_numpy(np.ascontiguousarray(Aq).view(np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(As, dtype=np.float32)).cuda())


def run_a4(Aq_d, As_d, dev, out=None):
    return w4.gemm_a4(Aq_d, As_d, dev["Wq"], dev["S"], dev["Z"], out=out)


def gen_a4(M, K, N, seed):
    return synth.generate_custom(M, K, N, seed=seed, act4=True)


# ------------------------------------------------------------- activation quantizer
def _activations(M, K, seed):
    """bfloat16 activations with rows and groups spanning many binades, zero groups,
    one-signed groups, bfloat16 subnormals and values near the bfloat16 maximum."""
    r = np.random.default_rng(seed)
    A = r.standard_normal((M, K)).astype(np.float32) * np.float32(2.0) ** r.integers(-20, 20, size=(M, 1)).astype(np.float32)
    G = K // 128
    for m in range(min(M, 6)):
        g = m % G
        cols = slice(128 * g, 128 * g + 128)
        if m == 0:
            A[m, cols] = 0.0
        elif m == 1:
            A[m, cols] = np.abs(A[m, cols])
        elif m == 2:
            A[m, cols] = (r.standard_normal(128) * 2.0 ** -128).astype(np.float32)  # bfloat16 subnormals
        elif m == 3:
            A[m, cols] = (r.uniform(-1, 1, 128) * 3.0e38).astype(np.float32)
        elif m == 4:
            A[m, cols] = (r.integers(-6, 7, 128) + 0.5).astype(np.float32)  # ties once the scale is 1
            A[m, 128 * g] = 7.0
    return synth.f32_to_bf16_bits(A)


@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (7, 1152), (32, 4096), (33, 11008), (160, 3584), (3, 1 << 17)])
def test_a4_quantize_bit_exact(orc, M, K):
    log(f"a4 quantize M={M} K={K}")
    Ab = _activations(M, K, seed=M * 7 + K)
    Aq, As = w4.quantize_activations(torch.from_numpy(Ab.view(np.int16)).cuda().view(torch.bfloat16))
    rAq, rAs = orc.quantize_activations(Ab)
    assert np.array_equal(As.cpu().numpy().view(np.uint32), rAs.view(np.uint32)), "scales differ"
    assert np.array_equal(Aq.cpu().numpy().view(np.uint32), rAq), "codes differ"


# ------------------------------------------------------------------- the W4A4 product
GRID_M = [1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64]
GRID_K = [128, 256, 1152]
GRID_N = [1, 3, 8, 63, 64, 65, 257]


@pytest.mark.parametrize("M", GRID_M)
def test_grid_a4(orc, M):
    worst = 0.0
    for K in GRID_K:
        for N in GRID_N:
            log(f"w4a4 grid M={M} K={K} N={N}")
            x = gen_a4(M, K, N, seed=1)
            Aq_d, As_d = dev_a4(x.Aq, x.As)
            C = run_a4(Aq_d, As_d, to_dev(x)).cpu().numpy()
            Cr, Cabs = orc.gemm_a4(x.Aq, x.As, x.Wq, x.S, x.Z)
            worst = max(worst, check(C, Cr, Cabs, f"w4a4 M={M} K={K} N={N}"))
    log(f"w4a4 grid M={M}: worst error / bound = {worst:.3g}")


@pytest.mark.parametrize("M,K,N", [(5, 4096, 64), (1, 11008, 4096), (32, 4096, 12288), (32, 11008, 4096),
                                   (7, 8192, 200), (100, 1024, 130)])
def test_split_k_shapes_a4(orc, M, K, N):
    p = w4.plan(M, K, N, a4=True)
    log(f"w4a4 split-K M={M} K={K} N={N} plan={p}")
    x = gen_a4(M, K, N, seed=2)
    Aq_d, As_d = dev_a4(x.Aq, x.As)
    C = run_a4(Aq_d, As_d, to_dev(x)).cpu().numpy()
    cols = np.unique(np.r_[0, N - 1, np.random.default_rng(3).integers(0, N, 64)])
    Cr, Cabs = orc.gemm_a4(x.Aq, x.As, x.Wq, x.S, x.Z, cols=cols)
    check(C[:, cols], Cr, Cabs, f"w4a4 split M={M} K={K} N={N}")


def test_balanced_plan_a4(orc):
    M, K, N = 1, 1024, 19200
    p = w4.plan(M, K, N, a4=True)
    log(f"w4a4 balanced plan={p}")
    x = gen_a4(M, K, N, seed=21)
    Aq_d, As_d = dev_a4(x.Aq, x.As)
    dev = to_dev(x)
    C1 = run_a4(Aq_d, As_d, dev)
    C2 = run_a4(Aq_d, As_d, dev)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2), "w4a4 plan not reproducible"
    Cr, Cabs = orc.gemm_a4(x.Aq, x.As, x.Wq, x.S, x.Z)
    check(C1.cpu().numpy(), Cr, Cabs, "w4a4 balanced")


@pytest.mark.parametrize("M,K,N", [(5, 384, 72), (16, 1152, 64), (1, 4096, 33), (40, 256, 130), (24, 384, 72),
                                   (32, 1152, 130)])
def test_one_hot_correctly_rounded_a4(orc, M, K, N):
    x = gen_a4(M, K, N, seed=4)
    dev = to_dev(x)
    r = np.random.default_rng(5)
    As = np.exp2(r.integers(-20, 20, size=x.As.shape)).astype(np.float32)  # power-of-two scales
    for (m0, k0, c0) in ((0, 0, 7), (M - 1, K - 1, -8), (M // 2, 131, 3), (0, K // 2 + 5, -1)):
        qa = np.zeros((M, K), np.int64)
        qa[m0, k0] = c0
        Aq = ((qa + 8).astype(np.uint32).reshape(M, K // 8, 8) << (4 * np.arange(8, dtype=np.uint32))).sum(
            axis=2, dtype=np.uint32)
        log(f"w4a4 one-hot M={M} K={K} N={N} m0={m0} k0={k0} code={c0}")
        Aq_d, As_d = dev_a4(Aq, As)
        C = run_a4(Aq_d, As_d, dev).cpu().numpy()
        Cr, _ = orc.gemm_a4(Aq, As, x.Wq, x.S, x.Z)
        assert np.array_equal(C, Cr.astype(np.float32)), f"one-hot ({m0},{k0}) not the rounded exact product"


def test_zero_cases_exact_a4(orc):
    M, K, N = 7, 1152, 129
    x = gen_a4(M, K, N, seed=6)
    dev = to_dev(x)
    zero_codes = np.full(x.Aq.shape, 0x88888888, np.uint32)  # every activation code 0
    Aq_d, As_d = dev_a4(zero_codes, x.As)
    assert np.all(run_a4(Aq_d, As_d, dev).cpu().numpy() == 0.0)
    Aq_d, As_d = dev_a4(x.Aq, np.zeros_like(x.As))
    assert np.all(run_a4(Aq_d, As_d, dev).cpu().numpy() == 0.0)
    q = np.repeat(x.Z & 0xF, 128, axis=0).astype(np.uint8)  # q = z: every weight is zero
    dev["Wq"] = torch.from_numpy(orc.pack(q).view(np.int32)).cuda()
    Aq_d, As_d = dev_a4(x.Aq, x.As)
    assert np.all(run_a4(Aq_d, As_d, dev).cpu().numpy() == 0.0)


def test_quantize_then_gemm_a4(orc):
    # bfloat16 activations through a4_quantize and w4a4_gemm on the device, against the
    # oracle's quantizer and product; and beside the W4A16 product of the same activations
    M, K, N = 32, 4096, 1000
    x = synth.generate_custom(M, K, N, seed=7)
    dev = to_dev(x)
    Aq_d, As_d = w4.quantize_activations(dev["A"])
    C = run_a4(Aq_d, As_d, dev).cpu().numpy()
    rAq, rAs = orc.quantize_activations(x.A)
    Cr, Cabs = orc.gemm_a4(rAq, rAs, x.Wq, x.S, x.Z)
    check(C, Cr, Cabs, "quantize then w4a4")
    C16, Cabs16 = orc.gemm(x.A, x.Wq, x.S, x.Z)
    rel = np.abs(Cr - C16).max() / np.abs(C16).max()
    log(f"4-bit activations vs bfloat16 activations: max |dC| / max |C| = {rel:.3g}")
    assert rel < 0.5  # the quantization error of 4-bit activations, not a mismatch of layouts


def test_poisoned_output_and_graph_replay_a4(orc):
    shapes = [(32, 4096, 12288), (32, 11008, 4096), (1, 4096, 22016)]
    inputs = [gen_a4(M, K, N, seed=11 + i) for i, (M, K, N) in enumerate(shapes)]
    devs = [(dev_a4(x.Aq, x.As), to_dev(x)) for x in inputs]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = [run_a4(a[0], a[1], d) for a, d in devs]
    torch.cuda.synchronize()
    for x, e, (M, K, N) in zip(inputs, eager, shapes):
        cols = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 32)])
        Cr, Cabs = orc.gemm_a4(x.Aq, x.As, x.Wq, x.S, x.Z, cols=cols)
        check(e.cpu().numpy()[:, cols], Cr, Cabs, f"w4a4 eager {M}x{K}x{N}")
    outs = [torch.full_like(e, float("nan")) for e in eager]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for (a, d), o in zip(devs, outs):
            run_a4(a[0], a[1], d, out=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        log(f"w4a4 graph replay {rep}")
        for e, o in zip(eager, outs):
            assert torch.equal(e, o), "replay differs from the eager call"


def test_workload_w4a4_draft_every_element(orc):
    # one whole layer (qkv, o, gate_up, down) and the last GEMM of the step, every element
    wl = synth.WORKLOADS["llama2-7b-w4a4-draft-m32"]
    for spec in list(wl.gemms[:4]) + [wl.gemms[-1]]:
        x = synth.generate(spec)
        log(f"w4a4 workload gemm {spec.name} M={spec.M} K={spec.K} N={spec.N} "
            f"plan={w4.plan(spec.M, spec.K, spec.N, a4=True)}")
        Aq_d, As_d = dev_a4(x.Aq, x.As)
        C = run_a4(Aq_d, As_d, to_dev(x)).cpu().numpy()
        Cr, Cabs = orc.gemm_a4(x.Aq, x.As, x.Wq, x.S, x.Z)
        check(C, Cr, Cabs, f"{spec.name} (every element)")


def test_maximum_size_a4(orc):
    # activation codes just under 2 GiB (M * K / 2 bytes), the largest array the kernel's
    # 32-bit byte offsets address; sampled rows (edges, row-block boundaries) and all columns
    M, K, N = 32767, 131072, 8
    assert M * K // 2 < 1 << 31
    p = w4.plan(M, K, N, a4=True)
    log(f"w4a4 maximum size M={M} K={K} N={N} plan={p}")
    x = synth.generate_custom(1, K, N, seed=31)  # weights; activations drawn below
    r = np.random.default_rng(32)
    Aq = r.integers(0, 1 << 32, size=(M, K // 8), dtype=np.uint32)
    As = ((2.5 + 0.3 * np.abs(r.standard_normal((M, K // 128)))) / 7.0).astype(np.float32)
    Aq_d, As_d = dev_a4(Aq, As)
    C = run_a4(Aq_d, As_d, to_dev(x)).cpu().numpy()
    del Aq_d, As_d
    rows = np.unique(np.r_[0, 15, 16, M - 17, M - 16, M - 1, r.integers(0, M, 6)]).astype(np.int64)
    Cr, Cabs = orc.gemm_a4(Aq[rows], As[rows], x.Wq, x.S, x.Z)
    check(C[rows], Cr, Cabs, f"w4a4 max size M={M} K={K} N={N}")
