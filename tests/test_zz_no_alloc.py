"""The entry point that allocates nothing (w4a16_gemm_noalloc), through the C ABI, against
the allocating entry point (w4a16_gemm) on the same inputs: same plan and kernels, so the
results must agree bit for bit, and both must meet the oracle's tolerance."""
import numpy as np
import pytest
import torch

import int4_weight_only_gemm_amd as w4
import oracle
import synth
from gpu_helpers import check, log, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(dev, out, stream):
    w4.gemm_noalloc_raw(dev["A"].data_ptr(), dev["Wq"].data_ptr(), dev["S"].data_ptr(), dev["Z"].data_ptr(),
                        out.data_ptr(), out.shape[0], dev["A"].shape[1], out.shape[1], stream.cuda_stream)


def _alloc(dev, out, stream):
    w4.gemm_raw(dev["A"].data_ptr(), dev["Wq"].data_ptr(), dev["S"].data_ptr(), dev["Z"].data_ptr(),
                out.data_ptr(), out.shape[0], dev["A"].shape[1], out.shape[1], stream.cuda_stream)


# two calls in a row on each path, the second smaller: small-M split plans (tall and wide,
# balanced), an unsplit plan, the bf16 kernel's split slices, and its (tile, group) steps
# shared out evenly
CASES = [((5, 18944, 3584), (3, 3584, 4608)), ((5, 3584, 37888), (1, 1536, 17920)),
         ((160, 4096, 12288), (64, 3584, 3584)), ((7, 1536, 1536), (2, 256, 96)),
         ((40, 3584, 37888), (17, 2048, 40003))]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: "x".join(map(str, c)))
def test_noalloc_matches_allocating_entry_point(first, second):
    orc = oracle.get()
    s = torch.cuda.Stream()
    for i, (M, K, N) in enumerate((first, second)):
        x = synth.generate_custom(M, K, N, seed=71 + i)
        dev = to_dev(x)
        ref = torch.full((M, N), float("nan"), device="cuda")
        got = torch.full((M, N), float("nan"), device="cuda")
        log(f"noalloc call {i}: M={M} K={K} N={N} plan={w4.plan(M, K, N)}")
        with torch.cuda.stream(s):
            _alloc(dev, ref, s)
            _noalloc(dev, got, s)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: noalloc differs from w4a16_gemm"
        cols = np.unique(np.r_[0, N - 1, np.random.default_rng(i).integers(0, N, 64)])
        Cr, Cabs = orc.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
        check(got.cpu().numpy()[:, cols], Cr, Cabs, f"noalloc call {i}")


def test_noalloc_captures_a_new_split_shape_without_warm_up():
    # the allocating entry point cannot capture the first call of a new split shape on a new
    # stream (its workspace would have to grow); the no-alloc one can, and its replays match
    # eager calls of the allocating one
    M, K, N = 5, 18944, 3072  # a split plan, on a stream that has never run it
    x = synth.generate_custom(M, K, N, seed=81)
    dev = to_dev(x)
    s = torch.cuda.Stream()
    out = torch.full((M, N), float("nan"), device="cuda")
    free0 = torch.cuda.mem_get_info()[0]
    g = torch.cuda.CUDAGraph()
    log("noalloc graph capture of a new split shape")
    with torch.cuda.graph(g, stream=s):
        _noalloc(dev, out, s)
    ref = torch.empty_like(out)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            _alloc(dev, ref, s)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs"
    del g
    log(f"free device memory before/after: {free0} {torch.cuda.mem_get_info()[0]}")


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    # a plan whose split slices (M*N*splits*4 bytes) exceed the 64 MiB scratch: a clear error
    # before anything is launched, and C is left as it was (real buffers of the right sizes)
    M, K, N = 1312, 6144, 7680  # 3 slices of M*N floats: 115 MiB
    p = w4.plan(M, K, N)
    log(f"noalloc oversize plan={p}")
    assert p["workspace_bytes"] > (64 << 20) - (256 << 10)
    x = synth.generate_custom(M, K, N, seed=83)
    dev = to_dev(x)
    out = torch.full((M, N), 7.0, device="cuda")
    s = torch.cuda.Stream()
    with pytest.raises(w4.W4Error) as e:
        _noalloc(dev, out, s)
    torch.cuda.synchronize()
    assert e.value.code == 6 and "scratch" in str(e.value)
    assert bool((out == 7.0).all())
