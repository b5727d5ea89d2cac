"""Shared helpers for the GPU tests: upload synthetic inputs, call the C-ABI through the
binding, compare with the oracle element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import int4_weight_only_gemm_amd as w4
import oracle

REL, ABS = 1e-4, 1e-6  # |C_gpu - C| <= 1e-4 * sum_k |A W| + 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x, device="cuda"):
    """GemmInputs -> dict of device tensors in the boundary's dtypes."""
    d = {
        "A": torch.from_numpy(np.ascontiguousarray(x.A).view(np.int16)).to(device).view(torch.bfloat16),
        "S": torch.from_numpy(np.ascontiguousarray(x.S).view(np.int16)).to(device).view(torch.float16),
        "Z": torch.from_numpy(np.ascontiguousarray(x.Z)).to(device),
    }
    if x.Wq is not None:
        d["Wq"] = torch.from_numpy(np.ascontiguousarray(x.Wq).view(np.int32)).to(device)
    if x.q is not None:
        d["q"] = torch.from_numpy(np.ascontiguousarray(x.q)).to(device)
    return d


def host_words(x):
    """Packed words on the host: drawn directly, or packed by the oracle from the codes."""
    if x.Wq is not None:
        return x.Wq
    return oracle.get().pack(x.q)


def run(dev, out=None):
    return w4.gemm(dev["A"], dev["Wq"], dev["S"], dev["Z"], out=out)


def check(C_gpu: np.ndarray, C_ref: np.ndarray, Cabs: np.ndarray, what: str) -> float:
    """Assert the element-wise tolerance; return the worst error as a fraction of the bound
    1e-4*Cabs+1e-6 (for the log)."""
    C_gpu = np.asarray(C_gpu, np.float64)
    assert C_gpu.shape == C_ref.shape, (what, C_gpu.shape, C_ref.shape)
    assert np.all(np.isfinite(C_gpu)), f"{what}: non-finite output"
    err = np.abs(C_gpu - C_ref)
    bound = REL * Cabs + ABS
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at {tuple(i)}: "
                             f"gpu={C_gpu[tuple(i)]!r} ref={C_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return float(np.max(err / bound)) if err.size else 0.0
