"""Seeded synthetic inputs for the W4A16 GEMM: shapes, value distributions, RNG streams.

This module is shared by the oracle side (tests, the CPU baseline) and the HIP side
(tests, bench). It draws random numbers and lays them out in the boundary's storage
formats; it performs none of the GEMM's arithmetic (no unpacking, no dequantization,
no products or sums).

Workload shapes come from the models the pages measure:
  * "When Do Quantized Drafts Help Speculative Decoding?", section "Current pilot setup":
    a Qwen2.5-7B-Instruct target verifying a Qwen2.5-1.5B-Instruct draft at gamma=4, batch 1;
    the interpretation item (c) sweeps gamma over 2..6.
  * the same page, section "What is open": Llama2-7B at batch 32, the batched regime, and
    whether the ceiling holds at batch 8 and 16 (the Qwen2.5-7B verify at 40 and 80 rows).
  * "The Free Half of Speculative Decoding", third paragraph: the target is quantized to
    INT4 with AWQ (weight-only), the draft may be quantized as well.
The per-layer (K, N) sizes are the public architectures of those models (hidden size,
fused q/k/v width, fused gate/up width, MLP width); the pages do not print them.

Value recipe (the pages give no distribution; these are the stated synthetic inputs):
  A  ~ N(0, 1) drawn in float32, rounded to bfloat16 (round-to-nearest-even)
  q  ~ uniform integers 0..15   (4-bit codes); large workloads draw the packed u32 words
       directly, whose 8 nibbles are then i.i.d. uniform 0..15
  s  = |N(0, 1)| * 0.02 + 1e-3 computed in float64, rounded to float16 (RNE)
  z  ~ uniform integers 0..15, one byte each
8-bit weights (the GPTQ INT8 draft of "When Do Quantized Drafts Help Speculative Decoding?",
"Current pilot setup"): q and z uniform 0..255 (words: 4 i.i.d. uniform bytes), and the
4-bit scale recipe divided by 16, s = (|N(0, 1)| * 0.02 + 1e-3) / 16, so that the dequantized
weights span the same range as the 4-bit ones.
4-bit activations (the W4A4 draft of "When Do Quantized Drafts Help Speculative Decoding?",
"What is open"): codes uniform -8..7 as offset-binary nibbles (uniform u32 words), one
float32 scale per row and group of 128, (2.5 + 0.3 |N(0, 1)|) / 7, about what the largest
of 128 standard normal values gives.  The weights are the 4-bit recipe above.
Every (layer, projection) gets its own PCG64 stream spawned from
SeedSequence([0, workload_id, layer, projection_index]) so any single GEMM can be
regenerated without drawing the others.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

GROUP = 128  # quantization group length along K

# (K, N) per projection; K = input features, N = output features.
MODEL_SHAPES: Dict[str, Dict[str, Tuple[int, int]]] = {
    "qwen2.5-1.5b": {
        "qkv": (1536, 2048),
        "o": (1536, 1536),
        "gate_up": (1536, 17920),
        "down": (8960, 1536),
    },
    "qwen2.5-7b": {
        "qkv": (3584, 4608),
        "o": (3584, 3584),
        "gate_up": (3584, 37888),
        "down": (18944, 3584),
    },
    "llama2-7b": {
        "qkv": (4096, 12288),
        "o": (4096, 4096),
        "gate_up": (4096, 22016),
        "down": (11008, 4096),
    },
}
PROJ_ORDER = ("qkv", "o", "gate_up", "down")


@dataclasses.dataclass(frozen=True)
class GemmSpec:
    """One GEMM of a workload: C[M,N] = A[M,K] . W[K,N]."""
    name: str
    M: int
    K: int
    N: int
    seed: Tuple[int, ...]  # SeedSequence entropy for this GEMM's draws
    q_as_bytes: bool = False  # draw unpacked u8 codes (packed later by the pack entry point)
    bits: int = 4             # code width: 4 (W4A16) or 8 (W8A16)
    act4: bool = False        # 4-bit activations (W4A4) instead of bfloat16

    @property
    def weight_bytes(self) -> int:
        """Bytes of the quantized weight as stored at the boundary:
        K*N*bits/8 (codes) + 2*K*N/128 (fp16 scales) + K*N/128 (u8 zeros)."""
        g = self.K // GROUP
        return self.K * self.N * self.bits // 8 + 2 * g * self.N + g * self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.K * self.N


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    gemms: Tuple[GemmSpec, ...]

    @property
    def weight_bytes(self) -> int:
        return sum(g.weight_bytes for g in self.gemms)

    @property
    def flops(self) -> int:
        return sum(g.flops for g in self.gemms)


def _model_pass(wid: int, model: str, M: int, layers: int, bits: int = 4, act4: bool = False) -> Tuple[GemmSpec, ...]:
    out = []
    for layer in range(layers):
        for pi, proj in enumerate(PROJ_ORDER):
            K, N = MODEL_SHAPES[model][proj]
            out.append(GemmSpec(f"L{layer}.{proj}", M, K, N, (0, wid, layer, pi), bits=bits, act4=act4))
    return tuple(out)


def _gamma_sweep(wid: int, Ms=(3, 4, 5, 6, 7), copies: int = 28) -> Tuple[GemmSpec, ...]:
    # Weights are shared across M (same seed for the weight part), activations differ per M.
    out = []
    for M in Ms:
        for c in range(copies):
            for pi, proj in ((3, "down"), (2, "gate_up")):
                K, N = MODEL_SHAPES["qwen2.5-7b"][proj]
                out.append(GemmSpec(f"M{M}.C{c}.{proj}", M, K, N, (0, wid, c, pi, M)))
    return tuple(out)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload(
            "single-m5-k1536-n1536",
            "one W4A16 GEMM at M=5 (gamma=4 verify, batch 1), K=N=1536",
            (GemmSpec("single", 5, 1536, 1536, (0, 1, 0, 0), q_as_bytes=True),),
        ),
        Workload(
            "qwen2.5-1.5b-draft-m1",
            "draft step of a Qwen2.5-1.5B-shaped model, M=1, 28 layers x {qkv,o,gate_up,down}",
            _model_pass(2, "qwen2.5-1.5b", 1, 28),
        ),
        Workload(
            "qwen2.5-1.5b-draft-m1-w8",
            "draft step of a Qwen2.5-1.5B-shaped model with 8-bit weights (W8A16), M=1, "
            "28 layers x {qkv,o,gate_up,down}",
            _model_pass(8, "qwen2.5-1.5b", 1, 28, bits=8),
        ),
        Workload(
            "qwen2.5-7b-verify-m5",
            "verify pass of a Qwen2.5-7B-shaped target, M=gamma+1=5, 28 layers x {qkv,o,gate_up,down}",
            _model_pass(3, "qwen2.5-7b", 5, 28),
        ),
        Workload(
            "qwen2.5-7b-gamma-sweep",
            "Qwen2.5-7B down (18944x3584) and gate_up (3584x37888), 28 copies each, M in 3..7",
            _gamma_sweep(4),
        ),
        Workload(
            "qwen2.5-7b-batched-verify-m40",
            "batched verify of a Qwen2.5-7B-shaped target, batch 8 x (gamma+1) = 40 rows, "
            "28 layers x {qkv,o,gate_up,down}",
            _model_pass(6, "qwen2.5-7b", 40, 28),
        ),
        Workload(
            "qwen2.5-7b-batched-verify-m80",
            "batched verify of a Qwen2.5-7B-shaped target, batch 16 x (gamma+1) = 80 rows, "
            "28 layers x {qkv,o,gate_up,down}",
            _model_pass(7, "qwen2.5-7b", 80, 28),
        ),
        Workload(
            "llama2-7b-w4a4-draft-m32",
            "W4A4 draft step of a Llama-2-7B-shaped model at batch 32 (one token per sequence, M=32), "
            "32 layers x {qkv,o,gate_up,down}, 4-bit activations on the 4-bit weights",
            _model_pass(9, "llama2-7b", 32, 32, act4=True),
        ),
        Workload(
            "llama2-7b-batched-verify-m160",
            "batched verify of a Llama-2-7B-shaped target, M=32x5=160, 32 layers x {qkv,o,gate_up,down}",
            _model_pass(5, "llama2-7b", 160, 32),
        ),
    )
}


def with_copies(wl: Workload, copies: int) -> Workload:
    """The workload's GEMMs repeated `copies` times back to back, each copy with its own
    weights and activations (copy 0 is the workload itself).  Used to measure a small
    workload from HBM rather than from the on-chip caches."""
    if copies <= 1:
        return wl
    gemms = []
    for c in range(copies):
        for g in wl.gemms:
            seed = (g.seed[0], g.seed[1], g.seed[2] + 100000 * c) + tuple(g.seed[3:])
            gemms.append(dataclasses.replace(g, name=f"{g.name}.copy{c}", seed=seed))
    return Workload(f"{wl.name}-x{copies}", f"{wl.description}, {copies} distinct copies", tuple(gemms))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the u16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


@dataclasses.dataclass
class GemmInputs:
    """Host arrays in the boundary's storage formats (all C-contiguous)."""
    A: np.ndarray      # uint16 [M, K]   bfloat16 bit patterns, row-major
    Wq: np.ndarray     # uint32 [K*bits/32, N] packed codes (None if only q was drawn)
    q: Optional[np.ndarray]  # uint8 [K, N] unpacked codes, when drawn as bytes
    S: np.ndarray      # uint16 [K/128, N] float16 bit patterns
    Z: np.ndarray      # uint8 [K/128, N]  zero points (4-bit: low nibble used)
    Aq: Optional[np.ndarray] = None  # uint32 [M, K/8] 4-bit activation codes (W4A4), else None
    As: Optional[np.ndarray] = None  # float32 [M, K/128] activation scales (W4A4), else None


def _rng(seed: Tuple[int, ...]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def draw_activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def draw_scales(rng: np.random.Generator, G: int, N: int, bits: int = 4) -> np.ndarray:
    s = np.abs(rng.standard_normal((G, N))) * 0.02 + 1e-3
    if bits == 8:
        s = s / 16.0
    return s.astype(np.float16).view(np.uint16)


def draw_zeros(rng: np.random.Generator, G: int, N: int, bits: int = 4) -> np.ndarray:
    return rng.integers(0, 1 << bits, size=(G, N), dtype=np.uint8)


def draw_codes(rng: np.random.Generator, K: int, N: int, bits: int = 4) -> np.ndarray:
    return rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)


def draw_words(rng: np.random.Generator, K: int, N: int, bits: int = 4) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=(K * bits // 32, N), dtype=np.uint32)


def generate(spec: GemmSpec) -> GemmInputs:
    """Draw one GEMM's inputs. Weight draws use a stream that does not depend on M for the
    gamma sweep (its seed tuple ends with M; the weight stream drops that entry)."""
    M, K, N = spec.M, spec.K, spec.N
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    if spec.bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    G = K // GROUP
    wseed = spec.seed[:4]  # weight stream: shared by every M of a gamma-sweep copy
    wr = _rng(wseed + (1,))
    if spec.q_as_bytes:
        q = draw_codes(wr, K, N, spec.bits)
        Wq = None
    else:
        q = None
        Wq = draw_words(wr, K, N, spec.bits)
    S = draw_scales(wr, G, N, spec.bits)
    Z = draw_zeros(wr, G, N, spec.bits)
    ar = _rng(tuple(spec.seed) + (0,))
    A = draw_activations(ar, M, K)
    if spec.act4:
        Aq, As = draw_act4(ar, M, K)
        return GemmInputs(A=A, Wq=Wq, q=q, S=S, Z=Z, Aq=Aq, As=As)
    return GemmInputs(A=A, Wq=Wq, q=q, S=S, Z=Z)


def draw_act4(rng: np.random.Generator, M: int, K: int) -> Tuple[np.ndarray, np.ndarray]:
    """4-bit activation codes (offset-binary nibbles in uniform u32 words) and float32 scales."""
    Aq = rng.integers(0, 1 << 32, size=(M, K // 8), dtype=np.uint32)
    As = ((2.5 + 0.3 * np.abs(rng.standard_normal((M, K // GROUP)))) / 7.0).astype(np.float32)
    return Aq, As


def generate_custom(M: int, K: int, N: int, seed: int, q_as_bytes: bool = False,
                    z_range: Optional[Tuple[int, int]] = None, bits: int = 4, act4: bool = False) -> GemmInputs:
    """Inputs for an arbitrary shape (parity grids, edge cases) with the standard recipe."""
    spec = GemmSpec("custom", M, K, N, (0, 99 + (bits == 8), seed, M * 1_000_003 + K * 1009 + N), q_as_bytes,
                    bits=bits, act4=act4)
    x = generate(spec)
    if z_range is not None and z_range != (0, 1 << bits):
        r = _rng((0, 98, seed))
        x.Z = r.integers(z_range[0], z_range[1], size=x.Z.shape, dtype=np.uint8)
    return x


def iter_workload(name: str, limit: Optional[int] = None) -> Iterator[Tuple[GemmSpec, GemmInputs]]:
    wl = WORKLOADS[name]
    for i, spec in enumerate(wl.gemms):
        if limit is not None and i >= limit:
            return
        yield spec, generate(spec)


def workload_names() -> List[str]:
    return list(WORKLOADS)
