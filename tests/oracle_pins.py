"""Pins for the oracle: checks that tie it to something other than itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle disagrees
with what the mathematics or a worked example fixes. The pins are collected by
test_oracle_pins.py (run against the real oracle) and by test_oracle_mutants.py (run
against copies of the oracle with one plausible mistake planted, each of which must
fail at least one pin).

What pins what:
  * decoders: every one of the 65536 fp16 and bf16 bit patterns against numpy's own
    float16 and float32 conversions (hardware IEEE decoding, not the oracle's code);
  * packing: hand-worked words (tests/golden/pack_words.txt), round trips both ways,
    high-nibble masking;
  * the GEMM: hand-computed closed forms (tests/golden/closed_forms.txt), the identity
    case q=z+1, s=1 (row sums of A), the all-ones-A case (integer column sums of the
    codes), one-hot A (row extraction), q=z and s=0 (exact zeros), exact rational brute
    force with Python fractions on tiny shapes, a BLAS float64 matmul of an explicitly
    dequantized W at a mid size, power-of-two scaling, column sampling and thread-count
    invariance;
  * the binary16 encoder: numpy's IEEE binary32 -> binary16 conversion on every binary16
    value, every midpoint and random values;
  * the quantizer: values on the grid (exact scales, zeros and codes), ties at grid
    midpoints (to even), all-zero and one-signed groups, the half-step error bound and the
    scale's agreement with the range, power-of-two scaling, column and group permutations;
  * the 8-bit variant: hand-worked words (tests/golden/pack8_words.txt) and closed forms
    (tests/golden/closed_forms8.txt), round trips against numpy's byte view of the words,
    the identity and all-ones cases with zero points up to 254, one-hot rows, exact zeros,
    exact rational brute force, a BLAS float64 matmul of the dequantized W, column sampling,
    thread count and scale invariance;
  * 4-bit activations: hand-worked words (tests/golden/act4_words.txt), exact codes and
    scales on the grid, ties to even, all-zero groups, numpy's binary32 division for the
    scale with the half-step error bound, power-of-two scaling and negation; the W4A4
    product by hand-computed closed forms (tests/golden/closed_forms_a4.txt), rational brute
    force, a BLAS matmul, one-hot rows, exact zeros, the identity case, and equality with
    the W4A16 product where the dequantized activations are exact bfloat16 values.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------------------
# independent helpers (numpy / Python only; they do not call the oracle)
def np_bf16_to_f64(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def np_f16_to_f64(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def np_unpack(Wq):
    Wq = np.asarray(Wq, np.uint32)
    KB, N = Wq.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, :, None]
    return ((Wq[:, None, :] >> shifts) & 0xF).reshape(KB * 8, N).astype(np.uint8)


def np_pack(q):
    q = np.asarray(q, np.uint8) & 0xF
    K, N = q.shape
    q8 = q.reshape(K // 8, 8, N).astype(np.uint32)
    w = np.zeros((K // 8, N), np.uint32)
    for j in range(8):
        w |= q8[:, j, :] << np.uint32(4 * j)
    return w


def bf16_bits(values):
    """Exact bf16 encodings of values that are exactly representable."""
    v = np.asarray(values, np.float32)
    bits = v.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def f16_bits(values):
    v = np.asarray(values, np.float64)
    h = v.astype(np.float16)
    assert np.all(h.astype(np.float64) == v), "value not exactly representable in fp16"
    return h.view(np.uint16)


# ---------------------------------------------------------------------------------------
def pin_f16_decoder_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    ref = np_f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the sign of zero is kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


def pin_bf16_decoder_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_f64(bits)
    ref = np_bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _golden_pack_rows():
    rows = []
    with open(os.path.join(GOLDEN, "pack_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append(([int(p) for p in parts[:8]], int(parts[8], 16)))
    return rows


def pin_pack_golden(o):
    rows = _golden_pack_rows()
    assert len(rows) >= 8
    q = np.array([r[0] for r in rows], dtype=np.uint8).T.copy()  # [8, n]
    words = o.pack(q)
    assert words.shape == (1, len(rows))
    for i, (_, w) in enumerate(rows):
        assert int(words[0, i]) == w, f"golden row {i}: {int(words[0, i]):#010x} != {w:#010x}"
    # unpack returns the low nibbles of the golden inputs
    assert np.array_equal(o.unpack(words), q & 0xF)


def pin_pack_roundtrip(o):
    r = np.random.default_rng(7)
    q = r.integers(0, 16, size=(64, 37), dtype=np.uint8)
    w = o.pack(q)
    assert np.array_equal(o.unpack(w), q)
    assert np.array_equal(w, np_pack(q))
    words = r.integers(0, 1 << 32, size=(9, 13), dtype=np.uint32)
    assert np.array_equal(o.pack(o.unpack(words)), words)
    assert np.array_equal(o.unpack(words), np_unpack(words))


def pin_pack_high_nibble(o):
    r = np.random.default_rng(8)
    q = r.integers(0, 256, size=(32, 19), dtype=np.uint8)
    assert np.array_equal(o.pack(q), o.pack(q & 0xF))
    assert np.array_equal(o.unpack(o.pack(q)), q & 0xF)


def _closed_form_rows():
    rows = []
    with open(os.path.join(GOLDEN, "closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            K = int(parts[0])
            groups = [tuple(float(v) for v in p.split()) for p in parts[1:-1]]
            rows.append((K, groups, float(parts[-1])))
    return rows


def pin_closed_forms(o):
    rows = _closed_form_rows()
    assert len(rows) >= 4
    for K, groups, expect in rows:
        G = K // 128
        assert len(groups) == G
        N = 3
        A = np.zeros((2, K), np.float32)
        q = np.zeros((K, N), np.uint8)
        S = np.zeros((G, N), np.float64)
        Z = np.zeros((G, N), np.uint8)
        for g, (a, qq, zz, ss) in enumerate(groups):
            A[:, g * 128:(g + 1) * 128] = a
            q[g * 128:(g + 1) * 128, :] = int(qq)
            Z[g, :] = int(zz)
            S[g, :] = ss
        C, Cabs = o.gemm(bf16_bits(A), np_pack(q), f16_bits(S), Z)
        assert np.all(C == expect), (K, groups, C, expect)
        assert np.all(Cabs >= np.abs(C))


def pin_identity_rowsum(o):
    # q = z + 1 and s = 1 make W all ones, so C[m, n] is the row sum of A for every n.
    M, K, N = 3, 384, 11
    r = np.random.default_rng(11)
    A = synth.f32_to_bf16_bits(r.standard_normal((M, K), dtype=np.float32))
    Z = r.integers(0, 15, size=(K // 128, N), dtype=np.uint8)
    q = np.repeat(Z + 1, 128, axis=0).astype(np.uint8)
    S = f16_bits(np.ones((K // 128, N)))
    C, _ = o.gemm(A, np_pack(q), S, Z)
    a = np_bf16_to_f64(A)
    for m in range(M):
        rs = math.fsum(a[m])
        assert np.all(np.abs(C[m] - rs) <= K * 2.0 ** -53 * np.sum(np.abs(a[m])))


def pin_all_ones(o):
    # A = 1: C[m, n] = sum_g s[g,n] * (sum_{k in g} q[k,n] - 128 z[g,n]), integer inner sums.
    M, K, N = 2, 512, 9
    r = np.random.default_rng(12)
    q = r.integers(0, 16, size=(K, N), dtype=np.uint8)
    Z = r.integers(0, 16, size=(K // 128, N), dtype=np.uint8)
    S = synth.draw_scales(r, K // 128, N)
    A = bf16_bits(np.ones((M, K), np.float32))
    C, Cabs = o.gemm(A, np_pack(q), S, Z)
    s = np_f16_to_f64(S)
    for n in range(N):
        exact = Fraction(0)
        for g in range(K // 128):
            isum = int(q[g * 128:(g + 1) * 128, n].astype(np.int64).sum()) - 128 * int(Z[g, n])
            exact += Fraction(s[g, n]) * isum
        for m in range(M):
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(K) * Fraction(2) ** -53 * Fraction(Cabs[m, n])


def pin_one_hot(o):
    # A = a0 * e_{m0,k0}: row m0 of C is a0 * (q[k0,:] - z[g0,:]) * s[g0,:]; other rows are 0.
    M, K, N = 4, 384, 21
    x = synth.generate_custom(M, K, N, seed=13)
    q = np_unpack(x.Wq)
    s = np_f16_to_f64(x.S)
    for (m0, k0, a0) in ((0, 0, 1.0), (1, 7, -2.5), (3, 130, 0.375), (2, 255, 96.0), (1, 383, -0.0078125)):
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        C, _ = o.gemm(bf16_bits(A), x.Wq, x.S, x.Z)
        g0 = k0 // 128
        expect = a0 * (q[k0].astype(np.float64) - (x.Z[g0] & 0xF)) * s[g0]
        assert np.array_equal(C[m0], expect), (m0, k0)
        others = [m for m in range(M) if m != m0]
        assert np.all(C[others] == 0.0)


def pin_zero_cases(o):
    M, K, N = 3, 256, 17
    x = synth.generate_custom(M, K, N, seed=14)
    # q = z everywhere -> exactly zero
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)
    C, Cabs = o.gemm(x.A, np_pack(q), x.S, x.Z)
    assert np.all(C == 0.0) and np.all(Cabs == 0.0)
    # s = 0 -> exactly zero
    C, _ = o.gemm(x.A, x.Wq, np.zeros_like(x.S), x.Z)
    assert np.all(C == 0.0)


def pin_zero_high_nibble(o):
    M, K, N = 2, 256, 13
    x = synth.generate_custom(M, K, N, seed=15)
    r = np.random.default_rng(15)
    Zg = (x.Z | (r.integers(1, 16, size=x.Z.shape, dtype=np.uint8) << 4)).astype(np.uint8)
    C1, _ = o.gemm(x.A, x.Wq, x.S, x.Z)
    C2, _ = o.gemm(x.A, x.Wq, x.S, Zg)
    assert np.array_equal(C1, C2)


def _exact_gemm(A, Wq, S, Z):
    a = np_bf16_to_f64(A)
    q = np_unpack(Wq).astype(np.int64)
    s = np_f16_to_f64(S)
    z = (np.asarray(Z) & 0xF).astype(np.int64)
    M, K = a.shape
    N = q.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            g = k // 128
            w = Fraction(s[g, n]) * int(q[k, n] - z[g, n])
            for m in range(M):
                t = Fraction(a[m, k]) * w
                C[m][n] += t
                B[m][n] += abs(t)
    return C, B


def pin_brute_force(o):
    for (M, K, N, seed) in ((1, 128, 3, 1), (3, 256, 5, 2), (2, 128, 4, 3)):
        x = synth.generate_custom(M, K, N, seed=100 + seed)
        Zg = (x.Z | np.uint8(0xA0)).astype(np.uint8)  # high nibbles must not matter
        C, Cabs = o.gemm(x.A, x.Wq, x.S, Zg)
        Ce, Be = _exact_gemm(x.A, x.Wq, x.S, x.Z)
        bound_scale = Fraction(K) * Fraction(2) ** -53
        for m in range(M):
            for n in range(N):
                assert abs(Fraction(C[m, n]) - Ce[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)
                assert abs(Fraction(Cabs[m, n]) - Be[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)


def pin_numpy_matmul(o):
    # mid size: a BLAS float64 matmul of an explicitly dequantized W (numpy decoding)
    M, K, N = 5, 1536, 1536
    x = synth.generate(synth.WORKLOADS["single-m5-k1536-n1536"].gemms[0])
    Wq = np_pack(x.q)
    C, Cabs = o.gemm(x.A, Wq, x.S, x.Z)
    g = np.arange(K) // 128
    W = (x.q.astype(np.float64) - (x.Z[g] & 0xF)) * np_f16_to_f64(x.S)[g]
    Cn = np_bf16_to_f64(x.A) @ W
    assert np.all(np.abs(Cn - C) <= 1e-12 * Cabs)
    absn = np.abs(np_bf16_to_f64(x.A)) @ np.abs(W)
    assert np.all(np.abs(absn - Cabs) <= 1e-12 * Cabs)


def pin_power_of_two_scaling(o):
    M, K, N = 3, 256, 7
    x = synth.generate_custom(M, K, N, seed=16)
    C, _ = o.gemm(x.A, x.Wq, x.S, x.Z)
    A2 = bf16_bits(np_bf16_to_f64(x.A).astype(np.float32) * np.float32(4.0))
    C2, _ = o.gemm(A2, x.Wq, x.S, x.Z)
    assert np.array_equal(C2, 4.0 * C)
    S2 = f16_bits(np_f16_to_f64(x.S) * 0.5)
    C3, _ = o.gemm(x.A, x.Wq, S2, x.Z)
    assert np.array_equal(C3, 0.5 * C)


def pin_column_sampling_and_threads(o):
    M, K, N = 4, 512, 97
    x = synth.generate_custom(M, K, N, seed=17)
    C, Cabs = o.gemm(x.A, x.Wq, x.S, x.Z)
    C1, _ = o.gemm(x.A, x.Wq, x.S, x.Z, threads=1)
    assert np.array_equal(C, C1)
    cols = np.array([96, 0, 41, 41, 7], np.int64)
    Cs, Cabss = o.gemm(x.A, x.Wq, x.S, x.Z, cols=cols)
    assert np.array_equal(Cs, C[:, cols]) and np.array_equal(Cabss, Cabs[:, cols])


# ---------------------------------------------------------------------------------------
# The binary16 encoder and the quantizer (the producer side of the format)
def pin_f16_encoder_against_numpy(o):
    """binary32 -> binary16 must match numpy's IEEE conversion (ties to even): every
    binary16 value, every midpoint between neighbours, the overflow and underflow edges
    and random binary32 values."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = h[np.isfinite(h)].astype(np.float64)
    vals = np.unique(fin)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in binary64; representable in binary32
    rng = np.random.default_rng(5)
    rnd = np.r_[rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -26, 2.0 ** -14,
                2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]
    x32 = np.r_[vals, mids, -mids, rnd].astype(np.float32)
    with np.errstate(over="ignore"):
        want = x32.astype(np.float16).view(np.uint16)
    got = np.array([o.f32_to_f16(float(v)) for v in x32], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} encodings differ, first {x32[bad[0]]!r}: {got[bad[0]]:#06x} vs {want[bad[0]]:#06x}"


def _grid_group(s, z, reps=8):
    """128 values on the quantization grid (j - z) * s, j = 0..15, each repeated."""
    return np.repeat((np.arange(16) - z) * s, reps)


GRID_CASES = [(0.5, 6), (0.125, 0), (2.0 ** -10, 15), (3 * 2.0 ** -6, 8), (1.25, 3), (1024.0, 9)]


def pin_quantize_grid_exact(o):
    """Values on the grid (j - z)*s with the grid's ends present: the scale, zero and every
    code come back exactly (s, 15s and (j-z)s are exact in binary16 here)."""
    cols = [np.r_[_grid_group(s, z), _grid_group(s, z)[::-1]] for s, z in GRID_CASES]
    W = np.stack(cols, axis=1)  # K = 256: two groups, the second in reverse order
    Wq, S, Z = o.quantize(f16_bits(W))
    q = np.stack([np.r_[np.repeat(np.arange(16), 8), np.repeat(np.arange(16), 8)[::-1]] for _ in GRID_CASES], 1)
    assert np.array_equal(np_unpack(Wq), q), "codes differ on the grid"
    assert np.array_equal(S, np.tile(f16_bits([s for s, _ in GRID_CASES]), (2, 1))), "scales differ"
    assert np.array_equal(Z, np.tile(np.array([z for _, z in GRID_CASES], np.uint8), (2, 1))), "zeros differ"


def pin_quantize_ties_to_even(o):
    """Values halfway between grid points round to the even code offset (ties to even),
    with the grid's ends present so that s and z are those of the grid."""
    cols, want = [], []
    for s, z in GRID_CASES:
        mid = (np.arange(15) - z + 0.5) * s
        g = np.r_[-z * s, (15 - z) * s, np.resize(mid, 126)]
        cols.append(g)
        r = np.array([round(v) for v in np.resize(np.arange(15) - z + 0.5, 126)])  # Python round: ties to even
        want.append(np.r_[0, 15, r + z])
    Wq, S, Z = o.quantize(f16_bits(np.stack(cols, 1)))
    assert np.array_equal(np_unpack(Wq), np.stack(want, 1).astype(np.uint8)), "ties do not round to even"


def pin_quantize_all_zero(o):
    """An all-zero group (either sign of zero) takes s = binary16(2/15) and z = 8, so every
    code is 8 and dequantizes to 0 exactly."""
    W = np.zeros((256, 3), np.float64)
    bits = f16_bits(W)
    bits[128:, 1] = 0x8000  # -0.0
    Wq, S, Z = o.quantize(bits)
    s215 = np.array([np.float32(2) / np.float32(15)], np.float32).astype(np.float16).view(np.uint16)[0]
    assert np.all(S == s215) and np.all(Z == 8), "degenerate group parameters"
    assert np.all(np_unpack(Wq) == 8), "degenerate group codes"


def pin_quantize_one_signed_groups(o):
    """The range always holds 0: an all-positive group gets z = 0 and its largest value code
    15; an all-negative group with an exact scale gets z = 15 and its smallest value code 0."""
    rng = np.random.default_rng(6)
    pos = np.r_[2.0, rng.uniform(1.0, 2.0, 127)].astype(np.float16).astype(np.float64)
    neg = np.r_[-1.875, -0.5, rng.uniform(-1.875, -0.5, 126)].astype(np.float16).astype(np.float64)
    Wq, S, Z = o.quantize(f16_bits(np.stack([pos, neg], 1)))
    q = np_unpack(Wq)
    assert Z[0, 0] == 0 and q[0, 0] == 15, "all-positive group"
    assert np_f16_to_f64(S[0, 1]) == 0.125 and Z[0, 1] == 15 and q[0, 1] == 0, "all-negative group"
    assert q[:, 0].min() >= 7 and q[:, 1].max() <= 11, "codes outside the values' range"


def _dequant_error(W, Wq, S, Z):
    q = np_unpack(Wq).astype(np.float64)
    K, N = q.shape
    s = np.repeat(np_f16_to_f64(S), 128, axis=0)
    z = np.repeat(Z.astype(np.float64), 128, axis=0)
    return np.abs(W - (q - z) * s), s


def pin_quantize_error_bound(o):
    """Every element dequantizes to within about half a step of its value: the codes are the
    nearest grid points, and the grid spans the group's range (up to the scale's binary16
    rounding).  Scales track (max - min)/15 within binary16 rounding; zeros lie in 0..15."""
    rng = np.random.default_rng(7)
    K, N = 512, 67
    mag = 10.0 ** rng.integers(-4, 4, N)
    W = (rng.standard_normal((K, N)) * mag).astype(np.float16).astype(np.float64)
    W[:, 5] = np.abs(W[:, 5])
    W[:, 6] = -np.abs(W[:, 6])
    Wq, S, Z = o.quantize(f16_bits(W))
    err, s = _dequant_error(W, Wq, S, Z)
    assert np.all(err <= 0.51 * s), f"dequantization error {np.max(err / s):.3f} steps"
    Wg = W.reshape(K // 128, 128, N)
    rng_ = np.maximum(Wg.max(1), 0) - np.minimum(Wg.min(1), 0)
    half_ulp = np.maximum(2.0 ** -11 * rng_ / 15, 2.0 ** -25)  # relative, or absolute for subnormals
    assert np.all(np.abs(np_f16_to_f64(S) - rng_ / 15) <= half_ulp * 1.01), "scale off its range"
    assert Z.max() <= 15


def pin_quantize_power_of_two(o):
    """Scaling the weights by 2^3 or 2^-3 (exact in binary16 here) leaves codes and zeros
    unchanged and scales the scales by the same power of two."""
    rng = np.random.default_rng(8)
    W = rng.standard_normal((256, 33)).astype(np.float16).astype(np.float64)
    W[np.abs(W) < 2.0 ** -10] = 0.0  # stay clear of binary16 subnormals when scaled down
    base = o.quantize(f16_bits(W))
    for e in (3, -3):
        Wq, S, Z = o.quantize(f16_bits(W * 2.0 ** e))
        assert np.array_equal(Wq, base[0]) and np.array_equal(Z, base[2]), f"codes change under 2^{e}"
        assert np.array_equal(np_f16_to_f64(S), np_f16_to_f64(base[1]) * 2.0 ** e), f"scales under 2^{e}"


def pin_quantize_layout(o):
    """Columns and groups are independent: permuting columns, or swapping two groups of
    rows, permutes the outputs the same way."""
    rng = np.random.default_rng(9)
    W = rng.standard_normal((384, 19)).astype(np.float16).astype(np.float64)
    Wq, S, Z = o.quantize(f16_bits(W))
    perm = rng.permutation(19)
    Wq2, S2, Z2 = o.quantize(f16_bits(W[:, perm]))
    assert np.array_equal(Wq2, Wq[:, perm]) and np.array_equal(S2, S[:, perm]) and np.array_equal(Z2, Z[:, perm])
    Wsw = np.r_[W[256:], W[128:256], W[:128]]
    Wq3, S3, Z3 = o.quantize(f16_bits(Wsw))
    assert np.array_equal(Wq3, np.r_[Wq[32:], Wq[16:32], Wq[:16]]), "group order"
    assert np.array_equal(S3, S[::-1]) and np.array_equal(Z3, Z[::-1]), "group order of scales/zeros"


# ---------------------------------------------------------------------------------------
# The 8-bit variant (W8A16): codes and zero points 0..255, 4 codes per u32 along K.
def np_unpack8(Wq8):
    Wq8 = np.asarray(Wq8, np.uint32)
    KB, N = Wq8.shape
    shifts = (8 * np.arange(4, dtype=np.uint32))[None, :, None]
    return ((Wq8[:, None, :] >> shifts) & 0xFF).reshape(KB * 4, N).astype(np.uint8)


def np_pack8(q):
    # on this little-endian host the four bytes of a packed word are q[4kb..4kb+3] in order
    q = np.ascontiguousarray(np.asarray(q, np.uint8))
    K, N = q.shape
    return np.ascontiguousarray(q.reshape(K // 4, 4, N).transpose(0, 2, 1)).view("<u4").reshape(K // 4, N)


def pin_pack8_golden(o):
    rows = []
    with open(os.path.join(GOLDEN, "pack8_words.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                parts = line.split()
                rows.append(([int(p) for p in parts[:4]], int(parts[4], 16)))
    assert len(rows) >= 8
    q = np.array([r[0] for r in rows], dtype=np.uint8).T.copy()  # [4, n]
    words = o.pack8(q)
    assert words.shape == (1, len(rows))
    assert [int(w) for w in words[0]] == [r[1] for r in rows]
    assert np.array_equal(o.unpack8(words), q)


def pin_pack8_roundtrip(o):
    r = np.random.default_rng(21)
    q = r.integers(0, 256, size=(64, 23), dtype=np.uint8)
    assert np.array_equal(o.pack8(q), np_pack8(q))
    assert np.array_equal(o.unpack8(o.pack8(q)), q)
    w = r.integers(0, 1 << 32, size=(16, 9), dtype=np.uint32)
    assert np.array_equal(o.pack8(o.unpack8(w)), w)
    assert np.array_equal(o.unpack8(w), np_unpack8(w))


def pin_closed_forms8(o):
    rows = []
    with open(os.path.join(GOLDEN, "closed_forms8.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                parts = [p.strip() for p in line.split("|")]
                rows.append((int(parts[0]), [tuple(float(v) for v in p.split()) for p in parts[1:-1]],
                             float(parts[-1])))
    assert len(rows) >= 4
    for K, groups, expect in rows:
        G = K // 128
        assert len(groups) == G
        N = 5
        A = np.zeros((2, K), np.float32)
        q = np.zeros((K, N), np.uint8)
        S = np.zeros((G, N), np.float64)
        Z = np.zeros((G, N), np.uint8)
        for g, (a, qq, zz, ss) in enumerate(groups):
            A[:, g * 128:(g + 1) * 128] = a
            q[g * 128:(g + 1) * 128, :] = int(qq)
            Z[g, :] = int(zz)
            S[g, :] = ss
        C, Cabs = o.gemm(bf16_bits(A), np_pack8(q), f16_bits(S), Z, bits=8)
        assert np.all(C == expect), (K, groups, C, expect)
        assert np.all(Cabs >= np.abs(C))


def pin_identity_rowsum8(o):
    # q = z + 1 (z up to 254) and s = 1 make W all ones: every column is the row sum of A.
    M, K, N = 3, 384, 11
    r = np.random.default_rng(22)
    A = synth.f32_to_bf16_bits(r.standard_normal((M, K), dtype=np.float32))
    Z = r.integers(0, 255, size=(K // 128, N), dtype=np.uint8)
    Z[0, 0] = 254
    q = np.repeat(Z + 1, 128, axis=0).astype(np.uint8)
    S = f16_bits(np.ones((K // 128, N)))
    C, _ = o.gemm(A, np_pack8(q), S, Z, bits=8)
    a = np_bf16_to_f64(A)
    for m in range(M):
        rs = math.fsum(a[m])
        assert np.all(np.abs(C[m] - rs) <= K * 2.0 ** -53 * np.sum(np.abs(a[m])))


def pin_all_ones8(o):
    # A = 1: C[m, n] = sum_g s[g,n] * (sum_{k in g} q[k,n] - 128 z[g,n]), integer inner sums.
    M, K, N = 2, 512, 9
    r = np.random.default_rng(23)
    q = r.integers(0, 256, size=(K, N), dtype=np.uint8)
    Z = r.integers(0, 256, size=(K // 128, N), dtype=np.uint8)
    S = synth.draw_scales(r, K // 128, N, bits=8)
    A = bf16_bits(np.ones((M, K), np.float32))
    C, Cabs = o.gemm(A, np_pack8(q), S, Z, bits=8)
    s = np_f16_to_f64(S)
    for n in range(N):
        exact = Fraction(0)
        for g in range(K // 128):
            isum = int(q[g * 128:(g + 1) * 128, n].astype(np.int64).sum()) - 128 * int(Z[g, n])
            exact += Fraction(s[g, n]) * isum
        for m in range(M):
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(K) * Fraction(2) ** -53 * Fraction(Cabs[m, n])


def pin_one_hot8(o):
    # A = a0 * e_{m0,k0}: row m0 of C is a0 * (q[k0,:] - z[g0,:]) * s[g0,:], exactly.
    M, K, N = 4, 384, 21
    x = synth.generate_custom(M, K, N, seed=24, bits=8)
    q = np_unpack8(x.Wq)
    s = np_f16_to_f64(x.S)
    for (m0, k0, a0) in ((0, 0, 1.0), (1, 3, -2.5), (3, 129, 0.375), (2, 254, 96.0), (1, 383, -0.0078125)):
        A = np.zeros((M, K), np.float32)
        A[m0, k0] = a0
        C, _ = o.gemm(bf16_bits(A), x.Wq, x.S, x.Z, bits=8)
        g0 = k0 // 128
        expect = a0 * (q[k0].astype(np.float64) - x.Z[g0]) * s[g0]
        assert np.array_equal(C[m0], expect), (m0, k0)
        assert np.all(C[[m for m in range(M) if m != m0]] == 0.0)


def pin_zero_cases8(o):
    M, K, N = 3, 256, 17
    x = synth.generate_custom(M, K, N, seed=25, bits=8)
    q = np.repeat(x.Z, 128, axis=0).astype(np.uint8)
    C, Cabs = o.gemm(x.A, np_pack8(q), x.S, x.Z, bits=8)
    assert np.all(C == 0.0) and np.all(Cabs == 0.0)
    C, _ = o.gemm(x.A, x.Wq, np.zeros_like(x.S), x.Z, bits=8)
    assert np.all(C == 0.0)


def _exact_gemm8(A, Wq8, S, Z):
    a = np_bf16_to_f64(A)
    q = np_unpack8(Wq8).astype(np.int64)
    s = np_f16_to_f64(S)
    z = np.asarray(Z).astype(np.int64)
    M, K = a.shape
    N = q.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            g = k // 128
            w = Fraction(s[g, n]) * int(q[k, n] - z[g, n])
            for m in range(M):
                t = Fraction(a[m, k]) * w
                C[m][n] += t
                B[m][n] += abs(t)
    return C, B


def pin_brute_force8(o):
    for (M, K, N, seed) in ((1, 128, 3, 1), (3, 256, 5, 2), (2, 128, 4, 3)):
        x = synth.generate_custom(M, K, N, seed=200 + seed, bits=8)
        C, Cabs = o.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
        Ce, Be = _exact_gemm8(x.A, x.Wq, x.S, x.Z)
        bound_scale = Fraction(K) * Fraction(2) ** -53
        for m in range(M):
            for n in range(N):
                assert abs(Fraction(C[m, n]) - Ce[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)
                assert abs(Fraction(Cabs[m, n]) - Be[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)


def pin_numpy_matmul8(o):
    # mid size: a BLAS float64 matmul of an explicitly dequantized W (numpy decoding)
    M, K, N = 3, 1536, 2048
    x = synth.generate_custom(M, K, N, seed=26, bits=8)
    C, Cabs = o.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
    g = np.arange(K) // 128
    W = (np_unpack8(x.Wq).astype(np.float64) - x.Z[g]) * np_f16_to_f64(x.S)[g]
    Cn = np_bf16_to_f64(x.A) @ W
    assert np.all(np.abs(Cn - C) <= 1e-12 * Cabs)
    absn = np.abs(np_bf16_to_f64(x.A)) @ np.abs(W)
    assert np.all(np.abs(absn - Cabs) <= 1e-12 * Cabs)


def pin_w8_sampling_scaling_threads(o):
    M, K, N = 4, 512, 97
    x = synth.generate_custom(M, K, N, seed=27, bits=8)
    C, Cabs = o.gemm(x.A, x.Wq, x.S, x.Z, bits=8)
    C1, _ = o.gemm(x.A, x.Wq, x.S, x.Z, threads=1, bits=8)
    assert np.array_equal(C, C1)
    cols = np.array([96, 0, 41, 41, 7], np.int64)
    Cs, Cabss = o.gemm(x.A, x.Wq, x.S, x.Z, cols=cols, bits=8)
    assert np.array_equal(Cs, C[:, cols]) and np.array_equal(Cabss, Cabs[:, cols])
    S2 = f16_bits(np_f16_to_f64(x.S) * 2.0)  # exact: the 8-bit scales are far below the fp16 maximum
    C3, _ = o.gemm(x.A, x.Wq, S2, x.Z, bits=8)
    assert np.array_equal(C3, 2.0 * C)


# ---------------------------------------------------------------------------------------
# 4-bit activations (W4A4): symmetric codes per row and group of 128, offset-binary nibbles.
def np_act_codes(Aq):
    """Signed activation codes [M, K] from the packed words (numpy decoding)."""
    Aq = np.asarray(Aq, np.uint32)
    M, KB = Aq.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    return (((Aq[:, :, None] >> shifts) & 0xF).reshape(M, KB * 8).astype(np.int64) - 8)


def np_pack_act(qa):
    """Pack signed codes [M, K] (-8..7) into offset-binary words [M, K/8]."""
    u = (np.asarray(qa, np.int64) + 8).astype(np.uint32)
    M, K = u.shape
    u = u.reshape(M, K // 8, 8)
    w = np.zeros((M, K // 8), np.uint32)
    for j in range(8):
        w |= u[:, :, j] << np.uint32(4 * j)
    return w


def pin_a4_golden_words(o):
    rows = []
    with open(os.path.join(GOLDEN, "act4_words.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                parts = line.split()
                rows.append(([float(v) for v in parts[:8]], int(parts[8], 16)))
    assert len(rows) >= 5
    A = np.zeros((len(rows), 128), np.float32)
    for i, (vals, _) in enumerate(rows):
        A[i, 40:48] = vals  # the word of k = 40..47; the rest of the group is 0
    Aq, As = o.quantize_activations(bf16_bits(A))
    for i, (_, word) in enumerate(rows):
        assert As[i, 0] == 1.0, (i, As[i, 0])
        assert int(Aq[i, 5]) == word, (i, hex(int(Aq[i, 5])), hex(word))
        assert all(int(Aq[i, j]) == 0x88888888 for j in range(16) if j != 5)


def pin_a4_grid_exact(o):
    # A = qa * 2^e with some |qa| = 7 in each group: the scale is exactly 2^e, codes exact
    r = np.random.default_rng(41)
    M, K = 4, 512
    e = r.integers(-20, 20, size=(M, K // 128))
    qa = r.integers(-7, 8, size=(M, K))
    qa[:, ::128] = 7 * r.choice([-1, 1], size=(M, K // 128))
    A = (qa * np.exp2(np.repeat(e, 128, axis=1))).astype(np.float32)
    Aq, As = o.quantize_activations(bf16_bits(A))
    assert np.array_equal(As, np.exp2(e).astype(np.float32))
    assert np.array_equal(np_act_codes(Aq), qa)


def pin_a4_ties_to_even(o):
    r = np.random.default_rng(42)
    halves = r.integers(-6, 7, size=(3, 128)) + 0.5
    halves[:, 0] = 7.0
    Aq, As = o.quantize_activations(bf16_bits(halves.astype(np.float32)))
    expect = np.array([[round(v) for v in row] for row in halves])  # Python rounds ties to even
    assert np.all(As == 1.0)
    assert np.array_equal(np_act_codes(Aq), expect)


def pin_a4_zero_group(o):
    A = np.zeros((2, 256), np.float32)
    A[1, 128:] = 0.25
    A[0, 200] = -3.0
    Aq, As = o.quantize_activations(bf16_bits(A))
    assert As[0, 0] == 0.0 and As[1, 0] == 0.0
    assert np.all(Aq[:, :16] == 0x88888888)
    qa = np_act_codes(Aq)
    assert qa[0, 200] == -7 and np.all(np.delete(qa[0, 128:], 72) == 0)
    assert np.all(qa[1, 128:] == 7)


def pin_a4_error_bound_and_scale(o):
    # random activations: the scale is the group's largest magnitude over 7 (numpy binary32
    # division), every code is within half a step of A / scale, the largest element maps
    # to +-7, and no code leaves -8..7
    r = np.random.default_rng(43)
    M, K = 6, 1024
    A = r.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    A[2] *= np.float32(2.0 ** 30)
    A[3] *= np.float32(2.0 ** -30)
    Ab = bf16_bits(np_bf16_to_f64(synth.f32_to_bf16_bits(A)).astype(np.float32))
    Aq, As = o.quantize_activations(Ab)
    a = np_bf16_to_f64(Ab).reshape(M, K // 128, 128)
    amax = np.abs(a).max(axis=2).astype(np.float32)
    assert np.array_equal(As, amax / np.float32(7.0))
    qa = np_act_codes(Aq).reshape(M, K // 128, 128)
    assert qa.min() >= -8 and qa.max() <= 7
    s = As.astype(np.float64)[:, :, None]
    assert np.all(np.abs(a - s * qa) <= 0.5 * s * (1 + 2.0 ** -20))
    assert np.all(np.abs(qa).max(axis=2) == 7)


def pin_a4_scaling_and_sign(o):
    r = np.random.default_rng(44)
    A = synth.f32_to_bf16_bits(r.standard_normal((3, 384), dtype=np.float32))
    Aq, As = o.quantize_activations(A)
    a = np_bf16_to_f64(A)
    Aq2, As2 = o.quantize_activations(bf16_bits((a * 8.0).astype(np.float32)))
    assert np.array_equal(Aq2, Aq) and np.array_equal(As2, As * np.float32(8.0))
    Aq3, As3 = o.quantize_activations(bf16_bits((-a).astype(np.float32)))
    assert np.array_equal(As3, As) and np.array_equal(np_act_codes(Aq3), -np_act_codes(Aq))


def pin_a4_gemm_closed_forms(o):
    rows = []
    with open(os.path.join(GOLDEN, "closed_forms_a4.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                parts = [p.strip() for p in line.split("|")]
                rows.append((int(parts[0]), [tuple(float(v) for v in p.split()) for p in parts[1:-1]],
                             float(parts[-1])))
    assert len(rows) >= 4
    for K, groups, expect in rows:
        G = K // 128
        N = 3
        qa = np.zeros((2, K), np.int64)
        As = np.zeros((2, G), np.float32)
        q = np.zeros((K, N), np.uint8)
        S = np.zeros((G, N), np.float64)
        Z = np.zeros((G, N), np.uint8)
        for g, (c, sa, qq, zz, ss) in enumerate(groups):
            qa[:, g * 128:(g + 1) * 128] = int(c)
            As[:, g] = sa
            q[g * 128:(g + 1) * 128, :] = int(qq)
            Z[g, :] = int(zz)
            S[g, :] = ss
        assert np.all(As.astype(np.float64) == [[g[1] for g in groups]] * 2)
        C, Cabs = o.gemm_a4(np_pack_act(qa), As, np_pack(q), f16_bits(S), Z)
        assert np.all(C == expect), (K, groups, C, expect)
        assert np.all(Cabs >= np.abs(C))


def _a4_inputs(M, K, N, seed):
    x = synth.generate_custom(M, K, N, seed=seed)
    Aq, As = (lambda r: (np_pack_act(r.integers(-8, 8, size=(M, K))),
                         (np.abs(r.standard_normal((M, K // 128))) * 0.1 + 1e-3).astype(np.float32)))(
        np.random.default_rng(seed))
    return Aq, As, x


def _exact_gemm_a4(Aq, As, Wq, S, Z):
    qa = np_act_codes(Aq)
    q = np_unpack(Wq).astype(np.int64)
    s = np_f16_to_f64(S)
    z = (np.asarray(Z) & 0xF).astype(np.int64)
    M, K = qa.shape
    N = q.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    B = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            g = k // 128
            w = Fraction(s[g, n]) * int(q[k, n] - z[g, n])
            for m in range(M):
                t = Fraction(float(As[m, g])) * int(qa[m, k]) * w
                C[m][n] += t
                B[m][n] += abs(t)
    return C, B


def pin_a4_gemm_brute_force(o):
    for (M, K, N, seed) in ((1, 128, 3, 51), (3, 256, 5, 52), (2, 128, 4, 53)):
        Aq, As, x = _a4_inputs(M, K, N, seed)
        C, Cabs = o.gemm_a4(Aq, As, x.Wq, x.S, x.Z)
        Ce, Be = _exact_gemm_a4(Aq, As, x.Wq, x.S, x.Z)
        bound_scale = Fraction(K) * Fraction(2) ** -53
        for m in range(M):
            for n in range(N):
                assert abs(Fraction(C[m, n]) - Ce[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)
                assert abs(Fraction(Cabs[m, n]) - Be[m][n]) <= bound_scale * Be[m][n], (M, K, N, m, n)


def pin_a4_gemm_numpy_matmul(o):
    M, K, N = 5, 1536, 1024
    Aq, As, x = _a4_inputs(M, K, N, 54)
    C, Cabs = o.gemm_a4(Aq, As, x.Wq, x.S, x.Z)
    g = np.arange(K) // 128
    Ad = np_act_codes(Aq) * As.astype(np.float64)[:, g]
    W = (np_unpack(x.Wq).astype(np.float64) - (x.Z[g] & 0xF)) * np_f16_to_f64(x.S)[g]
    assert np.all(np.abs(Ad @ W - C) <= 1e-12 * Cabs)
    assert np.all(np.abs(np.abs(Ad) @ np.abs(W) - Cabs) <= 1e-12 * Cabs)


def pin_a4_gemm_one_hot_zero_identity(o):
    M, K, N = 4, 384, 21
    Aq, As, x = _a4_inputs(M, K, N, 55)
    q = np_unpack(x.Wq)
    s = np_f16_to_f64(x.S)
    for (m0, k0, c0) in ((0, 0, 1), (1, 7, -8), (3, 130, 7), (2, 383, -3)):
        qa = np.zeros((M, K), np.int64)
        qa[m0, k0] = c0
        C, _ = o.gemm_a4(np_pack_act(qa), As, x.Wq, x.S, x.Z)
        g0 = k0 // 128
        expect = float(As[m0, g0]) * c0 * (q[k0].astype(np.float64) - (x.Z[g0] & 0xF)) * s[g0]
        assert np.array_equal(C[m0], expect) and np.all(np.delete(C, m0, axis=0) == 0.0)
    C, Cabs = o.gemm_a4(np_pack_act(np.zeros((M, K), np.int64)), As, x.Wq, x.S, x.Z)
    assert np.all(C == 0.0) and np.all(Cabs == 0.0)
    C, _ = o.gemm_a4(Aq, As, np_pack(np.repeat(x.Z & 0xF, 128, axis=0)), x.S, x.Z)
    assert np.all(C == 0.0)
    # q = z + 1 and s = 1: every column is the row sum of the dequantized activations
    Zs = np.random.default_rng(56).integers(0, 15, size=x.Z.shape, dtype=np.uint8)
    C, _ = o.gemm_a4(Aq, As, np_pack(np.repeat(Zs + 1, 128, axis=0)), f16_bits(np.ones(x.S.shape)), Zs)
    rows = (np_act_codes(Aq) * As.astype(np.float64)[:, np.arange(K) // 128])
    for m in range(M):
        assert np.all(np.abs(C[m] - math.fsum(rows[m])) <= K * 2.0 ** -53 * np.abs(rows[m]).sum())


def pin_a4_gemm_matches_w4a16_on_exact_activations(o):
    # with power-of-two activation scales, sa * qa is an exact bfloat16: the W4A4 product
    # must equal the W4A16 product of those dequantized activations, bit for bit
    M, K, N = 3, 512, 40
    r = np.random.default_rng(57)
    Aq, _, x = _a4_inputs(M, K, N, 58)
    As = np.exp2(r.integers(-12, 12, size=(M, K // 128))).astype(np.float32)
    Ad = (np_act_codes(Aq) * As.astype(np.float64)[:, np.arange(K) // 128]).astype(np.float32)
    C4, _ = o.gemm_a4(Aq, As, x.Wq, x.S, x.Z)
    C16, _ = o.gemm(bf16_bits(Ad), x.Wq, x.S, x.Z)
    assert np.array_equal(C4, C16)
    cols = np.array([39, 0, 17], np.int64)
    Cs, _ = o.gemm_a4(Aq, As, x.Wq, x.S, x.Z, cols=cols, threads=1)
    assert np.array_equal(Cs, C4[:, cols])


ALL_PINS = [
    pin_f16_encoder_against_numpy,
    pin_quantize_grid_exact,
    pin_quantize_ties_to_even,
    pin_quantize_all_zero,
    pin_quantize_one_signed_groups,
    pin_quantize_error_bound,
    pin_quantize_power_of_two,
    pin_quantize_layout,
    pin_f16_decoder_exhaustive,
    pin_bf16_decoder_exhaustive,
    pin_pack_golden,
    pin_pack_roundtrip,
    pin_pack_high_nibble,
    pin_closed_forms,
    pin_identity_rowsum,
    pin_all_ones,
    pin_one_hot,
    pin_zero_cases,
    pin_zero_high_nibble,
    pin_brute_force,
    pin_numpy_matmul,
    pin_power_of_two_scaling,
    pin_column_sampling_and_threads,
    pin_pack8_golden,
    pin_pack8_roundtrip,
    pin_closed_forms8,
    pin_identity_rowsum8,
    pin_all_ones8,
    pin_one_hot8,
    pin_zero_cases8,
    pin_brute_force8,
    pin_numpy_matmul8,
    pin_w8_sampling_scaling_threads,
    pin_a4_golden_words,
    pin_a4_grid_exact,
    pin_a4_ties_to_even,
    pin_a4_zero_group,
    pin_a4_error_bound_and_scale,
    pin_a4_scaling_and_sign,
    pin_a4_gemm_closed_forms,
    pin_a4_gemm_brute_force,
    pin_a4_gemm_numpy_matmul,
    pin_a4_gemm_one_hot_zero_identity,
    pin_a4_gemm_matches_w4a16_on_exact_activations,
]
