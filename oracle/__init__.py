"""The oracle: a plain fp64 CPU reference for the W4A16 GEMM and its 8-bit variant (W8A16),
their packing rules, and the round-to-nearest quantizer that produces the 4-bit format
(binary32, as the pages' format is produced; see the C source).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in __graft_entry__ and the
bench's CPU-baseline leg may import this package. It shares no code with the HIP
library and never imports it.

The C source (w4a16_oracle.c) states the operation and the pages it follows; this
module builds it with gcc and wraps it with ctypes over numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "w4a16_oracle.c")
BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "liboracle_w4a16.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(out_path: str = LIB_PATH, source: str = SOURCE, extra_cflags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_cflags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out_path)
    return out_path


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes wrapper around one build of the oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            build(lib_path)
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        lib.oracle_w4a16_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, ctypes.c_int]
        lib.oracle_w4a16_gemm.restype = ctypes.c_int
        lib.oracle_w4_pack.argtypes = [vp, vp, i64, i64]
        lib.oracle_w4_pack.restype = ctypes.c_int
        lib.oracle_w4_unpack.argtypes = [vp, vp, i64, i64]
        lib.oracle_w4_unpack.restype = ctypes.c_int
        lib.oracle_decode_bf16_array.argtypes = [vp, vp, i64]
        lib.oracle_decode_f16_array.argtypes = [vp, vp, i64]
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_w4_quantize.argtypes = [vp, vp, vp, vp, i64, i64]
        lib.oracle_w4_quantize.restype = ctypes.c_int
        lib.oracle_w8a16_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, ctypes.c_int]
        lib.oracle_w8a16_gemm.restype = ctypes.c_int
        lib.oracle_w8_pack.argtypes = [vp, vp, i64, i64]
        lib.oracle_w8_pack.restype = ctypes.c_int
        lib.oracle_w8_unpack.argtypes = [vp, vp, i64, i64]
        lib.oracle_w8_unpack.restype = ctypes.c_int
        lib.oracle_a4_quantize.argtypes = [vp, vp, vp, i64, i64]
        lib.oracle_a4_quantize.restype = ctypes.c_int
        lib.oracle_w4a4_gemm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, ctypes.c_int]
        lib.oracle_w4a4_gemm.restype = ctypes.c_int
        self._lib = lib

    # -- decoders -----------------------------------------------------------------
    def bf16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.oracle_decode_bf16_array(_ptr(b), _ptr(out), b.size)
        return out

    def f16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.oracle_decode_f16_array(_ptr(b), _ptr(out), b.size)
        return out

    def f32_to_f16(self, x: float) -> int:
        """binary16 bits of a binary32 value, ties to even."""
        return int(self._lib.oracle_f32_to_f16(ctypes.c_float(x)))

    # -- quantizer ----------------------------------------------------------------
    def quantize(self, W_f16: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Round-to-nearest min/max quantizer (groups of 128 along K), see the C source.

        W_f16: uint16 binary16 bits [K, N].  Returns (Wq uint32 [K/8, N], S uint16 binary16
        bits [K/128, N], Z uint8 [K/128, N]).
        """
        W = np.ascontiguousarray(W_f16, dtype=np.uint16)
        K, N = W.shape
        Wq = np.empty((K // 8, N), dtype=np.uint32)
        S = np.empty((K // 128, N), dtype=np.uint16)
        Z = np.empty((K // 128, N), dtype=np.uint8)
        rc = self._lib.oracle_w4_quantize(_ptr(W), _ptr(Wq), _ptr(S), _ptr(Z), K, N)
        if rc:
            raise ValueError(f"oracle quantize rejected shape {W.shape}")
        return Wq, S, Z

    # -- packing ------------------------------------------------------------------
    def pack(self, q: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        K, N = q.shape
        out = np.empty((K // 8, N), dtype=np.uint32)
        rc = self._lib.oracle_w4_pack(_ptr(q), _ptr(out), K, N)
        if rc:
            raise ValueError(f"oracle pack rejected shape {q.shape}")
        return out

    def unpack(self, Wq: np.ndarray) -> np.ndarray:
        Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
        KB, N = Wq.shape
        out = np.empty((KB * 8, N), dtype=np.uint8)
        rc = self._lib.oracle_w4_unpack(_ptr(Wq), _ptr(out), KB * 8, N)
        if rc:
            raise ValueError(f"oracle unpack rejected shape {Wq.shape}")
        return out

    def pack8(self, q: np.ndarray) -> np.ndarray:
        """8-bit codes uint8 [K, N] -> uint32 [K/4, N] (byte j of a word holds k = 4 kb + j)."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        K, N = q.shape
        out = np.empty((K // 4, N), dtype=np.uint32)
        rc = self._lib.oracle_w8_pack(_ptr(q), _ptr(out), K, N)
        if rc:
            raise ValueError(f"oracle pack8 rejected shape {q.shape}")
        return out

    def unpack8(self, Wq8: np.ndarray) -> np.ndarray:
        Wq8 = np.ascontiguousarray(Wq8, dtype=np.uint32)
        KB, N = Wq8.shape
        out = np.empty((KB * 4, N), dtype=np.uint8)
        rc = self._lib.oracle_w8_unpack(_ptr(Wq8), _ptr(out), KB * 4, N)
        if rc:
            raise ValueError(f"oracle unpack8 rejected shape {Wq8.shape}")
        return out

    # -- 4-bit activations (W4A4) --------------------------------------------------
    def quantize_activations(self, A: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Symmetric 4-bit activations per row and group of 128 (see the C source).

        A: uint16 bfloat16 bits [M, K].  Returns (Aq uint32 [M, K/8] offset-binary nibbles,
        As float32 [M, K/128] scales).
        """
        A = np.ascontiguousarray(A, dtype=np.uint16)
        M, K = A.shape
        Aq = np.empty((M, K // 8), dtype=np.uint32)
        As = np.empty((M, K // 128), dtype=np.float32)
        rc = self._lib.oracle_a4_quantize(_ptr(A), _ptr(Aq), _ptr(As), M, K)
        if rc:
            raise ValueError(f"oracle a4 quantize rejected shape {A.shape}")
        return Aq, As

    def gemm_a4(self, Aq: np.ndarray, As: np.ndarray, Wq: np.ndarray, S: np.ndarray, Z: np.ndarray,
                cols: Optional[np.ndarray] = None, threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """W4A4: (C, Cabs) float64 [M, ncols] from 4-bit activations (Aq, As) and the 4-bit
        weight format (Wq [K/8, N], S, Z)."""
        Aq = np.ascontiguousarray(Aq, dtype=np.uint32)
        As = np.ascontiguousarray(As, dtype=np.float32)
        Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        Z = np.ascontiguousarray(Z, dtype=np.uint8)
        M, KB = Aq.shape
        K = KB * 8
        N = Wq.shape[1]
        if Wq.shape[0] * 8 != K or As.shape != (M, K // 128) or S.shape != (K // 128, N) or Z.shape != (K // 128, N):
            raise ValueError("inconsistent shapes")
        if cols is not None:
            cols = np.ascontiguousarray(cols, dtype=np.int64)
            nc = cols.size
        else:
            nc = N
        C = np.empty((M, nc), dtype=np.float64)
        Cabs = np.empty((M, nc), dtype=np.float64)
        rc = self._lib.oracle_w4a4_gemm(_ptr(Aq), _ptr(As), _ptr(Wq), _ptr(S), _ptr(Z), M, K, N, _ptr(cols), nc,
                                        _ptr(C), _ptr(Cabs), int(threads))
        if rc:
            raise ValueError(f"oracle rejected the shape M={M} K={K} N={N} (rc={rc})")
        return C, Cabs

    # -- the GEMM -----------------------------------------------------------------
    def gemm(self, A: np.ndarray, Wq: np.ndarray, S: np.ndarray, Z: np.ndarray,
             cols: Optional[np.ndarray] = None, threads: int = 0, bits: int = 4) -> Tuple[np.ndarray, np.ndarray]:
        """Return (C, Cabs), both float64 [M, ncols]: C = A.W and Cabs = sum_k |A.W| terms.

        A: uint16 bf16 bits [M,K]; Wq: uint32 [K*bits/32,N] (bits = 4: 8 codes per word,
        zeros' low nibble; bits = 8: 4 codes per word, full-byte zeros); S: uint16 fp16 bits
        [K/128,N]; Z: uint8 [K/128,N]; cols: optional int64 column indices.
        """
        if bits not in (4, 8):
            raise ValueError("bits must be 4 or 8")
        per_word = 32 // bits
        A = np.ascontiguousarray(A, dtype=np.uint16)
        Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        Z = np.ascontiguousarray(Z, dtype=np.uint8)
        M, K = A.shape
        KB, N = Wq.shape
        if KB * per_word != K or S.shape != (K // 128, N) or Z.shape != (K // 128, N):
            raise ValueError("inconsistent shapes")
        if cols is not None:
            cols = np.ascontiguousarray(cols, dtype=np.int64)
            nc = cols.size
        else:
            nc = N
        C = np.empty((M, nc), dtype=np.float64)
        Cabs = np.empty((M, nc), dtype=np.float64)
        fn = self._lib.oracle_w4a16_gemm if bits == 4 else self._lib.oracle_w8a16_gemm
        rc = fn(_ptr(A), _ptr(Wq), _ptr(S), _ptr(Z), M, K, N, _ptr(cols), nc, _ptr(C), _ptr(Cabs), int(threads))
        if rc:
            raise ValueError(f"oracle rejected the shape M={M} K={K} N={N} (rc={rc})")
        return C, Cabs


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The shared oracle instance (built on first use if the library is missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def within_tolerance(C_test: np.ndarray, C_ref: np.ndarray, Cabs: np.ndarray,
                     rel: float = 1e-4, abs_: float = 1e-6) -> np.ndarray:
    """Element-wise acceptance: |C_test - C_ref| <= rel * sum_k|A W| + abs_ (in float64)."""
    err = np.abs(np.asarray(C_test, dtype=np.float64) - C_ref)
    return err <= rel * Cabs + abs_
