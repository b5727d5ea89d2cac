"""Python binding of libw4a16.so: the group-wise INT4 weight-only GEMM for MI355X (gfx950).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream; every step of the computation runs in the library's HIP kernels. Importing this
package fails loudly when the library has not been built (there is no fallback).

    import int4_weight_only_gemm_amd as w4
    Wq = w4.pack(q_u8)                    # [K, N] uint8 codes -> [K/8, N] int32 words
    C = w4.gemm(A_bf16, Wq, s_f16, z_u8)  # [M, N] float32
    Wq8 = w4.pack(q_u8, bits=8)           # 8-bit codes -> [K/4, N] int32 words
    C = w4.gemm(A_bf16, Wq8, s_f16, z_u8, bits=8)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, List

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "w4a16.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m int4_weight_only_gemm_amd.build` "
        "(hipcc --offload-arch=gfx950); there is no CPU fallback")

# One HIP runtime per process: torch bundles its own libamdhip64.so.7 (and HSA runtime).
# Importing torch first makes the library's libamdhip64.so.7 dependency resolve to that
# already-loaded copy; loading the library first would bring in /opt/rocm's copy and torch
# would then start a second, conflicting runtime.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

STATUS = {
    0: "W4_OK",
    1: "W4_ERR_NULL",
    2: "W4_ERR_SHAPE",
    3: "W4_ERR_ALIGN",
    4: "W4_ERR_DEVICE",
    5: "W4_ERR_HIP",
    6: "W4_ERR_WORKSPACE",
    7: "W4_ERR_PLAN",
}


class W4Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = _lib.w4_last_error().decode(errors="replace")
        name = STATUS.get(code, str(code))
        super().__init__(f"{where}: {name}: {detail}")


class Plan(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int),
        ("tile_m", ctypes.c_int),
        ("tile_n", ctypes.c_int),
        ("m_blocks", ctypes.c_int),
        ("n_tiles", ctypes.c_int),
        ("splits", ctypes.c_int),
        ("groups_per_split", ctypes.c_int),
        ("full_tiles", ctypes.c_int),
        ("workgroups", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("group_stride", ctypes.c_int64),
    ]

    def as_dict(self) -> Dict[str, int]:
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib.w4a16_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.w4a16_gemm.restype = ctypes.c_int
_lib.w4a16_gemm_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.w4a16_gemm_noalloc.restype = ctypes.c_int
_lib.w4_pack.argtypes = [_vp, _vp, _i64, _i64, _vp]
_lib.w4_pack.restype = ctypes.c_int
_lib.w4_quantize.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _vp]
_lib.w4_quantize.restype = ctypes.c_int
_lib.w4_read_probe.argtypes = [_vp, _i64, _vp, _i64, _vp]
_lib.w4_read_probe.restype = ctypes.c_int
_lib.w4a16_plan.argtypes = [_i64, _i64, _i64, ctypes.POINTER(Plan)]
_lib.w4a16_plan.restype = ctypes.c_int
_lib.w8a16_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.w8a16_gemm.restype = ctypes.c_int
_lib.w8_pack.argtypes = [_vp, _vp, _i64, _i64, _vp]
_lib.w8_pack.restype = ctypes.c_int
_lib.w8a16_plan.argtypes = [_i64, _i64, _i64, ctypes.POINTER(Plan)]
_lib.w8a16_plan.restype = ctypes.c_int
_lib.w4a4_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.w4a4_gemm.restype = ctypes.c_int
_lib.w4a4_plan.argtypes = [_i64, _i64, _i64, ctypes.POINTER(Plan)]
_lib.w4a4_plan.restype = ctypes.c_int
_lib.a4_quantize.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp]
_lib.a4_quantize.restype = ctypes.c_int
_lib.w4_status_string.argtypes = [ctypes.c_int]
_lib.w4_status_string.restype = ctypes.c_char_p
_lib.w4_last_error.argtypes = []
_lib.w4_last_error.restype = ctypes.c_char_p


def lib() -> ctypes.CDLL:
    return _lib


def header_functions(path: str = HEADER) -> List[str]:
    """Names of the functions declared in include/w4a16.h."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\**\s*\b((?:w[48]|a4)\w*)\s*\(", text, flags=re.M)


def status_string(code: int) -> str:
    return _lib.w4_status_string(code).decode()


def _bits_fns(bits: int):
    if bits == 4:
        return _lib.w4a16_gemm, "w4a16_gemm", _lib.w4_pack, "w4_pack", _lib.w4a16_plan, "w4a16_plan"
    if bits == 8:
        return _lib.w8a16_gemm, "w8a16_gemm", _lib.w8_pack, "w8_pack", _lib.w8a16_plan, "w8a16_plan"
    raise ValueError("bits must be 4 or 8")


def plan(M: int, K: int, N: int, bits: int = 4, a4: bool = False) -> Dict[str, int]:
    """How the GEMM entry point for `bits`-wide codes (or, with a4, w4a4_gemm) would run a
    shape (host only)."""
    fn, name = (_lib.w4a4_plan, "w4a4_plan") if a4 else _bits_fns(bits)[4:]
    p = Plan()
    rc = fn(M, K, N, ctypes.byref(p))
    if rc:
        raise W4Error(rc, name)
    return p.as_dict()


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(t, name, dtype, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def gemm(A, Wq, scales, zeros, out=None, stream=None, bits: int = 4):
    """C[M,N] = A[M,K] . W[K,N] with W[k,n] = (q[k,n] - z[k/128,n]) * s[k/128,n].

    A: bfloat16 [M,K]; Wq: int32 (or uint32) [K*bits/32,N] packed codes; scales: float16
    [K/128,N]; zeros: uint8 [K/128,N]; out: optional float32 [M,N] (overwritten).
    bits = 4 calls w4a16_gemm (zeros' low nibble), bits = 8 calls w8a16_gemm (full bytes).
    """
    fn, name = _bits_fns(bits)[:2]
    import torch
    _check(A, "A", torch.bfloat16, 2)
    if Wq.dtype not in (torch.int32, torch.uint32):
        raise TypeError("Wq must be int32 or uint32")
    _check(Wq, "Wq", Wq.dtype, 2)
    _check(scales, "scales", torch.float16, 2)
    _check(zeros, "zeros", torch.uint8, 2)
    M, K = A.shape
    N = Wq.shape[1]
    if Wq.shape[0] * (32 // bits) != K or scales.shape != (K // 128, N) or zeros.shape != (K // 128, N):
        raise ValueError(f"inconsistent shapes A{tuple(A.shape)} Wq{tuple(Wq.shape)} "
                         f"scales{tuple(scales.shape)} zeros{tuple(zeros.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        _check(out, "out", torch.float32, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    rc = fn(A.data_ptr(), Wq.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
            out.data_ptr(), M, K, N, _stream_handle(stream))
    if rc:
        raise W4Error(rc, name)
    return out


def gemm_noalloc_raw(A_ptr: int, Wq_ptr: int, S_ptr: int, Z_ptr: int, C_ptr: int, M: int, K: int, N: int,
                     stream_handle: int = 0) -> None:
    """w4a16_gemm_noalloc on raw device pointers: the 4-bit GEMM with the library's fixed
    per-GPU scratch instead of an allocated workspace (no device allocation at all)."""
    rc = _lib.w4a16_gemm_noalloc(A_ptr, Wq_ptr, S_ptr, Z_ptr, C_ptr, M, K, N, stream_handle)
    if rc:
        raise W4Error(rc, "w4a16_gemm_noalloc")


def quantize_activations(A, stream=None):
    """4-bit activations: bfloat16 A [M, K] -> (Aq int32 [M, K/8] offset-binary codes,
    A_scales float32 [M, K/128]), symmetric per row and group of 128 (a4_quantize)."""
    import torch
    _check(A, "A", torch.bfloat16, 2)
    M, K = A.shape
    Aq = torch.empty((M, K // 8), dtype=torch.int32, device=A.device)
    As = torch.empty((M, K // 128), dtype=torch.float32, device=A.device)
    rc = _lib.a4_quantize(A.data_ptr(), Aq.data_ptr(), As.data_ptr(), M, K, _stream_handle(stream))
    if rc:
        raise W4Error(rc, "a4_quantize")
    return Aq, As


def gemm_a4(Aq, A_scales, Wq, scales, zeros, out=None, stream=None):
    """W4A4: C[M,N] from 4-bit activations (Aq int32 [M, K/8], A_scales float32 [M, K/128])
    and the 4-bit weight format (Wq int32 [K/8, N], scales float16, zeros uint8)."""
    import torch
    for t, name in ((Aq, "Aq"), (Wq, "Wq")):
        if t.dtype not in (torch.int32, torch.uint32):
            raise TypeError(f"{name} must be int32 or uint32")
        _check(t, name, t.dtype, 2)
    _check(A_scales, "A_scales", torch.float32, 2)
    _check(scales, "scales", torch.float16, 2)
    _check(zeros, "zeros", torch.uint8, 2)
    M, K = Aq.shape[0], Aq.shape[1] * 8
    N = Wq.shape[1]
    if (Wq.shape[0] * 8 != K or A_scales.shape != (M, K // 128) or scales.shape != (K // 128, N)
            or zeros.shape != (K // 128, N)):
        raise ValueError(f"inconsistent shapes Aq{tuple(Aq.shape)} A_scales{tuple(A_scales.shape)} "
                         f"Wq{tuple(Wq.shape)} scales{tuple(scales.shape)} zeros{tuple(zeros.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=Aq.device)
    else:
        _check(out, "out", torch.float32, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    rc = _lib.w4a4_gemm(Aq.data_ptr(), A_scales.data_ptr(), Wq.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                        out.data_ptr(), M, K, N, _stream_handle(stream))
    if rc:
        raise W4Error(rc, "w4a4_gemm")
    return out


def gemm_raw(A_ptr: int, Wq_ptr: int, S_ptr: int, Z_ptr: int, C_ptr: int, M: int, K: int, N: int,
             stream_handle: int = 0, bits: int = 4) -> None:
    """Direct C-ABI call on raw device pointers (no checks beyond the library's own)."""
    fn, name = _bits_fns(bits)[:2]
    rc = fn(A_ptr, Wq_ptr, S_ptr, Z_ptr, C_ptr, M, K, N, stream_handle)
    if rc:
        raise W4Error(rc, name)


def pack(q, out=None, stream=None, bits: int = 4):
    """Pack uint8 codes [K,N] into int32 words [K*bits/32,N]: 8 codes per word for bits = 4
    (high nibbles ignored), 4 codes per word for bits = 8."""
    import torch
    fn, name = _bits_fns(bits)[2:4]
    _check(q, "q", torch.uint8, 2)
    K, N = q.shape
    KB = K * bits // 32
    if out is None:
        out = torch.empty((KB, N), dtype=torch.int32, device=q.device)
    elif out.dtype not in (torch.int32, torch.uint32) or tuple(out.shape) != (KB, N):
        raise ValueError(f"out must be int32 [{KB}, N]")
    rc = fn(q.data_ptr(), out.data_ptr(), K, N, _stream_handle(stream))
    if rc:
        raise W4Error(rc, name)
    return out


def quantize(W, stream=None):
    """Round-to-nearest group-128 quantizer: float16 W [K, N] -> (Wq int32 [K/8, N],
    scales float16 [K/128, N], zeros uint8 [K/128, N]) in the storage format."""
    import torch
    _check(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty((K // 8, N), dtype=torch.int32, device=W.device)
    S = torch.empty((K // 128, N), dtype=torch.float16, device=W.device)
    Z = torch.empty((K // 128, N), dtype=torch.uint8, device=W.device)
    rc = _lib.w4_quantize(W.data_ptr(), Wq.data_ptr(), S.data_ptr(), Z.data_ptr(), K, N, _stream_handle(stream))
    if rc:
        raise W4Error(rc, "w4_quantize")
    return Wq, S, Z


def quantize_raw(W_ptr: int, Wq_ptr: int, S_ptr: int, Z_ptr: int, K: int, N: int, stream_handle: int = 0) -> None:
    """Direct C-ABI call of the quantizer on raw device pointers."""
    rc = _lib.w4_quantize(W_ptr, Wq_ptr, S_ptr, Z_ptr, K, N, stream_handle)
    if rc:
        raise W4Error(rc, "w4_quantize")


def read_probe(buf, blocks: int = 768, out=None, stream=None):
    """Streaming-read probe over a contiguous device tensor (size a multiple of 16 bytes).

    Returns the int32 [blocks, 4] per-wave XORs of the 32-bit words read (4 waves per
    block); XOR-reducing all of them gives the XOR of every word of the buffer.
    """
    import torch
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty((blocks, 4), dtype=torch.int32, device=buf.device)
    else:
        _check(out, "out", torch.int32, 2)
        if tuple(out.shape) != (blocks, 4):
            raise ValueError("out must be int32 [blocks, 4]")
    rc = _lib.w4_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, _stream_handle(stream))
    if rc:
        raise W4Error(rc, "w4_read_probe")
    return out


def read_probe_raw(src_ptr: int, nbytes: int, out_ptr: int, blocks: int, stream_handle: int = 0) -> None:
    """Direct C-ABI call of the streaming-read probe on raw device pointers."""
    rc = _lib.w4_read_probe(src_ptr, nbytes, out_ptr, blocks, stream_handle)
    if rc:
        raise W4Error(rc, "w4_read_probe")
