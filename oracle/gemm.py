"""ctypes wrapper for the GEMM oracle in ``gemm_ref.c``.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Operands are numpy arrays of the raw codes, viewed with any strides (numpy
views such as ``arr.transpose(...)`` or ``as_strided``): uint16 for fp16 bits,
uint8 for E4M3 / E8M0 bytes, float32 for fp32.  Their element strides are
handed to the C side unchanged, so transposed and batched views are
evaluated exactly as the data-layout page's shape:stride model says.

Parity: pinned in ``tests/test_oracle_gemm.py`` (codecs exhaustively against
numpy float16 and torch float8 conversions; GEMM against numpy fp64 matmul
on exact small-integer data, closed-form special cases, and the exactness of
power-of-two block scaling).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_ref.c")
LIB = os.path.join(HERE, "libgemm_oracle.so")

F16, F32, E4M3, E8M0, BF16, E2M1, E2M3, E3M2 = 1, 2, 3, 4, 5, 6, 7, 8


class _Tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 3),
        ("stride", ctypes.c_int64 * 3),
    ]


def build(force: bool = False) -> str:
    """Compile gemm_ref.c with gcc into libgemm_oracle.so (in-tree)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-D_GNU_SOURCE", SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER
        L.go_f16_decode.restype = ctypes.c_double
        L.go_f16_decode.argtypes = [ctypes.c_uint16]
        L.go_f16_encode.restype = ctypes.c_uint16
        L.go_f16_encode.argtypes = [ctypes.c_double]
        L.go_bf16_decode.restype = ctypes.c_double
        L.go_bf16_decode.argtypes = [ctypes.c_uint16]
        L.go_bf16_encode.restype = ctypes.c_uint16
        L.go_bf16_encode.argtypes = [ctypes.c_double]
        L.go_e2m1_decode.restype = ctypes.c_double
        L.go_e2m1_decode.argtypes = [ctypes.c_uint8]
        for name in ("go_e2m3_decode", "go_e3m2_decode"):
            getattr(L, name).restype = ctypes.c_double
            getattr(L, name).argtypes = [ctypes.c_uint8]
        L.go_fp6_code.restype = ctypes.c_uint8
        L.go_fp6_code.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.go_e4m3_decode.restype = ctypes.c_double
        L.go_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.go_e8m0_decode.restype = ctypes.c_double
        L.go_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.go_gemm.restype = ctypes.c_int
        L.go_gemm.argtypes = [P(_Tensor)] * 5 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                 ctypes.c_int32]
        L.go_gemm_points.restype = ctypes.c_int
        L.go_gemm_points.argtypes = [P(_Tensor)] * 5 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.c_int32, ctypes.c_int32]
        L.go_check.restype = ctypes.c_int64
        L.go_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                               P(ctypes.c_int64), P(ctypes.c_double), ctypes.c_int32]
        _lib = L
    return _lib


_DT = {np.dtype(np.uint16): F16, np.dtype(np.float16): F16, np.dtype(np.float32): F32}


def packed(storage: np.ndarray, shape: Sequence[int], strides: Sequence[int], dtype: int = None):
    """An operand given as raw storage plus a shape and ELEMENT strides, for
    formats numpy cannot view (E2M1, two elements per byte; E2M3 / E3M2, a
    6-bit little-endian bit stream)."""
    return ("packed", np.ascontiguousarray(storage), tuple(shape), tuple(strides), dtype)


def _is_packed(x) -> bool:
    return isinstance(x, tuple) and len(x) == 5 and x[0] == "packed"


def _tensor(arr, dtype: Optional[int] = None) -> _Tensor:
    t = _Tensor()
    if _is_packed(arr):
        _, storage, shape, strides, code = arr
        t.data = storage.ctypes.data
        t.dtype = code if code is not None else dtype
        t.rank = len(shape)
        for i in range(len(shape)):
            t.shape[i] = shape[i]
            t.stride[i] = strides[i]
        return t
    if arr is None:
        t.data = None
        t.dtype = 0
        t.rank = 2
        return t
    assert arr.ndim in (2, 3), arr.shape
    if dtype is None:
        dtype = _DT[arr.dtype]
    t.data = arr.ctypes.data
    t.dtype = dtype
    t.rank = arr.ndim
    for i in range(arr.ndim):
        t.shape[i] = arr.shape[i]
        assert arr.strides[i] % arr.itemsize == 0
        t.stride[i] = arr.strides[i] // arr.itemsize
    return t


def _args(a, b, c, sfa, sfb, mx: bool, bf16: bool = False):
    if mx:
        # block-scaled: E4M3 data with E8M0 scales unless the operands say
        # otherwise (packed E2M1 data, E4M3 scales for NVFP4)
        return (_tensor(a, E4M3), _tensor(b, E4M3), _tensor(c),
                _tensor(sfa, E8M0), _tensor(sfb, E8M0))
    if bf16:
        return (_tensor(a, BF16), _tensor(b, BF16), _tensor(c, BF16 if c is not None else None),
                _tensor(None), _tensor(None))
    return _tensor(a), _tensor(b), _tensor(c), _tensor(None), _tensor(None)


def _threads(nthreads: Optional[int]) -> int:
    if nthreads:
        return int(nthreads)
    return max(1, len(os.sched_getaffinity(0)))


def gemm(a: np.ndarray, b: np.ndarray, c: Optional[np.ndarray] = None,
         sfa: Optional[np.ndarray] = None, sfb: Optional[np.ndarray] = None,
         block_k: int = 32, nthreads: Optional[int] = None, bf16: bool = False
         ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Every element of D = A B^T + C.  ``a``: (batch?, M, K), ``b``:
    (batch?, N, K), ``c``: (batch?, M, N) or None.  With ``sfa``/``sfb`` the
    operands are E4M3 codes scaled per ``block_k`` K elements.  With
    ``bf16`` the uint16 codes of a, b and c are bf16 and D is rounded to
    bf16.  Returns (D codes as uint16 (batch, M, N), fp64 value before
    rounding, sum_k |A B| in fp64)."""
    mx = sfa is not None
    dims = lambda x: x[2] if _is_packed(x) else x.shape
    batch = max(dims(x)[0] if x is not None and len(dims(x)) == 3 else 1 for x in (a, b, c))
    M, N = dims(a)[-2], dims(b)[-2]
    d = np.empty((batch, M, N), np.uint16)
    ref = np.empty((batch, M, N), np.float64)
    absum = np.empty((batch, M, N), np.float64)
    ta, tb, tc, tsa, tsb = _args(a, b, c, sfa, sfb, mx, bf16)
    rc = lib().go_gemm(ctypes.byref(ta), ctypes.byref(tb), ctypes.byref(tc), ctypes.byref(tsa),
                       ctypes.byref(tsb), block_k, batch, d.ctypes.data, ref.ctypes.data,
                       absum.ctypes.data, _threads(nthreads), BF16 if bf16 else F16)
    if rc:
        raise ValueError(f"oracle gemm rejected the operands (code {rc})")
    return d, ref, absum


def gemm_points(a, b, c=None, sfa=None, sfb=None, points: np.ndarray = None,
                block_k: int = 32, nthreads: Optional[int] = None, bf16: bool = False):
    """As ``gemm`` but only at ``points`` (an int64 (count, 3) array of
    (batch, m, n)).  Returns (d codes, ref, absum), each of length count."""
    mx = sfa is not None
    pts = np.ascontiguousarray(points, dtype=np.int64)
    assert pts.ndim == 2 and pts.shape[1] == 3
    n = pts.shape[0]
    d = np.empty(n, np.uint16)
    ref = np.empty(n, np.float64)
    absum = np.empty(n, np.float64)
    ta, tb, tc, tsa, tsb = _args(a, b, c, sfa, sfb, mx, bf16)
    rc = lib().go_gemm_points(ctypes.byref(ta), ctypes.byref(tb), ctypes.byref(tc), ctypes.byref(tsa),
                              ctypes.byref(tsb), block_k, pts.ctypes.data, n, d.ctypes.data,
                              ref.ctypes.data, absum.ctypes.data, _threads(nthreads), BF16 if bf16 else F16)
    if rc:
        raise ValueError(f"oracle gemm rejected the operands (code {rc})")
    return d, ref, absum


def check(d: np.ndarray, d_ref: np.ndarray, absum: np.ndarray, bf16: bool = False) -> Tuple[int, int, float]:
    """The acceptance bound |D - D_ref| <= 2^-10 |D_ref| + 2^-13 S (2^-7 in
    place of 2^-10 for bf16 codes), per element.  Returns (violations,
    index of the worst element, its |D - D_ref| / bound)."""
    d = np.ascontiguousarray(d, dtype=np.uint16).ravel()
    d_ref = np.ascontiguousarray(d_ref, dtype=np.uint16).ravel()
    absum = np.ascontiguousarray(absum, dtype=np.float64).ravel()
    assert d.size == d_ref.size == absum.size
    wi = ctypes.c_int64(-1)
    wr = ctypes.c_double(0.0)
    bad = lib().go_check(d.ctypes.data, d_ref.ctypes.data, absum.ctypes.data, d.size,
                         ctypes.byref(wi), ctypes.byref(wr), BF16 if bf16 else F16)
    return int(bad), int(wi.value), float(wr.value)


def f16_decode(code: int) -> float:
    return lib().go_f16_decode(code)


def f16_encode(x: float) -> int:
    return lib().go_f16_encode(x)


def bf16_decode(code: int) -> float:
    return lib().go_bf16_decode(code)


def bf16_encode(x: float) -> int:
    return lib().go_bf16_encode(x)


def e2m1_decode(code: int) -> float:
    return lib().go_e2m1_decode(code)


def e2m3_decode(code: int) -> float:
    return lib().go_e2m3_decode(code)


def e3m2_decode(code: int) -> float:
    return lib().go_e3m2_decode(code)


def fp6_code(storage: np.ndarray, offset: int) -> int:
    """The 6-bit code at element offset ``offset`` of a packed byte array."""
    buf = np.ascontiguousarray(storage, dtype=np.uint8)
    return lib().go_fp6_code(buf.ctypes.data, offset)


def e4m3_decode(code: int) -> float:
    return lib().go_e4m3_decode(code)


def e8m0_decode(code: int) -> float:
    return lib().go_e8m0_decode(code)
