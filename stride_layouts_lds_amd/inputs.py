"""Seeded synthetic workloads for the strided-layout GEMM.

This module holds only random draws, their rounding to the storage formats
(numpy's float16 cast and torch's float8_e4m3fn cast, both round-to-nearest-
even) and the strides that lay them out.  It holds none of the GEMM's
arithmetic: no decoding, no products, no sums.  Both the HIP path and the CPU
oracle are fed from here, so they see identical bytes.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in fp64 in the
order A, B, C, SFA, SFB.  Each operand is drawn in its storage order (so a
transposed view is a real transposed layout of the same draws), then rounded.
Scale exponents are integers uniform in [-4, 4] stored as E8M0 bytes e + 127.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Sequence, Dict, Optional, Tuple

import numpy as np


PACKED = ("e2m1", "e2m3", "e3m2")  # sub-byte kinds, packed along the unit-stride axis


@dataclass
class HostOperand:
    """A host operand: raw codes (uint16 fp16 bits, uint8 E4M3/E8M0 bytes)
    in a flat storage array, and the (batch?, rows, cols) view with element
    strides."""
    storage: np.ndarray
    shape: Tuple[int, ...]
    strides: Tuple[int, ...]
    kind: str  # 'f16' | 'bf16' | 'e4m3' | 'e8m0' | 'e2m1' | 'e2m3' | 'e3m2' (packed, strides in elements)

    @property
    def view(self) -> np.ndarray:
        if self.kind in PACKED:
            raise TypeError("packed sub-byte codes have no numpy view")
        it = self.storage.itemsize
        return np.lib.stride_tricks.as_strided(
            self.storage, shape=self.shape, strides=tuple(s * it for s in self.strides),
            writeable=False)


@dataclass
class Workload:
    name: str
    M: int
    N: int
    K: int
    batch: int
    a: HostOperand
    b: HostOperand
    c: Optional[HostOperand] = None
    sfa: Optional[HostOperand] = None
    sfb: Optional[HostOperand] = None
    block_k: int = 32
    d_shape: Tuple[int, ...] = ()
    d_strides: Tuple[int, ...] = ()
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def mx(self) -> bool:
        return self.sfa is not None

    @property
    def bf16(self) -> bool:
        return self.a.kind == "bf16"

    @property
    def fp4(self) -> bool:
        return self.a.kind == "e2m1"

    @property
    def nvfp4(self) -> bool:
        return self.fp4 and self.sfa is not None and self.sfa.kind == "e4m3"

    @property
    def mxfp4(self) -> bool:
        return self.fp4 and self.sfa is not None and self.sfa.kind == "e8m0"

    @property
    def fp6(self) -> bool:
        return self.a.kind in ("e2m3", "e3m2")

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K


def _draw(rng: np.random.Generator, dist: str, n: int) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, n)
    if dist == "normal":
        return rng.standard_normal(n)
    if dist.startswith("int"):  # "int4": integers uniform in [-4, 4]
        r = int(dist[3:])
        return rng.integers(-r, r + 1, n).astype(np.float64)
    raise ValueError(dist)


def _f16_codes(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float16).view(np.uint16)


def _bf16_codes(x: np.ndarray) -> np.ndarray:
    import torch  # fp32 first, then torch's nearest-even bfloat16 conversion
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    import torch  # the cast rounds to nearest even; clamp first so it saturates
    t = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def matrix(rng, dist: str, batch: Optional[int], rows: int, cols: int, major: str,
           kind: str = "f16") -> HostOperand:
    """Draw a (batch?, rows, cols) operand.  ``major='row'``: cols contiguous
    (strides (rows*cols, cols, 1)); ``major='col'``: rows contiguous (strides
    (rows*cols, 1, rows)), i.e. the stride-swapped view of a stored
    (cols, rows) matrix."""
    nb = batch or 1
    x = _draw(rng, dist, nb * rows * cols)
    codes = _e4m3_codes(x) if kind == "e4m3" else _bf16_codes(x) if kind == "bf16" else _f16_codes(x)
    if major == "row":
        st = (rows * cols, cols, 1)
    elif major == "col":
        st = (rows * cols, 1, rows)
    else:
        raise ValueError(major)
    if batch is None:
        return HostOperand(codes, (rows, cols), st[1:], kind)
    return HostOperand(codes, (batch, rows, cols), st, kind)


def scales(rng, batch: Optional[int], rows: int, kblocks: int, lo: int = -4, hi: int = 4,
           pad: int = 0) -> HostOperand:
    """E8M0 scale codes 127 + e, e uniform in [lo, hi]; rows are kblocks + pad
    bytes apart (the pad bytes hold NaN codes, 0xFF, and are never read)."""
    rs = kblocks + pad
    e = rng.integers(lo, hi + 1, (batch or 1) * rows * rs)
    codes = (e + 127).astype(np.uint8)
    if pad:
        codes.reshape(-1, rs)[:, kblocks:] = 0xFF
    if batch is None:
        return HostOperand(codes, (rows, kblocks), (rs, 1), "e8m0")
    return HostOperand(codes, (batch, rows, kblocks), (rows * rs, rs, 1), "e8m0")


def e2m1_matrix(rng, batch: Optional[int], rows: int, cols: int) -> HostOperand:
    """(batch?, rows, cols) E2M1 codes, uniform over all 16, packed two per
    byte along cols (element 2i in the low nibble), rows cols apart."""
    nb = batch or 1
    codes = rng.integers(0, 16, (nb * rows, cols)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8).ravel()
    if batch is None:
        return HostOperand(packed, (rows, cols), (cols, 1), "e2m1")
    return HostOperand(packed, (batch, rows, cols), (rows * cols, cols, 1), "e2m1")


def e4m3_scales(rng, batch: Optional[int], rows: int, kblocks: int, lo: int = -4, hi: int = 4,
                mantissas: Sequence[int] = tuple(range(8))) -> HostOperand:
    """Positive E4M3 scale codes 2^e * (1 + m/8), e uniform in [lo, hi], m
    drawn from ``mantissas``."""
    n = (batch or 1) * rows * kblocks
    e = rng.integers(lo, hi + 1, n)
    m = rng.choice(np.array(mantissas), n)
    codes = (((e + 7) << 3) | m).astype(np.uint8)
    if batch is None:
        return HostOperand(codes, (rows, kblocks), (kblocks, 1), "e4m3")
    return HostOperand(codes, (batch, rows, kblocks), (rows * kblocks, kblocks, 1), "e4m3")


def nvfp4_workload(name: str, M: int, N: int, K: int, *, seed: int, batch: Optional[int] = None,
                   with_c: bool = False, exact: bool = False) -> Workload:
    """NVFP4: packed E2M1 A and B (codes uniform), one positive E4M3 scale
    per 16 K (exponents in [-4, 0], any mantissa, which keeps an 8192-term
    fp16 result finite; with ``exact``, exponents in [-2, 2] and mantissas 0
    or 4, so every partial sum is exact in fp32), C fp16 normal(0,1) if
    asked."""
    rng = np.random.default_rng(seed)
    a = e2m1_matrix(rng, batch, M, K)
    b = e2m1_matrix(rng, batch, N, K)
    kb = -(-K // 16)
    lo, hi, mans = (-2, 2, (0, 4)) if exact else (-4, 0, tuple(range(8)))
    sfa = e4m3_scales(rng, batch, M, kb, lo, hi, mans)
    sfb = e4m3_scales(rng, batch, N, kb, lo, hi, mans)
    c = matrix(rng, "int4" if exact else "normal", batch, M, N, "row") if with_c else None
    if batch is None:
        d_shape, d_strides = (M, N), (N, 1)
    else:
        d_shape, d_strides = (batch, M, N), (M * N, N, 1)
    return Workload(name, M, N, K, batch or 1, a, b, c, sfa, sfb, 16, d_shape, d_strides)


def mxfp4_workload(name: str, M: int, N: int, K: int, *, seed: int, batch: Optional[int] = None,
                   with_c: bool = False, exact: bool = False) -> Workload:
    """MXFP4: packed E2M1 A and B (codes uniform), one E8M0 scale per 32 K
    with exponents uniform in [-4, 0] (with ``exact``, [-1, 1], so every
    partial sum of a K <= 2048 problem is exact in fp32), C fp16 if asked."""
    rng = np.random.default_rng(seed)
    a = e2m1_matrix(rng, batch, M, K)
    b = e2m1_matrix(rng, batch, N, K)
    kb = -(-K // 32)
    lo, hi = (-1, 1) if exact else (-4, 0)
    sfa = scales(rng, batch, M, kb, lo, hi)
    sfb = scales(rng, batch, N, kb, lo, hi)
    c = matrix(rng, "int4" if exact else "normal", batch, M, N, "row") if with_c else None
    if batch is None:
        d_shape, d_strides = (M, N), (N, 1)
    else:
        d_shape, d_strides = (batch, M, N), (M * N, N, 1)
    return Workload(name, M, N, K, batch or 1, a, b, c, sfa, sfb, 32, d_shape, d_strides)


def fp6_matrix(rng, batch: Optional[int], rows: int, cols: int, kind: str, exact: bool = False) -> HostOperand:
    """(batch?, rows, cols) 6-bit codes packed along cols as one little-endian
    bit stream per row (code j at bits 6j .. 6j+5; 64-element rows are 48
    bytes), rows cols apart.  Codes are uniform over all 64, or with
    ``exact`` built from the fields sign | exponent | significand with
    significand 0 or half its range and the three exponents just above
    zero's (E2M3: 1 .. 3, E3M2: 3 .. 5) plus zero, the values
    {0, +-1, +-1.5, +-2, +-3, +-4, +-6}."""
    assert cols % 4 == 0
    nb = batch or 1
    if exact:
        if kind == "e2m3":
            fields = [(e << 3) | m for e in (1, 2, 3) for m in (0, 4)] + [0]
        else:
            fields = [(e << 2) | m for e in (3, 4, 5) for m in (0, 2)] + [0]
        mag = rng.choice(np.array(fields, np.uint8), (nb * rows, cols))
        codes = (mag | (rng.integers(0, 2, mag.shape).astype(np.uint8) << 5)).astype(np.uint8)
    else:
        codes = rng.integers(0, 64, (nb * rows, cols)).astype(np.uint8)
    bits = ((codes[:, :, None] >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8).reshape(nb * rows, 6 * cols)
    packed = np.packbits(bits, axis=1, bitorder="little").ravel()
    if batch is None:
        return HostOperand(packed, (rows, cols), (cols, 1), kind)
    return HostOperand(packed, (batch, rows, cols), (rows * cols, cols, 1), kind)


def mxfp6_workload(name: str, M: int, N: int, K: int, *, seed: int, kind: str = "e2m3",
                   batch: Optional[int] = None, with_c: bool = False, exact: bool = False) -> Workload:
    """MXFP6: packed 6-bit A and B of one format (codes uniform; ``exact``:
    see fp6_matrix), one E8M0 scale per 32 K with exponents uniform in
    [-4, 0] ([-1, 1] with ``exact``, every partial sum of a K <= 2048
    problem then exact in fp32), C fp16 if asked."""
    rng = np.random.default_rng(seed)
    a = fp6_matrix(rng, batch, M, K, kind, exact)
    b = fp6_matrix(rng, batch, N, K, kind, exact)
    kb = -(-K // 32)
    lo, hi = (-1, 1) if exact else (-4, 0)
    sfa = scales(rng, batch, M, kb, lo, hi)
    sfb = scales(rng, batch, N, kb, lo, hi)
    c = matrix(rng, "int4" if exact else "normal", batch, M, N, "row") if with_c else None
    if batch is None:
        d_shape, d_strides = (M, N), (N, 1)
    else:
        d_shape, d_strides = (batch, M, N), (M * N, N, 1)
    return Workload(name, M, N, K, batch or 1, a, b, c, sfa, sfb, 32, d_shape, d_strides)


def gemm_workload(name: str, M: int, N: int, K: int, *, seed: int, dist: str = "normal",
                  batch: Optional[int] = None, a_major: str = "row", b_major: str = "row",
                  with_c: bool = False, c_dist: Optional[str] = None, mx: bool = False,
                  block_k: int = 32, rng: Optional[np.random.Generator] = None,
                  scale_range: Tuple[int, int] = (-4, 4), scale_pad: int = 0, bf16: bool = False) -> Workload:
    """A generic seeded GEMM problem.  ``a_major``/``b_major`` say which of
    the two matrix dimensions is contiguous: 'row' = K-contiguous (TN
    convention), 'col' = M- (or N-) contiguous."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    kind = "e4m3" if mx else "bf16" if bf16 else "f16"
    a = matrix(rng, dist, batch, M, K, a_major, kind)
    b = matrix(rng, dist, batch, N, K, b_major, kind)
    c = matrix(rng, c_dist or dist, batch, M, N, "row", "bf16" if bf16 else "f16") if with_c else None
    sfa = sfb = None
    if mx:
        kb = -(-K // block_k)
        sfa = scales(rng, batch, M, kb, *scale_range, pad=scale_pad)
        sfb = scales(rng, batch, N, kb, *scale_range, pad=scale_pad)
    if batch is None:
        d_shape, d_strides = (M, N), (N, 1)
    else:
        d_shape, d_strides = (batch, M, N), (M * N, N, 1)
    return Workload(name, M, N, K, batch or 1, a, b, c, sfa, sfb, block_k, d_shape, d_strides)


def to_device(op: Optional[HostOperand]):
    """The same storage bytes on the current GPU, viewed with the same
    strides (a torch tensor); None stays None."""
    import torch
    if op is None:
        return None
    if op.kind == "e2m1":
        # packed pairs: torch's float4_e2m1fn_x2 holds two elements per item
        st = torch.from_numpy(np.ascontiguousarray(op.storage)).to("cuda").view(torch.float4_e2m1fn_x2)
        return st.as_strided(op.shape[:-1] + (op.shape[-1] // 2,), tuple(x // 2 for x in op.strides[:-1]) + (1,))
    if op.kind in ("e2m3", "e3m2"):
        # no torch dtype: the bytes on the device, described by a PackedTensor
        from .api import PackedTensor, SL_F6_E2M3, SL_F6_E3M2
        st = torch.from_numpy(np.ascontiguousarray(op.storage)).to("cuda")
        return PackedTensor(st, SL_F6_E2M3 if op.kind == "e2m3" else SL_F6_E3M2, op.shape, op.strides)
    st = torch.from_numpy(np.ascontiguousarray(op.storage))
    st = st.view({"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
                  "e8m0": torch.float8_e8m0fnu}[op.kind])
    return st.to("cuda").as_strided(op.shape, op.strides)


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def config1() -> Workload:
    """fp16 TN 256^3, uniform[-1,1], C = 0, seed 0."""
    return gemm_workload("fp16_tn_256", 256, 256, 256, seed=0, dist="uniform")


def config2(n: int = 4096, with_c: bool = True) -> Workload:
    """fp16 TN n^3 with C, all normal(0,1), seed 1 (n = 4096; 8192 for the
    large square case)."""
    return gemm_workload(f"fp16_tn_{n}" + ("_c" if with_c else ""), n, n, n, seed=1,
                         dist="normal", with_c=with_c)


def config3() -> Tuple[Workload, Workload]:
    """Ragged and skinny fp16 TN, uniform[-1,1], C = 0; one generator with
    seed 2 draws (4000,3000,2056) first, then (8192,128,8192)."""
    rng = np.random.default_rng(2)
    w1 = gemm_workload("fp16_tn_4000x3000x2056", 4000, 3000, 2056, seed=2, dist="uniform", rng=rng)
    w2 = gemm_workload("fp16_tn_8192x128x8192", 8192, 128, 8192, seed=2, dist="uniform", rng=rng)
    return w1, w2


def config4(case: str = "NN") -> Workload:
    """Batch 64 of 512^3, seed 3, normal(0,1), C = 0.  A is the stride-swapped
    view (M contiguous, strides (M*K, 1, M)).  'NN': B is K-contiguous;
    'NT': B is N-contiguous (strides (N*K, 1, N)).  'TN'/'TT' are the other two
    combinations with a K-contiguous A."""
    a_major = "col" if case[0] == "N" else "row"
    b_major = "row" if case[1] == "N" else "col"
    return gemm_workload(f"fp16_batched64_512_{case}", 512, 512, 512, seed=3, dist="normal",
                         batch=64, a_major=a_major, b_major=b_major)


def config5(n: int = 8192) -> Workload:
    """MXFP8: E4M3 data from normal(0,1), one E8M0 scale per 32 K per row,
    exponents uniform in [-4, 4], C = 0, seed 4."""
    return gemm_workload(f"mxfp8_tn_{n}", n, n, n, seed=4, dist="normal", mx=True)
