"""Shared helpers of the GPU tests: move seeded host operands to the device
with their strides, run the library, and check its output against the
oracle (full or at sampled points)."""

from __future__ import annotations

import os
import sys

import numpy as np

from oracle import gemm as OG
from stride_layouts_lds_amd.inputs import HostOperand, Workload, to_device  # noqa: F401


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_library(w: Workload, out=None, stream=None):
    """D from the HIP library for workload w (D row-major, allocated by torch)."""
    import torch
    from stride_layouts_lds_amd import api
    a, b, c = to_device(w.a), to_device(w.b), to_device(w.c)
    sfa, sfb = to_device(w.sfa), to_device(w.sfb)
    if out is None:
        out = torch.empty(w.d_shape, dtype=torch.bfloat16 if w.bf16 else torch.float16, device="cuda")
    api.gemm(a, b, c, out=out, sfa=sfa, sfb=sfb, block_k=w.block_k, stream=stream)
    torch.cuda.synchronize()
    return out


def d_codes(d) -> np.ndarray:
    import torch
    return d.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def _ora(op, scale: bool = False, nvfp4: bool = False):
    """An operand as the oracle takes it: a numpy view, or (packed E2M1 or
    6-bit data, NVFP4's E4M3 scales) raw storage with element strides."""
    if op is None:
        return None
    if op.kind in ("e2m1", "e2m3", "e3m2"):
        code = {"e2m1": OG.E2M1, "e2m3": OG.E2M3, "e3m2": OG.E3M2}[op.kind]
        return OG.packed(op.storage, op.shape, op.strides, code)
    if scale and nvfp4:
        return OG.packed(op.storage, op.shape, op.strides, OG.E4M3)
    return op.view


def _operands(w: Workload):
    nv = w.nvfp4  # E4M3 scales (MXFP4's E8M0 scales have numpy views)
    return (_ora(w.a), _ora(w.b), _ora(w.c), _ora(w.sfa, True, nv), _ora(w.sfb, True, nv))


def oracle_full(w: Workload, max_outputs: int = 1 << 23):
    """The oracle over every output element.  Large outputs go in bands of
    rows of A (and of C and A's scales), one call per band with a progress
    line, so that a long check keeps printing; each element is computed the
    same way either way."""
    ops = _operands(w)
    M = w.M
    if w.batch * M * w.N <= max_outputs or any(x is not None and not isinstance(x, np.ndarray) for x in ops):
        return OG.gemm(*ops, block_k=w.block_k, bf16=w.bf16)
    rows = max(1, max_outputs // (w.batch * w.N))
    parts = []
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        parts.append(oracle_rows(w, r0, r1))
        log(f"  oracle rows {r1} of {M}")
    return tuple(np.concatenate([p[i] for p in parts], axis=-2) for i in range(3))


def oracle_rows(w: Workload, r0: int, r1: int):
    """The oracle over output rows [r0, r1) of every batch: the same call on
    row bands of A, C and A's scales (numpy views; not for packed data)."""
    a, b, c, sfa, sfb = _operands(w)
    band = lambda x: None if x is None else x[..., r0:r1, :]
    assert all(x is None or isinstance(x, np.ndarray) for x in (a, c, sfa)), "row bands of numpy views only"
    return OG.gemm(band(a), b, band(c), band(sfa), sfb, block_k=w.block_k, bf16=w.bf16)


def oracle_points(w: Workload, pts: np.ndarray):
    return OG.gemm_points(*_operands(w), points=pts, block_k=w.block_k, bf16=w.bf16)


def sample_points(w: Workload, n: int, seed: int = 0) -> np.ndarray:
    """Random output points plus every corner and the last row / column
    (ragged edges), as (batch, m, n)."""
    rng = np.random.default_rng(seed)
    B, M, N = w.batch, w.M, w.N
    pts = [np.stack([rng.integers(0, B, n), rng.integers(0, M, n), rng.integers(0, N, n)], 1)]
    edge = []
    for b in {0, B - 1}:
        for m in {0, M - 1}:
            for nn in {0, N - 1}:
                edge.append((b, m, nn))
        for nn in rng.integers(0, N, 64):
            edge.append((b, M - 1, int(nn)))
        for m in rng.integers(0, M, 64):
            edge.append((b, int(m), N - 1))
    pts.append(np.array(edge, np.int64))
    return np.concatenate(pts).astype(np.int64)


def tile_points(w: Workload, tile: int = 256, seed: int = 0, max_batches: int = 8) -> np.ndarray:
    """Every row and every column of every tile x tile block of the output,
    at least once: in block (tm, tn), of r rows and c columns inside the
    output, the points (tm*tile + i % r, tn*tile + p(i % c)) for i below
    max(r, c) and a random permutation p, over up to max_batches batches (the first, the last and
    random ones between); plus sample_points' edges.  As (batch, m, n)."""
    rng = np.random.default_rng(seed)
    B, M, N = w.batch, w.M, w.N
    bs = sorted({0, B - 1} | set(rng.integers(0, B, max(0, max_batches - 2)).tolist())) if B > 0 else []
    out = []
    for b in bs:
        for tm in range(0, M, tile):
            for tn in range(0, N, tile):
                r, c = min(tile, M - tm), min(tile, N - tn)
                i = np.arange(max(r, c))
                m, n = tm + i % r, tn + rng.permutation(c)[i % c]
                out.append(np.stack([np.full(i.size, b), m, n], 1))
    out.append(sample_points(w, 0, seed))
    return np.concatenate(out).astype(np.int64)


def assert_within_bound(d: np.ndarray, d_ref: np.ndarray, absum: np.ndarray, what: str, bf16: bool = False) -> None:
    bad, wi, wr = OG.check(d, d_ref, absum, bf16=bf16)
    if bad:
        dec = OG.bf16_decode if bf16 else OG.f16_decode
        dd, rr = dec(int(d.ravel()[wi])), dec(int(d_ref.ravel()[wi]))
        rel = "2^-7" if bf16 else "2^-10"
        raise AssertionError(f"{what}: {bad} of {d.size} elements outside |D-Dref| <= {rel}|Dref| + 2^-13 S; "
                             f"worst index {wi}: D={dd} Dref={rr} S={absum.ravel()[wi]} "
                             f"(error/bound {wr:.3g})")


def dump(name: str, arr) -> None:
    """Save an array as <name>.npy in the directory named by SL_DUMP, for
    offline reading (a debug aid: nothing is written when it is unset)."""
    d = os.environ.get("SL_DUMP")
    if d:
        os.makedirs(d, exist_ok=True)
        np.save(os.path.join(d, name + ".npy"), np.asarray(arr))
