"""Parity of the HIP GEMM with the oracle, through the C ABI.

* exact: small-integer inputs make every product, partial sum and fp32
  accumulation exact, so the library's fp16 output must equal the oracle's
  bit for bit, over ragged multi-tile shapes, every majorness combination,
  batches, broadcasts, in-place C, K = 0 and the element-loader path;
* bounded: real-valued seeded inputs, every element within
  |D - D_ref| <= 2^-10 |D_ref| + 2^-13 sum_k |A B|: every output element of
  the named workloads at their full sizes (the 8192^3 ones in bands of rows);
  for the other formats at 8192^3, every row and column of every 256 x 256
  block, random points and the edges, plus a finiteness check of every
  element.
"""

import os

import numpy as np
import pytest

from stride_layouts_lds_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stride_layouts_lds_amd import api as A
    A.lib()
    return A


def H():
    import gpu_helpers
    return gpu_helpers


# ------------------------------------------------------------------ exact

EXACT = [
    # M, N, K, batch, a_major, b_major, with_c
    (256, 256, 64, None, "row", "row", False),
    (300, 520, 200, None, "row", "row", True),
    (1, 1, 8, None, "row", "row", False),
    (17, 33, 8, None, "row", "row", True),
    (513, 257, 1000, None, "row", "row", True),
    (520, 264, 136, 2, "col", "row", False),
    (96, 80, 64, 3, "col", "col", True),
    (96, 80, 72, 3, "row", "col", False),
    (264, 136, 200, None, "col", "col", False),
    (100, 60, 40, None, "col", "row", False),   # M % 8 != 0: element loader for A
    (70, 90, 37, None, "row", "row", True),     # K % 8 != 0: element loaders
]


@pytest.mark.parametrize("case", EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_{c[4]}{c[5]}_c{int(c[6])}")
def test_exact_integer_parity(api, case):
    h = H()
    M, N, K, batch, am, bm, with_c = case
    w = I.gemm_workload("exact", M, N, K, seed=M + N + K, dist="int4", batch=batch, a_major=am, b_major=bm,
                        with_c=with_c)
    h.log(f"exact {case} plan={_plan(api, w)}")
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


# every fp16 tile configuration the planner can be told to use (SL_TILE),
# on K-contiguous operands, over several output tiles with ragged edges
F16_TILES = list(range(18)) + [19, 20]


@pytest.mark.parametrize("tile", F16_TILES)
def test_exact_parity_every_fp16_tile(api, tile, monkeypatch):
    h = H()
    monkeypatch.setenv("SL_TILE", str(tile))
    w = I.gemm_workload("tiles", 520, 300, 328, seed=tile, dist="int4", with_c=True)
    plan = _plan(api, w)
    h.log(f"tile {tile} plan={plan}")
    assert plan["kernel"] == api.K_F16
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


MN_DIRECT = [
    # M, N, K, batch, a_major, b_major, with_c: M- / N-contiguous operands
    # through the 8-wave kernel's direct M-major copy and transposing reads
    (520, 264, 136, 2, "col", "row", False),
    (256, 256, 64, None, "col", "col", True),
    (264, 520, 200, None, "row", "col", True),
    (512, 512, 512, 3, "col", "col", False),
    (136, 72, 1000, None, "col", "row", True),   # K-tiles past the ragged end of K
]


@pytest.mark.parametrize("tile", [4, 19])
@pytest.mark.parametrize("case", MN_DIRECT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_{c[4]}{c[5]}")
def test_exact_parity_m_major_direct_copy(api, case, tile, monkeypatch):
    """The 8-wave kernel (tile 4) and the ring kernel (tile 19) with direct
    M-major copies and transposing fragment reads."""
    h = H()
    monkeypatch.setenv("SL_TILE", str(tile))
    M, N, K, batch, am, bm, with_c = case
    w = I.gemm_workload("mn_direct", M, N, K, seed=M + 2 * N + K, dist="int4", batch=batch, a_major=am,
                        b_major=bm, with_c=with_c)
    plan = _plan(api, w)
    h.log(f"mn direct {case} plan={plan}")
    assert plan["tile_m"] == 256 and plan["a_load"] == (3 if am == "col" else 0)
    assert plan["b_load"] == (3 if bm == "col" else 0)
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


SPLITK = [
    # M, N, K, batch, with_c, forced split count (0: the planner's), expected splits
    (300, 72, 2056, None, True, 0, 7),    # 33 K-tiles: 7 splits of 5 (the last of 3)
    (130, 120, 1032, 2, False, 3, 3),
    (200, 70, 1000, None, True, 5, 4),    # N % 4 != 0: scalar partial stores; 16 K-tiles in 4 splits of 4
    (64, 64, 4096, None, False, 0, 8),
    (520, 136, 776, None, True, 2, 2),    # ragged last split (13 K-tiles: 7 + 6)
]


@pytest.mark.parametrize("case", SPLITK, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_s{c[6]}")
def test_splitk_exact_parity(api, case, monkeypatch):
    h = H()
    M, N, K, batch, with_c, force, want = case
    monkeypatch.setenv("SL_TILE", "16")
    if force:
        monkeypatch.setenv("SL_SPLITK", str(force))
    w = I.gemm_workload("splitk", M, N, K, seed=M + K, dist="int4", batch=batch, with_c=with_c)
    import torch
    out = torch.empty(w.d_shape, dtype=torch.float16, device="cuda")
    args = api.make_args(h.to_device(w.a), h.to_device(w.b), h.to_device(w.c), out, None, None, 32)
    plan = api.sl_gemm_plan(args)
    h.log(f"splitk {case} plan={plan}")
    assert plan["split_k"] == want and plan["tile_m"] == plan["tile_n"] == 128
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


def test_splitk_in_place_and_repeated_calls(api, monkeypatch):
    """C == D in place through a split-K plan, then the same call again on
    another stream, each call with its own caller-allocated workspace."""
    import torch
    h = H()
    monkeypatch.setenv("SL_TILE", "16")
    monkeypatch.setenv("SL_SPLITK", "4")
    w = I.gemm_workload("splitk_inplace", 264, 96, 1024, seed=9, dist="int4", with_c=True)
    a, b = h.to_device(w.a), h.to_device(w.b)
    d = h.to_device(w.c).contiguous().clone()
    api.gemm(a, b, d, out=d)
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        d2 = torch.zeros_like(d)
        api.gemm(a, b, None, out=d2, stream=s2.cuda_stream)
    torch.cuda.synchronize()
    d_ref, _, _ = h.oracle_full(w)
    assert np.array_equal(h.d_codes(d), d_ref[0])
    w0 = I.gemm_workload("splitk_inplace", 264, 96, 1024, seed=9, dist="int4", with_c=True)
    w0.c = None
    d0_ref, _, _ = h.oracle_full(w0)
    assert np.array_equal(h.d_codes(d2), d0_ref[0])


def _plan(api, w):
    import torch
    h = H()
    out = torch.empty(w.d_shape, dtype=torch.bfloat16 if w.bf16 else torch.float16, device="cuda")
    args = api.make_args(h.to_device(w.a), h.to_device(w.b), h.to_device(w.c), out, h.to_device(w.sfa),
                         h.to_device(w.sfb), w.block_k)
    p = api.sl_gemm_plan(args)
    return {k: p[k] for k in ("kernel", "a_load", "b_load", "tile_m", "tile_n", "workgroups", "lds_bytes", "split_k",
                                   "workspace_bytes")}


def test_odd_strides_take_the_element_loader(api):
    """Row stride K+3 and a column-strided view (every other K element)."""
    import torch
    h = H()
    rng = np.random.default_rng(21)
    M, N, K = 150, 130, 96
    a_st = rng.integers(-4, 5, (M, K + 3)).astype(np.float16)
    b_st = rng.integers(-4, 5, (N, 2 * K)).astype(np.float16)
    a = torch.from_numpy(a_st).cuda()[:, :K]
    b = torch.from_numpy(b_st).cuda()[:, ::2]
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    p = api.sl_gemm_plan(api.make_args(a, b, None, out))
    assert p["kernel"] == api.K_F16_GENERIC
    api.gemm(a, b, out=out)
    torch.cuda.synchronize()
    from oracle import gemm as OG
    d_ref, _, _ = OG.gemm(a_st.view(np.uint16)[:, :K], b_st.view(np.uint16)[:, ::2])
    assert np.array_equal(h.d_codes(out), d_ref[0])


RING = [
    # M, N, K, batch, with_c: the 4-wave ring kernel (tile 19) at one K-tile,
    # a K below one tile, ragged edges in M, N and K, batches, long K
    (256, 256, 64, None, False),
    (256, 256, 8, None, True),
    (520, 300, 328, None, True),
    (1000, 776, 1032, 2, True),
    (264, 520, 4104, None, False),
    # with C at 2, 3, 5, 8 and 9 K-tiles: the C lines loaded ahead during the
    # last eight K-tiles (a window that starts before the first one, with it,
    # or after it), full tiles for the row epilogue
    (512, 256, 128, None, True),
    (256, 512, 192, 2, True),
    (512, 512, 320, None, True),
    (512, 256, 512, None, True),
    (256, 512, 576, 2, True),
]


@pytest.mark.parametrize("case", RING, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_c{int(c[4])}")
def test_ring_kernel_exact_parity(api, case, monkeypatch):
    h = H()
    monkeypatch.setenv("SL_TILE", "19")
    M, N, K, batch, with_c = case
    w = I.gemm_workload("ring", M, N, K, seed=M + N + K + 19, dist="int4", batch=batch, with_c=with_c)
    plan = _plan(api, w)
    h.log(f"ring {case} plan={plan}")
    assert plan["lds_bytes"] == 163840  # five 32 KiB operand K-tiles: the ring kernel
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


def test_ring_kernel_in_place(api, monkeypatch):
    """C == D through the ring kernel: every C element is read before its
    D element is written."""
    import torch
    h = H()
    monkeypatch.setenv("SL_TILE", "19")
    w = I.gemm_workload("ring_inplace", 520, 264, 200, seed=23, dist="int4", with_c=True)
    d_ref, _, _ = h.oracle_full(w)
    c = h.to_device(w.c).contiguous()
    api.gemm(h.to_device(w.a), h.to_device(w.b), c, out=c)
    torch.cuda.synchronize()
    assert np.array_equal(h.d_codes(c), d_ref[0])


def test_in_place_c_equals_d(api):
    import torch
    h = H()
    w = I.gemm_workload("inplace", 200, 136, 128, seed=5, dist="int4", with_c=True)
    d_ref, _, _ = h.oracle_full(w)
    c = h.to_device(w.c).contiguous()
    api.gemm(h.to_device(w.a), h.to_device(w.b), c, out=c)
    torch.cuda.synchronize()
    assert np.array_equal(h.d_codes(c), d_ref[0])


def test_k_zero_gives_c(api):
    import torch
    h = H()
    M, N = 70, 40
    c = torch.randn(M, N).half().cuda()
    a = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((N, 0), dtype=torch.float16, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    api.gemm(a, b, c, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), c.cpu())
    api.gemm(a, b, None, out=out)
    torch.cuda.synchronize()
    assert not out.cpu().any()


def test_empty_is_a_noop(api):
    import torch
    a = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    b = torch.zeros((32, 64), dtype=torch.float16, device="cuda")
    out = torch.zeros((0, 32), dtype=torch.float16, device="cuda")
    api.gemm(a, b, out=out)
    torch.cuda.synchronize()


def test_broadcast_b_across_batch(api):
    import torch
    h = H()
    rng = np.random.default_rng(22)
    nb, M, N, K = 4, 136, 72, 64
    A = rng.integers(-4, 5, (nb, M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda().unsqueeze(0).expand(nb, N, K)  # batch stride 0
    out = api.gemm(a, b)
    torch.cuda.synchronize()
    from oracle import gemm as OG
    bv = np.lib.stride_tricks.as_strided(B.view(np.uint16), (nb, N, K), (0, 2 * K, 2))
    d_ref, _, _ = OG.gemm(A.view(np.uint16), bv)
    assert np.array_equal(h.d_codes(out), d_ref)


@pytest.mark.parametrize("tile", [19, 4])
@pytest.mark.parametrize("M,N", [(512, 256), (300, 264)], ids=["rows", "quads"])
def test_ring_kernel_broadcast_a_and_c(api, M, N, tile, monkeypatch):
    """A and C shared across a batch of B (batch stride 0 on both) through
    the ring kernel (tile 19) and the 8-wave kernel (tile 4), with the row
    epilogue (full tiles) and the per-quad one (ragged edges)."""
    import torch
    h = H()
    monkeypatch.setenv("SL_TILE", str(tile))
    rng = np.random.default_rng(M + N)
    nb, K = 3, 576
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (nb, N, K)).astype(np.float16)
    C = rng.integers(-64, 65, (M, N)).astype(np.float16)
    a = torch.from_numpy(A).cuda().unsqueeze(0).expand(nb, M, K)
    c = torch.from_numpy(C).cuda().unsqueeze(0).expand(nb, M, N)
    out = api.gemm(a, torch.from_numpy(B).cuda(), c)
    torch.cuda.synchronize()
    from oracle import gemm as OG
    av = np.lib.stride_tricks.as_strided(A.view(np.uint16), (nb, M, K), (0, 2 * K, 2))
    cv = np.lib.stride_tricks.as_strided(C.view(np.uint16), (nb, M, N), (0, 2 * N, 2))
    d_ref, _, _ = OG.gemm(av, B.view(np.uint16), cv)
    assert np.array_equal(h.d_codes(out), d_ref)


@pytest.mark.parametrize("with_c", [False, True], ids=["noc", "c"])
@pytest.mark.parametrize("M,N", [(300, 261), (512, 387), (520, 384)])
def test_ring_192_edges(api, M, N, with_c, monkeypatch):
    """The 256 x 192 ring tile at the edges: M and N not multiples of the
    tile, N not a multiple of 4 (D and C rows padded to a multiple of 4, so
    the rows are vector-aligned while the quad that crosses N is stored
    element by element); the padding columns are never written."""
    import torch
    h = H()
    monkeypatch.setenv("SL_TILE", "20")
    rng = np.random.default_rng(M * 7 + N)
    K, NP = 200, (N + 3) // 4 * 4
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    Cf = rng.integers(-64, 65, (M, NP)).astype(np.float16)
    c = torch.from_numpy(Cf).cuda()[:, :N] if with_c else None
    dbuf = torch.full((M, NP), float("nan"), dtype=torch.float16, device="cuda")
    out = dbuf[:, :N]
    args = api.make_args(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), c, out)
    plan = api.sl_gemm_plan(args)
    h.log(f"ring 192 edges M={M} N={N} c={with_c} plan={plan}")
    assert plan["tile_n"] == 192
    api.gemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), c, out=out)
    torch.cuda.synchronize()
    from oracle import gemm as OG
    cv = np.ascontiguousarray(Cf[:, :N]).view(np.uint16) if with_c else None
    d_ref, _, _ = OG.gemm(A.view(np.uint16), B.view(np.uint16), cv)
    assert np.array_equal(h.d_codes(out), d_ref[0])
    # the padding columns are never written
    assert torch.isnan(dbuf[:, N:]).all().item()


# zero strides inside the matrix dimensions: C as a bias row (0, 1) or a
# column (1, 0), A or B with row stride 0 (every row the same), on full
# 256 x 256 tiles (row epilogues; the ring kernel's C-line prefetch) and on
# ragged ones (per-quad epilogue); the planner's tile, the 8-wave tile and
# the ring tile
ZERO_STRIDE = [
    # M, N, K, which operand broadcasts, how
    (512, 512, 576, "c", "row"),
    (512, 512, 576, "c", "col"),
    (300, 264, 200, "c", "row"),
    (300, 264, 200, "c", "col"),
    (512, 512, 320, "a", "row"),
    (300, 264, 200, "a", "row"),
    (512, 512, 320, "b", "row"),
    (300, 264, 200, "b", "row"),
    (264, 96, 1024, "c", "row"),   # split-K (skinny output): the reduction reads C
]


@pytest.mark.parametrize("tile", [None, 4, 19, 20])
@pytest.mark.parametrize("case", ZERO_STRIDE, ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[3]}_{c[4]}")
def test_zero_stride_inside_the_matrix(api, case, tile, monkeypatch):
    """A zero stride inside a matrix dimension reads one element for every
    index along it ("CuTe 中 A、B 如何加载到 MMA 寄存器", section 3, the
    broadcast stride; "数据布局及其记号", "Shape-Stride 模型"): exact-integer
    parity with the oracle over the same zero-strided views."""
    import torch
    h = H()
    M, N, K, which, how = case
    if tile is not None:
        if K < 64 or (M, N) == (264, 96):
            pytest.skip("the forced tiles are for outputs without a K-split")
        monkeypatch.setenv("SL_TILE", str(tile))
    rng = np.random.default_rng(M + N + K + ord(which))
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    u16 = lambda x: x.view(np.uint16)
    a_dev, b_dev = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    av, bv, cv, c_dev = u16(A), u16(B), None, None
    if which == "a":
        row = rng.integers(-4, 5, (1, K)).astype(np.float16)
        a_dev = torch.from_numpy(row).cuda().expand(M, K)                   # strides (0, 1)
        av = np.lib.stride_tricks.as_strided(u16(row), (M, K), (0, 2))
    elif which == "b":
        row = rng.integers(-4, 5, (1, K)).astype(np.float16)
        b_dev = torch.from_numpy(row).cuda().expand(N, K)
        bv = np.lib.stride_tricks.as_strided(u16(row), (N, K), (0, 2))
    else:
        if how == "row":   # a bias row: C[m, n] = bias[n], strides (0, 1)
            vec = rng.integers(-64, 65, (1, N)).astype(np.float16)
            c_dev = torch.from_numpy(vec).cuda().expand(M, N)
            cv = np.lib.stride_tricks.as_strided(u16(vec), (M, N), (0, 2))
        else:              # a column: C[m, n] = col[m], strides (1, 0)
            vec = rng.integers(-64, 65, (M, 1)).astype(np.float16)
            c_dev = torch.from_numpy(vec).cuda().expand(M, N)
            cv = np.lib.stride_tricks.as_strided(u16(vec), (M, N), (2, 0))
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    args = api.make_args(a_dev, b_dev, c_dev, out)
    h.log(f"zero stride {case} tile={tile} strides a{tuple(a_dev.stride())} b{tuple(b_dev.stride())} "
          f"c{tuple(c_dev.stride()) if c_dev is not None else None} plan={api.sl_gemm_plan(args)}")
    api.gemm(a_dev, b_dev, c_dev, out=out)
    torch.cuda.synchronize()
    from oracle import gemm as OG
    d_ref, _, _ = OG.gemm(av, bv, cv)
    mism = np.count_nonzero(h.d_codes(out) != d_ref[0])
    assert mism == 0, f"{mism} elements differ"


MX_EXACT = [
    # M, N, K, batch, scale row padding, kernel the planner must pick when
    # asked for the 8-wave tile
    (256, 256, 128, None, 0, 4),
    (300, 200, 384, None, 0, 4),
    (64, 520, 256, None, 0, 4),
    (130, 260, 112, None, 0, 4),   # last scale block covers 16 of its 32 K
    (136, 128, 256, 2, 0, 4),      # batched scales
    (256, 264, 256, None, 4, 4),   # padded scale rows, still dword aligned
    (256, 264, 256, None, 1, 3),   # scale rows 9 bytes apart: byte-load kernel
    (300, 264, 512, None, 0, 4),   # 16 blocks per row: 16-byte scale copies every 4 K-tiles
    (256, 200, 1536, 2, 0, 4),     # batched, 48 blocks per row
    (264, 136, 1024, None, 16, 4),  # padded rows 48 bytes apart: 16-byte copies
    (264, 136, 512, None, 4, 4),   # rows 20 bytes apart: dword copies
    (300, 200, 208, None, 0, 3),   # 7 scale blocks per row: byte-load kernel
    (72, 96, 96, 3, 0, 3),
]


@pytest.mark.parametrize("case", MX_EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_p{c[4]}_k{c[5]}")
def test_mx_exact_parity(api, case, monkeypatch):
    """E4M3 integers and scale exponents in [-2, 2]: every product is a
    multiple of 2^-4 below 2^8 and every partial sum stays exact in fp32."""
    h = H()
    monkeypatch.setenv("SL_TILE", "4")
    M, N, K, batch, pad, kernel = case
    w = I.gemm_workload("mx_exact", M, N, K, seed=K + M, dist="int4", batch=batch, mx=True,
                        scale_range=(-2, 2), scale_pad=pad)
    plan = _plan(api, w)
    h.log(f"mx exact {case} plan={plan}")
    assert plan["kernel"] == kernel
    if kernel == 4:  # 16-byte scale copies (two 8 KiB buffers) iff rows allow them
        kb = -(-K // 32)
        s16 = kb % 16 == 0 and (kb + pad) % 16 == 0
        assert plan["lds_bytes"] == 2 * 512 * 128 + (2 * 512 * 16 if s16 else 2 * 512 * 4)
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


MX_RING = [
    # M, N, K, batch, scale row padding, with C: the 4-wave MXFP8 ring kernel
    # (16-byte scale chunks, so K is a multiple of 512 or just below one)
    (256, 256, 512, None, 0, False),    # one tile, one group of four K-tiles, row epilogue
    (264, 136, 496, None, 0, True),     # ragged M, N and K: per-quad epilogue
    (256, 200, 1536, 2, 0, True),       # batched, 48 blocks per row
    (264, 136, 1024, None, 16, False),  # padded scale rows 48 bytes apart
    (512, 512, 2048, None, 0, True),    # four full tiles, 16 K-tiles, row epilogue with C
]


@pytest.mark.parametrize("case", MX_RING, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_p{c[4]}_c{int(c[5])}")
def test_mx_ring_exact_parity(api, case, monkeypatch):
    h = H()
    monkeypatch.setenv("SL_TILE", "19")
    M, N, K, batch, pad, with_c = case
    w = I.gemm_workload("mx_ring", M, N, K, seed=K + M + 7, dist="int4", batch=batch, mx=True,
                        scale_range=(-2, 2), scale_pad=pad, with_c=with_c)
    plan = _plan(api, w)
    h.log(f"mx ring {case} plan={plan}")
    assert plan["kernel"] == api.K_MX_W4R and plan["lds_bytes"] == 163840
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


@pytest.mark.parametrize("tile", [1, 3, 4, 19])
def test_mx_kernels_agree_on_one_input(api, tile, monkeypatch):
    """The same normal-valued MXFP8 problem through each MX kernel (tile
    forced), every element within the bound."""
    h = H()
    monkeypatch.setenv("SL_TILE", str(tile))
    w = I.gemm_workload("mx_tiles", 300, 264, 512, seed=77, dist="normal", mx=True, with_c=True)
    plan = _plan(api, w)
    h.log(f"mx tile {tile} plan={plan}")
    assert plan["kernel"] == {4: api.K_MX_W8, 19: api.K_MX_W4R}.get(tile, api.K_MX)
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, f"mx tile {tile}")


# ------------------------------------------------------------------ bounded

SMALL = [
    ("normal_c", dict(M=520, N=264, K=320, dist="normal", with_c=True)),
    ("uniform_ragged", dict(M=333, N=251, K=264, dist="uniform")),
    ("batched_nn", dict(M=136, N=128, K=200, dist="normal", batch=3, a_major="col", b_major="row")),
    ("batched_nt", dict(M=128, N=136, K=96, dist="normal", batch=2, a_major="col", b_major="col")),
    ("mx", dict(M=300, N=264, K=512, dist="normal", mx=True)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_bounded_small(api, name, kw):
    h = H()
    M, N, K = kw.pop("M"), kw.pop("N"), kw.pop("K")
    w = I.gemm_workload(name, M, N, K, seed=31, **kw)
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, name)


def test_config1_full(api):
    h = H()
    w = I.config1()
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, w.name)


def _full(api, w):
    """Every output element against the oracle's, within the bound."""
    import time
    h = H()
    h.log(f"{w.name}: plan {_plan(api, w)}")
    d = h.d_codes(h.run_library(w)).reshape(w.batch, w.M, w.N)
    t0 = time.perf_counter()
    d_ref, _, absum = h.oracle_full(w)
    h.log(f"{w.name}: oracle over all {d_ref.size} outputs in {time.perf_counter() - t0:.1f} s")
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, w.name, bf16=w.bf16)


def _sampled(api, w, n=3000):
    """Every row and column of every 256 x 256 block once (h.tile_points),
    plus n random points and the edges; every element must be finite."""
    import torch
    h = H()
    h.log(f"{w.name}: plan {_plan(api, w)}")
    out = h.run_library(w)
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    d = h.d_codes(out).reshape(w.batch, w.M, w.N)
    pts = np.concatenate([h.tile_points(w), h.sample_points(w, n)])
    d_ref, _, absum = h.oracle_points(w, pts)
    h.assert_within_bound(d[pts[:, 0], pts[:, 1], pts[:, 2]], d_ref, absum, w.name, bf16=w.bf16)


# The 8192^3 workloads: the library runs once (kept for the module) and
# every output element is checked against the oracle in bands of rows, one
# test per band, so each test takes well under a minute of oracle time.
_BIG = {}


def _full_band(api, make, band, bands):
    h = H()
    key = make.__name__
    if key not in _BIG:
        _BIG.clear()
        w = make()
        h.log(f"{w.name}: plan {_plan(api, w)}")
        _BIG[key] = (w, h.d_codes(h.run_library(w)).reshape(w.batch, w.M, w.N))
    w, d = _BIG[key]
    r0, r1 = band * w.M // bands, (band + 1) * w.M // bands
    d_ref, _, absum = h.oracle_rows(w, r0, r1)
    h.assert_within_bound(d[:, r0:r1], d_ref, absum, f"{w.name} rows {r0}..{r1 - 1}", bf16=w.bf16)
    if band == bands - 1:
        _BIG.clear()


def _config2_8192():
    return I.config2(8192)


def _config5_8192():
    return I.config5(8192)


def test_config2_4096_with_c(api):
    _full(api, I.config2(4096))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("band", range(4))
def test_config2_8192_with_c(api, band):
    _full_band(api, _config2_8192, band, 4)


def test_config3_ragged_and_skinny(api):
    for w in I.config3():
        _full(api, w)


@pytest.mark.parametrize("case", ["NN", "NT", "TN", "TT"])
def test_config4_batched_strided(api, case):
    _full(api, I.config4(case))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("band", range(8))
def test_config5_mxfp8_8192(api, band):
    _full_band(api, _config5_8192, band, 8)


# ------------------------------------------------------------------ bf16

BF16_EXACT = [
    # M, N, K, batch, a_major, b_major, with_c, forced tile (None: planner)
    (300, 520, 200, None, "row", "row", True, None),
    (520, 264, 136, 2, "col", "row", False, 4),      # M-major direct copy
    (264, 136, 200, None, "col", "col", True, None),  # register-transposing loader
    (70, 90, 37, None, "row", "row", True, None),     # element loaders
    (300, 72, 2056, None, "row", "row", True, 16),    # split-K
    (520, 300, 328, None, "row", "row", True, 17),
    (520, 300, 328, None, "row", "row", True, 7),
    (520, 300, 328, None, "row", "row", True, 15),
    (520, 300, 328, None, "row", "row", True, 5),
    (520, 300, 328, None, "row", "row", True, 19),
    (1000, 776, 1032, 2, "row", "row", True, 19),
    (520, 300, 328, None, "row", "row", True, 20),
    (264, 520, 200, 2, "col", "row", True, 19),   # M-major A through the ring kernel's direct copies
    (512, 512, 320, None, "col", "row", True, 4),  # 8-wave kernel, full tiles: row epilogue with C
    (512, 256, 128, 2, "row", "row", True, 4),
]


@pytest.mark.parametrize("case", BF16_EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_{c[4]}{c[5]}_t{c[7]}")
def test_bf16_exact_parity(api, case, monkeypatch):
    h = H()
    M, N, K, batch, am, bm, with_c, tile = case
    if tile is not None:
        monkeypatch.setenv("SL_TILE", str(tile))
    w = I.gemm_workload("bf16_exact", M, N, K, seed=M + N + K + 1, dist="int4", batch=batch, a_major=am,
                        b_major=bm, with_c=with_c, bf16=True)
    h.log(f"bf16 exact {case} plan={_plan(api, w)}")
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


def test_bf16_bounded_and_sampled(api):
    h = H()
    w = I.gemm_workload("bf16_normal", 520, 264, 320, seed=41, dist="normal", with_c=True, bf16=True)
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, w.name, bf16=True)
    _full(api, I.gemm_workload("bf16_tn_4096_c", 4096, 4096, 4096, seed=1, dist="normal", with_c=True,
                               bf16=True))


@pytest.mark.parametrize("bf16", [False, True], ids=["f16", "bf16"])
def test_output_rounding_ties_to_even(api, bf16):
    """Sums that fall exactly halfway between two representable outputs:
    D[m][n] = 1 + t_m with t_m = (2j+1) * ulp/2 (and quarter-ulps), so the
    library's fp32 -> 16-bit conversion must round ties to the even code,
    bit for bit with the oracle."""
    import torch
    h = H()
    ulp = 2.0 ** -7 if bf16 else 2.0 ** -10
    ts = [(2 * j + 1) * ulp / 2 for j in range(8)] + [ulp / 4, 3 * ulp / 4, -ulp / 4, -(2 * 3 + 1) * ulp / 4]
    M, N, K = len(ts), 16, 32
    a = np.zeros((M, K)); b = np.zeros((N, K))
    a[:, 0] = 1.0; a[:, 1] = ts
    b[:, 0] = 1.0; b[:, 1] = 1.0
    dt = torch.bfloat16 if bf16 else torch.float16
    at = torch.from_numpy(a).to(dt); bt = torch.from_numpy(b).to(dt)
    assert torch.equal(at.double(), torch.from_numpy(a)), "inputs must be exact"
    out = api.gemm(at.cuda(), bt.cuda())
    torch.cuda.synchronize()
    from oracle import gemm as OG
    codes = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    d_ref, ref, _ = OG.gemm(codes(at), codes(bt), bf16=bf16)
    assert np.array_equal(ref[0][:, 0], 1.0 + np.array(ts))
    assert np.array_equal(h.d_codes(out), d_ref[0])


# ------------------------------------------------------------------ NVFP4

NVFP4_EXACT = [
    # M, N, K, batch, with_c
    (256, 256, 64, None, False),
    (300, 264, 512, None, True),
    (136, 72, 96, 2, True),      # K ends half way through a 64-wide K-tile
    (136, 72, 128, 3, True),     # batched, K whole K-tiles (decoded ahead when forced)
    (520, 300, 1024, None, False),
    (512, 512, 320, None, True),   # full tiles with C: the row epilogue; an odd number of K-tiles
]


@pytest.mark.parametrize("case", NVFP4_EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_c{int(c[4])}")
@pytest.mark.parametrize("mode", [None, 19, "decode"])
def test_nvfp4_exact_parity(api, case, mode, monkeypatch):
    """Packed E2M1 data, E4M3 scales 2^[-2,2] x {1, 1.5}: every decoded
    product and partial sum is exact in fp32, so D must equal the oracle
    bit for bit.  The automatic plan at these sizes (the fused 8-wave
    kernel), the fused 4-wave ring schedule (tile 19, 128 KiB of LDS), and
    the operands decoded ahead into the workspace followed by the fp16 ring
    kernel (forced here; the automatic plan from 2048^3 on), which needs K a
    multiple of 64 and otherwise keeps the fused kernel."""
    h = H()
    if mode == 19:
        monkeypatch.setenv("SL_TILE", "19")
    elif mode == "decode":
        monkeypatch.setenv("SL_NV_DECODE", "1")
    M, N, K, batch, with_c = case
    w = I.nvfp4_workload("nvfp4_exact", M, N, K, seed=M + K, batch=batch, with_c=with_c, exact=True)
    plan = _plan(api, w)
    h.log(f"nvfp4 exact {case} {mode} plan={plan}")
    # scale rows of a multiple of 8 bytes take the paired loader (5), others the per-tile one (4)
    kind = 5 if (K // 16) % 8 == 0 and os.environ.get("SL_NV_PAIRS", "1") != "0" else 4
    decoded = mode == "decode" and K % 64 == 0
    nb = batch or 1
    assert plan["kernel"] == api.K_NVFP4 and plan["a_load"] == plan["b_load"] == (0 if decoded else kind)
    assert plan["lds_bytes"] == (163840 if decoded else 131072 if mode == 19 and K > 0 else 2 * 512 * 128)
    assert plan["workspace_bytes"] == ((nb * M * K * 2 + 255) // 256 * 256 + nb * N * K * 2 if decoded else 0)
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


@pytest.mark.parametrize("mode", [None, "decode"])
def test_nvfp4_column_major_scales(api, mode, monkeypatch):
    """E4M3 scales held column-major (the K block the fast index is not):
    the fused kernel's per-tile loader and the decode-ahead kernel both
    address them through their strides; D equals the oracle bit for bit."""
    import torch
    h = H()
    if mode == "decode":
        monkeypatch.setenv("SL_NV_DECODE", "1")
    M, N, K = 264, 136, 512
    w = I.nvfp4_workload("nvfp4_cm_scales", M, N, K, seed=11, with_c=True, exact=True)
    a, b, c = h.to_device(w.a), h.to_device(w.b), h.to_device(w.c)
    sfa, sfb = h.to_device(w.sfa), h.to_device(w.sfb)
    cm = lambda x: x.t().contiguous().t()  # same values, strides (1, rows)
    sfa_cm, sfb_cm = cm(sfa), cm(sfb)
    assert sfa_cm.stride() == (1, M) and torch.equal(sfa_cm.view(torch.uint8), sfa.view(torch.uint8))
    out = torch.full(w.d_shape, float("nan"), dtype=torch.float16, device="cuda")
    args = api.make_args(a, b, c, out, sfa_cm, sfb_cm, w.block_k)
    plan = api.sl_gemm_plan(args)
    h.log(f"nvfp4 column-major scales {mode} plan={plan}")
    assert plan["a_load"] == (0 if mode == "decode" else 4)
    api.gemm(a, b, c, out=out, sfa=sfa_cm, sfb=sfb_cm, block_k=w.block_k)
    torch.cuda.synchronize()
    d_ref, _, _ = h.oracle_full(w)
    got = h.d_codes(out)
    assert np.array_equal(got.reshape(d_ref.shape), d_ref), f"{np.count_nonzero(got.reshape(d_ref.shape) != d_ref)} differ"


def test_nvfp4_bounded_and_sampled_8192(api):
    h = H()
    w = I.nvfp4_workload("nvfp4_1024", 1024, 520, 2048, seed=3, with_c=True)
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, w.name)
    _sampled(api, I.nvfp4_workload("nvfp4_8192", 8192, 8192, 8192, seed=6), n=1500)


# ------------------------------------------------------------------ MXFP4

MXFP4_EXACT = [
    # M, N, K, batch, with_c
    (256, 256, 512, None, False),
    (300, 264, 1024, None, True),
    (136, 72, 512, 2, True),
    (520, 300, 2048, None, False),
]


@pytest.mark.parametrize("case", MXFP4_EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_c{int(c[4])}")
def test_mxfp4_exact_parity(api, case):
    """Packed E2M1 data with E8M0 scales 2^[-1,1]: every product and partial
    sum is exact in fp32, so D must equal the oracle bit for bit."""
    h = H()
    M, N, K, batch, with_c = case
    w = I.mxfp4_workload("mxfp4_exact", M, N, K, seed=M + K + 1, batch=batch, with_c=with_c, exact=True)
    plan = _plan(api, w)
    h.log(f"mxfp4 exact {case} plan={plan}")
    assert plan["kernel"] == api.K_MXFP4
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp6"])
def test_packed_operand_spanning_3gib(api, fmt):
    """A packed operand whose 512 rows sit 6 MiB apart spans 3 GiB, past the
    32-bit byte range of one buffer resource, while each 256-row tile spans
    1.5 GiB: the kernels address every tile from its own first row."""
    import torch
    h = H()
    M, N, K = 512, 256, 512
    row_bytes = 6 << 20
    if fmt == "mxfp4":
        w = I.mxfp4_workload("mxfp4_span", M, N, K, seed=31, exact=True)
        per_row = K // 2
    else:
        w = I.mxfp6_workload("mxfp6_span", M, N, K, seed=32, kind="e2m3", exact=True)
        per_row = K // 4 * 3
    a_rows = np.ascontiguousarray(w.a.storage).reshape(M, per_row)
    buf = torch.empty((M, row_bytes), dtype=torch.uint8, device="cuda")
    buf[:, :per_row] = torch.from_numpy(a_rows).cuda()
    if fmt == "mxfp4":
        a = buf.view(torch.float4_e2m1fn_x2).as_strided((M, K // 2), (row_bytes, 1))
    else:
        a = api.PackedTensor(buf.view(-1), api.SL_F6_E2M3, (M, K), (row_bytes // 3 * 4, 1))
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    api.gemm(a, I.to_device(w.b), None, out=out, sfa=I.to_device(w.sfa), sfb=I.to_device(w.sfb), block_k=32)
    torch.cuda.synchronize()
    d_ref, _, _ = h.oracle_full(w)
    assert np.array_equal(h.d_codes(out), d_ref[0])


def test_mxfp4_sampled_8192(api):
    _sampled(api, I.mxfp4_workload("mxfp4_8192", 8192, 8192, 8192, seed=7), n=1500)


# ------------------------------------------------------------------ MXFP6

MXFP6_EXACT = [
    # M, N, K, batch, with_c, format
    (256, 256, 512, None, False, "e2m3"),
    (256, 256, 512, None, False, "e3m2"),
    (300, 264, 1024, None, True, "e2m3"),
    (136, 72, 512, 2, True, "e3m2"),
    (520, 300, 2048, None, False, "e2m3"),
    (520, 300, 2048, None, False, "e3m2"),
]


@pytest.mark.parametrize("case", MXFP6_EXACT, ids=lambda c: "x".join(map(str, c[:3])) + f"_b{c[3]}_c{int(c[4])}_{c[5]}")
def test_mxfp6_exact_parity(api, case):
    """Packed 6-bit data (values {0, +-1, +-1.5, +-2, +-3, +-4, +-6}) with
    E8M0 scales 2^[-1,1]: every product and partial sum is exact in fp32,
    so D must equal the oracle bit for bit."""
    h = H()
    M, N, K, batch, with_c, kind = case
    w = I.mxfp6_workload("mxfp6_exact", M, N, K, seed=M + K + 2, kind=kind, batch=batch, with_c=with_c, exact=True)
    plan = _plan(api, w)
    h.log(f"mxfp6 exact {case} plan={plan}")
    assert plan["kernel"] == api.K_MXFP6
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    mism = np.count_nonzero(d.reshape(d_ref.shape) != d_ref)
    assert mism == 0, f"{mism} elements differ"


@pytest.mark.parametrize("kind", ["e2m3", "e3m2"])
def test_mxfp6_bounded(api, kind):
    """All 64 codes, scale exponents [-4, 0], ragged M and N: within the
    acceptance bound everywhere."""
    h = H()
    w = I.mxfp6_workload("mxfp6_bounded", 390, 200, 1024, seed=31, kind=kind, with_c=True)
    h.log(f"mxfp6 bounded {kind} plan={_plan(api, w)}")
    d = h.d_codes(h.run_library(w))
    d_ref, _, absum = h.oracle_full(w)
    h.assert_within_bound(d.reshape(d_ref.shape), d_ref, absum, w.name)


def test_mxfp6_sampled_8192(api):
    _sampled(api, I.mxfp6_workload("mxfp6_8192", 8192, 8192, 8192, seed=8), n=1500)
