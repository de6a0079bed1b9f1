"""The C-ABI library on the host (no GPU): it loads, exports every symbol
include/sl.h declares, validates descriptors before any HIP call, selects
loaders and tiles, and its exported layout maps equal the oracle's
bit for bit.  No compute call is made here."""

import os
import re

import numpy as np
import pytest

from oracle import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def api():
    from stride_layouts_lds_amd import api as A
    if not os.path.exists(A.LIB_PATH):
        from stride_layouts_lds_amd import build
        build.build(verbose=False)
    A.lib()
    return A


def header_functions():
    text = open(os.path.join(ROOT, "include", "sl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[\w\s\*]*?\b(sl_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(api):
    declared = header_functions()
    assert "sl_gemm" in declared and len(declared) >= 10
    assert sorted(api.EXPORTS) == declared
    for name in declared:
        assert hasattr(api.lib(), name), name


def test_abi_version_and_strings(api):
    text = open(os.path.join(ROOT, "include", "sl.h")).read()
    assert api.abi_version() == int(re.search(r"#define SL_ABI_VERSION (\d+)", text).group(1))
    for code in api.STATUS:
        assert api.status_string(code) and api.status_string(code) != "unknown status"
    assert api.status_string(12345) == "unknown status"


# ------------------------------------------------------------------ validation

F16 = 1
BASE_A, BASE_B, BASE_C, BASE_D = 0x100000000, 0x200000000, 0x300000000, 0x400000000


def rowmajor(ptr, shape, dtype=F16):
    st = [0] * len(shape)
    acc = 1
    for i in reversed(range(len(shape))):
        st[i] = acc
        acc *= shape[i]
    return ptr, dtype, shape, st


def plan(api, a, b, c=None, d=None, sfa=None, sfb=None, block_k=32):
    D = lambda x: api.desc(*x) if x is not None else None
    return api.sl_gemm_plan(api.make_args(D(a), D(b), D(c), D(d), D(sfa), D(sfb), block_k))


def err(api, *args, **kw):
    with pytest.raises(api.SLError) as e:
        plan(api, *args, **kw)
    return e.value.name


def test_plan_tn_square(api):
    p = plan(api, rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (8192, 8192)), None,
             rowmajor(BASE_D, (8192, 8192)))
    assert p["kernel"] == api.K_F16 and p["a_load"] == 0 and p["b_load"] == 0
    assert (p["tile_m"], p["tile_n"], p["tile_k"]) == (256, 256, 64)
    assert p["workgroups"] == 32 * 32


def test_plan_transposed_views_select_loaders(api):
    nb, M, N, K = 64, 512, 512, 512
    a_mn = (BASE_A, F16, (nb, M, K), (M * K, 1, M))          # M contiguous (stride-swapped view)
    b_k = (BASE_B, F16, (nb, N, K), (N * K, K, 1))           # K contiguous
    b_n = (BASE_B, F16, (nb, N, K), (N * K, 1, N))           # N contiguous
    d = (BASE_D, F16, (nb, M, N), (M * N, N, 1))
    # the 8-wave 256x256 tile copies M- (N-) contiguous operands straight
    # into an M-major LDS tile (loader 3)
    p = plan(api, a_mn, b_k, None, d)
    assert (p["a_load"], p["b_load"]) == (3, 0) and p["batch"] == nb and p["tile_m"] == 256
    p = plan(api, a_mn, b_n, None, d)
    assert (p["a_load"], p["b_load"]) == (3, 3)
    # other tiles keep the register-transposing loader (loader 1)
    os.environ["SL_TILE"] = "0"
    try:
        p = plan(api, a_mn, b_n, None, d)
    finally:
        del os.environ["SL_TILE"]
    assert (p["a_load"], p["b_load"]) == (1, 1)
    # an odd stride or a misaligned base goes to the element loader
    odd = (BASE_A, F16, (M, K), (K + 1, 1))
    p = plan(api, odd, rowmajor(BASE_B, (N, K)), None, rowmajor(BASE_D, (M, N)))
    assert p["kernel"] == api.K_F16_GENERIC and p["a_load"] == 2
    mis = (BASE_A + 2, F16, (M, K), (K, 1))
    p = plan(api, mis, rowmajor(BASE_B, (N, K)), None, rowmajor(BASE_D, (M, N)))
    assert p["a_load"] == 2


def test_validation_errors(api):
    A = rowmajor(BASE_A, (64, 32))
    B = rowmajor(BASE_B, (48, 32))
    Dd = rowmajor(BASE_D, (64, 48))
    assert err(api, (BASE_A, 2, (64, 32), (32, 1)), B, None, Dd) == "SL_ERR_DTYPE"
    assert err(api, A, rowmajor(BASE_B, (48, 31)), None, Dd) == "SL_ERR_SHAPE"
    assert err(api, A, B, None, rowmajor(BASE_D, (64, 47))) == "SL_ERR_SHAPE"
    assert err(api, A, B, rowmajor(BASE_C, (63, 48)), Dd) == "SL_ERR_SHAPE"
    assert err(api, (BASE_A, F16, (64, 32), (-32, 1)), B, None, Dd) == "SL_ERR_LAYOUT"
    assert err(api, (BASE_A, F16, (64, 32), (32, 1)), B, None, (BASE_D, F16, (64, 48), (0, 1))) == "SL_ERR_LAYOUT"
    assert err(api, (BASE_A + 1, F16, (64, 32), (32, 1)), B, None, Dd) == "SL_ERR_ALIGN"
    assert err(api, (0, F16, (64, 32), (32, 1)), B, None, Dd) == "SL_ERR_NULL"
    # D overlapping an input
    assert err(api, A, B, None, (BASE_A + 64, F16, (64, 48), (48, 1))) == "SL_ERR_ALIAS"
    # C == D in place is allowed; C overlapping D otherwise is not
    plan(api, A, B, Dd, Dd)
    assert err(api, A, B, (BASE_D + 2, F16, (64, 48), (48, 1)), Dd) == "SL_ERR_ALIAS"
    # batch mismatch
    assert err(api, rowmajor(BASE_A, (3, 64, 32)), B, None, rowmajor(BASE_D, (2, 64, 48))) == "SL_ERR_SHAPE"
    # rank
    with pytest.raises(api.SLError):
        api.sl_gemm_plan(api.make_args(api.desc(BASE_A, F16, (1, 1, 64, 32)[:3], (1, 32, 1)),
                                       api.desc(*B), None, api.desc(*Dd)))


def test_degenerate_sizes_are_noops(api):
    p = plan(api, rowmajor(BASE_A, (0, 32)), rowmajor(BASE_B, (48, 32)), None, rowmajor(BASE_D, (0, 48)))
    assert p["m"] == 0 and p["workgroups"] == 0
    # K = 0: D = C, still a launch (A and B may be NULL)
    p = plan(api, (0, F16, (64, 0), (0, 1)), (0, F16, (48, 0), (0, 1)), rowmajor(BASE_C, (64, 48)),
             rowmajor(BASE_D, (64, 48)))
    assert p["k"] == 0 and p["workgroups"] > 0


def test_broadcast_inputs_allowed(api):
    # one B for every batch (batch stride 0), and a zero row stride on A
    p = plan(api, rowmajor(BASE_A, (4, 64, 32)), (BASE_B, F16, (4, 48, 32), (0, 32, 1)), None,
             rowmajor(BASE_D, (4, 64, 48)))
    assert p["batch"] == 4
    plan(api, (BASE_A, F16, (64, 32), (0, 1)), rowmajor(BASE_B, (48, 32)), None, rowmajor(BASE_D, (64, 48)))


def test_mx_validation(api):
    E4, E8 = 3, 4
    M = N = K = 256
    a = (BASE_A, E4, (M, K), (K, 1))
    b = (BASE_B, E4, (N, K), (K, 1))
    sa = (BASE_C, E8, (M, K // 32), (K // 32, 1))
    sb = (BASE_C + 0x10000, E8, (N, K // 32), (K // 32, 1))
    d = rowmajor(BASE_D, (M, N))
    p = plan(api, a, b, None, d, sa, sb)
    assert p["kernel"] in (api.K_MX, api.K_MX_W8) and p["tile_k"] == 128
    # a full-chip problem takes the 8-wave kernel when the scale rows are
    # whole dwords, the 4-wave byte-load kernel otherwise
    M4 = N4 = 4096
    a4, b4 = (BASE_A, E4, (M4, K), (K, 1)), (BASE_B, E4, (N4, K), (K, 1))
    s4a, s4b = (BASE_C, E8, (M4, K // 32), (K // 32, 1)), (BASE_C + 0x100000, E8, (N4, K // 32), (K // 32, 1))
    d4 = rowmajor(BASE_D, (M4, N4))
    p = plan(api, a4, b4, None, d4, s4a, s4b)
    assert p["kernel"] == api.K_MX_W8 and p["threads"] == 512 and p["tile_m"] == p["tile_n"] == 256
    assert p["lds_bytes"] == 2 * (256 + 256) * (128 + 4)
    s9 = (BASE_C, E8, (M4, K // 32), (9, 1))
    assert plan(api, a4, b4, None, d4, s9, s4b)["kernel"] == api.K_MX
    K2 = 208  # 7 scale blocks per row
    a2, b2 = (BASE_A, E4, (M4, K2), (224, 1)), (BASE_B, E4, (N4, K2), (224, 1))
    s2a, s2b = (BASE_C, E8, (M4, 8), (8, 1)), (BASE_C + 0x100000, E8, (N4, 8), (8, 1))
    assert plan(api, a2, b2, None, d4, s2a[:2] + ((M4, 7), (8, 1)), s2b[:2] + ((N4, 7), (8, 1)))["kernel"] == api.K_MX
    assert err(api, a, b, None, d, sa, sb, block_k=16) == "SL_ERR_SHAPE"
    assert err(api, a, b, None, d, sa, (BASE_C + 0x10000, E8, (N, 7), (7, 1))) == "SL_ERR_SHAPE"
    assert err(api, a, b, None, d, None, None) == "SL_ERR_DTYPE"
    assert err(api, (BASE_A, E4, (M, K), (1, M)), b, None, d, sa, sb) == "SL_ERR_LAYOUT"


# ------------------------------------------------------------------ maps

@pytest.mark.parametrize("instr", [0, 1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("operand", [0, 1, 2])
def test_fragment_maps_equal_oracle(api, instr, operand):
    got = api.query_fragment_map(instr, operand)
    tv = L.INSTR_MAPS[instr][operand]
    want = np.array(tv.table(), np.int32)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("instr", [2, 3])
def test_scale_map_equal_oracle(api, instr):
    got = api.query_fragment_map(instr, 3)
    rows = 16 if instr == 2 else 32
    want = np.array([(l, 0) + L.mfma_scale_owner(rows, l) for l in range(64)], np.int32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("variant", [1, 2, 3, 4])
def test_lds_map_is_the_xor_swizzle(api, variant):
    offs, es = api.query_lds_map(variant, 0)
    rows, cols = offs.shape
    assert rows * cols * es == rows * 128
    # a bijection onto the tile's bytes (element granularity)
    assert sorted((offs // es).ravel().tolist()) == list(range(rows * cols))
    # equal to Swizzle<3, 4, 3 + shift> of the row-major byte offset (the
    # byte form of the pages' Swizzle<3,3,3> on fp16 elements) with
    # Swizzle<1, 4, 7 + shift> composed on top (chunk bit 0 ^= row bit 4)
    shift = int(os.environ.get("SL_SWZ", "0") or 0) and 1
    for r in range(rows):
        for k in range(cols):
            x = L.swizzle_bms(r * 128 + k * es, 3, 4, 3 + shift)
            assert offs[r, k] == L.swizzle_bms(x, 1, 4, 7 + shift)


@pytest.mark.parametrize("variant,instr", [(1, 0), (3, 2), (4, 3)])
def test_fragment_addresses_compose_maps(api, variant, instr):
    got = api.query_fragment_addresses(variant, 0)
    tv = L.INSTR_MAPS[instr][0]
    es = 2 if instr < 2 else 1
    shift = int(os.environ.get("SL_SWZ", "0") or 0) and 1
    want = [L.swizzle_bms(L.swizzle_bms(r * 128 + c * es, 3, 4, 3 + shift), 1, 4, 7 + shift)
            for _, _, r, c in tv.table()]
    assert got.tolist() == want


def test_fragment_reads_conflict_free_under_the_page_bank_model(api):
    """Under the data-layout page's bank model (32 banks x 4 B, 16-byte
    accesses served 8 lanes per pass) every ds_read_b128 of a fragment load
    takes the minimum 8 passes with the default swizzle, and 8x that
    without it.  On gfx950 the hardware counter decides."""
    addrs = api.query_fragment_addresses(1, 0).reshape(64, 8)[:, 0]
    assert L.bank_conflict_passes(addrs.tolist(), 16, 32, 4, 8) == 8
    plain = [r * 128 + c * 2 for _, v, r, c in L.MFMA16_F16_A.table() if v == 0]
    assert L.bank_conflict_passes(plain, 16, 32, 4, 8) == 64


def _gfx950_b128_passes(addrs):
    """Cycles of one ds_read_b128 under the gfx950 behaviour the LDS
    conflict counter shows: 64 banks of 4 bytes, one pass per lane set
    {0-7, 16-23}, {8-15, 24-31}, {32-39, 48-55}, {40-47, 56-63}, a pass
    taking as many cycles as the most distinct dwords on one bank."""
    total = 0
    for g in range(4):
        base = 32 * (g // 2) + 8 * (g % 2)
        lanes = list(range(base, base + 8)) + list(range(base + 16, base + 24))
        banks = {}
        for l in lanes:
            for w in range(4):
                dw = addrs[l] // 4 + w
                banks.setdefault(dw % 64, set()).add(dw)
        total += max(len(v) for v in banks.values())
    return total


@pytest.mark.parametrize("variant,slots_per_piece", [(1, 8), (3, 16), (4, 16)])
def test_fragment_reads_conflict_free_on_gfx950(api, variant, slots_per_piece):
    """The 16-byte fragment reads of each kernel variant (MFMA tile 0,
    k-slice 0, both pieces of an f8 fragment) take the minimum 4 passes,
    where the plain SWIZZLE_128B rule takes 8 for the 32-row instruction."""
    addr = api.query_fragment_addresses(variant, 0)
    per_lane = addr.reshape(64, -1)
    pieces = per_lane.shape[1] // slots_per_piece
    for piece in range(pieces):
        base = per_lane[:, piece * slots_per_piece]
        assert _gfx950_b128_passes(base.tolist()) == 4, (variant, piece)
    # the plain rule on the 32-row f8 instruction: rows r and r + 16 collide
    plain = [L.swizzle_bms(r * 128 + c, 3, 4, 3) for _, v, r, c in L.MFMA32_F8_A.table() if v == 0]
    assert _gfx950_b128_passes(plain) == 8


def _gfx950_b64_passes(addrs):
    """Cycles of one ds_read_b64 under the behaviour measured on gfx950: 64
    banks of 4 bytes, one pass per 32 lanes (0-31, 32-63), a pass taking as
    many cycles as the most distinct dwords on one bank."""
    total = 0
    for base in (0, 32):
        banks = {}
        for l in range(base, base + 32):
            for w in range(2):
                dw = addrs[l] // 4 + w
                banks.setdefault(dw % 64, set()).add(dw)
        total += max(len(v) for v in banks.values())
    return total


def test_mxfp6_packed_rows_on_gfx950():
    """The 4-wave MX kernel's packed 6-bit K-tiles: a row's 96 bytes are 6
    chunks of 16 bytes, rows 96 bytes apart, chunk c of row r at chunk
    (c + (r >> 4) & 1) mod 6.  Lane half h = lane / 32 takes blocks 2h
    (k-slice 0: a 16-byte read of chunk 3h and an 8-byte read of the low
    half of chunk 3h + 1) and 2h + 1 (slice 1: the high half of chunk 3h + 1
    and chunk 3h + 2).  The 16-byte reads take the minimum passes on every
    32-row block; the 8-byte reads take two (every lane of a 32-lane pass
    reads the same half of a chunk, so only half the banks are reachable),
    which the loader accepts for a quarter fewer copies than 128-byte rows.
    The copy (64 consecutive chunks per instruction) puts every byte of the
    K-tile exactly once where these reads find it."""
    def pos(r, c):
        return 96 * r + 16 * ((c + ((r >> 4) & 1)) % 6)

    for slot in (0, 32768):
        for row0 in range(0, 256, 32):
            rows = [row0 + (l & 31) for l in range(64)]
            h = [l >> 5 for l in range(64)]
            b128_0 = [slot + pos(rows[l], 3 * h[l]) for l in range(64)]
            b64_0 = [slot + pos(rows[l], 3 * h[l] + 1) for l in range(64)]
            b64_1 = [slot + pos(rows[l], 3 * h[l] + 1) + 8 for l in range(64)]
            b128_1 = [slot + pos(rows[l], 3 * h[l] + 2) for l in range(64)]
            assert _gfx950_b128_passes(b128_0) == 4 and _gfx950_b128_passes(b128_1) == 4, (slot, row0)
            assert _gfx950_b64_passes(b64_0) == 4 and _gfx950_b64_passes(b64_1) == 4, (slot, row0)
    # the copy: chunk g = 64 instruction + lane of the tile is physical chunk
    # g % 6 of row g / 6 and holds the row's chunk (g % 6 - (row >> 4) & 1) mod 6
    lds = {}
    for g in range(256 * 6):
        r, p = divmod(g, 6)
        c = (p - ((r >> 4) & 1)) % 6
        for x in range(16):
            assert 16 * g + x not in lds
            lds[16 * g + x] = (r, 16 * c + x)
    assert len(lds) == 256 * 96
    for r in range(256):
        for h in range(2):
            blk0 = [lds[pos(r, 3 * h) + x] for x in range(16)] + [lds[pos(r, 3 * h + 1) + x] for x in range(8)]
            blk1 = [lds[pos(r, 3 * h + 1) + 8 + x] for x in range(8)] + [lds[pos(r, 3 * h + 2) + x] for x in range(16)]
            assert blk0 == [(r, 48 * h + x) for x in range(24)], (r, h)
            assert blk1 == [(r, 48 * h + 24 + x) for x in range(24)], (r, h)


def test_plan_split_k_for_skinny_outputs(api):
    """An 8192 x 128 x 8192 output fills 64 tiles of 128 x 128: the planner
    splits K four ways (256 workgroups); a square 4096^3 is not split."""
    p = plan(api, rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (128, 8192)), None, rowmajor(BASE_D, (8192, 128)))
    assert (p["split_k"], p["tile_m"], p["tile_n"], p["workgroups"]) == (4, 128, 128, 256)
    p = plan(api, rowmajor(BASE_A, (4096, 4096)), rowmajor(BASE_B, (4096, 4096)), None, rowmajor(BASE_D, (4096, 4096)))
    assert p["split_k"] == 1
    # short K: no split (fewer than 4 K-tiles of 64 per split)
    p = plan(api, rowmajor(BASE_A, (256, 256)), rowmajor(BASE_B, (256, 256)), None, rowmajor(BASE_D, (256, 256)))
    assert p["split_k"] == 1


def test_planner_environment_overrides(api, monkeypatch):
    """The environment overrides sl.h lists change the plan as stated, and a
    value a shape cannot use leaves the planner's own choice (SL_GROUP_M
    changes only the tile order inside the kernels, which the plan does not
    report)."""
    sq = (rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (8192, 8192)), None, rowmajor(BASE_D, (8192, 8192)))
    base = plan(api, *sq)
    assert base["threads"] == 256 and base["lds_bytes"] == 5 * 32768  # the 4-wave ring kernel
    monkeypatch.setenv("SL_TILE", "4")
    p = plan(api, *sq)
    assert p["threads"] == 512 and (p["tile_m"], p["tile_n"]) == (256, 256)
    monkeypatch.setenv("SL_TILE", "99")
    assert plan(api, *sq) == base
    monkeypatch.delenv("SL_TILE")

    sk = (rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (128, 8192)), None, rowmajor(BASE_D, (8192, 128)))
    monkeypatch.setenv("SL_SPLITK", "2")
    p = plan(api, *sk)
    assert p["split_k"] == 2 and p["workspace_bytes"] == 2 * 8192 * 128 * 4
    monkeypatch.delenv("SL_SPLITK")

    # MXFP8 with 16 scale blocks per row: the ring kernel, or without
    # 16-byte scale chunks the 8-wave one
    E4, E8, M, K = 3, 4, 4096, 512
    mx = ((BASE_A, E4, (M, K), (K, 1)), (BASE_B, E4, (M, K), (K, 1)), None, rowmajor(BASE_D, (M, M)),
          (BASE_C, E8, (M, K // 32), (K // 32, 1)), (BASE_C + 0x100000, E8, (M, K // 32), (K // 32, 1)))
    assert plan(api, *mx)["kernel"] == api.K_MX_W4R
    monkeypatch.setenv("SL_SCALE16", "0")
    assert plan(api, *mx)["kernel"] == api.K_MX_W8
    monkeypatch.delenv("SL_SCALE16")

    # NVFP4: the paired loader (5), or one K-tile per fetch (4)
    E2, N, K = 6, 256, 1024
    nv = ((BASE_A, E2, (512, K), (K, 1)), (BASE_B, E2, (N, K), (K, 1)), None, rowmajor(BASE_D, (512, N)),
          (BASE_C, E4, (512, K // 16), (K // 16, 1)), (BASE_C + 0x100000, E4, (N, K // 16), (K // 16, 1)))
    assert (plan(api, *nv, block_k=16)["a_load"]) == 5
    monkeypatch.setenv("SL_NV_PAIRS", "0")
    assert (plan(api, *nv, block_k=16)["a_load"]) == 4
    monkeypatch.delenv("SL_NV_PAIRS")

    # M- and N-contiguous operands of the 8-wave kernel: direct copies (3),
    # or the register-transposing loader (1)
    nb, M, N, K = 64, 512, 512, 512
    mn = ((BASE_A, F16, (nb, M, K), (M * K, 1, M)), (BASE_B, F16, (nb, N, K), (N * K, 1, N)), None,
          (BASE_D, F16, (nb, M, N), (M * N, N, 1)))
    assert (plan(api, *mn)["a_load"], plan(api, *mn)["b_load"]) == (3, 3)
    monkeypatch.setenv("SL_MN_LOADER", "1")
    assert (plan(api, *mn)["a_load"], plan(api, *mn)["b_load"]) == (1, 1)
    monkeypatch.delenv("SL_MN_LOADER")

    # NVFP4 decoded ahead (a_load 0, a workspace) when forced, else fused
    monkeypatch.setenv("SL_NV_DECODE", "1")
    p = plan(api, *nv, block_k=16)
    assert p["a_load"] == 0 and p["workspace_bytes"] == 512 * 1024 * 2 + 256 * 1024 * 2


def test_split_k_workspace_is_the_callers(api):
    """A split-K plan needs a caller workspace of splits * batch * M * N fp32:
    the plan and sl_gemm_workspace_bytes report its size, and sl_gemm
    rejects a missing, short, misaligned or overlapping one before any HIP
    call (so these run without a GPU).  Unsplit plans need none."""
    a, b, d = rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (128, 8192)), rowmajor(BASE_D, (8192, 128))
    args = api.make_args(api.desc(*a), api.desc(*b), None, api.desc(*d))
    need = 4 * 8192 * 128 * 4
    assert api.sl_gemm_workspace_bytes(args) == need
    assert api.sl_gemm_plan(args)["workspace_bytes"] == need

    def status(ws, nbytes):
        args.workspace, args.workspace_bytes = ws, nbytes
        with pytest.raises(api.SLError) as e:
            api.sl_gemm(args, 0)
        return e.value.name

    free = 0x500000000
    assert status(None, 0) == "SL_ERR_NULL"
    assert status(None, need) == "SL_ERR_NULL"
    assert status(free, need - 1) == "SL_ERR_SHAPE"
    assert status(free, -1) == "SL_ERR_SHAPE"
    assert status(free + 8, need) == "SL_ERR_ALIGN"
    assert status(BASE_D - 16, need) == "SL_ERR_ALIAS"      # runs into D
    assert status(BASE_A + 4096, need) == "SL_ERR_ALIAS"    # inside A
    assert status(BASE_B - need + 16, need) == "SL_ERR_ALIAS"
    sq = api.make_args(api.desc(*rowmajor(BASE_A, (4096, 4096))), api.desc(*rowmajor(BASE_B, (4096, 4096))), None,
                       api.desc(*rowmajor(BASE_D, (4096, 4096))))
    assert api.sl_gemm_workspace_bytes(sq) == 0 and api.sl_gemm_plan(sq)["workspace_bytes"] == 0
    empty = api.make_args(api.desc(*rowmajor(BASE_A, (0, 64))), api.desc(*rowmajor(BASE_B, (128, 64))), None,
                          api.desc(*rowmajor(BASE_D, (0, 128))))
    assert api.sl_gemm_workspace_bytes(empty) == 0
    assert api.lib().sl_gemm_workspace_bytes(None, None) == -1  # SL_ERR_NULL


def test_no_alloc_rejects_plans_beyond_its_scratch(api, monkeypatch):
    """sl_gemm_no_alloc serves a split-K plan from a static scratch of
    SL_NO_ALLOC_SCRATCH_BYTES: a plan needing more returns SL_ERR_SHAPE
    before any HIP call (so this runs without a GPU), whatever workspace
    the arguments carry; the header and the binding state one size."""
    text = open(os.path.join(ROOT, "include", "sl.h")).read()
    assert api.SL_NO_ALLOC_SCRATCH_BYTES == eval(
        re.search(r"#define SL_NO_ALLOC_SCRATCH_BYTES \((\d+)LL << (\d+)\)", text).expand(r"\1 << \2"))
    monkeypatch.setenv("SL_TILE", "16")
    monkeypatch.setenv("SL_SPLITK", "8")
    M, N, K = 1024, 1152, 8192
    args = api.make_args(api.desc(*rowmajor(BASE_A, (M, K))), api.desc(*rowmajor(BASE_B, (N, K))), None,
                         api.desc(*rowmajor(BASE_D, (M, N))))
    need = api.sl_gemm_workspace_bytes(args)
    assert need == 8 * M * N * 4 > api.SL_NO_ALLOC_SCRATCH_BYTES
    args.workspace, args.workspace_bytes = 0x500000000, need
    with pytest.raises(api.SLError) as e:
        api.sl_gemm_no_alloc(args, 0)
    assert e.value.name == "SL_ERR_SHAPE" and "static scratch" in str(e.value)


def test_m_major_tile_is_a_chunk_swizzle(api):
    """The M-major LDS tile (operands copied with M contiguous): a bijection
    onto 256 x 64 halves in which every 16-byte chunk holds 8 consecutive
    rows of one K-row (what one 16-byte direct copy moves)."""
    offs, es = api.query_lds_map(5, 0)
    assert offs.shape == (256, 64) and es == 2
    assert sorted((offs // 2).ravel().tolist()) == list(range(256 * 64))
    for k in range(64):
        for c in range(32):
            col = offs[8 * c:8 * c + 8, k]
            assert col[0] % 16 == 0 and np.array_equal(col - col[0], np.arange(8) * 2)
            assert col[0] // 512 == k  # K-row k occupies bytes [512 k, 512 k + 512)


def test_m_major_fragment_by_transposing_reads(api):
    """Fill an LDS image through the M-major tile map, apply the transposing
    read (its lane semantics as pinned on the device) to the addresses each
    lane supplies, and check that every lane receives exactly its MFMA
    16x16x32 fragment: (row l % 16, k 8 (l / 16) + v)."""
    offs, _ = api.query_lds_map(5, 0)
    code = lambda r, k: (r * 64 + k) & 0xFFFF
    lds = np.zeros(256 * 64, np.int64)
    for r in range(256):
        for k in range(64):
            lds[offs[r, k] // 2] = code(r, k)
    addr = api.query_fragment_addresses(5, 0).reshape(64, 2)
    got = [[], []]
    for rd in range(2):
        got[rd] = L.ds_read_tr16_b64_expected(addr[:, rd].tolist(), lds.tolist())
    want = {(l, v): code(r, c) for l, v, r, c in L.MFMA16_F16_A.table()}
    for l in range(64):
        frag = got[0][l] + got[1][l]
        assert frag == [want[(l, v)] for v in range(8)], l


def test_bf16_dtypes(api):
    """bf16 operands take bf16 C and D; mixing 16-bit formats is rejected."""
    BF = 5
    A = (BASE_A, BF, (64, 32), (32, 1))
    B = (BASE_B, BF, (48, 32), (32, 1))
    Dbf = (BASE_D, BF, (64, 48), (48, 1))
    p = plan(api, A, B, (BASE_C, BF, (64, 48), (48, 1)), Dbf)
    assert p["kernel"] == api.K_F16
    assert err(api, A, B, None, rowmajor(BASE_D, (64, 48))) == "SL_ERR_DTYPE"      # f16 D
    assert err(api, A, rowmajor(BASE_B, (48, 32)), None, Dbf) == "SL_ERR_DTYPE"    # f16 B
    assert err(api, A, B, rowmajor(BASE_C, (64, 48)), Dbf) == "SL_ERR_DTYPE"       # f16 C
    # ping-pong tiles are fp16 only: a bf16 plan asked for one falls back to the planner's choice
    os.environ["SL_TILE"] = "9"
    try:
        p = plan(api, (BASE_A, BF, (4096, 4096), (4096, 1)), (BASE_B, BF, (4096, 4096), (4096, 1)), None,
                 (BASE_D, BF, (4096, 4096), (4096, 1)))
    finally:
        del os.environ["SL_TILE"]
    assert p["tile_m"] == 256 and p["threads"] == 256 and p["lds_bytes"] == 5 * 256 * 128


def test_ring_tile_choice(api):
    """fp16 and bf16 outputs with K-contiguous operands that fill the chip
    take the 4-wave ring kernels (tile 19, 256x256; tile 20, 256x192; 256
    threads, five 32 KiB operand K-tiles); K = 0 and an explicit other tile
    do not; M/N-contiguous operands take it only when asked for tile 19."""
    big = [rowmajor(BASE_A, (8192, 8192)), rowmajor(BASE_B, (8192, 8192)), rowmajor(BASE_C, (8192, 8192)),
           rowmajor(BASE_D, (8192, 8192))]
    p = plan(api, *big)
    assert (p["tile_m"], p["tile_n"], p["threads"], p["lds_bytes"]) == (256, 256, 256, 163840)
    # K = 0: the ring kernel runs at least one K-tile, so the 8-wave kernel does it
    k0 = plan(api, rowmajor(BASE_A, (4096, 0)), rowmajor(BASE_B, (4096, 0)), rowmajor(BASE_C, (4096, 4096)),
              rowmajor(BASE_D, (4096, 4096)))
    assert k0["threads"] == 512
    # M- or N-contiguous operands: the 8-wave kernel with direct M-major
    # copies, or the ring kernel with them when asked for tile 19
    a_mn = (BASE_A, F16, (8192, 8192), (1, 8192))
    p = plan(api, a_mn, big[1], None, big[3])
    assert p["threads"] == 512 and p["a_load"] == 3
    os.environ["SL_TILE"] = "19"
    try:
        p = plan(api, a_mn, big[1], None, big[3])
    finally:
        del os.environ["SL_TILE"]
    assert p["threads"] == 256 and p["a_load"] == 3 and p["lds_bytes"] == 163840
    # a ragged output that 256x192 tiles fill better: the 256x192 ring kernel
    r = plan(api, rowmajor(BASE_A, (4000, 2056)), rowmajor(BASE_B, (3000, 2056)), None, rowmajor(BASE_D, (4000, 3000)))
    assert (r["tile_m"], r["tile_n"], r["threads"], r["lds_bytes"]) == (256, 192, 256, 163840)
    for tile, threads in (("4", 512), ("19", 256)):
        os.environ["SL_TILE"] = tile
        try:
            p = plan(api, *big)
            k0 = plan(api, rowmajor(BASE_A, (4096, 0)), rowmajor(BASE_B, (4096, 0)), None,
                      rowmajor(BASE_D, (4096, 4096)))
        finally:
            del os.environ["SL_TILE"]
        assert p["threads"] == threads and k0["threads"] == 512
    text = api.describe_plan(api.make_args(*(api.desc(*x) for x in big), None, None, 32))
    assert "ring of five operand K-tiles" in text and "163840 LDS bytes" in text


def test_nvfp4_plan_and_validation(api):
    """NVFP4: packed E2M1 operands with E4M3 scales per 16 K go to the
    dequantising 8-wave kernel (E8M0 scales per 32 make it MXFP4); other
    scale pairings and packed layouts the loader cannot take are rejected."""
    E2, E4, E8 = 6, 3, 4
    M, N, K = 512, 256, 1024
    a = (BASE_A, E2, (M, K), (K, 1))
    b = (BASE_B, E2, (N, K), (K, 1))
    sa = (BASE_C, E4, (M, K // 16), (K // 16, 1))
    sb = (BASE_C + 0x100000, E4, (N, K // 16), (K // 16, 1))
    d = rowmajor(BASE_D, (M, N))
    p = plan(api, a, b, None, d, sa, sb, block_k=16)
    # scale rows K-contiguous on 8-byte boundaries: the paired loader (5)
    assert p["kernel"] == api.K_NVFP4 and (p["a_load"], p["b_load"]) == (5, 5)
    assert p["tile_m"] == p["tile_n"] == 256 and p["tile_k"] == 64 and p["lds_bytes"] == 2 * 512 * 64 * 2
    # scale rows padded to an odd length, or column-major scales: the per-tile loader (4)
    sa_odd = (BASE_C, E4, (M, K // 16), (K // 16 + 1, 1))
    assert plan(api, a, b, None, d, sa_odd, sb, block_k=16)["a_load"] == 4
    sa_cm = (BASE_C, E4, (M, K // 16), (1, M))
    assert plan(api, a, b, None, d, sa_cm, sb, block_k=16)["a_load"] == 4
    s8a = (BASE_C, E8, (M, K // 32), (K // 32, 1))
    s8b = (BASE_C + 0x100000, E8, (N, K // 32), (K // 32, 1))
    assert plan(api, a, b, None, d, s8a, s8b, block_k=32)["kernel"] == api.K_MXFP4
    assert err(api, a, b, None, d, s8a, s8b, block_k=16) == "SL_ERR_DTYPE"
    assert err(api, a, b, None, d, sa, sb, block_k=32) == "SL_ERR_DTYPE"
    assert err(api, a, b, None, d, sa, s8b, block_k=16) == "SL_ERR_DTYPE"
    # K % 32 != 0, an N-contiguous B, a row stride that is not a multiple of 32
    K2 = 1008
    assert err(api, (BASE_A, E2, (M, K2), (K2, 1)), (BASE_B, E2, (N, K2), (K2, 1)), None, d,
               (BASE_C, E4, (M, K2 // 16), (K2 // 16, 1)), (BASE_C + 0x100000, E4, (N, K2 // 16), (K2 // 16, 1)),
               block_k=16) == "SL_ERR_LAYOUT"
    assert err(api, a, (BASE_B, E2, (N, K), (1, N)), None, d, sa, sb, block_k=16) == "SL_ERR_LAYOUT"
    assert err(api, (BASE_A, E2, (M, K), (K + 16, 1)), b, None, d, sa, sb, block_k=16) == "SL_ERR_LAYOUT"


def test_nvfp4_large_products_decode_ahead(api, monkeypatch):
    """From 2048^3 on, NVFP4 operands are decoded to fp16 rows in the
    caller's workspace (A, then B from the next 256-byte boundary) and the
    fp16 ring kernel runs on them; SL_NV_DECODE=0, an SL_TILE choice, or K
    not a multiple of 64 keep the fused kernels, and a missing workspace is
    an error before any HIP call."""
    E2, E4 = 6, 3

    def nv(M, N, K, batch=None):
        sh = lambda r, c: (r, c) if batch is None else (batch, r, c)
        st = lambda r, c: (c, 1) if batch is None else (r * c, c, 1)
        return ((BASE_A, E2, sh(M, K), st(M, K)), (BASE_B, E2, sh(N, K), st(N, K)), None,
                (BASE_D, F16, sh(M, N), st(M, N)),
                (BASE_C, E4, sh(M, K // 16), st(M, K // 16)),
                (BASE_C + 0x40000000, E4, sh(N, K // 16), st(N, K // 16)))

    big = nv(8192, 8192, 8192)
    p = plan(api, *big, block_k=16)
    assert p["kernel"] == api.K_NVFP4 and (p["a_load"], p["b_load"]) == (0, 0)
    assert (p["threads"], p["lds_bytes"], p["workgroups"]) == (256, 5 * 32768, 1024)
    assert p["workspace_bytes"] == 2 * 8192 * 8192 * 2
    p = plan(api, *nv(2048, 2048, 2048), block_k=16)
    assert p["a_load"] == 0 and p["workspace_bytes"] == 2 * 2048 * 2048 * 2
    p = plan(api, *nv(2048, 2048, 1024), block_k=16)   # below 2^33 multiply-adds
    assert p["a_load"] == 5 and p["workspace_bytes"] == 0
    p = plan(api, *nv(300, 264, 512, batch=256), block_k=16)   # the batch counts: 2^33.2
    assert p["a_load"] == 0 and p["workspace_bytes"] == (256 * 300 * 512 * 2 + 255) // 256 * 256 + 256 * 264 * 512 * 2
    p = plan(api, *nv(4096, 4096, 4128), block_k=16)   # K % 64 != 0 (258-byte scale rows: loader 4)
    assert p["a_load"] == 4 and p["workspace_bytes"] == 0
    monkeypatch.setenv("SL_TILE", "19")
    assert plan(api, *big, block_k=16)["a_load"] == 5
    monkeypatch.delenv("SL_TILE")
    monkeypatch.setenv("SL_NV_DECODE", "0")
    assert plan(api, *big, block_k=16)["workspace_bytes"] == 0
    monkeypatch.delenv("SL_NV_DECODE")
    D = lambda x: api.desc(*x) if x is not None else None
    args = api.make_args(*[D(x) for x in big], 16)
    assert api.sl_gemm_workspace_bytes(args) == 2 * 8192 * 8192 * 2
    with pytest.raises(api.SLError) as e:
        api.sl_gemm(args, 0)
    assert e.value.name == "SL_ERR_NULL"


def test_mxfp6_plan(api):
    """MXFP6 (packed 6-bit E2M3 or E3M2, E8M0 per 32 K) goes to the 8-wave
    scaled-MFMA kernel with 128-wide K-tiles (96 bytes per row); rows must
    be multiples of 64 elements apart, K a multiple of 512, both operands
    in one 6-bit format."""
    F6A, F6B, E8, E4 = 7, 8, 4, 3
    M, N, K = 512, 256, 1024
    a = (BASE_A, F6A, (M, K), (K, 1))
    b = (BASE_B, F6A, (N, K), (K, 1))
    sa = (BASE_C, E8, (M, K // 32), (K // 32, 1))
    sb = (BASE_C + 0x100000, E8, (N, K // 32), (K // 32, 1))
    d = rowmajor(BASE_D, (M, N))
    p = plan(api, a, b, None, d, sa, sb, block_k=32)
    assert p["kernel"] == api.K_MXFP6 and p["tile_k"] == 128 and p["threads"] == 256
    assert p["lds_bytes"] == 5 * 256 * 128  # the 4-wave ring kernel
    p2 = plan(api, (BASE_A, F6B, (M, K), (K, 1)), (BASE_B, F6B, (N, K), (K, 1)), None, d, sa, sb, block_k=32)
    assert p2["kernel"] == api.K_MXFP6
    # mixed formats, E4M3 scales, block 16
    assert err(api, a, (BASE_B, F6B, (N, K), (K, 1)), None, d, sa, sb, block_k=32) == "SL_ERR_DTYPE"
    assert err(api, a, b, None, d, (BASE_C, E4, (M, K // 32), (K // 32, 1)),
               (BASE_C + 0x100000, E4, (N, K // 32), (K // 32, 1)), block_k=32) == "SL_ERR_DTYPE"
    assert err(api, a, b, None, d, sa, sb, block_k=16) == "SL_ERR_DTYPE"
    # K % 512, a row stride not a multiple of 64, an N-contiguous B, a base off 16 bytes
    K2 = 768
    assert err(api, (BASE_A, F6A, (M, K2), (K2, 1)), (BASE_B, F6A, (N, K2), (K2, 1)), None, d,
               (BASE_C, E8, (M, K2 // 32), (K2 // 32, 1)), (BASE_C + 0x100000, E8, (N, K2 // 32), (K2 // 32, 1)),
               block_k=32) == "SL_ERR_LAYOUT"
    assert err(api, (BASE_A, F6A, (M, K), (K + 32, 1)), b, None, d, sa, sb, block_k=32) == "SL_ERR_LAYOUT"
    assert err(api, a, (BASE_B, F6A, (N, K), (1, N)), None, d, sa, sb, block_k=32) == "SL_ERR_LAYOUT"
    assert err(api, (BASE_A + 8, F6A, (M, K), (K, 1)), b, None, d, sa, sb, block_k=32) == "SL_ERR_LAYOUT"
    # an output overlapping the packed A (bytes = 3/4 of the elements)
    assert err(api, a, b, None, (BASE_A + M * K * 3 // 4 - 2, 1, (M, N), (N, 1)), sa, sb, block_k=32) == "SL_ERR_ALIAS"
    assert plan(api, a, b, None, (BASE_A + M * K * 3 // 4, 1, (M, N), (N, 1)), sa, sb, block_k=32)["kernel"] == 7


def test_size_limits(api):
    """Dimensions past 2^31 - 1 are SL_ERR_SHAPE before any HIP call.  An
    operand has no whole-span limit (every kernel addresses a tile from its
    own first row with 64-bit pointers): only a 256-row tile must span less
    than 2^31 bytes, for the vector loaders of 16-bit operands (else the
    element loader) and for packed and scale operands (else SL_ERR_SHAPE)."""
    big = 1 << 31
    assert err(api, rowmajor(BASE_A, (big, 64)), rowmajor(BASE_B, (64, 64)), None,
               (BASE_D, 1, (big, 64), (64, 1))) == "SL_ERR_SHAPE"
    assert err(api, rowmajor(BASE_A, (64, big)), rowmajor(BASE_B, (64, big)), None,
               rowmajor(BASE_D, (64, 64))) == "SL_ERR_SHAPE"
    # a 4 GiB fp16 operand plans with the vector loader
    p = plan(api, rowmajor(BASE_A, (131072, 16384)), rowmajor(BASE_B, (64, 16384)), None,
             rowmajor(BASE_D, (131072, 64)))
    assert p["a_load"] == 0
    # a row stride that puts a 256-row tile past 2^31 bytes takes the element loader
    p = plan(api, (BASE_A, 1, (512, 64), (1 << 23, 1)), rowmajor(BASE_B, (256, 64)), None,
             rowmajor(BASE_D, (512, 256)))
    assert p["a_load"] == 2
    # packed E2M1: a 2 GiB operand and its 8 MiB of scales plan
    E2, E8 = 6, 4
    M, K = 1 << 18, 16384
    sa = (BASE_C, E8, (M, K // 32), (K // 32, 1))
    sb = (0x2000000000, E8, (256, K // 32), (K // 32, 1))
    p = plan(api, (BASE_A, E2, (M, K), (K, 1)), (BASE_B, E2, (256, K), (K, 1)), None,
             rowmajor(0x1000000000, (M, 256)), sa, sb, block_k=32)
    assert p["kernel"] == api.K_MXFP4
    # ... but not rows 32 MiB apart: one 256-row tile would span 8 GiB
    rs = 1 << 26
    assert err(api, (BASE_A, E2, (512, K), (rs, 1)), (BASE_B, E2, (256, K), (K, 1)), None,
               rowmajor(0x1000000000, (512, 256)), (BASE_C, E8, (512, K // 32), (K // 32, 1)), sb,
               block_k=32) == "SL_ERR_SHAPE"
    # nor scale rows 16 MiB apart
    assert err(api, (BASE_A, E2, (512, K), (K, 1)), (BASE_B, E2, (256, K), (K, 1)), None,
               rowmajor(0x1000000000, (512, 256)), (BASE_C, E8, (512, K // 32), (1 << 24, 1)), sb,
               block_k=32) == "SL_ERR_SHAPE"


def test_mxfp4_plan(api):
    """MXFP4 (packed E2M1, E8M0 per 32 K) goes to the 4-wave scaled-MFMA
    ring kernel with 256-wide K-tiles (the 8-wave one when asked for tile 4
    or K = 0); K must be a multiple of 512."""
    E2, E8 = 6, 4
    M, N, K = 512, 256, 1024
    a = (BASE_A, E2, (M, K), (K, 1))
    b = (BASE_B, E2, (N, K), (K, 1))
    sa = (BASE_C, E8, (M, K // 32), (K // 32, 1))
    sb = (BASE_C + 0x100000, E8, (N, K // 32), (K // 32, 1))
    d = rowmajor(BASE_D, (M, N))
    p = plan(api, a, b, None, d, sa, sb, block_k=32)
    assert p["kernel"] == api.K_MXFP4 and p["tile_k"] == 256 and p["threads"] == 256
    assert p["lds_bytes"] == 5 * 256 * 128
    os.environ["SL_TILE"] = "4"
    try:
        p4 = plan(api, a, b, None, d, sa, sb, block_k=32)
    finally:
        del os.environ["SL_TILE"]
    assert p4["threads"] == 512 and p4["lds_bytes"] == 2 * 768 * 128 - 2 * 256 * 128 + 2 * 768 * 16 - 2 * 256 * 16
    z = plan(api, (BASE_A, E2, (M, 0), (512, 1)), (BASE_B, E2, (N, 0), (512, 1)), None, d,
             (BASE_C, E8, (M, 0), (16, 1)), (BASE_C + 0x100000, E8, (N, 0), (16, 1)), block_k=32)
    assert z["threads"] == 512
    K2 = 768
    assert err(api, (BASE_A, E2, (M, K2), (K2, 1)), (BASE_B, E2, (N, K2), (K2, 1)), None, d,
               (BASE_C, E8, (M, K2 // 32), (K2 // 32, 1)), (BASE_C + 0x100000, E8, (N, K2 // 32), (K2 // 32, 1)),
               block_k=32) == "SL_ERR_LAYOUT"
