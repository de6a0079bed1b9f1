"""Pins of the layout oracle against what the pages fix.

Each test checks an oracle function against a value the pages print
(tests/golden/page_values.json), a brute-force construction, or numpy/torch
stride semantics -- never against a retyped copy of the oracle's own formula.
"""

import itertools

import numpy as np
import pytest

from oracle import layout as L


# ---------------------------------------------------------------- core algebra

def test_tile_layout_equals_tile_major_enumeration(golden):
    g = golden["tile_layout"]
    shape, stride = tuple(g["shape"]), tuple(g["stride"])
    R, C = g["matrix"]
    tr, tc = g["tile"]
    # brute force: lay tiles out row-major, elements row-major inside a tile
    pos = {}
    addr = 0
    for ti in range(R // tr):
        for tj in range(C // tc):
            for i in range(tr):
                for j in range(tc):
                    pos[(ti * tr + i, tj * tc + j)] = addr
                    addr += 1
    got = {}
    for i in range(R):
        for j in range(C):
            got[(i, j)] = L.mem(L.eval_flat(i * C + j, shape, stride, "rowmajor"))
    assert got == pos
    assert sorted(got.values()) == list(range(R * C))  # bijection


def test_tile_layout_unflatten_as_printed(golden):
    # the page prints c0 = x//16, c1 = (x//8)%2, c2 = (x//4)%2, c3 = x%4 and
    # then c0 = i//2, c1 = i%2, c2 = j//4, c3 = j%4 for x = 8i + j
    for i in range(8):
        for j in range(8):
            assert L.unflatten_rowmajor(8 * i + j, (4, 2, 2, 4)) == (i // 2, i % 2, j // 4, j % 4)


def test_row_major_matches_numpy(golden):
    g = golden["row_major_4x4"]
    ref = np.arange(16).reshape(4, 4)
    for i in range(4):
        for j in range(4):
            assert L.mem(L.crd2idx((i, j), tuple(g["shape"]), tuple(g["stride"]))) == ref[i, j]


def test_transpose_is_stride_swap(golden):
    torch = pytest.importorskip("torch")
    g = golden["transpose"]
    t = torch.arange(12).reshape(*g["shape"])
    assert tuple(t.stride()) == tuple(g["stride"])
    tt = t.T
    assert tuple(tt.shape) == tuple(g["t_shape"]) and tuple(tt.stride()) == tuple(g["t_stride"])
    flat = t.flatten()
    for i in range(4):
        for j in range(3):
            off = L.mem(L.crd2idx((i, j), tuple(g["t_shape"]), tuple(g["t_stride"])))
            assert flat[off].item() == tt[i, j].item() == t[j, i].item()


def test_colex_and_rowmajor_differ_only_in_order():
    # same leaves, same dot product when the coordinate tuple is the same
    shape = (3, 4, 5)
    for x in range(60):
        c = L.unflatten_colex(x, shape)
        assert c == (x % 3, (x // 3) % 4, x // 12)
        r = L.unflatten_rowmajor(x, shape)
        assert r == (x // 20, (x // 5) % 4, x % 5)


# ---------------------------------------------------------------- named axes

def test_m8n8_fragment(golden):
    g = golden["m8n8_fragment"]
    assert g["row"] * 8 + g["col"] == g["cell"]
    assert L.m8n8_position(g["row"], g["col"]) == (g["laneid"], g["reg"])
    seen = set()
    for r in range(8):
        for c in range(8):
            seen.add(L.m8n8_position(r, c))
    assert seen == {(l, s) for l in range(32) for s in range(2)}


def test_m8n8_agrees_with_ldmatrix_x1_formula(golden):
    # a second page states the same map from the lane side
    for t in range(golden["ldmatrix_x1_formula"]["lanes"]):
        row, col0 = t // 4, (t % 4) * 2
        assert L.m8n8_position(row, col0) == (t, 0)
        assert L.m8n8_position(row, col0 + 1) == (t, 1)


def test_tmem_sfa_replication(golden):
    g = golden["tmem_sfa"]
    assert L.tmem_sfa_positions(g["m"], g["sfk"]) == [tuple(p) for p in g["positions"]]
    # the four copies of one element never share a cell with another m
    cells = {}
    for m in range(128):
        for sfk in range(4):
            for p in L.tmem_sfa_positions(m, sfk):
                assert p not in cells
                cells[p] = (m, sfk)
    assert len(cells) == 128 * 4 * 4


def test_mesh_replication_and_offset(golden):
    g = golden["mesh"]
    base = L.crd2idx(tuple(g["coord"]), L.MESH_BASE_SHAPE, L.MESH_BASE_STRIDE)
    assert base.get("gpuid_y") == g["gpuid_y"] and base.get("m") == g["m"]
    reps = L.replicate(base, [(2, L.Ax(1, "gpuid_x"))])
    devs = sorted((p.get("gpuid_x", 0), p["gpuid_y"]) for p in reps)
    assert devs == [tuple(d) for d in g["replicated_devices"]]
    assert all(p["m"] == g["m"] for p in reps)
    off = L.offset(base, L.Ax(1, "gpuid_x"))
    assert (off["gpuid_x"], off["gpuid_y"]) == tuple(g["offset_device"]) and off["m"] == g["m"]


# ---------------------------------------------------------------- sm80 TV maps

def test_sm80_A_lane0(golden):
    g = golden["sm80_A_lane0"]
    got = [L.SM80_16x8x16_A(0, v) for v in range(8)]
    assert got == [tuple(x) for x in g["mk"]]
    # offsets in sA = (16,16):(16,1)
    offs = [L.mem(L.crd2idx((m, k), (16, 16), (16, 1))) for m, k in got]
    assert offs == g["smem_offset"]
    assert L.SM80_16x8x16_A.inverse()[(0, 9)] == (g["A09_lane"], g["A09_slot"])


def test_sm80_A_bijection_and_printed_inverse():
    inv = L.SM80_16x8x16_A.inverse()  # asserts bijection onto 16x16
    for (m, k), tv in inv.items():
        assert L.sm80_A_inverse(m, k) == tv


def test_sm80_A_element_set_agrees_with_excalidraw(golden):
    g = golden["thread5_elements"]
    got = {L.SM80_16x8x16_A(g["lane"], v) for v in range(8)}
    assert got == {tuple(x) for x in g["mk"]}


def test_sm80_B_map(golden):
    inv = L.SM80_16x8x16_B.inverse()  # bijection onto 8x16 (n,k)
    for (n, k), tv in inv.items():
        assert L.sm80_B_inverse(n, k) == tv
    assert [L.SM80_16x8x16_B(0, v) for v in range(4)] == [tuple(x) for x in golden["sm80_B_lane0"]["nk"]]


def test_partition_views(golden):
    g = golden["sm80_partition"]
    # the printed smem view of lane 0 reproduces the offsets of its values
    sh = (2, 2, 2)
    for v in range(8):
        m, k = L.SM80_16x8x16_A(0, v)
        assert L.mem(L.crd2idx(v, sh, tuple(g["tCsA_stride0"]))) == 16 * m + k
    # make_fragment_like's block keeps the shape and packs the values
    assert L.fragment_block(sh, tuple(g["tCsA_stride0"])) == (sh, tuple(g["tCrA_stride0"]))
    assert [L.mem(L.crd2idx(v, sh, tuple(g["tCrA_stride0"]))) for v in range(8)] == list(range(8))


def test_broadcast_block(golden):
    g = golden["broadcast_block"]
    sh = tuple(g["shape"])
    atom_stride = (1, L.STATIC_ZERO, 8)
    assert L.filter_zeros(atom_stride, sh) == tuple(g["compact_shape"])
    shape, stride = L.fragment_block(sh, atom_stride)
    assert shape == sh and stride == tuple(g["block_stride"])
    assert L.cosize(shape, stride) == g["cosize"]
    assert L.mem(L.crd2idx((0, 1, 0), shape, stride)) == L.mem(L.crd2idx((0, 0, 0), shape, stride)) == 0
    # a runtime zero is not a static broadcast: it keeps its own slot
    assert L.fragment_block(sh, (1, 0, 8))[1] == (1, 2, 4)


def test_exercise_row_stride_24(golden):
    g = golden["exercises"]
    # sA = (16,24):(24,1): lane 0's smem offsets follow ((2,2,2)):(1,192,8)
    for v in range(8):
        m, k = L.SM80_16x8x16_A(0, v)
        assert L.mem(L.crd2idx(v, (2, 2, 2), tuple(g["row_stride_24_partition_stride0"]))) == 24 * m + k
    assert L.fragment_block((2, 2, 2), tuple(g["row_stride_24_partition_stride0"]))[1] == (1, 2, 4)


def test_full_config_fragment_layout(golden):
    g = golden["full_config"]
    # Swizzle<3,3,3> reading reproduces the printed runtime strides
    assert [L.swizzle_bms(s, 3, 3, 3) for s in g["unswizzled_strides"]] == g["swizzled_strides"]
    # make_ordered_layout: static 2048 before the dynamic (144, 288)
    rest = L.ordered_rest((4, (2, 2)), (L.Ord(2048, True), (L.Ord(144, False), L.Ord(288, False))))
    assert rest == (g["rest_stride"][0], tuple(g["rest_stride"][1]))
    # tiled_product: rest strides scaled by the block's cosize (8)
    shape_a, block_a = L.fragment_block((2, 2, 2), (1, 512, 72))
    cos = L.cosize(shape_a, block_a)
    assert cos == 8
    tcra_rest = L.scale_strides(rest, cos)
    assert tcra_rest == (g["tCrA_rest_stride"][0], tuple(g["tCrA_rest_stride"][1]))
    tcra_shape = ((2, 2, 2), 4, (2, 2))
    tcra_stride = (block_a,) + tcra_rest
    # printed: offset_A(v,m,k) = v + 8m + 32k
    offs = set()
    for v, m, k in itertools.product(range(8), range(4), range(4)):
        o = L.mem(L.crd2idx((v, m, k), tcra_shape, tcra_stride))
        assert o == v + 8 * m + 32 * k
        offs.add(o)
    assert offs == set(range(128))
    # B: block (2,2):(1,2), rest (8,(2,2)); printed offset_B = v + 4n + 32k
    shape_b, block_b = L.fragment_block((2, 2), (1, 8))
    rest_b = L.scale_strides(L.ordered_rest((8, (2, 2)), (L.Ord(1024, True), (L.Ord(144, False), L.Ord(288, False)))),
                             L.cosize(shape_b, block_b))
    for v, n, k in itertools.product(range(4), range(8), range(4)):
        assert L.mem(L.crd2idx((v, n, k), ((2, 2), 8, (2, 2)), (block_b,) + rest_b)) == v + 4 * n + 32 * k


def test_exercise_tXrB_regroup(golden):
    g = golden["exercises"]
    v, j, k = g["tXrB"]
    tcrb = (v % 4, 2 * j + v // 4, k)
    assert tcrb == tuple(g["tCrB"])
    shape_b, block_b = L.fragment_block((2, 2), (1, 8))
    stride = (block_b, 4, (32, 64))
    assert L.mem(L.crd2idx(tcrb, ((2, 2), 8, (2, 2)), stride)) == g["tCrB_offset"]


def test_ldmatrix_chain(golden):
    g = golden["ldmatrix_chain"]
    src = ((32, 8), (8, 1))
    ref = ((32, (2, 4)), (2, (1, 64)))
    e_src = L.mem(L.crd2idx(tuple(g["src"]), *src))
    e_dst = L.mem(L.crd2idx(tuple(g["dst"]), *ref))
    assert e_src == e_dst == g["e"]
    # right_inverse of the reference layout, by brute force over its domain
    inv = {}
    for t in range(32):
        for v in range(8):
            inv[L.mem(L.crd2idx((t, v), *ref))] = t + 32 * v
    assert sorted(inv) == list(range(256))
    tv = inv[g["e"]]
    assert tv == g["tv"]
    q = L.SM80_16x8x16_A.q(tv % 32, tv // 32)
    assert q == g["q"] and (q % 16, q // 16) == tuple(g["mk"])
    # every source lane reads one contiguous, 16-B aligned row of sA, and
    # source and destination agree on the matrix coordinate of every element
    for ts in range(32):
        coords = []
        for vs in range(8):
            e = L.mem(L.crd2idx((ts, vs), *src))
            r = inv[e]
            coords.append(L.SM80_16x8x16_A(r % 32, r // 32))
        ms = {m for m, _ in coords}
        ks = [k for _, k in coords]
        assert len(ms) == 1 and ks == list(range(ks[0], ks[0] + 8))
        assert (16 * coords[0][0] + coords[0][1]) * 2 % 16 == 0
        if str(ts) in g["source_row_starts"]:
            assert list(coords[0]) == g["source_row_starts"][str(ts)]
    # the hardware moves element e from the source (ts,vs) with Src = e to
    # the destination (td,vd) with Dst = e; the matrix coordinate that
    # arrives there must be the one the MMA expects in that slot
    dst = ((32, (2, 4)), (2, (1, 64)))
    for td in range(32):
        for vd in range(8):
            e = L.mem(L.crd2idx((td, vd), *dst))
            r = inv[e]
            assert L.SM80_16x8x16_A(r % 32, r // 32) == L.SM80_16x8x16_A(td, vd)


# ---------------------------------------------------------------- swizzle

def test_xor_toy(golden):
    g = golden["xor_toy"]
    row1 = [None] * 8
    for c in range(8):
        row1[L.xor_toy_mapped_col(1, c)] = c  # physical slot -> logical column
    assert row1 == g["row1"]
    assert [8 * 1 + c for c in row1] == g["row1_ptx"]
    col = 3
    plain = [r * 8 + col for r in range(8)]
    swz = [r * 8 + L.xor_toy_mapped_col(r, col) for r in range(8)]
    kw = dict(bytes_per_lane=1, n_banks=8, bank_bytes=1, lanes_per_pass=8)
    assert L.bank_conflict_passes(plain, **kw) == g["cycles_rowmajor"]
    assert L.bank_conflict_passes(swz, **kw) == g["cycles_swizzled"]


def test_swizzle_is_a_bijection():
    for b, m, s in [(3, 3, 3), (2, 3, 3), (3, 4, 3), (3, 3, 4)]:
        n = 1 << (b + m + s + 1)
        assert sorted(L.swizzle_bms(o, b, m, s) for o in range(n)) == list(range(n))


def test_bank_model_nvidia_passes():
    # 32 banks x 4 B: 16-B accesses go 8 lanes per pass; 32 lanes reading
    # consecutive 16-B chunks take 4 conflict-free passes
    addrs = [16 * l for l in range(32)]
    assert L.bank_conflict_passes(addrs, 16, 32, 4, 8) == 4
    # all 32 lanes on one 128-B-strided column: 8-way within each pass
    addrs = [128 * l for l in range(32)]
    assert L.bank_conflict_passes(addrs, 16, 32, 4, 8) == 4 * 8
    # broadcast: same address in a pass costs one cycle
    assert L.bank_conflict_passes([0] * 8, 16, 32, 4, 8) == 1


# ---------------------------------------------------------------- CDNA4 maps

@pytest.mark.parametrize("instr", sorted(L.INSTR_MAPS))
def test_cdna4_maps_are_bijections(instr):
    for tv in L.INSTR_MAPS[instr]:
        tv.inverse()


def test_probe_expectation_shape():
    # the expected one-hot probe output has exactly one nonzero row/column
    code = lambda l, s: l * 8 + s + 1
    out = L.probe_expected_onehot_A(0, 17, 3, code)
    nz = [(l, i) for l in range(64) for i in range(4) if out[l][i]]
    assert len(nz) == 16
    m0, _ = L.MFMA16_F16_A(17, 3)
    assert all(L.MFMA16_D(l, i)[0] == m0 for l, i in nz)
