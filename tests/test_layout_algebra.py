"""The library's host layout algebra (sl_layout_op) and plan trace
(sl_describe_plan), on the CPU.

The algebra is pinned to the layouts the pages print
(tests/golden/page_values.json: the fragment page's partition, broadcast
block, full configuration, ldmatrix chain and exercises), to the oracle's
fragment construction (oracle/layout.py) on random atoms, and to brute force:
every operation is checked as a function on small random layouts, evaluated
here by a plain colex evaluator of the layout text.  The plan trace is pinned
to the library's exported instruction and LDS maps (which the GPU probes pin
to the hardware) and to the kernels' documented epilogue and tile order.
"""

import itertools
import os
import random

import numpy as np
import pytest

from oracle import layout as L


@pytest.fixture(scope="module")
def api():
    from stride_layouts_lds_amd import api as A
    if not os.path.exists(A.LIB_PATH):
        from stride_layouts_lds_amd import build
        build.build(verbose=False)
    A.lib()
    return A


# ----------------------------------------------------------- test evaluator

def parse(text):
    """'(4,(2,2)):(1,(4,8))' -> (shape tree, stride tree) of ints ('_' dropped)."""
    def tree(s, i):
        if s[i] == "(":
            out, i = [], i + 1
            while True:
                t, i = tree(s, i)
                out.append(t)
                if s[i] == ",":
                    i += 1
                    continue
                assert s[i] == ")"
                return tuple(out), i + 1
        j = i
        while j < len(s) and (s[j].isdigit() or s[j] == "_"):
            j += 1
        return int(s[i:j].lstrip("_")), j
    s = text.replace(" ", "")
    shape, i = tree(s, 0)
    assert s[i] == ":"
    stride, i = tree(s, i + 1)
    assert i == len(s)
    return shape, stride


def leaves(t):
    return [x for e in t for x in leaves(e)] if isinstance(t, tuple) else [t]


def ev(text_or_pair, x):
    """Offset of flat index x (first mode fastest)."""
    shape, stride = parse(text_or_pair) if isinstance(text_or_pair, str) else text_or_pair
    off = 0
    for s, d in zip(leaves(shape), leaves(stride)):
        off += (x % s) * d
        x //= s
    return off


def size_of(text):
    return int(np.prod(leaves(parse(text)[0]), dtype=np.int64))


def text(shape, stride):
    def t(x):
        return "(" + ",".join(t(e) for e in x) + ")" if isinstance(x, tuple) else str(x)
    return t(shape) + ":" + t(stride)


# ------------------------------------------------- the pages' printed layouts

def test_partition_is_the_smem_tile_composed_with_lane0_values(api, golden):
    # lane 0's values of the SM80 A TV layout in tile coordinates q = m + 16k
    tv = L.SM80_16x8x16_A
    # the values' q-steps: v0 -> k+1 (16), v1 -> m+8 (8), v2 -> k+8 (128)
    lane0 = "((2,2,2),1,1):((16,8,128),0,0)"
    for v in range(8):
        m, k = tv(0, v)
        assert ev(lane0, v) == m + 16 * k
    got = api.layout_op("composition", "(16,16):(16,1)", lane0)
    s0 = golden["sm80_partition"]["tCsA_stride0"]
    assert got == "((2,2,2),1,1):((%d,%d,%d),0,0)" % tuple(s0)
    assert [ev(got, v) for v in range(8)] == golden["sm80_A_lane0"]["smem_offset"]
    # exercise 1: row stride 24 changes 128 into 192, the fragment stays
    s24 = golden["exercises"]["row_stride_24_partition_stride0"]
    got24 = api.layout_op("composition", "(16,16):(24,1)", lane0)
    assert got24 == "((2,2,2),1,1):((%d,%d,%d),0,0)" % tuple(s24)
    marked = "((_2,_2,_2),_1,_1):((_%d,_%d,_%d),_0,_0)"
    r0 = golden["sm80_partition"]["tCrA_stride0"]
    want = "((2,2,2),1,1):((%d,%d,%d),0,0)" % tuple(r0)
    assert api.layout_op("fragment_like", marked % tuple(s0)) == want
    assert api.layout_op("fragment_like", marked % tuple(s24)) == want


def test_fragment_block_steps(api, golden):
    g = golden["broadcast_block"]
    # filter_zeros: only the static zero is a broadcast
    assert api.layout_op("filter_zeros", "(2,2,2):(_1,_0,_8)") == "(%d,%d,%d):(1,0,8)" % tuple(g["compact_shape"])
    assert api.layout_op("filter_zeros", "(2,2,2):(_1,0,_8)") == "(2,2,2):(1,0,8)"
    assert api.layout_op("compact_left", "(%d,%d,%d)" % tuple(g["compact_shape"])) == \
        "(2,1,2):(%d,%d,%d)" % tuple(g["block_stride"])
    assert api.layout_op("compact_left", "(2,2,2)") == "(2,2,2):(1,2,4)"
    blk = api.layout_op("fragment_like", "((2,2,2),1):((_1,_0,_8),_0)")
    assert blk == "((2,2,2),1):((%d,%d,%d),0)" % tuple(g["block_stride"])
    atom = "(2,2,2):(%d,%d,%d)" % tuple(g["block_stride"])
    assert int(api.layout_op("cosize", atom)) == g["cosize"]
    assert ev(atom, 0) == ev(atom, 2) == 0  # (0,1,0) shares (0,0,0)'s slot
    # a run-time zero keeps its own slot
    assert api.layout_op("fragment_like", "((2,2,2),1):((_1,0,_8),_0)") == "((2,2,2),1):((1,2,4),0)"
    # the small example's rest: (1,1):(0,0)
    assert api.layout_op("make_ordered", "(1,1)", "(_0,_0)") == "(1,1):(0,0)"


def test_full_config_rest_fragment_and_tensor_like(api, golden):
    g = golden["full_config"]
    sw = g["swizzled_strides"]  # the printed run-time strides 72, 144, 288
    part = "((_2,_2,_2),_4,(_2,_2)):((_1,_512,%d),_2048,(%d,%d))" % tuple(sw)
    rs = g["rest_stride"]
    # static 2048 first, then the run-time (144, 288) as they appear
    assert api.layout_op("make_ordered", "(4,(2,2))", "(_2048,(%d,%d))" % tuple(sw[1:])) == \
        "(4,(2,2)):(%d,(%d,%d))" % (rs[0], *rs[1])
    # by value alone (all static) the K modes would come first
    assert api.layout_op("make_ordered", "(4,(2,2))", "(_2048,(_%d,_%d))" % tuple(sw[1:])) == "(4,(2,2)):(4,(1,2))"
    tr = g["tCrA_rest_stride"]
    frag = api.layout_op("fragment_like", part)
    assert frag == "((2,2,2),4,(2,2)):((1,2,4),%d,(%d,%d))" % (tr[0], *tr[1])
    # offset_A(v, m, k) = v + 8m + 32k over all 128 values
    for v, m, k in itertools.product(range(8), range(4), range(4)):
        assert ev(frag, v + 8 * m + 32 * k) == v + 8 * m + 32 * k
    # make_tensor_like scatters the atom to slots 0..3 and 16..19
    tl = api.layout_op("tensor_like", part)
    assert tl == "((2,2,2),4,(2,2)):((1,2,16),4,(32,64))"
    assert sorted(ev(tl, v) for v in range(8)) == [0, 1, 2, 3, 16, 17, 18, 19]
    # the static marks survive when asked for
    assert api.layout_op("fragment_like", part, mark_static=True).startswith("((_2,_2,_2),_4,(_2,_2)):((_1,_2,_4)")
    # exercise 2 on the B fragment built the same way: tCrB(2,3,0) is slot 14
    ex = golden["exercises"]
    b_part = "((_2,_2),_8,(_2,_2)):((_1,_8),_1024,(%d,%d))" % tuple(sw[1:])
    b_frag = api.layout_op("fragment_like", b_part)
    v, n, k = ex["tCrB"]
    assert ev(b_frag, v + 4 * n + 32 * k) == ex["tCrB_offset"]
    for v, n, k in itertools.product(range(4), range(8), range(4)):
        assert ev(b_frag, v + 4 * n + 32 * k) == v + 4 * n + 32 * k


def test_right_inverse_chain(api, golden):
    g = golden["ldmatrix_chain"]
    # the copy's reference layout: its right inverse takes e = 129 to tv 160
    inv_ref = api.layout_op("right_inverse", "(32,(2,4)):(2,(1,64))")
    assert ev(inv_ref, g["e"]) == g["tv"]
    # the A TV layout takes tv 160 to q = 144 = A(0,9); its inverse goes back
    tv = "((4,8),(2,2,2)):((32,1),(16,8,128))"
    assert ev(tv, g["tv"]) == g["q"] == g["mk"][0] + 16 * g["mk"][1]
    inv = api.layout_op("right_inverse", tv)
    assert size_of(inv) == 256 and ev(inv, g["q"]) == g["tv"]
    assert all(ev(tv, ev(inv, q)) == q for q in range(256))
    # and the tile layout of the data-layout page is a bijection
    t = golden["tile_layout"]
    tl = text(tuple(t["shape"]), tuple(t["stride"]))
    inv_t = api.layout_op("right_inverse", tl)
    assert size_of(inv_t) == 64 and all(ev(tl, ev(inv_t, i)) == i for i in range(64))


# ------------------------------------------------------------ brute force

def rand_pow2_layout(rng, n_modes, max_stride=64):
    shape = tuple(rng.choice([1, 2, 4, 8]) for _ in range(n_modes))
    stride = tuple(rng.choice([0, 1, 2, 4, 8, 16, 32, max_stride]) for _ in range(n_modes))
    return shape, stride


def rand_bijection(rng, shapes):
    order = list(range(len(shapes)))
    rng.shuffle(order)
    stride = [0] * len(shapes)
    cur = 1
    for i in order:
        stride[i] = cur
        cur *= shapes[i]
    return tuple(shapes), tuple(stride)


def test_coalesce_keeps_the_function(api):
    rng = random.Random(1)
    for _ in range(200):
        sh, st = rand_pow2_layout(rng, rng.randint(1, 5))
        t = text(sh, st)
        c = api.layout_op("coalesce", t)
        n = int(np.prod(sh))
        assert size_of(c) == n
        assert all(ev(c, i) == ev(t, i) for i in range(n)), (t, c)


def test_composition_is_function_composition(api):
    # A o B equals A(B(i)) when B's modes reach disjoint bits of A's
    # (power-of-two) coordinates, so the by-mode composition adds without
    # carries: B is a sub-layout of a compact bijection, some modes dropped
    # or broadcast
    rng = random.Random(2)
    for _ in range(300):
        a = rand_bijection(rng, [rng.choice([2, 4, 8]) for _ in range(rng.randint(1, 4))])
        na = int(np.prod(a[0]))
        bits = [1 << rng.choice([1, 1, 2, 3]) for _ in range(6)]
        while np.prod(bits) > na:
            bits.pop()
        if not bits:
            continue
        sb, db = rand_bijection(rng, bits)
        keep = [i for i in range(len(sb)) if rng.random() < 0.8] or [0]
        sb = tuple(sb[i] for i in keep)
        db = tuple(0 if rng.random() < 0.1 else db[i] for i in keep)
        b = text(sb, db)
        # hierarchical B: group its first two modes
        if len(sb) >= 2 and rng.random() < 0.5:
            b = text(((sb[0], sb[1]),) + sb[2:], ((db[0], db[1]),) + db[2:])
        c = api.layout_op("composition", text(*a), b)
        nb = int(np.prod(sb))
        assert size_of(c) == nb
        assert all(ev(c, i) == ev(a, ev(b, i)) for i in range(nb)), (a, b, c)
    # non-powers of two: the stride 2 splits A's mode of 6 into (2,3)
    a, b = "(6,4):(4,1)", "(3,4):(2,6)"
    c = api.layout_op("composition", a, b)
    assert c == "(3,4):(8,1)"
    assert all(ev(c, i) == ev(a, ev(b, i)) for i in range(12))


def test_complement_fills_the_codomain(api):
    rng = random.Random(3)
    for _ in range(200):
        sh = [rng.choice([2, 3, 4]) for _ in range(rng.randint(2, 4))]
        full = rand_bijection(rng, sh)
        keep = [i for i in range(len(sh)) if rng.random() < 0.6] or [0]
        a = text(tuple(full[0][i] for i in keep), tuple(full[1][i] for i in keep))
        total = int(np.prod(sh))
        c = api.layout_op("complement", a, total)
        joint = "(%s,%s)" % tuple(x.split(":")[0] for x in (a, c)), "(%s,%s)" % tuple(x.split(":")[1] for x in (a, c))
        jt = joint[0] + ":" + joint[1]
        n = size_of(jt)
        assert n == total, (a, c)
        assert sorted(ev(jt, i) for i in range(n)) == list(range(total)), (a, c)


def test_right_inverse_round_trip(api):
    rng = random.Random(4)
    for _ in range(200):
        sh = [rng.choice([2, 3, 4, 5]) for _ in range(rng.randint(1, 4))]
        a = text(*rand_bijection(rng, sh))
        r = api.layout_op("right_inverse", a)
        n = int(np.prod(sh))
        assert size_of(r) == n
        assert all(ev(a, ev(r, i)) == i for i in range(n)), (a, r)
    # a layout with a hole: the inverse covers the contiguous prefix only
    r = api.layout_op("right_inverse", "(2,4):(1,4)")
    assert size_of(r) == 2 and all(ev("(2,4):(1,4)", ev(r, i)) == i for i in range(2))


def test_zipped_divide_regroups_the_same_elements(api):
    rng = random.Random(5)
    for _ in range(60):
        M, K = rng.choice([8, 16, 24, 32]), rng.choice([8, 16, 32])
        bm, bk = rng.choice([4, 8]), rng.choice([4, 8])
        rs, cs = (K, 1) if rng.random() < 0.5 else (1, M)
        a = "(%d,%d):(%d,%d)" % (M, K, rs, cs)
        z = api.layout_op("zipped_divide", a, "(%d,%d):(1,1)" % (bm, bk))
        tm = M // bm
        for idx in range(M * K):
            i, j = idx % (bm * bk), idx // (bm * bk)
            ti, tk = i % bm, i // bm
            ri, rk = j % tm, j // tm
            assert ev(z, idx) == (ri * bm + ti) * rs + (rk * bk + tk) * cs
    # a ragged mode: 300 rows in tiles of 128 -> 3 tiles, the last partial
    assert api.layout_op("zipped_divide", "(300,64):(64,1)", "(128,64):(1,1)") == \
        "((128,64),(3,1)):((64,1),(8192,0))"


def test_make_ordered_is_compact_in_the_given_order(api):
    rng = random.Random(6)
    for _ in range(100):
        n = rng.randint(1, 5)
        sh = [rng.choice([1, 2, 3, 4]) for _ in range(n)]
        order = [(rng.randint(0, 50), rng.random() < 0.6) for _ in range(n)]
        ot = "(" + ",".join(("_%d" if s else "%d") % v for v, s in order) + ")"
        got = api.layout_op("make_ordered", "(" + ",".join(map(str, sh)) + ")", ot)
        # the oracle's make_ordered_layout
        want = L.ordered_rest(tuple(sh), tuple(L.Ord(v, s) for v, s in order))
        assert parse(got)[1] == want, (sh, order, got)


def test_fragment_like_matches_the_oracle(api):
    rng = random.Random(7)
    for _ in range(100):
        na = rng.randint(1, 3)
        atom_sh = tuple(rng.choice([1, 2, 4]) for _ in range(na))
        atom_st = tuple(rng.choice([L.STATIC_ZERO, 1, 8, 128, 0]) for _ in range(na))
        nr = rng.randint(1, 3)
        rest_sh = tuple(rng.choice([1, 2, 4]) for _ in range(nr))
        rest_ord = tuple(L.Ord(rng.choice([0, 16, 32, 64, 2048]), rng.random() < 0.5) for _ in range(nr))

        def lit(x):
            # a static zero is a broadcast; a bare 0 is a run-time zero
            return "_0" if x == L.STATIC_ZERO else "0" if x == 0 else "_%d" % x
        part = "((%s),%s):((%s),%s)" % (
            ",".join(map(str, atom_sh)), ",".join(map(str, rest_sh)),
            ",".join(lit(x) for x in atom_st),
            ",".join(("_%d" if o.static else "%d") % o.value for o in rest_ord))
        got = parse(api.layout_op("fragment_like", part))
        shape_b, block_b = L.fragment_block(atom_sh, atom_st)
        rest = L.scale_strides(L.ordered_rest(rest_sh, rest_ord), L.cosize(shape_b, block_b))
        assert got == ((atom_sh,) + rest_sh, (tuple(block_b),) + tuple(rest)), part


def test_layout_op_errors(api):
    def status(fn):
        with pytest.raises(api.SLError) as e:
            fn()
        return e.value.name
    assert status(lambda: api.layout_op("composition", "(3,5):(5,1)", "2:2")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("parse", "(4,2):(1")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("parse", "(4,2):(1,2,3)")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("eval", "(4,2):(1,4)", 8)) == "SL_ERR_SHAPE"
    assert status(lambda: api.layout_op("zipped_divide", "(4,2):(1,4)", "4:1")) == "SL_ERR_LAYOUT"
    import ctypes
    lib = api.lib()
    assert lib.sl_layout_op(99, b"4:1", None, ctypes.create_string_buffer(64), 64, None) == -9
    assert lib.sl_layout_op(0, None, None, ctypes.create_string_buffer(64), 64, None) == -1
    need = ctypes.c_int64(0)
    small = ctypes.create_string_buffer(4)
    assert lib.sl_layout_op(0, b"(4,(2,2)):(1,(4,8))", None, small, 4, ctypes.byref(need)) == -3
    assert need.value == len("(4,(2,2)):(1,(4,8))") + 1
    assert api.layout_op("parse", "( 4 , (2,2) ) : ( 1 , (4,8) )") == "(4,(2,2)):(1,(4,8))"
    assert api.layout_op("size", "(4,(2,3))") == "24" and api.layout_op("cosize", "(4,2):(2,1)") == "8"
    # empty modes and sizes past 2^62 are errors, never a crash or a wrapped value
    assert status(lambda: api.layout_op("composition", "(0,4):(1,0)", "2:1")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("composition", "(4,4):(1,4)", "(0,2):(1,4)")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("zipped_divide", "(0,8):(8,1)", "(4,4):(1,1)")) == "SL_ERR_LAYOUT"
    assert api.layout_op("size", "(0,8)") == "0" and api.layout_op("cosize", "(0,8):(8,1)") == "0"
    big = "(1000000000000,1000000000000):(1,1000000000000)"
    assert status(lambda: api.layout_op("size", big)) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("cosize", big)) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("compact_left", "(1000000000000,1000000000000)")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("parse", "(1" + "0" * 19 + "):(1)")) == "SL_ERR_LAYOUT"
    assert status(lambda: api.layout_op("parse", "(" * 40 + "1" + ")" * 40 + ":" + "(" * 40 + "1" + ")" * 40)) \
        == "SL_ERR_LAYOUT"


# ------------------------------------------------------------ the plan trace

BASE_A, BASE_B, BASE_C, BASE_D = 0x100000000, 0x200000000, 0x300000000, 0x400000000


def rowmajor(ptr, shape, dtype=1):
    st, acc = [0] * len(shape), 1
    for i in reversed(range(len(shape))):
        st[i] = acc
        acc *= shape[i]
    return ptr, dtype, shape, st


def trace(api, a, b, c=None, d=None, sfa=None, sfb=None, block_k=32):
    D = lambda x: api.desc(*x) if x is not None else None
    args = api.make_args(D(a), D(b), D(c), D(d), D(sfa), D(sfb), block_k)
    t = api.describe_plan(args)
    return t, api.describe_stages(t), api.sl_gemm_plan(args)


def swizzled(byte, row_bytes):
    row, b = byte // row_bytes, byte % row_bytes
    s = (row ^ ((row >> 4) & 1)) & (row_bytes // 16 - 1)
    return row * row_bytes + 16 * ((b // 16) ^ s) + b % 16


INSTRS = {1: 0, 3: 2, 4: 3, 6: 5, 7: 7}  # kernel family -> instruction id of its operand map


def check_instr_lines(api, st, kernel):
    instr = INSTRS[kernel]
    fm = api.query_fragment_map(instr, 0)
    R = 16 if instr in (0, 2) else 32
    for lane, slot, row, col in fm:
        assert ev(st["A_instr"], lane + 64 * slot) == row + R * col
    dm = api.query_fragment_map(instr, 2)
    for lane, reg, row, col in dm:
        # the instruction's rows are our n (B is its first operand)
        assert ev(st["D_instr"], lane + 64 * reg) == col + R * row


@pytest.mark.parametrize("tile,fn", [(4, 4), (19, 8)])
def test_trace_fp16_square(api, tile, fn, monkeypatch):
    """Tile 4: 8 waves, each 128x64 (4 instruction tiles along N); tile 19
    (the automatic choice): 4 waves, each 128x128 (8 along N)."""
    monkeypatch.setenv("SL_TILE", str(tile))
    n = 8192
    t, st, p = trace(api, rowmajor(BASE_A, (n, n)), rowmajor(BASE_B, (n, n)), rowmajor(BASE_C, (n, n)),
                     rowmajor(BASE_D, (n, n)))
    assert p["threads"] == (512 if tile == 4 else 256)
    for name in ("A_instr", "A", "A_tiles", "A_lds", "A_copy", "A_wave", "A_lane0", "A_frag", "B_wave",
                 "D_instr", "acc", "D_lane0", "D", "C", "D_tiles", "tile_order", "workgroup_tile"):
        assert name in st, name
        assert api.layout_op("parse", st[name]) == st[name]
    assert "Swizzle<3,4,3> then Swizzle<1,4,7>" in t
    check_instr_lines(api, st, 1)
    assert st["A_tiles"] == "((256,64),(32,128)):((8192,1),(2097152,64))"
    # the wave partition: element (row, k) of the K-major tile, through the
    # swizzle, is where the kernel's fragment reads land
    lds, es = api.query_lds_map(1, 0)
    fm = api.query_fragment_map(0, 0)
    fa = api.query_fragment_addresses(1, 0)
    for lane, slot, row, col in fm:
        for i, ks in itertools.product(range(8), range(2)):
            e = ev(st["A_wave"], lane + 64 * (slot + 8 * (i + 8 * ks)))
            assert divmod(e, 64) == (16 * i + row, 32 * ks + col)
            assert swizzled(2 * e, 128) == lds[16 * i + row, 32 * ks + col]
            if i == 0 and ks == 0:
                assert swizzled(2 * e, 128) == fa[lane * 8 + slot]
    # registers: one K slice, 8 halves per instruction tile, tiles in order
    assert st["A_frag"] == "((8),8):((1),8)" and st["B_frag"] == f"((8),{fn}):((1),8)"
    # every copy instruction fills 1 KiB of LDS, the tile once
    assert sorted(ev(st["A_copy"], x) for x in range(size_of(st["A_copy"]))) == list(range(0, 256 * 128, 16))
    # accumulators: lane 0's (r, i, j) is D(16 i, 16 j + r)
    for r, i, j in itertools.product(range(4), range(8), range(fn)):
        assert ev(st["D_lane0"], r + 4 * (i + 8 * j)) == 16 * i * n + 16 * j + r
        assert ev(st["acc"], r + 4 * (i + 8 * j)) == (i * fn + j) * 4 + r
    # workgroup -> tile: XCD x = b % 8 takes order range x*128.., the order
    # walks groups of 8 tile-rows column by column
    tiles_m = n // 256
    for b in range(p["workgroups"]):
        idx = (b % 8) * (p["workgroups"] // 8) + b // 8
        g, within = divmod(idx, 8 * tiles_m)
        tm, tn = g * 8 + within % 8, within // 8
        assert ev(st["workgroup_tile"], b) == tm + tiles_m * tn


def test_trace_m_major_and_mx(api):
    n = 4096
    _, st, p = trace(api, (BASE_A, 1, (n, n), (1, n)), rowmajor(BASE_B, (n, n)), None, rowmajor(BASE_D, (n, n)))
    assert p["a_load"] == 3 and st["A_lds"] == "(256,64):(1,256)"
    fm = api.query_fragment_map(0, 0)
    for lane, slot, row, col in fm:
        for i, ks in itertools.product(range(8), range(2)):
            e = ev(st["A_wave"], lane + 64 * (slot + 8 * (i + 8 * ks)))
            assert divmod(e, 256) == (32 * ks + col, 16 * i + row)


@pytest.mark.parametrize("tile,fn", [(None, 4), (4, 2)])
def test_trace_mx(api, tile, fn, monkeypatch):
    """MXFP8 on 32x32x64: the automatic choice (the 4-wave ring kernel, each
    wave 128x128: 4 instruction tiles along N) and the 8-wave kernel (tile 4,
    each wave 128x64: 2 along N)."""
    if tile is not None:
        monkeypatch.setenv("SL_TILE", str(tile))
    n = 4096
    # bytes (row, k) of the 128-byte tile rows
    t, st, p = trace(api, rowmajor(BASE_A, (n, n), 3), rowmajor(BASE_B, (n, n), 3), None,
                     rowmajor(BASE_D, (n, n)), rowmajor(BASE_C, (n, n // 32), 4),
                     rowmajor(0x500000000, (n, n // 32), 4))
    assert p["kernel"] == (api.K_MX_W4R if tile is None else api.K_MX_W8)
    if tile is None:
        assert p["lds_bytes"] == 5 * 256 * 128 and "straight into registers" in t
    check_instr_lines(api, st, 4)
    lds, es = api.query_lds_map(4, 0)
    fm = api.query_fragment_map(3, 0)
    for lane, slot, row, col in fm:
        for i, ks in itertools.product(range(4), range(2)):
            e = ev(st["A_wave"], lane + 64 * (slot + 32 * (i + 4 * ks)))
            assert divmod(e, 128) == (32 * i + row, 64 * ks + col)
            assert swizzled(e, 128) == lds[32 * i + row, 64 * ks + col]
    for lane in range(64):
        assert ev(st["scale_instr"], lane) == lane % 32 + 32 * (lane // 32)
    for r, i, j in itertools.product(range(16), range(4), range(fn)):
        # register r of tile (i, j): n = 8 (r / 4) + r % 4 for lane 0
        assert ev(st["D_lane0"], r + 16 * (i + 4 * j)) == 32 * i * n + 32 * j + 8 * (r // 4) + r % 4


def test_trace_other_plans(api):
    # ragged skinny: no single workgroup layout, still every stage
    t, st, p = trace(api, rowmajor(BASE_A, (300, 72)), rowmajor(BASE_B, (2056, 72)), None,
                     rowmajor(BASE_D, (300, 2056)))
    assert "A_wave" in st and "not one layout" in t
    # split-K: the workspace stage
    t, st, p = trace(api, rowmajor(BASE_A, (300, 2056)), rowmajor(BASE_B, (72, 2056)), None,
                     rowmajor(BASE_D, (300, 72)))
    assert p["split_k"] > 1 and "workspace" in st
    # MXFP4 (packed E2M1 rows, E8M0 scales) and NVFP4 (E4M3 scales per 16)
    n = 1024
    fp4 = lambda ptr, shape: (ptr, 6, shape, (shape[1], 1))
    _, st, p = trace(api, fp4(BASE_A, (n, n)), fp4(BASE_B, (n, n)), None, rowmajor(BASE_D, (n, n)),
                     rowmajor(BASE_C, (n, n // 32), 4), rowmajor(0x500000000, (n, n // 32), 4))
    assert p["kernel"] == api.K_MXFP4 and "SFA" in st
    check_instr_lines(api, st, 6)
    _, st, p = trace(api, fp4(BASE_A, (n, n)), fp4(BASE_B, (n, n)), None, rowmajor(BASE_D, (n, n)),
                     rowmajor(BASE_C, (n, n // 16), 3), rowmajor(0x500000000, (n, n // 16), 3), block_k=16)
    assert p["kernel"] == api.K_NVFP4 and st["SFA"] == "(1024,64):(64,1)"
    # MXFP6: the LDS tile in bits, the wave partition through the probed map
    fp6 = lambda ptr, shape: (ptr, 7, shape, (shape[1], 1))
    t6, st, p = trace(api, fp6(BASE_A, (n, n)), fp6(BASE_B, (n, n)), None, rowmajor(BASE_D, (n, n)),
                      rowmajor(BASE_C, (n, n // 32), 4), rowmajor(0x500000000, (n, n // 32), 4))
    assert p["kernel"] == api.K_MXFP6 and "E2M3" in t6
    check_instr_lines(api, st, 7)
    # the 4-wave kernel's packed rows: value k of a K-tile at bit 6 k of its 768-bit row (the chunk
    # rotation is stated in the line's note); lane half h = col / 32 of the instruction's operand map
    # takes the K-tile's blocks 2h (K slice 0) and 2h + 1 (slice 1)
    assert st["A_lds"] == "(256,128):(768,6)"
    for lane, slot, row, col in api.query_fragment_map(7, 0):
        for i, ks in itertools.product(range(4), range(2)):
            e = ev(st["A_wave"], lane + 64 * (slot + 32 * (i + 4 * ks)))
            k = 32 * (2 * (col // 32) + ks) + col % 32
            assert divmod(e, 768) == (32 * i + row, 6 * k)
    # an empty product and an invalid one
    t, _, _ = trace(api, rowmajor(BASE_A, (0, 64)), rowmajor(BASE_B, (64, 64)), None, rowmajor(BASE_D, (0, 64)))
    assert "empty" in t
    with pytest.raises(api.SLError) as e:
        trace(api, rowmajor(BASE_A, (64, 64)), rowmajor(BASE_B, (64, 32)), None, rowmajor(BASE_D, (64, 64)))
    assert e.value.name == "SL_ERR_SHAPE"
