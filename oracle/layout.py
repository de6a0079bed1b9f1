"""Layout oracle (LO): shape:stride layouts evaluated with plain integers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  No numpy, no GPU code,
nothing shared with the HIP library.

Sources (cited by page title and section):

* "数据布局及其记号" (mlc.ai, data-layout chapter), section "Shape-Stride 模型":
  a layout ``S[(shape):(strides)]`` maps a logical index to a position by the
  dot product of the index with the strides; a transpose is a stride swap.
* same page, section "Tile Layout": a flat index ``x`` is unflattened by the
  shape with the LAST mode fastest (``c0 = x // 16`` ... ``c3 = x % 4`` for
  shape (4,2,2,4)), then dotted with the strides.  Section "一般的 Layout 函数"
  generalises this; its display formulas did not survive extraction, and the
  reading taken is ``c_i = (x // prod_{j>i} e_j) % e_i``, ``f(x) = sum c_i s_i``.
* same page, section "命名轴": strides may carry a named physical axis
  (``@laneid``, ``@reg``, ``@TLane``, ``@m`` ...); the function then returns one
  sum per axis.
* same page, section "Replication 与 Offset": ``R[n : s@axis]`` adds copies at
  ``r*s`` for r in 0..n-1; ``O[s@axis]`` adds a fixed shift.
* same page, section "Swizzle Layout": XOR of the row into the column.
* "CuTe 中 A、B 如何加载到 MMA 寄存器" (blog.qingsen.net), section 2: a TV layout
  takes (lane, value), each unflattened with the FIRST mode fastest
  (``t = t0 + 4*t1``, ``v = v0 + 2*v1 + 4*v2``), and returns the matrix index
  ``q = m + 16*k``.

Parity: every function here is pinned in ``tests/test_oracle_layout.py`` by
values the pages print, by brute-force constructions, or by numpy/torch stride
semantics.  The CDNA4 operand maps at the bottom are NOT fixed by the pages
(they are hardware facts): parity unpinned by the pages, pinned instead by the
device probes in ``tests/test_gpu_probes.py``.
"""

from __future__ import annotations

from dataclasses import dataclass
from itertools import product
from typing import Dict, Iterable, List, Sequence, Tuple, Union


# ---------------------------------------------------------------------------
# Basic nested-tuple helpers
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Ax:
    """A stride tagged with a named physical axis, e.g. ``Ax(4, 'laneid')``
    is the page's ``4@laneid``.  A plain int stride is on the memory axis
    ``m``."""
    value: int
    axis: str


Stride = Union[int, Ax, tuple]
MEM = "m"


def flatten(t) -> list:
    """Depth-first, left-to-right leaves of a nested tuple."""
    if isinstance(t, tuple):
        out = []
        for e in t:
            out.extend(flatten(e))
        return out
    return [t]


def size(shape) -> int:
    """Number of logical coordinates of a (nested) shape."""
    n = 1
    for e in flatten(shape):
        n *= e
    return n


# ---------------------------------------------------------------------------
# Unflatten: the two conventions the pages use
# ---------------------------------------------------------------------------

def unflatten_rowmajor(x: int, shape: Sequence[int]) -> Tuple[int, ...]:
    """Flat shape, last mode fastest (data-layout page, "Tile Layout")."""
    assert 0 <= x < size(tuple(shape))
    coords = []
    for e in reversed(shape):
        coords.append(x % e)
        x //= e
    return tuple(reversed(coords))


def unflatten_colex(x: int, shape):
    """Nested shape, first mode fastest, applied recursively (CuTe page,
    section 2: ``t = t0 + 4*t1``)."""
    if not isinstance(shape, tuple):
        assert 0 <= x < shape
        return x
    assert 0 <= x < size(shape)
    coords = []
    for e in shape:
        n = size(e)
        coords.append(unflatten_colex(x % n, e))
        x //= n
    return tuple(coords)


# ---------------------------------------------------------------------------
# Evaluation (dot product), with named axes
# ---------------------------------------------------------------------------

def _accumulate(out: Dict[str, int], c: int, s) -> None:
    if isinstance(s, Ax):
        out[s.axis] = out.get(s.axis, 0) + c * s.value
    else:
        out[MEM] = out.get(MEM, 0) + c * s


def crd2idx(coord, shape, stride) -> Dict[str, int]:
    """Hierarchical coordinate -> position, one sum per axis.

    An integer coordinate given for a nested mode is first unflattened
    colexicographically inside that mode (CuTe convention: ``tCrA(5,0,0)``
    addresses value 5 of the (2,2,2) mode)."""
    out: Dict[str, int] = {}
    _crd2idx(coord, shape, stride, out)
    return out


def _crd2idx(coord, shape, stride, out):
    if isinstance(shape, tuple):
        if not isinstance(coord, tuple):
            coord = unflatten_colex(coord, shape)
        assert isinstance(stride, tuple) and len(coord) == len(shape) == len(stride)
        for c, e, s in zip(coord, shape, stride):
            _crd2idx(c, e, s, out)
    else:
        assert not isinstance(coord, tuple) and 0 <= coord < shape, (coord, shape)
        _accumulate(out, coord, stride)


def mem(pos: Dict[str, int]) -> int:
    """The memory-axis component of a position."""
    return pos.get(MEM, 0)


def eval_flat(x: int, shape, stride, order: str = "rowmajor") -> Dict[str, int]:
    """The general layout function of the data-layout page: unflatten the
    flat index ``x`` by the (flattened) shape, then dot with the strides.
    ``order`` names the unflatten convention (``'rowmajor'``: the data-layout
    page; ``'colex'``: CuTe)."""
    fs, ft = flatten(shape), flatten(stride)
    if order == "rowmajor":
        c = unflatten_rowmajor(x, fs)
    elif order == "colex":
        c = unflatten_colex(x, tuple(fs))
    else:
        raise ValueError(order)
    out: Dict[str, int] = {}
    for ci, si in zip(c, ft):
        _accumulate(out, ci, si)
    return out


def cosize(shape, stride) -> int:
    """1 + largest memory offset the layout reaches (strides >= 0)."""
    hi = 0
    for e, s in zip(flatten(shape), flatten(stride)):
        assert not isinstance(s, Ax)
        hi += (e - 1) * s
    return hi + 1


# ---------------------------------------------------------------------------
# Replication and offset (data-layout page, "Replication 与 Offset")
# ---------------------------------------------------------------------------

def replicate(pos: Dict[str, int], reps: Sequence[Tuple[int, Ax]]) -> List[Dict[str, int]]:
    """All positions of ``base + R[n0:s0@a0] + R[n1:s1@a1] ...``."""
    out = []
    for rs in product(*[range(n) for n, _ in reps]):
        p = dict(pos)
        for r, (_, s) in zip(rs, reps):
            _accumulate(p, r, s)
        out.append(p)
    return out


def offset(pos: Dict[str, int], shift: Ax) -> Dict[str, int]:
    """``base + O[s@axis]``: shifts the position, no copies."""
    p = dict(pos)
    _accumulate(p, 1, shift)
    return p


# ---------------------------------------------------------------------------
# TV layouts: (lane, value) -> matrix coordinate
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class TV:
    """A (thread, value) layout whose codomain is the column-major index
    ``q = row + rows*col`` of a ``rows x cols`` tile (CuTe page, section 2,
    ``q = m + 16*k``)."""
    shape: tuple   # (lane_shape, value_shape)
    stride: tuple  # (lane_stride, value_stride)
    rows: int
    cols: int

    @property
    def lanes(self) -> int:
        return size(self.shape[0])

    @property
    def values(self) -> int:
        return size(self.shape[1])

    def q(self, lane: int, value: int) -> int:
        return mem(crd2idx((lane, value), self.shape, self.stride))

    def __call__(self, lane: int, value: int) -> Tuple[int, int]:
        q = self.q(lane, value)
        return q % self.rows, q // self.rows

    def table(self) -> List[Tuple[int, int, int, int]]:
        """All (lane, value, row, col) tuples, lane-major."""
        return [(t, v) + self(t, v) for t in range(self.lanes) for v in range(self.values)]

    def inverse(self) -> Dict[Tuple[int, int], Tuple[int, int]]:
        """(row, col) -> (lane, value); asserts the map is a bijection."""
        inv = {}
        for t, v, r, c in self.table():
            assert (r, c) not in inv, f"not injective at {(r, c)}"
            inv[(r, c)] = (t, v)
        assert len(inv) == self.rows * self.cols, "not onto"
        return inv


# -- sm80 m16n8k16 (CuTe page, sections 2 and 5) ---------------------------

# ALayout = ((4,8),(2,2,2)):((32,1),(16,8,128)) onto the 16x16 A tile (m,k).
SM80_16x8x16_A = TV(shape=((4, 8), (2, 2, 2)), stride=((32, 1), (16, 8, 128)), rows=16, cols=16)

# B in CuTe's (n,k) indexing: n = t/4, k = 2*(t%4) + v%2 + 8*(v/2); with
# codomain q = n + 8*k this is lane (4,8):(16,1), value (2,2):(8,64).
SM80_16x8x16_B = TV(shape=((4, 8), (2, 2)), stride=((16, 1), (8, 64)), rows=8, cols=16)


def sm80_A_inverse(m: int, k: int) -> Tuple[int, int]:
    """Inverse printed on the CuTe page, section 2 (integer division)."""
    return 4 * (m % 8) + (k % 8) // 2, k % 2 + 2 * (m // 8) + 4 * (k // 8)


def sm80_B_inverse(n: int, k: int) -> Tuple[int, int]:
    """Inverse printed on the CuTe page, section 5."""
    return 4 * n + (k % 8) // 2, k % 2 + 2 * (k // 8)


# -- m8n8 register fragment (data-layout page, "Register Fragment") ---------

M8N8_FRAGMENT_SHAPE = (8, 4, 2)
M8N8_FRAGMENT_STRIDE = (Ax(4, "laneid"), Ax(1, "laneid"), Ax(1, "reg"))


def m8n8_position(row: int, col: int) -> Tuple[int, int]:
    """(laneid, reg) of element (row, col) through the page's layout
    ``S[(8,4,2):(4@laneid,1@laneid,1@reg)]`` applied to x = 8*row + col."""
    p = eval_flat(8 * row + col, M8N8_FRAGMENT_SHAPE, M8N8_FRAGMENT_STRIDE, "rowmajor")
    return p.get("laneid", 0), p.get("reg", 0)


# ---------------------------------------------------------------------------
# Fragment-layout construction (CuTe page, section 3 and the source notes)
# ---------------------------------------------------------------------------

STATIC_ZERO = "_0"  # marks a compile-time zero stride (broadcast)


def filter_zeros(stride, shape):
    """Replace the shape of every static-zero-stride leaf by 1 (section 3)."""
    if isinstance(shape, tuple):
        return tuple(filter_zeros(s, e) for s, e in zip(stride, shape))
    return 1 if stride == STATIC_ZERO else shape


def compact_left(shape, current: int = 1):
    """LayoutLeft compact strides; a size-1 leaf gets stride 0 and leaves the
    running product unchanged (section 3).  Returns (strides, next)."""
    if isinstance(shape, tuple):
        out = []
        for e in shape:
            s, current = compact_left(e, current)
            out.append(s)
        return tuple(out), current
    if shape == 1:
        return 0, current
    return current, current * shape


def fragment_block(atom_shape, atom_stride):
    """The compact layout of one atom's values: keeps the original shape,
    re-strides it column-major over the non-broadcast leaves (section 3)."""
    strides, _ = compact_left(filter_zeros(atom_stride, atom_shape))
    return atom_shape, strides


@dataclass(frozen=True)
class Ord:
    """One leaf of the ordering information ``make_ordered_layout`` receives:
    the original stride value and whether it was a compile-time constant."""
    value: int
    static: bool


def ordered_rest(shape, order):
    """``make_ordered_layout`` as the source notes of the CuTe page describe
    it: leaves get compact strides in increasing order of their ``Ord``; a
    static order compares by value, a dynamic order ranks after every static
    one, and dynamic ones keep their order of appearance.  Size-1 leaves get
    stride 0."""
    leaves = flatten(shape)
    ords = flatten(order)
    assert len(ords) == len(leaves) and all(isinstance(o, Ord) for o in ords)
    rank = sorted(range(len(leaves)),
                  key=lambda i: (0, ords[i].value, i) if ords[i].static else (1, 0, i))
    strides = [0] * len(leaves)
    cur = 1
    for i in rank:
        if leaves[i] != 1:
            strides[i] = cur
            cur *= leaves[i]
    it = iter(strides)

    def rebuild(s):
        if isinstance(s, tuple):
            return tuple(rebuild(e) for e in s)
        return next(it)
    return rebuild(shape)


def scale_strides(stride, k: int):
    if isinstance(stride, tuple):
        return tuple(scale_strides(s, k) for s in stride)
    return stride * k


# ---------------------------------------------------------------------------
# Swizzle (data-layout page, "Swizzle Layout")
# ---------------------------------------------------------------------------

def xor_toy_mapped_col(row: int, logical_col: int) -> int:
    """The 8x8 toy: ``mapped_col = logical_col XOR row``."""
    return logical_col ^ row


def swizzle_bms(offset: int, b: int, m: int, s: int) -> int:
    """``Swizzle<B,M,S>`` as read here: XOR bits [M+S, M+S+B) into [M, M+B).
    The pages name ``Swizzle<3,3,3>`` without a definition; this reading makes
    the 16-B chunk index of a 128-B row (fp16 bits 3..5) XOR the row-in-8
    (bits 6..8), i.e. the SWIZZLE_128B rule, and reproduces the printed
    strides 72, 144, 288 of the full configuration's partition_A."""
    mask = (1 << b) - 1
    return offset ^ (((offset >> (m + s)) & mask) << m)


def bank_conflict_passes(byte_addrs: Sequence[int], bytes_per_lane: int,
                         n_banks: int, bank_bytes: int, lanes_per_pass: int) -> int:
    """Number of serialized bank cycles for one LDS access instruction under a
    parameterised bank model (the data-layout page's model is 32 banks of 4 B
    with 32/16/8 lanes per pass for 4/8/16 B).  Lanes are grouped
    consecutively into passes; within a pass, distinct words on one bank
    serialise, identical words broadcast.  Returns the total cycles over all
    passes (1 per pass when conflict-free)."""
    total = 0
    for p0 in range(0, len(byte_addrs), lanes_per_pass):
        per_bank: Dict[int, set] = {}
        for a in byte_addrs[p0:p0 + lanes_per_pass]:
            for w in range(a // bank_bytes, (a + bytes_per_lane) // bank_bytes):
                per_bank.setdefault(w % n_banks, set()).add(w)
        total += max(len(v) for v in per_bank.values())
    return total


# ---------------------------------------------------------------------------
# Block-scale packing and the device mesh (data-layout page)
# ---------------------------------------------------------------------------

def tmem_sfa_positions(m: int, sfk: int) -> List[Tuple[int, int, int]]:
    """(TLane, TCol, byte) copies of SFA[m, sfk] after the 32x128b base
    packing (local_lane = m % 32, TCol = m // 32, byte = sfk) and the
    four-partition replication ``R[4 : 32@TLane]``."""
    base = crd2idx((m % 32, m // 32, sfk), (32, 4, 4), (Ax(1, "TLane"), Ax(1, "TCol"), Ax(1, "byte")))
    return [(p.get("TLane", 0), p.get("TCol", 0), p.get("byte", 0))
            for p in replicate(base, [(4, Ax(32, "TLane"))])]


MESH_BASE_SHAPE = (2, 4, 8)
MESH_BASE_STRIDE = (Ax(1, "gpuid_y"), Ax(8, "m"), Ax(1, "m"))


# ---------------------------------------------------------------------------
# CDNA4 (gfx950) matrix-core operand maps, in the same TV algebra.
# These are hardware facts not fixed by the pages: parity unpinned by the
# pages, pinned by the device probes.  Lane l = l0 + L0*l1 (colex).
# ---------------------------------------------------------------------------

# v_mfma_f32_16x16x32_f16, operand A (16 x 32, q = m + 16k): m = l0, k = 8*l1 + v
MFMA16_F16_A = TV(shape=((16, 4), 8), stride=((1, 128), 16), rows=16, cols=32)
# operand B indexed (n, k): same form with n for m
MFMA16_F16_B = TV(shape=((16, 4), 8), stride=((1, 128), 16), rows=16, cols=32)
# accumulator D (16 x 16, q = m + 16n): n = l0, m = 4*l1 + i
MFMA16_D = TV(shape=((16, 4), 4), stride=((16, 4), 1), rows=16, cols=16)

# v_mfma_f32_32x32x16_f16, A (32 x 16): m = l0, k = 8*l1 + v
MFMA32_F16_A = TV(shape=((32, 2), 8), stride=((1, 256), 32), rows=32, cols=16)
MFMA32_F16_B = TV(shape=((32, 2), 8), stride=((1, 256), 32), rows=32, cols=16)
# D (32 x 32): n = l0, m = 8*(i//4) + 4*l1 + i%4
MFMA32_D = TV(shape=((32, 2), (4, 4)), stride=((32, 4), (1, 8)), rows=32, cols=32)

# The scaled f8 instructions take 32 bytes per lane in two 16-byte halves,
# v = v0 + 16*v1.  Which bytes share one E8M0 scale fixes the absolute k
# order: the block-scaled product of the data-layout page ("Replication 与
# Offset": sfk = k // K_blk) gives one scale to 32 CONSECUTIVE k, and the
# bytes that share a scale lane are v0 < 16 of lanes l1 = 2b, 2b+1 (16x16x128)
# or l1 = 0, 1 (32x32x64) in half v1.  The k order consistent with both is:
# v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 data, A (16 x 128):
#   m = l0, k = 16*l1 + v0 + 64*v1
MFMA16_F8_A = TV(shape=((16, 4), (16, 2)), stride=((1, 256), (16, 1024)), rows=16, cols=128)
MFMA16_F8_B = TV(shape=((16, 4), (16, 2)), stride=((1, 256), (16, 1024)), rows=16, cols=128)
# v_mfma_scale_f32_32x32x64_f8f6f4, A (32 x 64): m = l0, k = 16*l1 + v0 + 32*v1
MFMA32_F8_A = TV(shape=((32, 2), (16, 2)), stride=((1, 512), (32, 1024)), rows=32, cols=64)
MFMA32_F8_B = TV(shape=((32, 2), (16, 2)), stride=((1, 512), (32, 1024)), rows=32, cols=64)


# The same instructions with E2M1 data (format 4) take 16 bytes per lane,
# 32 nibbles, low nibble first.  Nibble v of lane l = l0 + R*l1 holds
# (m = l0, k = 32*l1 + v): 32 consecutive k, the k-block of 32 that scale
# lane l1 covers.  (Pinned by the device probe; the f8 byte order, with its
# two halves 64 or 32 k apart, does not carry over.)
# v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 A (16 x 128): q = m + 16 k
MFMA16_F4_A = TV(shape=((16, 4), 32), stride=((1, 512), 16), rows=16, cols=128)
# v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 A (32 x 64): q = m + 32 k
MFMA32_F4_A = TV(shape=((32, 2), 32), stride=((1, 1024), 32), rows=32, cols=64)

# The same instructions with 6-bit data (format 2 E2M3, format 3 E3M2): a
# lane's 32 values are one little-endian bit stream over six dwords (value v
# at bits 6v .. 6v+5).  Reading: value v of lane l = l0 + R*l1 holds
# (m = l0, k = 32*l1 + v), the E2M1 order (32 values per lane, one k-block
# of 32 per scale lane).  Parity unpinned by the pages; pinned by the device
# probe.
MFMA16_F6_A = TV(shape=((16, 4), 32), stride=((1, 512), 16), rows=16, cols=128)
MFMA32_F6_A = TV(shape=((32, 2), 32), stride=((1, 1024), 32), rows=32, cols=64)


def mfma_scale_owner(rows: int, lane: int) -> Tuple[int, int]:
    """(row, k-block of 32) whose E8M0 scale lane ``lane`` supplies for the
    scaled f8 instructions: row = lane % rows, block = lane // rows (blocks
    counted in the k order above)."""
    return lane % rows, lane // rows


INSTR_MAPS = {
    # id: (A map, B map, D map)   -- ids match the library's query ids
    0: (MFMA16_F16_A, MFMA16_F16_B, MFMA16_D),
    1: (MFMA32_F16_A, MFMA32_F16_B, MFMA32_D),
    2: (MFMA16_F8_A, MFMA16_F8_B, MFMA16_D),
    3: (MFMA32_F8_A, MFMA32_F8_B, MFMA32_D),
    4: (MFMA16_F4_A, MFMA16_F4_A, MFMA16_D),
    5: (MFMA32_F4_A, MFMA32_F4_A, MFMA32_D),
    6: (MFMA16_F6_A, MFMA16_F6_A, MFMA16_D),
    7: (MFMA32_F6_A, MFMA32_F6_A, MFMA32_D),
}


def probe_expected_onehot_A(instr: int, lane: int, slot: int, code) -> List[List[float]]:
    """Expected accumulator registers [lane][i] of one matrix-core instruction
    when A holds 1 at (lane, slot) and 0 elsewhere, and B holds ``code(l, s)``
    at each of its (lane, slot): D(m, n) = sum_k A(m,k) B(n,k) = B(n, k0) on
    row m0 and 0 elsewhere."""
    amap, bmap, dmap = INSTR_MAPS[instr]
    m0, k0 = amap(lane, slot)
    binv = bmap.inverse()
    out = [[0.0] * dmap.values for _ in range(dmap.lanes)]
    for l in range(dmap.lanes):
        for i in range(dmap.values):
            m, n = dmap(l, i)
            if m == m0:
                out[l][i] = float(code(*binv[(n, k0)]))
    return out


def probe_expected_onehot_B(instr: int, lane: int, slot: int, code) -> List[List[float]]:
    """As ``probe_expected_onehot_A`` with the roles swapped: B holds 1 at
    (lane, slot), A holds ``code``; D is nonzero on column n0 only."""
    amap, bmap, dmap = INSTR_MAPS[instr]
    n0, k0 = bmap(lane, slot)
    ainv = amap.inverse()
    out = [[0.0] * dmap.values for _ in range(dmap.lanes)]
    for l in range(dmap.lanes):
        for i in range(dmap.values):
            m, n = dmap(l, i)
            if n == n0:
                out[l][i] = float(code(*ainv[(m, k0)]))
    return out


def ds_read_tr16_b64_expected(addr: Sequence[int], lds_halves: Sequence[int]) -> List[List[int]]:
    """Reading taken for gfx950's transposing LDS read ds_read_b64_tr_b16
    (a hardware fact the pages do not cover; parity unpinned by the pages,
    pinned by the device probe).  The 64 lanes form 4 groups of 16; lane
    p of a group supplies the byte address of a 64-bit block (4 halves).
    The group's 16 blocks are read as a 4 x 16 matrix whose row j is the
    blocks of lanes 4j..4j+3 side by side, and lane i receives column i:
    element j of lane i is half i % 4 of the block of lane 4j + i // 4.
    Returns the 4 halves each lane receives."""
    out = []
    for lane in range(64):
        g, i = lane // 16, lane % 16
        vals = []
        for j in range(4):
            src = 16 * g + 4 * j + i // 4
            vals.append(lds_halves[addr[src] // 2 + i % 4])
        out.append(vals)
    return out
