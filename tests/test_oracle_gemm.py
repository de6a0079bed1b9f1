"""Pins of the GEMM oracle (oracle/gemm_ref.c) against independent sources.

* codecs: exhaustively against numpy float16 and torch float8 conversions;
* GEMM: against numpy fp64 matmul on small-integer data where every product
  and partial sum is exact (so any summation order gives the same bits),
  through transposed, batched and broadcast views;
* closed forms: A = 0 gives C, A = I gives B^T + C, one-hot A and B hit one
  element;
* MX: unit scales reduce to the fp16 GEMM of the decoded E4M3 values, and a
  +1 on one E8M0 byte doubles exactly that block's contribution;
* the acceptance bound on hand-made cases.
"""

import numpy as np
import pytest

from oracle import gemm as G

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _built():
    G.build()


# ---------------------------------------------------------------- codecs

def test_f16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([G.f16_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy_rne():
    rng = np.random.default_rng(123)
    xs = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        rng.uniform(-70000, 70000, 2000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, np.inf, -np.inf],
    ])
    # every exact midpoint between adjacent finite fp16 values (tie cases)
    pos = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([xs, mids, -mids])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([G.f16_encode(float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], got[i], ref[i]) for i in bad[:5]]


def test_e4m3_decode_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([G.e4m3_decode(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # S.1111.111
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e8m0_decode_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([G.e8m0_decode(i) for i in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


# ---------------------------------------------------------------- helpers

def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def dec(codes):
    return np.asarray(codes, np.uint16).view(np.float16).astype(np.float64)


def strided(storage, shape, strides):
    it = storage.itemsize
    return np.lib.stride_tricks.as_strided(storage, shape=shape, strides=[s * it for s in strides])


# ---------------------------------------------------------------- fp16 GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 3), (37, 29, 64), (64, 33, 17)])
def test_gemm_exact_integers_vs_numpy(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = rng.integers(-4, 5, (M, K))
    b = rng.integers(-4, 5, (N, K))
    c = rng.integers(-100, 101, (M, N))
    d, ref, absum = G.gemm(f16(a), f16(b), f16(c))
    want = a.astype(np.float64) @ b.T.astype(np.float64) + c
    assert np.array_equal(ref[0], want)
    assert np.array_equal(d[0], f16(want))
    assert np.array_equal(absum[0], np.abs(a).astype(np.float64) @ np.abs(b).T.astype(np.float64))


@pytest.mark.parametrize("a_major,b_major", [("row", "row"), ("col", "row"), ("row", "col"), ("col", "col")])
def test_gemm_strided_batched_views(a_major, b_major):
    """Transposed (stride-swapped) and batched views, addressed only through
    their strides, agree with numpy on the same logical matrices."""
    rng = np.random.default_rng(7)
    nb, M, N, K = 3, 19, 23, 40
    A = rng.integers(-4, 5, (nb, M, K))
    B = rng.integers(-4, 5, (nb, N, K))
    if a_major == "row":
        a = strided(f16(A).ravel(), (nb, M, K), (M * K, K, 1))
    else:  # store (nb, K, M), view as (nb, M, K) with strides (M*K, 1, M)
        a = strided(f16(A.transpose(0, 2, 1)).ravel().copy(), (nb, M, K), (M * K, 1, M))
    if b_major == "row":
        b = strided(f16(B).ravel(), (nb, N, K), (N * K, K, 1))
    else:
        b = strided(f16(B.transpose(0, 2, 1)).ravel().copy(), (nb, N, K), (N * K, 1, N))
    d, ref, _ = G.gemm(a, b)
    want = np.einsum("bmk,bnk->bmn", A.astype(np.float64), B.astype(np.float64))
    assert np.array_equal(ref, want)


def test_gemm_broadcast_batch_stride_zero():
    rng = np.random.default_rng(8)
    nb, M, N, K = 4, 9, 11, 16
    A = rng.integers(-4, 5, (nb, M, K))
    B = rng.integers(-4, 5, (N, K))
    b = strided(f16(B).ravel(), (nb, N, K), (0, K, 1))  # one B for every batch
    d, ref, _ = G.gemm(f16(A), b)
    want = np.einsum("bmk,nk->bmn", A.astype(np.float64), B.astype(np.float64))
    assert np.array_equal(ref, want)


def test_gemm_real_values_vs_numpy():
    rng = np.random.default_rng(9)
    M, N, K = 33, 47, 130
    A = dec(f16(rng.standard_normal((M, K))))
    B = dec(f16(rng.standard_normal((N, K))))
    C = dec(f16(rng.standard_normal((M, N))))
    _, ref, absum = G.gemm(f16(A), f16(B), f16(C))
    want = A @ B.T + C
    S = np.abs(A) @ np.abs(B).T
    assert np.all(np.abs(ref[0] - want) <= 1e-13 * (S + np.abs(C)))
    np.testing.assert_allclose(absum[0], np.abs(A) @ np.abs(B).T, rtol=1e-13)


def test_gemm_closed_forms():
    rng = np.random.default_rng(10)
    M = K = 24
    N = 20
    B = dec(f16(rng.standard_normal((N, K))))
    C = dec(f16(rng.standard_normal((M, N)))) + 0.0
    # A = 0: D = C bit for bit
    d, _, absum = G.gemm(f16(np.zeros((M, K))), f16(B), f16(C))
    assert np.array_equal(dec(d[0]), C) and not absum.any()
    # A = I: D = fp16(B^T + C)
    d, ref, _ = G.gemm(f16(np.eye(M)), f16(B), f16(C))
    assert np.array_equal(ref[0], B.T + C)
    assert np.array_equal(d[0], f16(B.T + C))
    # one-hot A and B meeting at k0: a single 1 at (m0, n0)
    A1 = np.zeros((M, K)); A1[5, 17] = 1
    B1 = np.zeros((N, K)); B1[13, 17] = 1; B1[2, 16] = 1
    _, ref, _ = G.gemm(f16(A1), f16(B1))
    want = np.zeros((M, N)); want[5, 13] = 1
    assert np.array_equal(ref[0], want)


def test_gemm_points_equal_full():
    rng = np.random.default_rng(11)
    nb, M, N, K = 2, 13, 17, 50
    A = f16(rng.standard_normal((nb, M, K)))
    B = f16(rng.standard_normal((nb, N, K)))
    C = f16(rng.standard_normal((nb, M, N)))
    d, ref, absum = G.gemm(A, B, C)
    pts = np.stack([rng.integers(0, nb, 40), rng.integers(0, M, 40), rng.integers(0, N, 40)], 1)
    dp, rp, sp = G.gemm_points(A, B, C, points=pts)
    assert np.array_equal(dp, d[pts[:, 0], pts[:, 1], pts[:, 2]])
    assert np.array_equal(rp, ref[pts[:, 0], pts[:, 1], pts[:, 2]])
    assert np.array_equal(sp, absum[pts[:, 0], pts[:, 1], pts[:, 2]])


# ---------------------------------------------------------------- MX GEMM

def e4m3(x):
    return torch.from_numpy(np.clip(np.asarray(x, np.float32), -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_mx_unit_scales_equal_fp16_gemm_of_decoded_values():
    rng = np.random.default_rng(12)
    M, N, K = 21, 18, 96
    a8 = e4m3(rng.standard_normal((M, K)))
    b8 = e4m3(rng.standard_normal((N, K)))
    sfa = np.full((M, K // 32), 127, np.uint8)
    sfb = np.full((N, K // 32), 127, np.uint8)
    _, ref_mx, _ = G.gemm(a8, b8, sfa=sfa, sfb=sfb)
    # every E4M3 value is exactly an fp16 value
    _, ref_16, _ = G.gemm(f16(e4m3_values(a8)), f16(e4m3_values(b8)))
    assert np.array_equal(ref_mx, ref_16)


def test_mx_scales_vs_numpy():
    rng = np.random.default_rng(13)
    M, N, K = 17, 19, 160  # K = 5 blocks
    a8 = e4m3(rng.standard_normal((M, K)))
    b8 = e4m3(rng.standard_normal((N, K)))
    sfa = (rng.integers(-4, 5, (M, K // 32)) + 127).astype(np.uint8)
    sfb = (rng.integers(-4, 5, (N, K // 32)) + 127).astype(np.uint8)
    _, ref, _ = G.gemm(a8, b8, sfa=sfa, sfb=sfb)
    sa = torch.from_numpy(sfa).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    sb = torch.from_numpy(sfb).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    A = e4m3_values(a8) * np.repeat(sa, 32, axis=1)
    B = e4m3_values(b8) * np.repeat(sb, 32, axis=1)
    # E4M3 x 2^e values have few significant bits: every product and partial
    # sum here is exact in fp64, so the comparison is exact
    assert np.array_equal(ref[0], A @ B.T)


def test_mx_one_scale_step_doubles_one_block():
    rng = np.random.default_rng(14)
    M, N, K = 8, 6, 128
    a8 = e4m3(rng.standard_normal((M, K)))
    b8 = e4m3(rng.standard_normal((N, K)))
    sfa = (rng.integers(-4, 5, (M, 4)) + 127).astype(np.uint8)
    sfb = (rng.integers(-4, 5, (N, 4)) + 127).astype(np.uint8)
    _, base, _ = G.gemm(a8, b8, sfa=sfa, sfb=sfb)
    m0, kb = 3, 2
    sfa2 = sfa.copy(); sfa2[m0, kb] += 1
    _, bumped, _ = G.gemm(a8, b8, sfa=sfa2, sfb=sfb)
    # the block's own contribution, from the block alone
    a_blk = np.zeros_like(a8); a_blk[:, 32 * kb:32 * kb + 32] = a8[:, 32 * kb:32 * kb + 32]
    _, part, _ = G.gemm(a_blk, b8, sfa=sfa, sfb=sfb)
    diff = bumped[0] - base[0]
    assert np.array_equal(diff[m0], part[0, m0])
    assert not np.delete(diff, m0, axis=0).any()


# ---------------------------------------------------------------- acceptance

def test_check_bound():
    one = int(f16(1.0))
    up1, up2 = one + 1, one + 2         # 1 + 2^-10, 1 + 2^-9
    d_ref = np.array([one, one, one, one], np.uint16)
    absum = np.zeros(4)
    assert G.check(np.array([one, up1, one, one], np.uint16), d_ref, absum)[0] == 0
    bad, wi, _ = G.check(np.array([one, up2, one, one], np.uint16), d_ref, absum)
    assert bad == 1 and wi == 1
    # the S term admits a larger error
    absum2 = np.array([0, 2.0 ** 4, 0, 0])
    assert G.check(np.array([one, up2, one, one], np.uint16), d_ref, absum2)[0] == 0
    # NaN never passes
    assert G.check(np.array([0x7e00], np.uint16), np.array([0x7e00], np.uint16), np.zeros(1))[0] == 1


# ---------------------------------------------------------------- bf16

def _bf16_values():
    codes = np.arange(65536, dtype=np.uint16)
    return codes, torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_decode_all_codes():
    codes, ref = _bf16_values()
    got = np.array([G.bf16_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_encode_is_nearest_even_by_brute_force():
    """Every finite code round-trips; and for values between codes (random,
    exact midpoints, subnormal, near overflow) the encoder returns the
    nearest finite bf16, ties to the even code, found by search over the
    decoded table (itself pinned to torch above)."""
    codes, vals = _bf16_values()
    pos = [(v, int(c)) for c, v in zip(codes, vals) if np.isfinite(v) and v > 0 and not (int(c) & 0x8000)]
    pos.sort()
    pv = np.array([v for v, _ in pos])
    pc = [c for _, c in pos]
    for c, v in zip(codes, vals):
        if np.isfinite(v):
            assert G.bf16_encode(float(v)) == int(c)
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(0, 1, 300) * 2.0 ** rng.integers(-140, 128, 300))
    xs += [0.5 * (pv[i] + pv[i + 1]) for i in rng.integers(0, len(pv) - 1, 300)]  # exact midpoints
    xs += [2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126 * (1 - 2.0 ** -9)]
    for x in xs:
        i = int(np.searchsorted(pv, x))
        if i == 0:
            cand = [(0.0, 0)] + [(pv[0], pc[0])]
        elif i >= len(pv):
            cand = [(pv[-1], pc[-1])]
        else:
            cand = [(pv[i - 1], pc[i - 1]), (pv[i], pc[i])]
        best = min(cand, key=lambda t: (abs(t[0] - x), t[1] & 1))
        if x >= pv[-1] + 0.5 * (pv[-1] - pv[-2]):
            best = (np.inf, 0x7F80)  # at or past the midpoint to 2^128: infinity
        assert G.bf16_encode(float(x)) == best[1], x
        assert G.bf16_encode(-float(x)) == best[1] | 0x8000, x


def test_bf16_gemm_exact_integers_vs_numpy():
    rng = np.random.default_rng(8)
    M, N, K = 33, 20, 48
    a = rng.integers(-4, 5, (M, K)).astype(np.float64)
    b = rng.integers(-4, 5, (N, K)).astype(np.float64)
    c = rng.integers(-4, 5, (M, N)).astype(np.float64)
    enc = lambda x: np.array([G.bf16_encode(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)
    d, ref, absum = G.gemm(enc(a), enc(b).T.copy().T, enc(c), bf16=True)
    want = a @ b.T + c
    assert np.array_equal(ref[0], want)
    assert np.array_equal(d[0], enc(want))
    assert np.array_equal(absum[0], np.abs(a) @ np.abs(b).T)


def test_check_bound_bf16():
    one = G.bf16_encode(1.0)
    up1, up2 = one + 1, one + 2         # 1 + 2^-7, 1 + 2^-6
    d_ref = np.array([one, one], np.uint16)
    assert G.check(np.array([one, up1], np.uint16), d_ref, np.zeros(2), bf16=True)[0] == 0
    assert G.check(np.array([one, up2], np.uint16), d_ref, np.zeros(2), bf16=True)[0] == 1


# ---------------------------------------------------------------- E2M1 / NVFP4

def test_e2m1_decode_special_values_and_structure():
    """OCP MX v1.0 E2M1: smallest subnormal 0.5, smallest normal 1.0, largest
    6.0, sign-magnitude, no infinities or NaN; every value is an E4M3 value
    (the E4M3 decoder is pinned to torch above)."""
    v = [G.e2m1_decode(c) for c in range(16)]
    pos = v[:8]
    assert pos[0] == 0.0 and pos[1] == 0.5 and pos[2] == 1.0 and pos[7] == 6.0
    assert all(pos[i] < pos[i + 1] for i in range(7))
    assert all(v[8 + i] == -pos[i] for i in range(8)) and np.signbit(v[8])
    assert all(np.isfinite(x) for x in v)
    e4m3 = {G.e4m3_decode(c) for c in range(256)}
    assert all(x in e4m3 for x in v)
    # one significand bit: each binade [2^e, 2^(e+1)) holds exactly {2^e, 1.5 * 2^e}
    assert pos[2:] == [1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """(rows, K) nibble codes -> (rows, K/2) bytes, element 2i in the low nibble."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_nvfp4_gemm_vs_numpy():
    """Packed E2M1 operands with one E4M3 scale per 16 K: the oracle equals
    numpy's fp64 matmul of the decoded, block-scaled values (all exact)."""
    rng = np.random.default_rng(12)
    M, N, K = 24, 18, 64
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    # E4M3 scales from a small exact set (powers of two and 1.5 * powers)
    scale_codes = np.array([c for c in range(256) if G.e4m3_decode(c) in (0.25, 0.5, 0.75, 1.0, 1.5, 2.0, 3.0)],
                           np.uint8)
    sa = rng.choice(scale_codes, (M, K // 16)).astype(np.uint8)
    sb = rng.choice(scale_codes, (N, K // 16)).astype(np.uint8)
    dec2 = np.vectorize(G.e2m1_decode)
    dec8 = np.vectorize(G.e4m3_decode)
    a_real = dec2(ca) * np.repeat(dec8(sa), 16, axis=1)
    b_real = dec2(cb) * np.repeat(dec8(sb), 16, axis=1)
    A = G.packed(_pack_e2m1(ca), (M, K), (K, 1), G.E2M1)
    B = G.packed(_pack_e2m1(cb), (N, K), (K, 1), G.E2M1)
    SA = G.packed(sa, (M, K // 16), (K // 16, 1), G.E4M3)
    SB = G.packed(sb, (N, K // 16), (K // 16, 1), G.E4M3)
    d, ref, absum = G.gemm(A, B, None, SA, SB, block_k=16)
    assert np.array_equal(ref[0], a_real @ b_real.T)
    assert np.array_equal(absum[0], np.abs(a_real) @ np.abs(b_real).T)
    # the same values with the odd elements' nibbles swapped differ: the
    # packing order is observed
    swapped = G.packed((_pack_e2m1(ca) >> 4) | (_pack_e2m1(ca) << 4) & 0xF0, (M, K), (K, 1), G.E2M1)
    _, ref2, _ = G.gemm(swapped, B, None, SA, SB, block_k=16)
    a_sw = dec2(ca.reshape(M, K // 2, 2)[:, :, ::-1].reshape(M, K)) * np.repeat(dec8(sa), 16, axis=1)
    assert np.array_equal(ref2[0], a_sw @ b_real.T)


def test_mxfp4_gemm_vs_numpy():
    """Packed E2M1 operands with one E8M0 scale per 32 K (MXFP4): the oracle
    equals numpy's fp64 matmul of the decoded, block-scaled values."""
    rng = np.random.default_rng(13)
    M, N, K = 20, 26, 128
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sa = rng.integers(124, 131, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(124, 131, (N, K // 32)).astype(np.uint8)
    dec2 = np.vectorize(G.e2m1_decode)
    a_real = dec2(ca) * np.repeat(2.0 ** (sa.astype(np.float64) - 127), 32, axis=1)
    b_real = dec2(cb) * np.repeat(2.0 ** (sb.astype(np.float64) - 127), 32, axis=1)
    A = G.packed(_pack_e2m1(ca), (M, K), (K, 1), G.E2M1)
    B = G.packed(_pack_e2m1(cb), (N, K), (K, 1), G.E2M1)
    d, ref, absum = G.gemm(A, B, None, sa, sb, block_k=32)
    assert np.array_equal(ref[0], a_real @ b_real.T)


# ------------------------------------------------------------------ MXFP6

def _fp8_values(dtype):
    import torch
    return torch.arange(256, dtype=torch.uint8).view(dtype).double().numpy()


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_decode_against_the_8_bit_formats(fmt):
    """OCP MX v1.0 FP6: the 32 non-negative E2M3 codes are, in increasing
    order, exactly the E4M3 values in [0, 7.5] on the 1/8 grid (three
    significand bits, subnormal step 1/8, max 7.5); the E3M2 codes likewise
    the E5M2 values in [0, 28] on the 1/16 grid (two significand bits,
    subnormal step 1/16, max 28).  The 8-bit values come from torch's float8
    types; bit 5 is the sign; no infinities or NaN."""
    import torch
    if fmt == "e2m3":
        dec, ref, top, grid = G.e2m3_decode, _fp8_values(torch.float8_e4m3fn), 7.5, 8
    else:
        dec, ref, top, grid = G.e3m2_decode, _fp8_values(torch.float8_e5m2), 28.0, 16
    v = [dec(c) for c in range(64)]
    pos = v[:32]
    want = sorted({x for x in ref if np.isfinite(x) and 0 <= x <= top and (x * grid) == int(x * grid)})
    assert pos == want and len(want) == 32 and pos[-1] == top
    assert all(v[32 + i] == -pos[i] for i in range(32)) and np.signbit(v[32])
    assert all(np.isfinite(x) for x in v)


def _pack_fp6(codes: np.ndarray) -> np.ndarray:
    """(rows, K) 6-bit codes -> (rows, 3K/4) bytes: each row one little-endian
    bit stream, code j at bits 6j .. 6j+5 (numpy's bit unpacking, written
    independently of the oracle's extraction)."""
    rows, K = codes.shape
    bits = ((codes[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(rows, 6 * K)
    return np.packbits(bits, axis=1, bitorder="little")


def test_fp6_packing_order():
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 64, (3, 64)).astype(np.uint8)
    packed_rows = _pack_fp6(codes)
    assert packed_rows.shape == (3, 48)
    flat = packed_rows.reshape(-1)
    for r in range(3):
        for j in range(64):
            assert G.fp6_code(flat, r * 64 + j) == codes[r, j]
    # byte-level check of the first four codes (three bytes)
    c = codes[0, :4].astype(int)
    word = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18)
    assert list(flat[:3]) == [word & 255, (word >> 8) & 255, (word >> 16) & 255]


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2")])
def test_mxfp6_gemm_vs_numpy(fa, fb):
    """Packed 6-bit operands with one E8M0 scale per 32 K (MXFP6): the oracle
    equals numpy's fp64 matmul of the decoded, block-scaled values."""
    rng = np.random.default_rng(22)
    M, N, K = 18, 22, 128
    ca = rng.integers(0, 64, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 64, (N, K)).astype(np.uint8)
    sa = rng.integers(124, 131, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(124, 131, (N, K // 32)).astype(np.uint8)
    code = {"e2m3": G.E2M3, "e3m2": G.E3M2}
    dec = {"e2m3": np.vectorize(G.e2m3_decode), "e3m2": np.vectorize(G.e3m2_decode)}
    a_real = dec[fa](ca) * np.repeat(2.0 ** (sa.astype(np.float64) - 127), 32, axis=1)
    b_real = dec[fb](cb) * np.repeat(2.0 ** (sb.astype(np.float64) - 127), 32, axis=1)
    A = G.packed(_pack_fp6(ca), (M, K), (K, 1), code[fa])
    B = G.packed(_pack_fp6(cb), (N, K), (K, 1), code[fb])
    d, ref, absum = G.gemm(A, B, None, sa, sb, block_k=32)
    assert np.array_equal(ref[0], a_real @ b_real.T)
    assert np.array_equal(absum[0], np.abs(a_real) @ np.abs(b_real).T)
    # a transposed storage of A (K rows of M packed codes) through strides
    # (1, M): element (m, k) at offset k*M + m
    At = G.packed(_pack_fp6(np.ascontiguousarray(ca.T).reshape(1, -1)), (M, K), (1, M), code[fa])
    _, ref_t, _ = G.gemm(At, B, None, sa, sb, block_k=32)
    assert np.array_equal(ref_t[0], ref[0])
