"""Device probes: the operand maps of the matrix-core instructions and the
LDS data paths, observed on the hardware, against the maps written in the
oracle's TV algebra.  These maps are hardware facts the pages do not fix
(parity unpinned by the pages); the probes pin them."""

import numpy as np
import pytest

from oracle import gemm as OG
from oracle import layout as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stride_layouts_lds_amd import api as A
    A.lib()
    return A


def _expected_f16(instr, mode):
    code = lambda l, s: l * 8 + s + 1
    f = L.probe_expected_onehot_A if mode == 0 else L.probe_expected_onehot_B
    return np.array([f(instr, c // 8, c % 8, code) for c in range(512)], np.float32)


@pytest.mark.parametrize("instr", [0, 1])
@pytest.mark.parametrize("mode", [0, 1])
def test_probe_f16_maps(api, instr, mode):
    from gpu_helpers import dump, log
    log(f"probe f16 instr={instr} mode={mode}")
    got = api.probe_mfma(instr, mode).cpu().numpy()
    dump(f"probe_f16_{instr}_{mode}", got)
    want = _expected_f16(instr, mode)
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} registers differ"


E4M3_BASE = 0x20


def _expected_f8(instr, mode):
    amap, bmap, dmap = L.INSTR_MAPS[instr]
    R = 16 if instr == 2 else 32
    dec = np.array([OG.e4m3_decode(E4M3_BASE + x) for x in range(64)], np.float32)
    dm = np.array([[dmap(l, i)[0] for i in range(dmap.values)] for l in range(64)])
    dn = np.array([[dmap(l, i)[1] for i in range(dmap.values)] for l in range(64)])
    binv, ainv = bmap.inverse(), amap.inverse()
    owner = {L.mfma_scale_owner(R, s): s for s in range(64)}
    out = np.zeros((64 * 32, 64, dmap.values), np.float32)
    for c in range(64 * 32):
        hl, hs = c // 32, c % 32
        if mode in (0, 1, 4):
            m0, k0 = amap(hl, hs)
            mask = dm == m0
            if mode == 4:
                out[c][mask] = 2.0 ** (owner[(m0, k0 // 32)] - 32)
            else:
                ls = np.array([binv[(n, k0)] for n in range(R)])  # (lane, slot) of B(n, k0)
                out[c][mask] = dec[ls[dn[mask], 0 if mode == 0 else 1]]
        else:
            n0, k0 = bmap(hl, hs)
            mask = dn == n0
            if mode == 5:
                out[c][mask] = 2.0 ** (owner[(n0, k0 // 32)] - 32)
            else:
                ls = np.array([ainv[(m, k0)] for m in range(R)])
                out[c][mask] = dec[ls[dm[mask], 0 if mode == 2 else 1]]
    return out


@pytest.mark.parametrize("instr", [2, 3])
@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_probe_f8_maps(api, instr, mode):
    from gpu_helpers import dump, log
    log(f"probe f8 instr={instr} mode={mode}")
    got = api.probe_mfma(instr, mode).cpu().numpy()
    dump(f"probe_f8_{instr}_{mode}", got)
    want = _expected_f8(instr, mode)
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} registers differ"


@pytest.mark.parametrize("mode", [0, 1])
def test_probe_direct_to_lds(api, mode):
    """A 16-byte direct HBM->LDS load of one wave writes lane l's bytes at
    LDS base + 16*l, whatever global address the lane fetched."""
    import torch
    from gpu_helpers import dump, log
    log(f"probe lds dma mode={mode}")
    rng = np.random.default_rng(5)
    src = (np.arange(1024) * 37 + 11).astype(np.uint8)
    perm = rng.permutation(64).astype(np.int32)
    if mode == 0:
        perm[[3, 17, 40]] = -1  # out-of-range lanes: must land as zeros
    got = api.probe_lds(mode, torch.from_numpy(src).cuda(), torch.from_numpy(perm).cuda()).cpu().numpy()
    dump(f"probe_lds_{mode}", got)
    want = np.full(4096, 0xA5, np.uint8)
    for l in range(64):
        want[16 * l:16 * l + 16] = 0 if perm[l] < 0 else src[16 * perm[l]:16 * perm[l] + 16]
    assert np.array_equal(got, want)


def test_probe_direct_to_lds_dword(api):
    """A 4-byte direct HBM->LDS load of one wave writes lane l's bytes at
    LDS base + 4*l."""
    import torch
    from gpu_helpers import log
    log("probe lds dma dword")
    rng = np.random.default_rng(6)
    src = (np.arange(1024) * 29 + 5).astype(np.uint8)
    perm = rng.permutation(256)[:64].astype(np.int32)
    got = api.probe_lds(3, torch.from_numpy(src).cuda(), torch.from_numpy(perm).cuda()).cpu().numpy()
    want = np.full(4096, 0xA5, np.uint8)
    for l in range(64):
        want[4 * l:4 * l + 4] = src[4 * perm[l]:4 * perm[l] + 4]
    assert np.array_equal(got, want)


def test_probe_ds_read_tr16(api):
    import torch
    from gpu_helpers import dump, log
    log("probe ds_read_b64_tr_b16")
    halves = np.arange(2048, dtype=np.uint16)
    # lane l of group g: 64-bit block at row (4g + i//4), columns 4*(i%4).. of
    # a matrix with 32 halves per row
    addr = np.array([((4 * (l // 16) + (l % 16) // 4) * 32 + 4 * (l % 4)) * 2 for l in range(64)], np.int32)
    got = api.probe_lds(2, torch.from_numpy(halves.view(np.uint8).copy()).cuda(),
                        torch.from_numpy(addr).cuda()).cpu().numpy()
    got = got[:512].view(np.uint16).reshape(64, 4)
    dump("probe_tr16", got)
    want = np.array(L.ds_read_tr16_b64_expected(addr.tolist(), halves.tolist()), np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("instr", [2, 3])
def test_probe_e2m1_operand_map(api, instr):
    """A in E2M1 one-hot at (lane, nibble) against an E4M3 B whose map is
    pinned above: the output row gives m and the B codes (lane-coded, then
    byte-coded) give k, i.e. the E2M1 (lane, nibble) -> (m, k) map, compared
    with the reading in the oracle."""
    from gpu_helpers import dump, log
    log(f"probe e2m1 instr={instr}")
    got6 = api.probe_mfma(instr, 6).cpu().numpy()
    got7 = api.probe_mfma(instr, 7).cpu().numpy()
    amap, bmap, dmap = L.INSTR_MAPS[instr]
    famap = L.MFMA16_F4_A if instr == 2 else L.MFMA32_F4_A
    dec = {float(OG.e4m3_decode(E4M3_BASE + x)): x for x in range(64)}
    measured, bad = {}, 0
    for c in range(64 * 32):
        hl, hs = c // 32, c % 32
        nz6 = np.argwhere(got6[c] != 0)
        if len(nz6) == 0:
            measured[(hl, hs)] = None
            continue
        l, i = nz6[0]
        m, n = dmap(int(l), int(i))
        lane_b = dec[float(got6[c][l, i])]
        slot_b = dec[float(got7[c][l, i])]
        nb, kb = bmap(lane_b, slot_b)
        measured[(hl, hs)] = (m, kb)
        if (m, kb) != famap(hl, hs):
            bad += 1
    if bad:
        dump(f"probe_e2m1_{instr}", np.array([[h, s_, *(measured[(h, s_)] or (-1, -1))]
                                               for h in range(64) for s_ in range(32)], np.int32))
    assert bad == 0, f"{bad} of 2048 (lane, nibble) differ from the reading; e.g. " + str(
        [(k, v, famap(*k)) for k, v in list(measured.items()) if v != famap(*k)][:6])


def _measured_onehot_map(api, instr, mode_lane, mode_slot):
    """(lane, value) -> (m, k) of a one-hot A against the byte-coded E4M3 B
    (lane codes in mode_lane, slot codes in mode_slot); None where the
    one-hot produced no output."""
    got_l = api.probe_mfma(instr, mode_lane).cpu().numpy()
    got_s = api.probe_mfma(instr, mode_slot).cpu().numpy()
    amap, bmap, dmap = L.INSTR_MAPS[instr]
    dec = {float(OG.e4m3_decode(E4M3_BASE + x)): x for x in range(64)}
    measured = {}
    for c in range(64 * 32):
        hl, hs = c // 32, c % 32
        nz = np.argwhere(got_l[c] != 0)
        if len(nz) == 0:
            measured[(hl, hs)] = None
            continue
        l, i = nz[0]
        m, n = dmap(int(l), int(i))
        lane_b, slot_b = dec.get(float(got_l[c][l, i])), dec.get(float(got_s[c][l, i]))
        if lane_b is None or slot_b is None:
            measured[(hl, hs)] = (-2, -2)  # not a single B value: the one-hot did not read as 1.0
            continue
        measured[(hl, hs)] = (m, bmap(lane_b, slot_b)[1])
    return measured


@pytest.mark.parametrize("instr", [2, 3])
@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_probe_fp6_operand_map(api, instr, fmt):
    """A in a 6-bit format (E2M3 or E3M2), one-hot 1.0 at (lane, value) with
    a lane's 32 values packed as a little-endian bit stream, against the
    pinned E4M3 B: the measured (lane, value) -> (m, k) map against the
    oracle's reading."""
    from gpu_helpers import dump, log
    log(f"probe fp6 instr={instr} fmt={fmt}")
    modes = (8, 9) if fmt == "e2m3" else (10, 11)
    measured = _measured_onehot_map(api, instr, *modes)
    want = L.MFMA16_F6_A if instr == 2 else L.MFMA32_F6_A
    bad = [(k, v, want(*k)) for k, v in measured.items() if v != want(*k)]
    if bad:
        dump(f"probe_fp6_{fmt}_{instr}", np.array([[h, s_, *(measured[(h, s_)] or (-1, -1))]
                                                   for h in range(64) for s_ in range(32)], np.int32))
    assert not bad, f"{len(bad)} of 2048 (lane, value) differ from the reading; e.g. {bad[:6]}"
