"""The 4-wave 256x256 kernels (gemm_f16_w4r_kernel, gemm_mx_w4r_kernel) issue
their MFMAs as inline assembly on accumulators pinned to AGPRs, so the
compiler inserts no wait states around them and would not notice if it moved
an accumulator while an MFMA still writes it.  These host checks read the
library's own gfx950 code (the device code objects built from gemm_f16.hip
and gemm_mx.hip, disassembled with ROCm's llvm-objdump) and verify, for the instantiations listed in KERNELS (fp16 and
bf16 with K- or M-major loaders and 256- or 192-wide tiles, MXFP8, MXFP6 and
MXFP4; row and per-quad epilogues):

- the accumulators never move between the first and the last MFMA (no AGPR
  reads, writes or copies, no scratch traffic anywhere in the kernel);
- every MFMA accumulates in place, and an accumulator is written again only
  after at least 16 other instructions (straight-line, and around the
  K-loop);
- no vector-ALU write reaches an MFMA operand (data or scale) within 4
  instructions;
- after the last MFMA, at least 18 wait states pass before the first
  accumulator is read (the instruction's passes plus two need fewer);
- every s_barrier comes after a wait for all of the wave's LDS reads
  (lgkmcnt(0)) with no LDS read between: after the barrier other waves
  overwrite the ring slots this wave has just read.  The wait is issued
  through the compiler's builtin, which its wait-count pass may merge with a
  neighbouring wait; this checks that it survives as a full LDS wait.
"""

import os
import re
import subprocess

import pytest

LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
# name: (symbol, MFMAs of one K-loop iteration, MFMAs after the loop).
# 16-bit ring kernels: element type, epilogue through LDS rows or per
# accumulator quad, loaders (K-major, or M-major direct copies), tile width
# tile width and whether every K-tile is whole (copies without per-lane masks)
F16 = "_ZN2sl12_GLOBAL__N_119gemm_f16_w4r_kernelILi0ELi{d}ELb{r}ELi{al}ELi{bl}ELi{bn}ELb{kf}EEEvNS_10GemmParamsE"
KERNELS = {
    f"{dt}_{ep}{kn}": (F16.format(d=d, r=r, al=0, bl=0, bn=256, kf=kf), 128, 32)
    for d, dt in ((0, "fp16"), (1, "bf16")) for r, ep in ((1, "rows"), (0, "quads"))
    for kf, kn in ((0, ""), (1, "_kfull"))
}
KERNELS.update({
    f"{dt}_mn{al}{bl}_{ep}": (F16.format(d=d, r=r, al=al, bl=bl, bn=256, kf=0), 128, 32)
    for d, dt in ((0, "fp16"), (1, "bf16"))
    for al, bl in ((3, 0), (0, 3), (3, 3)) for r, ep in ((1, "rows"), (0, "quads"))
})
KERNELS.update({f"{dt}_256x192{kn}": (F16.format(d=d, r=0, al=0, bl=0, bn=192, kf=kf), 96, 24)
                for d, dt in ((0, "fp16"), (1, "bf16")) for kf, kn in ((0, ""), (1, "_kfull"))})
# NVFP4 on the ring schedule (decoding loaders, per K-tile or per pair)
KERNELS.update({
    f"nvfp4_{pn}_{ep}": (f"_ZN2sl12_GLOBAL__N_121gemm_nvfp4_w4r_kernelILi0ELb{pr}ELb{r}EEEvNS_10GemmParamsE", 128, 32)
    for pr, pn in ((1, "pairs"), (0, "tiles")) for r, ep in ((1, "rows"), (0, "quads"))
})
# the MX ring kernel: 128 scaled MFMAs per loop iteration (four K-tiles of 32
# for 8- and 6-bit data, two of 64 for E2M1), 8 after it
# (whole K-tiles for every format; E4M3 also with a partial last K-tile)
KERNELS.update({
    f"{fn}_{ep}{kn}": (f"_ZN2sl12_GLOBAL__N_118gemm_mx_w4r_kernelILi0ELb{r}ELi{f}ELb{kf}EEEvNS_10GemmParamsE", 128, 8)
    for f, fn in ((0, "mxfp8"), (2, "mxfp6_e2m3"), (3, "mxfp6_e3m2"), (4, "mxfp4")) for r, ep in ((1, "rows"), (0, "quads"))
    for kf, kn in ((1, ""), (0, "_kpart")) if kf == 1 or f == 0
})


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    from stride_layouts_lds_amd import api as A
    if not os.path.exists(A.LIB_PATH):
        from stride_layouts_lds_amd import build
        build.build(verbose=False)
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not found under {LLVM}")
    d = tmp_path_factory.mktemp("code")
    fat = d / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", A.LIB_PATH, str(d / "x")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    assert starts, "no offload bundle in the library"
    cos = []
    for k, a in enumerate(starts):
        b = starts[k + 1] if k + 1 < len(starts) else len(data)
        bundle = d / f"b{k}.bin"
        bundle.write_bytes(data[a:b])
        co = d / f"b{k}.co"
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={bundle}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True, capture_output=True)
        cos.append(str(co))
    return cos


def disassemble(cos, symbol):
    for co in cos:
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", f"--disassemble-symbols={symbol}",
                            co], check=True, capture_output=True, text=True)
        lines = [l.split("//")[0].strip() for l in r.stdout.splitlines()]
        lines = [l for l in lines if l and not l.endswith(">:") and not l.startswith("Disassembly")
                 and ":" not in l.split()[0]]
        if any(l.startswith("v_mfma") for l in lines):
            return lines
    raise AssertionError(f"{symbol} not found in the library's code objects")


def regs(tok):
    m = re.match(r"([vas])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([vas])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.mark.parametrize("dtype", sorted(KERNELS))
def test_ring_kernel_accumulator_discipline(code_objects, dtype):
    symbol, in_loop, after = KERNELS[dtype]
    L = disassemble(code_objects, symbol)
    ops = [l.replace(",", " ").split() for l in L]
    mf = [k for k, o in enumerate(ops) if o[0].startswith("v_mfma")]
    assert len(mf) == in_loop + after, f"{len(mf)} MFMAs ({in_loop} in the K-loop and {after} after it expected)"
    first, last = mf[0], mf[-1]

    assert not [l for l in L if l.startswith("scratch_")], "scratch traffic"
    moved = [L[k] for k in range(first, last) if ops[k][0].startswith("v_accvgpr")]
    assert not moved, f"accumulators moved inside the MFMA stream: {moved[:3]}"

    # accumulate in place; the same accumulator rewritten only after >= 16
    # instructions, in straight-line order and around the K-loop (the first
    # 128 MFMAs, taken cyclically)
    for k in mf:
        assert ops[k][1] == ops[k][4], f"not accumulating in place: {L[k]}"
    seen = {}
    for k in mf:
        if ops[k][1] in seen:
            assert k - seen[ops[k][1]] >= 16, f"{L[k]} within 16 instructions of its previous write"
        seen[ops[k][1]] = k
    loop = mf[:in_loop]
    span = loop[-1] - loop[0] + 1
    for a in range(in_loop):
        for b in range(a + 1, in_loop):
            if ops[loop[a]][1] == ops[loop[b]][1]:
                assert loop[a] + span - loop[b] >= 16, "accumulator rewritten too soon around the loop"

    # no vector-ALU write to an MFMA operand within 4 instructions
    last_write = {}
    for k, o in enumerate(ops):
        if o[0].startswith("v_mfma"):
            # operands A and B, and the scale registers of the scaled form
            for r in regs(o[2]) | regs(o[3]) | set().union(*(regs(x) for x in o[5:7])):
                w = last_write.get(r)
                assert w is None or k - w >= 4, f"{L[w]} feeds {L[k]} too closely"
        elif o[0].startswith("v_") and len(o) > 1:
            for r in regs(o[1]):
                last_write[r] = k

    # wait states between the last MFMA and the first instruction that reads
    # an accumulator (an AGPR copy, or an LDS or memory write of AGPR data)
    reads = [k for k in range(last + 1, len(L)) if any(regs(t) and next(iter(regs(t)))[0] == "a" for t in ops[k][1:])]
    assert reads, "accumulators never read"
    nops = sum(int(o[1]) + 1 for o in ops[last + 1:reads[0]] if o[0] == "s_nop")
    assert nops >= 18, f"{nops} wait states before the first accumulator read ({L[reads[0]]})"



def disassemble_cfg(cos, symbol):
    """(instruction, successor indices) per instruction of the symbol, from
    the disassembly's addresses and branch targets."""
    for co in cos:
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", f"--disassemble-symbols={symbol}",
                            co], check=True, capture_output=True, text=True)
        ins = []
        for line in r.stdout.splitlines():
            m = re.match(r"\s+(\S.*?)\s*//\s*([0-9A-Fa-f]+):", line)
            if m:
                t = re.search(r"<[^>+]+\+0x([0-9a-fA-F]+)>", line)
                ins.append((m.group(1).strip(), int(m.group(2), 16), int(t.group(1), 16) if t else None))
        if any(i[0].startswith("v_mfma") for i in ins):
            break
    else:
        raise AssertionError(f"{symbol} not found in the library's code objects")
    base = ins[0][1]
    at = {addr: k for k, (_, addr, _) in enumerate(ins)}
    succ = []
    for k, (text, addr, off) in enumerate(ins):
        op = text.split()[0]
        nxt = [] if op in ("s_branch", "s_endpgm", "s_setpc_b64") or k + 1 == len(ins) else [k + 1]
        if op.startswith("s_cbranch") or op == "s_branch":
            assert off is not None and base + off in at, f"branch target of {text} not found"
            nxt.append(at[base + off])
        succ.append(nxt)
    return [i[0] for i in ins], succ


def unwaited_lds_before(text, succ, b):
    """An LDS instruction from which some path reaches instruction b without
    passing an s_waitcnt with lgkmcnt(0), or None."""
    pred = [[] for _ in text]
    for k, ss in enumerate(succ):
        for j in ss:
            pred[j].append(k)
    seen, stack = set(), list(pred[b])
    while stack:
        k = stack.pop()
        if k in seen:
            continue
        seen.add(k)
        t = text[k]
        if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
            continue
        if t.startswith("ds_"):
            return t
        stack.extend(pred[k])
    return None


def test_unwaited_lds_walk_on_small_graphs():
    """The path walk on hand-made instruction lists: a straight line, a
    branch around the wait, and a loop whose back edge skips it."""
    line = ["ds_read_b128 v[0:3], v4", "s_waitcnt lgkmcnt(0)", "s_barrier"]
    assert unwaited_lds_before(line, [[1], [2], []], 2) is None
    assert unwaited_lds_before(["ds_read_b128 v[0:3], v4", "s_waitcnt lgkmcnt(1)", "s_barrier"], [[1], [2], []], 2)
    # 0: read, 1: conditional branch to 3 (skips the wait at 2), 3: barrier
    br = ["ds_read_b128 v[0:3], v4", "s_cbranch_scc1 1", "s_waitcnt lgkmcnt(0)", "s_barrier"]
    assert unwaited_lds_before(br, [[1], [2, 3], [3], []], 3) == br[0]
    # loop 0..3 with the barrier at its top: 0 barrier, 1 wait, 2 read, 3 branch back to 0
    lp = ["s_barrier", "s_waitcnt lgkmcnt(0)", "ds_read_b128 v[0:3], v4", "s_cbranch_scc1 -4"]
    assert unwaited_lds_before(lp, [[1], [2], [3], [0]], 0) == lp[2]
    lp_ok = ["s_barrier", "ds_read_b128 v[0:3], v4", "s_waitcnt lgkmcnt(0)", "s_cbranch_scc1 -4"]
    assert unwaited_lds_before(lp_ok, [[1], [2], [3], [0]], 0) is None


@pytest.mark.parametrize("dtype", sorted(KERNELS))
def test_ring_kernel_barriers_follow_lds_waits(code_objects, dtype):
    text, succ = disassemble_cfg(code_objects, KERNELS[dtype][0])
    bars = [k for k, t in enumerate(text) if t.split()[0] == "s_barrier"]
    assert bars, "no barrier"
    for b in bars:
        # every path into the barrier passes a full LDS wait after its last
        # LDS instruction (or has none)
        t = unwaited_lds_before(text, succ, b)
        assert t is None, f"a path reaches the barrier at {b} from {t} without an lgkmcnt(0) wait"
