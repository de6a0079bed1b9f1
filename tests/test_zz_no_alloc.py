"""sl_gemm_no_alloc, the entry point for callers that cannot allocate device
memory, against sl_gemm through the C ABI: the same plans and kernels, with
a split-K plan's partial sums in the library's static device scratch
instead of the caller's workspace.  Two split-K calls in a row (the second
smaller, on the scratch the first left behind), then an unsplit one; each
output must equal sl_gemm's bit for bit, and the oracle's (integer data,
exact sums).  NVFP4, which sl_gemm decodes ahead into its workspace from
2048^3 on, runs the fused kernel here: the same D."""

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


CALLS = [
    # M, N, K, with C, forced tile / K-split (None: the planner's), splits the plan must have
    (8192, 128, 8192, False, None, 4),   # the skinny workload: 16 MiB of partial sums
    (1000, 120, 3000, True, (16, 4), 4),  # smaller and ragged, after the first
    (512, 512, 256, True, None, 1),      # no split: the scratch is not touched
]


def test_no_alloc_matches_sl_gemm(api, monkeypatch):
    import torch
    h = H()
    for M, N, K, with_c, force, splits in CALLS:
        if force:
            monkeypatch.setenv("SL_TILE", str(force[0]))
            monkeypatch.setenv("SL_SPLITK", str(force[1]))
        else:
            monkeypatch.delenv("SL_TILE", raising=False)
            monkeypatch.delenv("SL_SPLITK", raising=False)
        w = I.gemm_workload("no_alloc", M, N, K, seed=M + N + K, dist="int4", with_c=with_c)
        a, b, c = h.to_device(w.a), h.to_device(w.b), h.to_device(w.c)
        ref = torch.full(w.d_shape, float("nan"), dtype=torch.float16, device="cuda")
        out = torch.full(w.d_shape, float("nan"), dtype=torch.float16, device="cuda")
        args = api.make_args(a, b, c, ref)
        plan = api.sl_gemm_plan(args)
        h.log(f"no_alloc {M}x{N}x{K} c={with_c} plan={plan}")
        assert plan["split_k"] == splits
        assert plan["workspace_bytes"] <= api.SL_NO_ALLOC_SCRATCH_BYTES
        api.set_workspace(args, api.workspace_for(args))
        api.sl_gemm(args)
        args_na = api.make_args(a, b, c, out)  # no workspace: the static scratch serves
        api.sl_gemm_no_alloc(args_na)
        torch.cuda.synchronize()
        got, want = h.d_codes(out), h.d_codes(ref)
        assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} elements differ from sl_gemm"
        d_ref, _, _ = h.oracle_full(w)
        assert np.array_equal(got, d_ref[0]), f"{np.count_nonzero(got != d_ref[0])} elements differ from the oracle"


def test_no_alloc_nvfp4_uses_the_fused_kernels(api, monkeypatch):
    """NVFP4 with its operands decoded ahead (forced here; sl_gemm's plan
    from 2048^3 on) against sl_gemm_no_alloc, which keeps the fused kernel
    and needs no workspace: the same D bit for bit, and the oracle's (exact
    data and scales)."""
    import torch
    h = H()
    monkeypatch.delenv("SL_TILE", raising=False)
    monkeypatch.setenv("SL_NV_DECODE", "1")
    M, N, K = 512, 264, 1024
    w = I.nvfp4_workload("no_alloc_nvfp4", M, N, K, seed=7, with_c=True, exact=True)
    a, b, c = h.to_device(w.a), h.to_device(w.b), h.to_device(w.c)
    sfa, sfb = h.to_device(w.sfa), h.to_device(w.sfb)
    ref = torch.full(w.d_shape, float("nan"), dtype=torch.float16, device="cuda")
    out = torch.full(w.d_shape, float("nan"), dtype=torch.float16, device="cuda")
    args = api.make_args(a, b, c, ref, sfa, sfb, w.block_k)
    plan = api.sl_gemm_plan(args)
    h.log(f"no_alloc nvfp4 {M}x{N}x{K} plan={plan}")
    assert plan["a_load"] == 0 and plan["workspace_bytes"] > 0  # decoded ahead
    api.set_workspace(args, api.workspace_for(args))
    api.sl_gemm(args)
    api.sl_gemm_no_alloc(api.make_args(a, b, c, out, sfa, sfb, w.block_k))
    torch.cuda.synchronize()
    got, want = h.d_codes(out), h.d_codes(ref)
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} elements differ from sl_gemm"
    d_ref, _, _ = h.oracle_full(w)
    assert np.array_equal(got.reshape(d_ref.shape), d_ref), "differs from the oracle"
