"""Size limits on the GPU: operands larger than 4 GiB, K = 2^20 through the
split-K path, a strided view spanning 8 GiB on the element loader, and
thousands of batches, each against the oracle (sampled points where the full
product is too large).  Values are small integers, so the fp32 sums are exact
and the comparisons are within the acceptance bound (exact in practice)."""

import numpy as np
import pytest

from stride_layouts_lds_amd.inputs import HostOperand, Workload

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


def int_codes(rng, rows, cols, chunk=8192):
    """(rows, cols) fp16 codes of integers in [-4, 4], drawn in row chunks
    to keep the host's temporaries small."""
    out = np.empty((rows, cols), np.uint16)
    for r in range(0, rows, chunk):
        n = min(chunk, rows - r)
        out[r:r + n] = rng.integers(-4, 5, (n, cols), dtype=np.int8).astype(np.float16).view(np.uint16)
    return out


def workload(name, a, b, M, N, K, c=None, batch=1):
    d_shape = (M, N) if batch == 1 and a.ndim == 2 else (batch, M, N)
    d_strides = (N, 1) if len(d_shape) == 2 else (M * N, N, 1)

    def op(x):
        if x is None:
            return None
        st = tuple(s // x.itemsize for s in x.strides)
        return HostOperand(x.reshape(-1) if x.flags.c_contiguous else x, x.shape, st, "f16")
    return Workload(name, M, N, K, batch, op(a), op(b), op(c), None, None, 32, d_shape, d_strides)


def check_sampled(api, w, n=600, split=None):
    """Runs w once (inputs copied to the device once), checks the plan's
    K-split if asked, and compares sampled outputs with the oracle."""
    import torch
    h = H()
    a, b, c = h.to_device(w.a), h.to_device(w.b), h.to_device(w.c)
    out = torch.empty(w.d_shape, dtype=torch.float16, device="cuda")
    args = api.make_args(a, b, c, out)
    ws = api.workspace_for(args)
    api.set_workspace(args, ws)
    plan = api.sl_gemm_plan(args)
    h.log(f"{w.name}: plan {plan}")
    if split is not None:
        assert plan["split_k"] == split
    api.sl_gemm(args)
    torch.cuda.synchronize()
    d = h.d_codes(out).reshape(w.batch, w.M, w.N)
    pts = h.sample_points(w, n)
    d_ref, _, absum = h.oracle_points(w, pts)
    h.assert_within_bound(d[pts[:, 0], pts[:, 1], pts[:, 2]], d_ref, absum, w.name)
    del a, b, c, out
    torch.cuda.empty_cache()


def test_operand_larger_than_4gib(api):
    """A is 131072 x 16384 fp16 (4 GiB, K-contiguous): every tile's copies
    are addressed from the tile's own base, so only a tile (256 rows) must
    fit the 32-bit buffer range."""
    rng = np.random.default_rng(41)
    M, N, K = 131072, 64, 16384
    a = int_codes(rng, M, K)
    b = int_codes(rng, N, K)
    check_sampled(api, workload("a_4gib", a, b, M, N, K))


def test_k_of_2_pow_20_split(api):
    """K = 1048576 on a 128 x 128 output: split-K with 8 splits of 2048
    K-tiles each."""
    rng = np.random.default_rng(42)
    M, N, K = 128, 128, 1 << 20
    check_sampled(api, workload("k_2e20", int_codes(rng, M, K), int_codes(rng, N, K), M, N, K), n=300, split=8)


def test_row_stride_spanning_8gib(api):
    """A (512, 64) viewed with a row stride of 2^23 elements (8 GiB between
    its first and last row): the element loader's 64-bit offsets."""
    import torch
    h = H()
    rng = np.random.default_rng(43)
    M, N, K = 512, 256, 64
    rs = 1 << 23
    a = int_codes(rng, M, K)
    b = int_codes(rng, N, K)
    big = torch.empty(M * rs, dtype=torch.float16, device="cuda")
    a_dev = big.as_strided((M, K), (rs, 1))
    a_dev.copy_(torch.from_numpy(a).view(torch.float16).cuda())
    b_dev = torch.from_numpy(b).view(torch.float16).cuda()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    args = api.make_args(a_dev, b_dev, None, out)
    plan = api.sl_gemm_plan(args)
    h.log(f"row stride 2^23 plan {plan}")
    assert plan["a_load"] == 2  # the element loader
    api.sl_gemm(args)
    torch.cuda.synchronize()
    w = workload("rs_2e23", a, b, M, N, K)
    d_ref, _, _ = h.oracle_full(w)
    d = h.d_codes(out)
    assert np.count_nonzero(d.reshape(d_ref.shape) != d_ref) == 0
    del big
    torch.cuda.empty_cache()


def test_4096_batches_with_broadcast_b(api):
    """4096 batches of a ragged 40 x 24 x 72 product, B broadcast over the
    batch (stride 0), C present: exact."""
    h = H()
    rng = np.random.default_rng(44)
    batch, M, N, K = 4096, 40, 24, 72
    a = int_codes(rng, batch * M, K).reshape(batch, M, K)
    b = int_codes(rng, N, K)
    c = int_codes(rng, batch * M, N).reshape(batch, M, N)
    w = workload("batch_4096", a, b, M, N, K, c=c, batch=batch)
    w.b = HostOperand(b.reshape(-1), (batch, N, K), (0, K, 1), "f16")  # broadcast over the batch
    d = h.d_codes(h.run_library(w))
    d_ref, _, _ = h.oracle_full(w)
    assert np.count_nonzero(d.reshape(d_ref.shape) != d_ref) == 0
