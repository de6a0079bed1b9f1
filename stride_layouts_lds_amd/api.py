"""ctypes binding of ``include/sl.h`` with the same names.

Argument marshalling only: every step of the GEMM runs in the HIP library.
PyTorch supplies device memory and the current HIP stream.  If the library
is not built, every call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstride_layouts_lds.so")

SL_F16, SL_F32, SL_F8_E4M3, SL_E8M0, SL_BF16, SL_F4_E2M1, SL_F6_E2M3, SL_F6_E3M2 = 1, 2, 3, 4, 5, 6, 7, 8
K_F16, K_F16_GENERIC, K_MX, K_MX_W8, K_NVFP4, K_MXFP4, K_MXFP6, K_MX_W4R = 1, 2, 3, 4, 5, 6, 7, 8
STATUS = {0: "SL_OK", -1: "SL_ERR_NULL", -2: "SL_ERR_DTYPE", -3: "SL_ERR_SHAPE", -4: "SL_ERR_LAYOUT",
          -5: "SL_ERR_ALIGN", -6: "SL_ERR_ALIAS", -7: "SL_ERR_ARCH", -8: "SL_ERR_LAUNCH", -9: "SL_ERR_ARG"}

# every symbol include/sl.h declares
EXPORTS = ["sl_gemm", "sl_gemm_no_alloc", "sl_gemm_plan", "sl_gemm_workspace_bytes", "sl_status_string", "sl_last_error_message",
           "sl_abi_version", "sl_query_fragment_map", "sl_query_lds_map", "sl_query_fragment_addresses", "sl_probe_mfma",
           "sl_probe_lds", "sl_layout_op", "sl_describe_plan"]

# sl_layout_op operations (include/sl.h)
LA_OPS = {"parse": 0, "coalesce": 1, "composition": 2, "complement": 3, "right_inverse": 4,
          "zipped_divide": 5, "filter_zeros": 6, "compact_left": 7, "make_ordered": 8,
          "logical_product": 9, "tiled_product": 10, "fragment_like": 11, "tensor_like": 12,
          "eval": 13, "size": 14, "cosize": 15}
SL_LA_MARK_STATIC = 256
SL_NO_ALLOC_SCRATCH_BYTES = 32 << 20  # the static scratch of sl_gemm_no_alloc (include/sl.h)


class sl_layout(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


class sl_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("layout", sl_layout)]


class sl_gemm_args(ctypes.Structure):
    _fields_ = [("a", sl_tensor), ("b", sl_tensor), ("c", sl_tensor), ("d", sl_tensor), ("sfa", sl_tensor),
                ("sfb", sl_tensor), ("block_k", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_int64)]


class sl_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("a_load", ctypes.c_int32), ("b_load", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("split_k", ctypes.c_int32), ("workgroups", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int32), ("batch", ctypes.c_int64), ("m", ctypes.c_int64),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


class SLError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m stride_layouts_lds_amd.build` "
                               "(the GEMM has no other implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.sl_gemm.restype = i32
        L.sl_gemm.argtypes = [P(sl_gemm_args), vp]
        L.sl_gemm_no_alloc.restype = i32
        L.sl_gemm_no_alloc.argtypes = [P(sl_gemm_args), vp]
        L.sl_gemm_plan.restype = i32
        L.sl_gemm_plan.argtypes = [P(sl_gemm_args), P(sl_plan)]
        L.sl_gemm_workspace_bytes.restype = i32
        L.sl_gemm_workspace_bytes.argtypes = [P(sl_gemm_args), P(i64)]
        L.sl_status_string.restype = ctypes.c_char_p
        L.sl_status_string.argtypes = [i32]
        L.sl_last_error_message.restype = ctypes.c_char_p
        L.sl_last_error_message.argtypes = []
        L.sl_abi_version.restype = i32
        L.sl_query_fragment_map.restype = i32
        L.sl_query_fragment_map.argtypes = [i32, i32, vp, vp, vp, vp, i64, P(i64)]
        L.sl_query_lds_map.restype = i32
        L.sl_query_lds_map.argtypes = [i32, i32, vp, i64, P(i32), P(i32), P(i32)]
        L.sl_query_fragment_addresses.restype = i32
        L.sl_query_fragment_addresses.argtypes = [i32, i32, vp, i64, P(i64)]
        L.sl_probe_mfma.restype = i32
        L.sl_probe_mfma.argtypes = [i32, i32, vp, i64, P(i64), vp]
        L.sl_probe_lds.restype = i32
        L.sl_probe_lds.argtypes = [i32, vp, vp, vp, vp]
        L.sl_layout_op.restype = i32
        L.sl_layout_op.argtypes = [i32, ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, i64, P(i64)]
        L.sl_describe_plan.restype = i32
        L.sl_describe_plan.argtypes = [P(sl_gemm_args), ctypes.c_char_p, i64, P(i64)]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise SLError(status, lib().sl_last_error_message().decode())


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def desc(data: int, dtype: int, shape: Sequence[int], strides: Sequence[int]) -> sl_tensor:
    """A raw descriptor: pointer, sl_dtype, shape and element strides."""
    t = sl_tensor()
    t.data = data or None
    t.dtype = dtype
    t.layout.rank = len(shape)
    for i, (n, s) in enumerate(zip(shape, strides)):
        t.layout.shape[i] = int(n)
        t.layout.stride[i] = int(s)
    return t


def _torch_dtype_code(x, override: Optional[int]) -> int:
    import torch
    if override is not None:
        return override
    table = {torch.float16: SL_F16, torch.bfloat16: SL_BF16, torch.float32: SL_F32, torch.float8_e4m3fn: SL_F8_E4M3,
             torch.float8_e8m0fnu: SL_E8M0}
    if x.dtype not in table:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return table[x.dtype]


class PackedTensor:
    """Packed sub-byte data torch has no dtype for (6-bit E2M3 / E3M2): the
    storage bytes (a device uint8 tensor), the sl_dtype code, and the
    (batch?, rows, cols) shape with strides in elements."""

    def __init__(self, storage, dtype: int, shape, strides):
        self.storage, self.dtype, self.shape, self.strides = storage, dtype, tuple(shape), tuple(strides)


def tensor_desc(x, dtype: Optional[int] = None) -> sl_tensor:
    """Descriptor of a torch tensor or PackedTensor (None: absent operand)."""
    if isinstance(x, PackedTensor):
        return desc(x.storage.data_ptr(), x.dtype, x.shape, x.strides)
    if x is None:
        t = sl_tensor()
        t.data = None
        t.dtype = 0
        t.layout.rank = 2
        return t
    import torch
    if x.dtype == torch.float4_e2m1fn_x2:
        # two E2M1 elements per item, packed along the unit-stride last axis
        if x.stride(-1) != 1:
            raise ValueError("packed E2M1 needs a unit stride on the last axis")
        shape = tuple(x.shape[:-1]) + (2 * x.shape[-1],)
        strides = tuple(2 * s for s in x.stride()[:-1]) + (1,)
        return desc(x.data_ptr(), SL_F4_E2M1, shape, strides)
    return desc(x.data_ptr(), _torch_dtype_code(x, dtype), tuple(x.shape), tuple(x.stride()))


def make_args(a, b, c=None, d=None, sfa=None, sfb=None, block_k: int = 32, workspace=None) -> sl_gemm_args:
    """Arguments from descriptors (sl_tensor) or torch tensors; ``workspace``
    is a device tensor (its bytes) or None."""
    args = sl_gemm_args()
    for name, v in (("a", a), ("b", b), ("c", c), ("d", d), ("sfa", sfa), ("sfb", sfb)):
        setattr(args, name, v if isinstance(v, sl_tensor) else tensor_desc(v))
    args.block_k = block_k
    set_workspace(args, workspace)
    return args


def set_workspace(args: sl_gemm_args, workspace) -> None:
    """Point args at a device tensor's bytes as the split-K workspace (None: none)."""
    if workspace is None:
        args.workspace, args.workspace_bytes = None, 0
    else:
        args.workspace = workspace.data_ptr() or None
        args.workspace_bytes = workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# the entry points
# ---------------------------------------------------------------------------

def sl_gemm(args: sl_gemm_args, stream: Optional[int] = None) -> None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    _check(lib().sl_gemm(ctypes.byref(args), ctypes.c_void_p(stream)))


def sl_gemm_no_alloc(args: sl_gemm_args, stream: Optional[int] = None) -> None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    _check(lib().sl_gemm_no_alloc(ctypes.byref(args), ctypes.c_void_p(stream)))


def sl_gemm_workspace_bytes(args: sl_gemm_args) -> int:
    n = ctypes.c_int64(0)
    _check(lib().sl_gemm_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def workspace_for(args: sl_gemm_args, device=None):
    """A torch uint8 device tensor of the workspace bytes the plan needs
    (None when it needs none)."""
    n = sl_gemm_workspace_bytes(args)
    if n == 0:
        return None
    import torch
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def sl_gemm_plan(args: sl_gemm_args) -> dict:
    p = sl_plan()
    _check(lib().sl_gemm_plan(ctypes.byref(args), ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in sl_plan._fields_}


def gemm(a, b, c=None, out=None, sfa=None, sfb=None, block_k: int = 32, stream: Optional[int] = None,
         workspace=None):
    """D = A B^T + C on torch tensors (any strides).  ``a``: (batch?, M, K)
    fp16, bf16 or float8_e4m3fn; ``b``: (batch?, N, K); ``c``: (batch?, M, N)
    of D's dtype (bf16 for bf16 operands, else fp16) or None; ``sfa``/``sfb``: float8_e8m0fnu scales (batch?, rows, K/32) for
    the MX form.  A plan's workspace (split-K partial sums, or NVFP4
    operands decoded to fp16) is ``workspace`` (a device tensor) or, when
    None, a torch allocation of the size the library asks for.  Returns ``out`` (allocated by torch if None)."""
    import torch
    if out is None:
        batch = max(x.shape[0] if x is not None and x.dim() == 3 else 0 for x in (a, b, c))
        shape = (a.shape[-2], b.shape[-2]) if batch == 0 else (batch, a.shape[-2], b.shape[-2])
        out = torch.empty(shape, dtype=torch.bfloat16 if a.dtype == torch.bfloat16 else torch.float16,
                          device=a.device)
    args = make_args(a, b, c, out, sfa, sfb, block_k)
    if workspace is None:
        workspace = workspace_for(args, out.device)
    set_workspace(args, workspace)
    sl_gemm(args, stream)
    return out


def _text_call(fn) -> str:
    """Runs fn(buffer, capacity, needed) and grows the buffer once if needed."""
    need = ctypes.c_int64(0)
    buf = ctypes.create_string_buffer(1 << 14)
    st = fn(buf, len(buf), ctypes.byref(need))
    if st == -3 and need.value > len(buf):
        buf = ctypes.create_string_buffer(need.value)
        st = fn(buf, len(buf), ctypes.byref(need))
    _check(st)
    return buf.value.decode()


def layout_op(op: str, a: str, b=None, mark_static: bool = False) -> str:
    """sl_layout_op by name: layout_op("composition", "(16,16):(16,1)", "(2,2,2):(16,8,128)")."""
    code = LA_OPS[op] | (SL_LA_MARK_STATIC if mark_static else 0)
    bb = None if b is None else str(b).encode()
    return _text_call(lambda buf, cap, need: lib().sl_layout_op(code, a.encode(), bb, buf, cap, need))


def describe_plan(args: sl_gemm_args) -> str:
    """sl_describe_plan: the layout of every stage of the planned GEMM."""
    return _text_call(lambda buf, cap, need: lib().sl_describe_plan(ctypes.byref(args), buf, cap, need))


def describe_stages(text: str) -> dict:
    """{name: layout text} of the stage lines of a describe_plan trace."""
    out = {}
    for line in text.splitlines():
        if line.startswith("#") or ": " not in line:
            continue
        name, rest = line.split(": ", 1)
        out[name] = rest.split("  #", 1)[0].strip()
    return out


def status_string(s: int) -> str:
    return lib().sl_status_string(s).decode()


def abi_version() -> int:
    return lib().sl_abi_version()


def query_fragment_map(instr: int, operand: int) -> np.ndarray:
    """(count, 4) int32 rows of (lane, slot, row, col)."""
    n = ctypes.c_int64(0)
    _check(lib().sl_query_fragment_map(instr, operand, None, None, None, None, 0, ctypes.byref(n)))
    cols = [np.zeros(n.value, np.int32) for _ in range(4)]
    _check(lib().sl_query_fragment_map(instr, operand, *[c.ctypes.data for c in cols], n.value, ctypes.byref(n)))
    return np.stack(cols, 1)


def query_lds_map(variant: int, operand: int) -> Tuple[np.ndarray, int]:
    """((rows, cols) int64 byte offsets, element bytes)."""
    r, c, e = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().sl_query_lds_map(variant, operand, None, 0, ctypes.byref(r), ctypes.byref(c), ctypes.byref(e)))
    out = np.zeros(r.value * c.value, np.int64)
    _check(lib().sl_query_lds_map(variant, operand, out.ctypes.data, out.size, ctypes.byref(r), ctypes.byref(c),
                                  ctypes.byref(e)))
    return out.reshape(r.value, c.value), e.value


def query_fragment_addresses(variant: int, operand: int) -> np.ndarray:
    n = ctypes.c_int64(0)
    _check(lib().sl_query_fragment_addresses(variant, operand, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, np.int64)
    _check(lib().sl_query_fragment_addresses(variant, operand, out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def probe_mfma(instr: int, mode: int, stream: Optional[int] = None):
    """Run the operand-map probe; returns a cuda float32 tensor
    (cases, 64 lanes, accumulator registers)."""
    import torch
    regs = 4 if instr in (0, 2) else 16
    cases = 64 * (8 if instr < 2 else 32)
    out = torch.zeros((cases, 64, regs), dtype=torch.float32, device="cuda")
    nc = ctypes.c_int64(0)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(lib().sl_probe_mfma(instr, mode, ctypes.c_void_p(out.data_ptr()), out.numel(), ctypes.byref(nc),
                               ctypes.c_void_p(stream)))
    return out


def probe_lds(mode: int, src, perm, stream: Optional[int] = None):
    """LDS data-path probe on cuda tensors (src uint8, perm int32[64])."""
    import torch
    out = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(lib().sl_probe_lds(mode, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(perm.data_ptr()),
                              ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream)))
    return out
