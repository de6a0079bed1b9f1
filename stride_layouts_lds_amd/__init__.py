"""stride_layouts_lds_amd: a strided-layout fp16 / MXFP8 GEMM for MI355X (gfx950).

The compute path is the HIP library ``libstride_layouts_lds.so`` behind the
C ABI declared in ``include/sl.h``; ``stride_layouts_lds_amd.api`` is a thin
ctypes binding with the same names.  Importing the package loads nothing;
the library is opened on first use and a missing library is an error.
"""

__all__ = ["api", "inputs"]
