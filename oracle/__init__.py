"""Oracle for the strided-layout GEMM: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package; only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark do.  The oracle shares no code,
headers, tables or helpers with the HIP library.

Two parts:

* ``oracle.layout`` (pure-integer Python): the shape:stride layout function,
  both unflatten conventions, named axes, TV maps, XOR swizzle, and the worked
  maps printed on the pages ("CuTe 中 A、B 如何加载到 MMA 寄存器" and
  "数据布局及其记号"), plus the CDNA4 matrix-core operand maps written in the
  same algebra.
* ``oracle.gemm`` (ctypes wrapper around ``gemm_ref.c``, built with gcc): the
  triple-loop fp64 GEMM ``D = A*B^T + C`` over descriptor-addressed operands,
  its own fp16 / E4M3 / E8M0 codecs, and the per-element acceptance bound.

Parity status of every function is listed in each module's header.
"""
