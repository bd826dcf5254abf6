"""libgemm for MI355X (gfx950): C = alpha*(A x B) + beta*C on row-major operands.

The computation runs in hand-written HIP kernels inside ``libgemm.so``; this
package is a thin ctypes binding over its C ABI (``include/gemm.h``).
"""
