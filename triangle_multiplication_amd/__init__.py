"""libtrimul: forward triangle multiplicative update on AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(``include/trimul.h``); ``triangle_multiplication_amd.binding`` marshals torch
tensors to it.  Importing this package loads nothing; import ``binding`` to
load the compiled library (it raises if the library is not built).
"""
__all__ = ["binding", "inputs"]
