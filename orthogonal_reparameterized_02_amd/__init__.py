"""POET-X reparameterized linear layer for AMD Instinct MI355X (gfx950).

The compute path is libpoetx.so (hand-written HIP kernels behind a C ABI,
declared in include/poetx.h); `poetx` binds it under the same names and
`layer` drives one layer through it.  Importing this package loads nothing;
the library is opened on first use and a missing build raises.
"""

__all__ = ["poetx", "layer", "inputs"]
