"""orthogonal_equivalence_amd: the POET-X linear layer y = R W0 P x on MI355X.

The compute path is the HIP library libpoetx.so (C ABI declared in
include/poetx.h); `orthogonal_equivalence_amd.poetx` is its thin ctypes
binding. `orthogonal_equivalence_amd.inputs` draws the seeded synthetic
inputs. Importing this package loads nothing.
"""
__version__ = "0.1.0"
