"""Block-scaled FP8 (grouped) GEMM library for MI355X (gfx950).

The compute path is the HIP library ``libdgmi.so`` built from ``csrc/``;
this package holds its thin ctypes binding and the seeded synthetic input
generators.  Importing the package loads nothing; the library is opened on
first use of the binding.
"""
