"""Sparse-BitNet BitLinear hot path for AMD Instinct MI355X (gfx950).

The compute lives in a HIP shared library (libbitlinear.so, C ABI declared in
include/bitlinear.h).  This package holds its thin Python binding
(`sparse_linear_layers_group_amd.bitlinear`), the build step, and the seeded
synthetic-input generators (`synth`).  Importing the package loads nothing;
the binding loads the library on first use and raises if it is missing.
"""
