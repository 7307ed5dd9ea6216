"""MI355X-native ternary BitLinear (BitNet b1.58, I2_S) forward path.

The HIP library (``libbitlinear.so``, built from ``csrc/``) is loaded on first
use by :mod:`ternary_bit_linear_amd.api`; importing the package itself loads
nothing, so the seeded input generators in :mod:`.workloads` can be used on a
machine without the library or a GPU.
"""
