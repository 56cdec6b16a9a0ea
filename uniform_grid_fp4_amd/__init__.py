"""MI355X-native UFP4 hot path: fused RHT + 4-bit quantizer and block-scaled
4-bit GEMMs, as a C-ABI HIP library (libufp4.so) with a thin ctypes binding.

The binding is loaded lazily; `uniform_grid_fp4_amd.ufp4` holds the calls.
"""
