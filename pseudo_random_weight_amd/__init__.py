"""SeedLM seed-decoding matrix products for AMD MI355X (gfx950).

The package is the HIP library libseedmm.so (C ABI in include/seedmm.h) and its
Python binding `pseudo_random_weight_amd.seedmm`.  Build with
`python -m pseudo_random_weight_amd.build`.
"""
__all__ = ["seedmm"]
