"""Tile-hybrid dense / 2:4 sparse weights on MI355X (gfx950).

The compute lives in libhyb.so (HIP kernels behind the C ABI of
include/hyb.h); this package is its ctypes binding plus the seeded synthetic
workloads.  Importing the package does not load the library; the first call
that needs it does, and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    HybError, HybLayout, HybPacked, PackedWeight, allocate, bits_to_tensor, gemm,
    gemm_mfma, gemv, lib, pack, plan, tensor_to_bits, unpack,
)
