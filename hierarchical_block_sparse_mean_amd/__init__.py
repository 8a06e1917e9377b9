"""PISA (pyramid top-K block selection + block-sparse attention) on AMD
Instinct MI355X (gfx950).

The hot path lives in libpisa.so (HIP kernels behind the C ABI of
include/pisa.h); ``hierarchical_block_sparse_mean_amd.pisa`` is its ctypes
binding and ``hierarchical_block_sparse_mean_amd.inputs`` generates the
seeded synthetic workloads.  Importing this package loads nothing.
"""

__all__ = ["pisa", "inputs"]
