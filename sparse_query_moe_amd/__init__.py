"""MI355X (gfx950) Grouped Query Experts prefill layer.

The kernels and the C ABI live in libgqe.so (include/gqe.h); `gqe` is its
ctypes binding.  Build with `python -m sparse_query_moe_amd.build`.
"""
