"""MoDA (Mixture-of-Depths Attention) forward for AMD Instinct MI355X.

The work runs in libmoda.so (HIP kernels for gfx950 behind the C ABI of
include/moda.h); ``depth_wise_kv_amd.moda`` is its ctypes binding.  Import
``depth_wise_kv_amd.moda`` explicitly: it raises if the library is not built.
"""
