"""Width-sharded 2-D convolution for AMD MI355X (gfx950).

The compute path lives in the C-ABI library ``libsscnn.so`` (hand-written HIP
kernels, see ``include/sscnn.h``); ``spatially_sharded_cnn_amd.sscnn`` is its
thin ctypes binding.  Importing this package loads nothing: the binding loads
the library on first use and raises if it has not been built.
"""
__all__ = ["sscnn", "workloads"]
