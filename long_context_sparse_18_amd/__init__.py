"""MI355X-native Sparse GQA full-attention layer (Step 5 Preview).

The compute path is the C-ABI library ``libsgqa.so`` (hand-written HIP
kernels for gfx950); :mod:`long_context_sparse_18_amd.sgqa` is its thin
ctypes binding.  Importing this package loads nothing; the library is
loaded on first use and its absence is an error, never a fallback.
"""
from .configs import LayerShape, Workload, WORKLOADS, TINY, REAL, with_selection  # noqa: F401
