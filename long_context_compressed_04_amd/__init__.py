"""MI355X-native Compressed Sparse Attention (CSA) / Heavily Compressed Attention (HCA).

The compute path is the C-ABI shared library ``libcsa.so`` (hand-written HIP for
gfx950) declared in ``include/csa.h``; ``long_context_compressed_04_amd.csa`` is
its thin ctypes binding over torch device tensors.  ``workloads`` draws the
seeded synthetic inputs.
"""
__all__ = ["csa", "workloads"]
