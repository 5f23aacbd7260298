"""Shifted short attention and bounded-history attention for MI355X (gfx950).

The compute lives in ``libs2a.so`` (hand-written HIP kernels behind a C ABI declared in
``include/s2a.h``).  ``block_sparse_attention_41_amd.ops`` is a thin ctypes binding over
it; PyTorch only supplies device memory and the HIP stream.
"""
