"""Anchor-masked block-sparse cross-attention for MI355X (gfx950).

The compute lives in the HIP library ``libsxattn.so`` (C ABI, ``include/sxattn.h``);
``block_sparse_cross_anchor_amd.sxattn`` is a thin ctypes binding over it.
``block_sparse_cross_anchor_amd.synth`` draws seeded synthetic workloads.
"""

__all__ = ["sxattn", "synth"]
