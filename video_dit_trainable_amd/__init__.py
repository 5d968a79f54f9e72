"""VSA2 sparse-attention hot path for video DiTs on MI355X (gfx950).

The compute lives in ``libvsa2.so`` (hand-written HIP, C-ABI declared in
``include/vsa2.h``).  ``video_dit_trainable_amd.vsa2`` is the thin ctypes
binding; ``video_dit_trainable_amd.inputs`` makes the seeded synthetic
workloads.  Importing this package does not load the shared library.
"""

__all__ = ["configs", "inputs", "vsa2"]
