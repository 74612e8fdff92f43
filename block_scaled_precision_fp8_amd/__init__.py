"""bsfp8 -- block-scaled FP8 / NVFP4-style linear layers for AMD MI355X (gfx950).

The compute lives in ``libbsfp8.so`` (hand-written HIP kernels behind a C-ABI,
declared in ``include/bsfp8.h``).  ``lib`` is a thin ctypes binding with the
same entry-point names; ``synth`` draws the seeded synthetic inputs.
"""

__all__ = ["lib", "synth"]
