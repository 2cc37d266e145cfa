"""gated_delta_amd: the RDA gated-delta token mixer on MI355X (gfx950).

The compute lives in ``librda.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rda.h``).  ``gated_delta_amd.rda`` is the thin ctypes
binding with the same entry-point names; ``gated_delta_amd.synth`` draws the
seeded synthetic inputs.  Importing the package loads nothing; the binding
loads the library on first use and fails loudly if it is missing.
"""
__all__ = ["rda", "synth"]
