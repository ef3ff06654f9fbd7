"""MI355X (gfx950) implementation of the FlashLoop lazy-update loop step.

The HIP library ``libflashloop.so`` (built from ``csrc/``) holds every step of
the path; ``abi`` is its thin ctypes binding.  Submodules are imported on
demand so that ``configs`` and ``synth`` work without a GPU.
"""
__all__ = ["configs", "synth", "abi", "driver"]
