"""MI355X-native drafter LM heads (dense, SlimSpec low-rank, SpecVocab) and batched
speculative verification.

The compute path is the HIP library ``libspechead.so`` (built from ``csrc/``) behind the
C ABI declared in ``include/spechead.h``; ``spechead`` is its thin ctypes binding.
Importing this package does not load the library; ``spechead.load()`` does, and raises if
it is missing.  There is no CPU fallback.
"""
__all__ = ["spechead", "synth", "configs"]
