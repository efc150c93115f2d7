"""MI355X-native adaptive-precision causal attention prefill (APA).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, built to ``libapa.so``); ``mixed_precision_long_amd.apa``
is its thin Python binding.  ``inputs`` synthesises seeded workloads.
"""
__all__ = ["apa", "inputs"]
