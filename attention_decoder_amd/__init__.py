"""LFM3-1.7B hybrid decoder forward pass (prefill + decode) on MI355X (gfx950).

The compute lives in a C-ABI HIP library (``liblfm3.so``, built from ``csrc/``); ``lfm3`` is its
thin ctypes binding, and ``synth`` draws the seeded synthetic weights and inputs.
"""
