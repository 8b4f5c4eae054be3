"""KIVI-style low-bit KV cache with paged decode and prefill attention for MI355X (gfx950).

The HIP library (``libkivi.so``) is loaded by :mod:`kivi_quantized_kv_append_amd.kivi`
on first use; importing this package alone loads nothing.
"""
__all__ = ["kivi", "inputs"]
