"""Fused attention forward (Yat kernel, softmax, s^tau) for MI355X (gfx950).

The compute path is the C-ABI library ``libsfs_attn.so`` built from
``csrc/``; ``attn`` is its thin ctypes binding.  Importing this package loads
nothing: the library is opened on first use and its absence is an error.
"""
__all__ = ["attn", "workloads"]
