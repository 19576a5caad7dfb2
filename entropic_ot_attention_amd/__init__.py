"""Banded balanced Sinkhorn attention on MI355X (gfx950).

The compute path is the HIP library ``libsinkhorn_attn.so`` (sources in ``csrc/``),
reached through the ctypes binding in ``binding.py``.  Importing this package does
not load the library; ``entropic_ot_attention_amd.binding`` does, and raises if it
is missing.
"""

__all__ = ["binding", "workloads"]
