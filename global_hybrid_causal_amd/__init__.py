"""OLMo 3 per-layer hybrid (sliding-window / full) causal attention for MI355X.

The compute path is the HIP library ``libolmo3attn.so`` (C ABI declared in
``include/olmo3_attn.h``); ``global_hybrid_causal_amd.attn`` is a thin ctypes
binding with the same entry-point names.  Importing this package loads
nothing: the library is opened on first use of the binding, and the binding
raises if it is missing.
"""

LAYER_SLIDING = 0
LAYER_FULL = 1

__all__ = ["LAYER_SLIDING", "LAYER_FULL"]
