"""MI355X-native grouped-query attention (MHA / GQA / MQA): forward, decode,
mixed prefill + decode batches and backward.

The compute runs in ``libgqa_attn.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/gqa_attn.h``).  ``binding`` is a thin ctypes layer
over it: argument checks and marshalling only, no compute and no fallback.

Importing this package does not load the library; the first use of any
entry point does, and raises if it has not been built.
"""
from __future__ import annotations

__all__ = ["attn_fwd", "attn_fwd_strided", "attn_fwd_varlen", "attn_decode", "attn_decode_noalloc",
           "attn_decode_append", "attn_decode_slots", "attn_bwd",
           "attn_mixed", "decode_workspace_bytes", "bwd_workspace_bytes", "library_path",
           "GqaError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
