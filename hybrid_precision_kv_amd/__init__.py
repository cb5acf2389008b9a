"""Hybrid-precision KV attention (HyQuant method) for AMD MI355X.

The compute path is the HIP library ``libhyq.so`` (C ABI in ``include/hyq.h``); this package
only marshals torch tensors (device memory and the current stream) into its calls.  The
library is loaded on first use and its absence raises -- there is no CPU fallback.
"""
from .api import (HybridKVCache, Shape, anchor_count, append_token, decode_attn, prefill_attn,
                  prefill_workspace, quantize_kv, select_vlines, workspace_bytes)

__all__ = ["HybridKVCache", "Shape", "anchor_count", "append_token", "decode_attn", "prefill_attn",
           "prefill_workspace", "quantize_kv", "select_vlines", "workspace_bytes"]
