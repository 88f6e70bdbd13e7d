"""Hybrid paged GQA attention (Gemma-4-style local/global families) for AMD MI355X.

The compute lives in libgattn.so (hand-written gfx950 HIP kernels behind the C
ABI of include/gattn.h); this package is its Python binding plus the traffic
counters the benchmark uses. Importing it fails if the library is not built.
"""
from ._native import (GLOBAL, LIB_PATH, LOCAL, PAGE_SIZE, GattnError, Layer, gattn_abi_version, gattn_combine,
                      gattn_decode, gattn_decode_fp8kv, gattn_decode_graphs_bucket, gattn_decode_graphs_create,
                      gattn_decode_graphs_destroy, gattn_decode_graphs_launch, gattn_decode_noalloc,
                      gattn_decode_workspace_bytes, gattn_kv_append, gattn_kv_append_fp8, gattn_kv_offset,
                      gattn_layer_family, gattn_prefill, gattn_status_str, make_layer)

__all__ = ["GLOBAL", "LOCAL", "PAGE_SIZE", "LIB_PATH", "GattnError", "Layer", "make_layer", "gattn_abi_version",
           "gattn_status_str", "gattn_layer_family", "gattn_kv_offset", "gattn_decode_workspace_bytes",
           "gattn_decode", "gattn_decode_noalloc", "gattn_decode_fp8kv", "gattn_decode_graphs_create",
           "gattn_decode_graphs_bucket", "gattn_decode_graphs_launch", "gattn_decode_graphs_destroy", "gattn_prefill",
           "gattn_combine", "gattn_kv_append", "gattn_kv_append_fp8"]
