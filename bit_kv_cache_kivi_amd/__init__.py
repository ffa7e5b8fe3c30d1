"""Low-bit KV cache for block-diffusion language models on AMD MI355X (gfx950).

``from bit_kv_cache_kivi_amd import kvq`` loads libkvq.so (the C ABI in
include/kvq.h) and exposes ``kvq.KVCache`` with ``commit`` (quantize-on-commit)
and ``block_attn`` (fused dequantize-and-attend).  Build the library first with
``python bit_kv_cache_kivi_amd/build.py``.
"""
