"""CPU oracle for the low-bit block-diffusion KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package; only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library: it restates the method from the
pages (quantize on commit, then attention over the dequantized cache) in plain
NumPy, fp32 for quantization and fp64 for attention, and is checked against
closed forms, invariants and pure-Python brute force in tests/test_oracle.py.

Sources (pages, cited by title and section):
  * Tai et al., "KV Cache Quantization for Diffusion Language Models",
    Findings of EMNLP 2026 (ACL Anthology record, abstract): KIVI adapted to
    Fast-dLLM-style prefix and dual cache reuse; KProtect keeps per-layer K-cache
    entries in high precision while values get standard low-bit quantization.
  * "SoloQ: Calibration-Free Quantization for Diffusion Language Models"
    (summary page, block-diffusion paragraph): KV entries are quantized only
    when a block is committed; the block being denoised stays in full precision;
    keys use KIVI-style per-channel asymmetric quantization.  Same page, opening
    paragraph: a diffusion LM revisits bidirectional context every step.
  * MaskAhead / Q-MaskAhead abstract: attention computed directly from low-bit KV.
  * Elastic-Cache abstract, observation (1): masked tokens beyond the active
    window can be cached block-wise (the suffix of the dual cache).
  * SoloQ abstract and summary page: a hardware-native 4-bit floating-point
    format with per-block scales (oracle/mxfp4.py, as OCP MX FP4).
  * MaskAhead abstract: mask queries of the current block rank cached entries by
    their estimated contribution to the attention output; the block attends to
    the top-ranked ones (oracle/selection.py).

Parity status: every function here is pinned by tests against closed forms,
invariants or brute force; the pages themselves print no worked example, so no
value is pinned to a number printed on the pages.
"""
from .quant import asym_quantize, dequantize, to_bf16_f32
from .layout import (record_layout, pack_record, unpack_record, v_token_position,
                     HEADER_BYTES)
from .cache import OracleCache
from .attention import block_attention, attention_rows
from .rotation import rotate_f32, unrotate, rotation_matrix, hadamard
from . import selection
from . import mxfp4

__all__ = [
    "asym_quantize", "dequantize", "to_bf16_f32", "record_layout", "pack_record",
    "unpack_record", "v_token_position", "HEADER_BYTES", "OracleCache",
    "block_attention", "attention_rows", "rotate_f32", "unrotate", "rotation_matrix", "hadamard",
    "selection", "mxfp4",
]
