"""CPU oracle for SpeCache-style decode attention over a 1/2-bit KIVI cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the tests, the smoke
check in __graft_entry__ and the cpu_baseline leg of bench.py may import it;
the library (decode_attention_bit_kivi_amd) never does, and the two share no
code.  Inputs come from the separate `workloads` generator.

Sources (the pages this follows):
  [SpeCache]  "SpeCache: Speculative Key-Value Caching for Efficient Generation
              of LLMs" (papercache.org summary of arXiv:2503.16163).
  [SemKV]     "SemKV: ... semantic mixed-precision KV cache quantization"
              (bittide.aicompass.dev translation of arXiv 2608.28911), §2.1.

Arithmetic: numpy float64, except the quantizer's zero-point / scale / code
steps, which the bit-exact contract fixes in float32 in the order the
SpeCache §3 equations write them (numpy float32 ops are IEEE
round-to-nearest-even, like the GPU's).

Every function here has at least one pin in tests/test_oracle_pins.py that
checks it against something other than itself (closed forms printed on the
pages, library routines such as torch's scaled_dot_product_attention,
invariants, brute force).  No function is "parity unpinned".
"""
from .quantize import (
    quantize_keys, quantize_values, dequantize_keys, dequantize_values, zero_point_scale,
)
from .rank import rank_scores, rank_scores_mixed, topk_positions, score_topk
from .attention import mixed_attention, attention_probs
from .gather import gather_rows, resident_rows

__all__ = [
    "quantize_keys", "quantize_values", "dequantize_keys", "dequantize_values",
    "zero_point_scale", "rank_scores", "rank_scores_mixed", "topk_positions", "score_topk",
    "mixed_attention", "attention_probs", "gather_rows", "resident_rows",
]
