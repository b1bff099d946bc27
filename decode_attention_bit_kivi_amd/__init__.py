"""MI355X-native decode attention over a 1/2-bit KIVI-style KV cache with
SpeCache's speculative top-k prefetch of 16-bit rows.

The compute path is the HIP library libspecache.so (include/specache.h); this
package is its thin Python binding.  Build the library with
`python -m decode_attention_bit_kivi_amd.build`.
"""
from .api import (
    LowBitCache, empty_cache, lowbit_sizes, quantize_pack, score_topk, score_topk_workspace_size,
    gather_fp16, decode_attn, decode_attn_workspace_size, decode_step, decode_step_workspace_size,
    GatherStream, ComputeStream, gather_reuse, gather_fp16_missing, quantize_append, offload_fp16,
    decode_attn_fp16, flag_set, flag_wait, decode_step_noalloc,
)
from ._lib import SpecacheError

__all__ = [
    "LowBitCache", "empty_cache", "lowbit_sizes", "quantize_pack", "score_topk",
    "score_topk_workspace_size", "gather_fp16", "decode_attn", "decode_attn_workspace_size",
    "decode_step", "decode_step_workspace_size", "GatherStream", "ComputeStream", "gather_reuse", "gather_fp16_missing",
    "quantize_append", "offload_fp16", "decode_attn_fp16", "flag_set", "flag_wait", "decode_step_noalloc",
    "SpecacheError",
]
