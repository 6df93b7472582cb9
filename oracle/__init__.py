"""CPU oracle for paged FlashAttention: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables), and it does not import the
library's Python binding.

Sources (web pages, cited by title and section):
  [KVFA]  "大模型推理优化：KV Cache与FlashAttention实战"
          (LLM inference optimisation: KV Cache and FlashAttention in practice)
  [FAPKV] "Flash Attention与Paged KV Cache优化大模型计算效率"
          (Flash Attention and Paged KV Cache: optimising LLM compute efficiency)
  [KV3X]  "大模型推理优化实战：KV Cache + Flash Attention，让 Token 生成快 3 倍"
          (LLM inference in practice: KV Cache + Flash Attention, 3x faster tokens)
  [SYS]   "LLM推理系统优化：KV缓存管理与动态批处理技术"
          (LLM inference systems: KV-cache management and dynamic batching)

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed
forms, a library routine, brute force and invariants the pages fix.
"""
from .attention import (
    gather_sequence,
    visible_mask,
    attention_paged,
    decode_paged,
    decode_layered,
    append_pages,
)
from .backward import attention_backward_paged
from .quant import quantize_int8_pages, dequantize_int8_pages, append_int8_pages
from .counts import visible_pairs, attention_flops, kv_read_bytes, kv_bytes_per_token
from .twins import brute_force_attention, online_softmax_attention, split_partials, merge_partials

__all__ = [
    "gather_sequence", "visible_mask", "attention_paged", "decode_paged", "decode_layered",
    "append_pages", "quantize_int8_pages", "dequantize_int8_pages", "visible_pairs",
    "attention_flops", "kv_read_bytes", "kv_bytes_per_token", "brute_force_attention",
    "online_softmax_attention", "split_partials", "merge_partials", "attention_backward_paged",
]
