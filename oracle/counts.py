"""Algorithmic work counts: visible (query, key) pairs, FLOPs and bytes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Counting follows the definition: every visible (query, key) pair costs a
D-long dot product for the score and a D-long multiply-add into the output,
i.e. 4 * D FLOPs per pair per query head ([KV3X] "先搞懂：大模型推理为什么慢？"
counts attention work in pairs; the pair count is n(n-1)/2 when the diagonal
is excluded and n(n+1)/2 when each token also attends to itself).  Each K/V
element is read once per KV head (GQA sharing, [SYS] §2.1).  [SYS] §1 gives
the cache bytes per token as layers x (d_k + d_v) x bytes-per-value.
"""
from __future__ import annotations


def visible_pairs(q_len: int, ctx: int, causal: bool = True, window_left: int = -1) -> int:
    """Number of (query row, key) pairs with key visible, by direct count of
    each row's visible key range (closed form per row)."""
    total = 0
    for i in range(q_len):
        p = ctx - q_len + i
        hi = p if causal else ctx - 1
        lo = max(0, p - window_left) if window_left >= 0 else 0
        if hi >= lo:
            total += hi - lo + 1
    return total


def attention_flops(pairs: int, head_dim: int, num_q_heads: int) -> int:
    """4 * D FLOPs per visible pair per query head (QK^T and PV, 2 each)."""
    return 4 * head_dim * num_q_heads * pairs


def kv_read_bytes(ctx_lens, num_kv_heads: int, head_dim: int, elem_bytes: int,
                  scale_bytes_per_page_head: int = 0, page_size: int = 0) -> int:
    """Bytes of K and V a decode step must read: every valid token's K and V
    row once per KV head, plus (for int8 caches) one K and one V scale per
    (page touched, KV head)."""
    total = 0
    for c in ctx_lens:
        c = int(c)
        total += 2 * c * num_kv_heads * head_dim * elem_bytes
        if scale_bytes_per_page_head:
            pages = -(-c // page_size)
            total += 2 * pages * num_kv_heads * scale_bytes_per_page_head
    return total


def kv_bytes_per_token(num_layers: int, d_k: int, d_v: int, bytes_per_value: int) -> int:
    """[SYS] §1: cache bytes per token = L x (d_k + d_v) x bytes."""
    return num_layers * (d_k + d_v) * bytes_per_value
