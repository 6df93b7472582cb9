"""Exact scaled-dot-product attention over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (the plain definition, not the tiled algorithm):
  * [KVFA] §2.1 (KV Cache principle): query i attends to the cached keys
    0..i, weights softmax(q_i . K^T / sqrt(d)), output = weights . V.
  * [KV3X] "KV Cache：空间换时间的经典操作": the new token's K/V are appended to
    the cache first, then the query attends to the whole cache (so a decoded
    token sees itself).
  * [KVFA] §5.1 (the flash_attn_v2 call): softmax_scale defaults to
    1/sqrt(dim); causal masking; a local window of 128 (read here as the
    extent to the left of the query, the right side being closed by
    causality).
  * [SYS] §2.1 (GQA): query heads come in groups of G = Hq/Hkv that share
    one K/V head; the K/V head of query head h is h // G (the
    repeat_interleave form).
  * [FAPKV] §3.2 (paged cache design) and [SYS] §3.1 (paged attention): the
    cache is cut into fixed-size pages; a per-sequence table maps logical
    page n to a physical page; token t lives in logical page t // P, slot
    t % P.  A physical page holds (page_size, d_model) values, token-major,
    with d_model = Hkv * D, so a pool is [num_pages, P, Hkv, D].  K and V
    live in separate pools.
  * [KV3X] "传统 Attention vs Flash Attention" (comparison table): the tiled
    method is exact, so the oracle is the plain definition and the HIP path
    must match it up to rounding.

Causal alignment (the pages are silent for q_len < ctx): bottom-right, i.e.
query row i of a sequence with q_len queries and ctx keys sits at absolute
position p = ctx - q_len + i.  Key j is visible iff (not causal or j <= p)
and (window_left < 0 or p - j <= window_left).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x).astype(np.float64)


def gather_sequence(pool, block_row, n_tokens: int, page_size: int) -> np.ndarray:
    """Dense copy [n_tokens, Hkv, D] of one sequence's cache, read through its
    block-table row ([FAPKV] §3.2: logical page -> physical page).

    Token t comes from physical page block_row[t // page_size], slot
    t % page_size.  The values are returned in the pool's own dtype (a pure
    gather, no arithmetic).
    """
    pool = np.asarray(pool)
    block_row = np.asarray(block_row)
    t = np.arange(int(n_tokens))
    phys = block_row[t // page_size]
    slot = t % page_size
    return pool[phys, slot]


def visible_mask(q_len: int, ctx: int, causal: bool, window_left: int,
                 r0: int = 0, r1: int | None = None) -> np.ndarray:
    """Boolean [r1 - r0, ctx]: True where query row i (r0 <= i < r1) may
    attend to key j.  Row i sits at absolute position p = ctx - q_len + i."""
    r1 = q_len if r1 is None else r1
    i = np.arange(r0, r1)[:, None]
    j = np.arange(ctx)[None, :]
    p = ctx - q_len + i
    vis = np.ones((r1 - r0, ctx), dtype=bool)
    if causal:
        vis &= j <= p
    if window_left >= 0:
        vis &= (p - j) <= window_left
    return vis


def _attend_rows(q_rows, keys, values, scale, vis):
    """softmax(scale * q . K^T) . V for a block of rows, with a visibility mask.

    q_rows [R, D], keys [C, D], values [C, D], vis [R, C] -> (out [R, D], lse [R]).
    A row that sees no key returns out = 0, lse = -inf.
    """
    s = scale * (q_rows @ keys.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=1)
    num = e @ values
    out = np.zeros_like(num)
    ok = denom > 0
    out[ok] = num[ok] / denom[ok, None]
    lse = np.full(denom.shape, -np.inf)
    lse[ok] = m_safe[ok] + np.log(denom[ok])
    return out, lse


def attention_paged(q, cu_q, k_pool, v_pool, block_table, ctx_lens, page_size: int,
                    softmax_scale: float | None = None, causal: bool = True,
                    window_left: int = -1, k_scales=None, v_scales=None,
                    row_block: int = 512):
    """Exact attention of ragged query rows against a paged K/V cache.

    q          [total_q, Hq, D]   queries of all sequences, concatenated
    cu_q       [B+1]              prefix sums of per-sequence query counts
    k_pool     [N, P, Hkv, D]     key pages (float, or int8 codes with k_scales)
    v_pool     [N, P, Hkv, D]     value pages (same)
    block_table[B, max_pages]     physical page of logical page n of sequence b
    ctx_lens   [B]                keys of sequence b, including its queries' own
    k_scales, v_scales [N, Hkv]   fp32 scales when the pools hold int8 codes

    Returns (out [total_q, Hq, D], lse [total_q, Hq]) in float64, lse in
    natural log.  Rows are evaluated independently, ``row_block`` at a time,
    so a large problem never holds its whole score matrix; each row still
    materialises its full score row over the keys it can see.
    """
    q = _f64(q)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    block_table = np.asarray(block_table)
    total_q, hq, d = q.shape
    hkv = np.asarray(k_pool).shape[2]
    assert hq % hkv == 0, "query heads must be a multiple of KV heads"
    group = hq // hkv
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((total_q, hq, d))
    lse = np.full((total_q, hq), -np.inf)
    for b in range(len(ctx_lens)):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        q_len, ctx = q1 - q0, int(ctx_lens[b])
        if q_len == 0:
            continue
        assert ctx >= q_len, "every query row must be a position inside the cache"
        kb = gather_sequence(k_pool, block_table[b], ctx, page_size)
        vb = gather_sequence(v_pool, block_table[b], ctx, page_size)
        if k_scales is not None:
            # one scale per (physical page, KV head): look it up per token
            phys = np.asarray(block_table[b])[np.arange(ctx) // page_size]
            kb = _f64(kb) * _f64(np.asarray(k_scales))[phys][:, :, None]
            vb = _f64(vb) * _f64(np.asarray(v_scales))[phys][:, :, None]
        kb, vb = _f64(kb), _f64(vb)
        for r0 in range(0, q_len, row_block):
            r1 = min(q_len, r0 + row_block)
            vis = visible_mask(q_len, ctx, causal, window_left, r0, r1)
            # keys that no row of this block can see contribute exp(-inf) = 0
            cols = np.nonzero(vis.any(axis=0))[0]
            if cols.size == 0:
                continue
            c0, c1 = int(cols[0]), int(cols[-1]) + 1
            for h in range(hq):
                g = h // group
                o, l = _attend_rows(q[q0 + r0:q0 + r1, h, :], kb[c0:c1, g, :], vb[c0:c1, g, :],
                                    scale, vis[:, c0:c1])
                out[q0 + r0:q0 + r1, h, :] = o
                lse[q0 + r0:q0 + r1, h] = l
    return out, lse


def decode_paged(q, k_pool, v_pool, block_table, ctx_lens, page_size: int,
                 softmax_scale: float | None = None, window_left: int = -1,
                 k_scales=None, v_scales=None):
    """Single-token decode: q [B, Hq, D], one query per sequence at position
    ctx_b - 1, attending to every cached key 0..ctx_b-1 (the new token's own
    K/V already appended).  Same definition as ``attention_paged`` with
    q_len = 1 (causality is then implied)."""
    q = np.asarray(q)
    b = q.shape[0]
    cu_q = np.arange(b + 1)
    return attention_paged(q, cu_q, k_pool, v_pool, block_table, ctx_lens, page_size,
                           softmax_scale=softmax_scale, causal=True, window_left=window_left,
                           k_scales=k_scales, v_scales=v_scales)


def _cached_values(pool, scales, block_row, n_tokens: int, page_size: int) -> np.ndarray:
    """float64 [n_tokens, Hkv, D] of one sequence's first n_tokens cached
    positions; int8 codes are read back as code * scale of their (physical
    page, KV head) group ([SYS] §3.2)."""
    x = gather_sequence(pool, block_row, n_tokens, page_size)
    if scales is None:
        return _f64(x)
    phys = np.asarray(block_row)[np.arange(n_tokens) // page_size]
    return _f64(x) * _f64(np.asarray(scales))[phys][:, :, None]


def decode_layered(q, hi: dict, lo: dict, softmax_scale: float | None = None):
    """Single-token decode over a context held in two caches: the layered
    cache of [KVFA] §2.2 (the first tokens of a sequence kept at full
    precision, later ones int8 with group scales, [SYS] §3.2).

    q [B, Hq, D].  ``hi`` and ``lo`` are dicts with the pools ``k``, ``v``
    [N, P, Hkv, D], ``block_table`` [B, max_pages], ``lens`` [B],
    ``page_size`` and, for int8 pools, ``k_scales`` / ``v_scales`` [N, Hkv].
    Sequence b's keys are its lens_hi[b] positions in ``hi`` followed by its
    lens_lo[b] positions in ``lo``; its one query attends to all of them (no
    mask: the query is the last position).  Returns (out [B, Hq, D],
    lse [B, Hq]); a sequence without keys gets out = 0, lse = -inf.
    """
    q = _f64(q)
    nb, hq, d = q.shape
    hkv = np.asarray(hi["k"]).shape[2]
    group = hq // hkv
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((nb, hq, d))
    lse = np.full((nb, hq), -np.inf)
    for b in range(nb):
        n_hi = int(np.asarray(hi["lens"])[b])
        n_lo = int(np.asarray(lo["lens"])[b])
        parts_k, parts_v = [], []
        for part, n in ((hi, n_hi), (lo, n_lo)):
            row = np.asarray(part["block_table"])[b]
            parts_k.append(_cached_values(part["k"], part.get("k_scales"), row, n, part["page_size"]))
            parts_v.append(_cached_values(part["v"], part.get("v_scales"), row, n, part["page_size"]))
        keys = np.concatenate(parts_k, axis=0)
        values = np.concatenate(parts_v, axis=0)
        if keys.shape[0] == 0:
            continue
        vis = np.ones((1, keys.shape[0]), dtype=bool)
        for h in range(hq):
            g = h // group
            o, l = _attend_rows(q[b:b + 1, h, :], keys[:, g, :], values[:, g, :], scale, vis)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def append_pages(k_pool, v_pool, k_new, v_new, block_table, start_pos, cu_new, page_size: int):
    """Write new K/V rows into their page slots ([KV3X] "KV Cache 的工作原理":
    the cache grows by appending; [FAPKV] §3.2: the slot is found through the
    page table).  Row r of sequence b (r < n_new_b) goes to position
    start_pos[b] + r.  Returns new pools; a pure copy of bits (works on any
    dtype, including raw 16-bit words of bf16 data)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    block_table = np.asarray(block_table)
    for b in range(len(start_pos)):
        n0, n1 = int(cu_new[b]), int(cu_new[b + 1])
        for r in range(n1 - n0):
            pos = int(start_pos[b]) + r
            phys = int(block_table[b, pos // page_size])
            slot = pos % page_size
            k_out[phys, slot] = k_new[n0 + r]
            v_out[phys, slot] = v_new[n0 + r]
    return k_out, v_out
