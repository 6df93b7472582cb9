"""Gradients of paged attention with respect to Q, K and V, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed: the derivative of the attention definition used by
``attention.attention_paged`` (same masks, scale, GQA head map and page
layout) for an upstream gradient dO of the output.  The pages fix the
method of the backward pass, not its formulas: [KVFA] §3.1 and [FAPKV] §2.1
(recomputation) say the attention matrix is not stored by the forward pass
but recomputed from Q, K and the saved softmax statistics when gradients are
needed.  The oracle does not need that economy: it forms each row's
probabilities and differentiates the plain chain

    s = scale * q . K^T,   p = softmax(s) over the visible keys,   o = p . V

    dV   = sum over rows of p^T dO
    dp   = dO . V^T
    ds   = p * (dp - rowsum(dO * o))        (softmax Jacobian, one row)
    dQ   = scale * ds . K
    dK   = sum over rows of scale * ds^T q

Query heads of one GQA group read the same K/V head, so their dK / dV add
up.  dK and dV are returned in the cache's page layout: the gradient of key
position t of sequence b sits in page block_table[b][t // P], slot t % P;
slots no sequence uses stay zero.  A row that sees no key has o = 0 and
contributes nothing.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, gather_sequence, visible_mask


def attention_backward_paged(q, cu_q, k_pool, v_pool, block_table, ctx_lens, page_size: int, d_out,
                             softmax_scale: float | None = None, causal: bool = True, window_left: int = -1):
    """Returns (dq [total_q, Hq, D], dk_pool, dv_pool [N, P, Hkv, D]) in float64."""
    q = _f64(q)
    d_out = _f64(d_out)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    block_table = np.asarray(block_table)
    k_pool, v_pool = np.asarray(k_pool), np.asarray(v_pool)
    total_q, hq, d = q.shape
    hkv = k_pool.shape[2]
    group = hq // hkv
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    dq = np.zeros_like(q)
    dk_pool = np.zeros(k_pool.shape)
    dv_pool = np.zeros(v_pool.shape)
    for b in range(len(ctx_lens)):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        q_len, ctx = q1 - q0, int(ctx_lens[b])
        if q_len == 0 or ctx == 0:
            continue
        keys = _f64(gather_sequence(k_pool, block_table[b], ctx, page_size))     # [ctx, Hkv, D]
        vals = _f64(gather_sequence(v_pool, block_table[b], ctx, page_size))
        vis = visible_mask(q_len, ctx, causal, window_left)                      # [q_len, ctx]
        dk = np.zeros((ctx, hkv, d))
        dv = np.zeros((ctx, hkv, d))
        for h in range(hq):
            g = h // group
            qh, doh = q[q0:q1, h, :], d_out[q0:q1, h, :]
            kh, vh = keys[:, g, :], vals[:, g, :]
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s - m[:, None])
            den = e.sum(axis=1)
            p = np.divide(e, den[:, None], out=np.zeros_like(e), where=den[:, None] > 0)
            o = p @ vh
            dv[:, g, :] += p.T @ doh
            dp = doh @ vh.T
            ds = p * (dp - (doh * o).sum(axis=1)[:, None])
            dq[q0:q1, h, :] = scale * (ds @ kh)
            dk[:, g, :] += scale * (ds.T @ qh)
        t = np.arange(ctx)
        phys, slot = np.asarray(block_table[b])[t // page_size], t % page_size
        dk_pool[phys, slot] = dk
        dv_pool[phys, slot] = dv
    return dq, dk_pool, dv_pool
