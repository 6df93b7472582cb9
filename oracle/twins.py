"""Independent second forms of the attention definition, used only to check
the oracle itself.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``brute_force_attention``: pure-Python loops (one dot product per key, a
  softmax, a weighted sum), the per-key form of [KV3X]
  "先搞懂：大模型推理为什么慢？" (naive attention), with math.fsum.
* ``online_softmax_attention``: the block-by-block online softmax of [KV3X]
  "Flash Attention 的分块计算原理" (running max m, running sum l, rescale by
  exp(m_old - m_new)), with the accumulator kept unnormalised and divided by
  l once at the end.  The page's listing also divides each block's
  contribution by the new l and then divides by l again, which normalises
  twice; that step is read as a typo and not followed.
* ``split_partials`` / ``merge_partials``: the same running (m, l, O) state
  computed over disjoint key ranges and merged with the rescaling algebra.
"""
from __future__ import annotations

import math

import numpy as np


def brute_force_attention(q_rows, keys, values, scale, visible):
    """q_rows: list of R query vectors; keys/values: lists of C vectors;
    visible(i, j) -> bool.  Returns (out: list of R lists, lse: list of R)."""
    outs, lses = [], []
    for i, q in enumerate(q_rows):
        scores = []
        for j, k in enumerate(keys):
            if visible(i, j):
                scores.append((j, scale * math.fsum(float(a) * float(b) for a, b in zip(q, k))))
        if not scores:
            outs.append([0.0] * len(values[0]))
            lses.append(-math.inf)
            continue
        m = max(s for _, s in scores)
        w = [(j, math.exp(s - m)) for j, s in scores]
        z = math.fsum(e for _, e in w)
        out = [math.fsum(e * float(values[j][d]) for j, e in w) / z for d in range(len(values[0]))]
        outs.append(out)
        lses.append(m + math.log(z))
    return outs, lses


def online_softmax_attention(q, k, v, scale, vis, block: int):
    """q [R, D], k [C, D], v [C, D], vis [R, C] bool; key blocks of ``block``.
    Returns (out [R, D], lse [R]) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    r, d = q.shape
    m = np.full(r, -np.inf)
    l = np.zeros(r)
    acc = np.zeros((r, d))
    for j0 in range(0, k.shape[0], block):
        s = scale * (q @ k[j0:j0 + block].T)
        s = np.where(vis[:, j0:j0 + block], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        # a row that has seen no visible key yet keeps m = -inf: guard the
        # rescale so that exp(-inf - (-inf)) is never evaluated
        live = np.isfinite(m_new)
        corr = np.where(live, np.exp(np.where(live, m - np.where(live, m_new, 0.0), 0.0)), 1.0)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = l * corr + p.sum(axis=1)
        acc = acc * corr[:, None] + p @ v[j0:j0 + block]
        m = m_new
    out = np.zeros_like(acc)
    ok = l > 0
    out[ok] = acc[ok] / l[ok, None]
    lse = np.where(ok, np.where(ok, m, 0.0) + np.log(np.where(ok, l, 1.0)), -np.inf)
    return out, lse


def split_partials(q, k, v, scale, vis, bounds):
    """Running state (m, l, unnormalised O) of each key range [bounds[s], bounds[s+1])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        s = scale * (q @ k[a:b].T)
        s = np.where(vis[:, a:b], s, -np.inf)
        m = s.max(axis=1, initial=-np.inf)
        live = np.isfinite(m)
        e = np.where(live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
        parts.append((m, e.sum(axis=1), e @ v[a:b]))
    return parts


def merge_partials(parts):
    """Merge (m_s, l_s, O_s): M = max m_s, L = sum l_s e^(m_s - M),
    O = sum O_s e^(m_s - M) / L; lse = M + ln L."""
    ms = np.stack([p[0] for p in parts])
    big_m = ms.max(axis=0)
    live = np.isfinite(big_m)
    mm = np.where(live, big_m, 0.0)
    w = np.where(np.isfinite(ms), np.exp(np.where(np.isfinite(ms), ms, 0.0) - mm), 0.0)
    big_l = sum(w[s] * parts[s][1] for s in range(len(parts)))
    acc = sum(w[s][:, None] * parts[s][2] for s in range(len(parts)))
    out = np.zeros_like(acc)
    ok = big_l > 0
    out[ok] = acc[ok] / big_l[ok, None]
    lse = np.where(ok, mm + np.log(np.where(ok, big_l, 1.0)), -np.inf)
    return out, lse
