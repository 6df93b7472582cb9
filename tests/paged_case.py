"""Small random paged-attention problems for the CPU oracle tests.

Builds the pools, block table and ragged query layout, plus an independent
per-sequence dense copy of K/V made with plain Python loops (so the oracle's
own gather is checked, not reused).
"""
from __future__ import annotations

import math

import numpy as np


class Case:
    def __init__(self, seed, hq, hkv, d, page_size, seqs, causal=True, window_left=-1,
                 scale=None, spare_pages=2):
        """seqs: list of (q_len, ctx) per sequence."""
        r = np.random.default_rng(seed)
        self.hq, self.hkv, self.d, self.page_size = hq, hkv, d, page_size
        self.causal, self.window_left = causal, window_left
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.q_lens = [q for q, _ in seqs]
        self.ctx_lens = np.array([c for _, c in seqs], dtype=np.int64)
        pages = [-(-c // page_size) for _, c in seqs]
        self.num_pages = sum(pages) + spare_pages
        perm = r.permutation(self.num_pages)
        self.block_table = np.full((len(seqs), max(pages)), -1, dtype=np.int64)
        off = 0
        for b, n in enumerate(pages):
            self.block_table[b, :n] = perm[off:off + n]
            off += n
        self.k_pool = r.standard_normal((self.num_pages, page_size, hkv, d))
        self.v_pool = r.standard_normal((self.num_pages, page_size, hkv, d))
        self.cu_q = np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int64)
        self.q = r.standard_normal((int(self.cu_q[-1]), hq, d))

    def dense(self, b):
        """K, V of sequence b as nested lists [ctx][hkv][d], gathered by loops."""
        ks, vs = [], []
        for t in range(int(self.ctx_lens[b])):
            page = int(self.block_table[b][t // self.page_size])
            slot = t - (t // self.page_size) * self.page_size
            ks.append(self.k_pool[page][slot].tolist())
            vs.append(self.v_pool[page][slot].tolist())
        return ks, vs

    def visible(self, b):
        q_len, ctx = self.q_lens[b], int(self.ctx_lens[b])

        def f(i, j):
            pos = ctx - q_len + i
            if self.causal and j > pos:
                return False
            if self.window_left >= 0 and pos - j > self.window_left:
                return False
            return True
        return f

    def oracle_args(self):
        return (self.q, self.cu_q, self.k_pool, self.v_pool, self.block_table, self.ctx_lens,
                self.page_size)
