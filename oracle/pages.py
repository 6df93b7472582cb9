"""Page-pool bookkeeping and page copies, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is modelled:
  * [FAPKV] §3.2 (page table): the cache is cut into fixed-size physical
    pages; each sequence maps its logical page n (tokens n*P .. n*P+P-1) to
    a physical page; a page is allocated when a sequence first needs it.
  * [FAPKV] §5 (the leak fix): releasing a sequence removes its table
    entries as well as giving its pages back.
  * [KVFA] §4.1 and [SYS] §3.1 (zero-copy sharing of a common prompt):
    several sequences may hold the same physical page; a reference count
    per page says how many do, and a page is free again at zero.

Readings where the pages are silent (each listed in the design notes):
  * A sequence that is about to write into a page other sequences also hold
    (a partly filled last page) first gets a private copy of it: a fresh
    page takes its place and the pair (old, new) is reported for the device
    copy (copy-on-write).
  * Free pages are handed out lowest id first (any choice is valid; fixing
    one makes the tables comparable entry by entry).
  * An extend that needs more free pages than there are changes nothing.
"""
from __future__ import annotations

import numpy as np


class PagePoolModel:
    """Plain model of the page pool: lists and a set, no cleverness."""

    def __init__(self, num_pages: int, page_size: int, max_seqs: int, max_pages_per_seq: int):
        self.page_size = page_size
        self.max_pages = max_pages_per_seq
        self.refcount = [0] * num_pages
        self.rows = [[] for _ in range(max_seqs)]   # physical pages of each sequence, in logical order
        self.lens = [0] * max_seqs

    def free_pages(self) -> list:
        return [p for p, r in enumerate(self.refcount) if r == 0]

    def _take(self) -> int:
        p = min(self.free_pages())
        self.refcount[p] = 1
        return p

    def extend(self, seq: int, new_len: int) -> list:
        """Grow seq to new_len tokens; returns the copies [(src, dst)] to make
        before its new rows are written.  Raises MemoryError (no change) when
        free pages run out, ValueError on bad arguments."""
        length = self.lens[seq]
        if new_len < length:
            raise ValueError("a sequence does not shrink")
        have = -(-length // self.page_size)
        need = -(-new_len // self.page_size)
        if need > self.max_pages:
            raise ValueError("too many pages for one sequence")
        row = self.rows[seq]
        shared_tail = (new_len > length and length % self.page_size != 0
                       and self.refcount[row[have - 1]] > 1)
        if (need - have) + (1 if shared_tail else 0) > len(self.free_pages()):
            raise MemoryError("not enough free pages")
        copies = []
        if shared_tail:
            old = row[have - 1]
            new = self._take()
            self.refcount[old] -= 1
            row[have - 1] = new
            copies.append((old, new))
        for _ in range(need - have):
            row.append(self._take())
        self.lens[seq] = new_len
        return copies

    def fork(self, parent: int, child: int, n_tokens: int) -> None:
        """The empty sequence child shares the pages holding the first
        n_tokens of parent."""
        if parent == child or self.lens[child] != 0 or not 1 <= n_tokens <= self.lens[parent]:
            raise ValueError("bad fork")
        shared = self.rows[parent][: -(-n_tokens // self.page_size)]
        for p in shared:
            self.refcount[p] += 1
        self.rows[child] = list(shared)
        self.lens[child] = n_tokens

    def release(self, seq: int) -> None:
        for p in self.rows[seq]:
            self.refcount[p] -= 1
        self.rows[seq] = []
        self.lens[seq] = 0

    def block_table(self) -> np.ndarray:
        t = np.full((len(self.rows), self.max_pages), -1, dtype=np.int32)
        for s, row in enumerate(self.rows):
            t[s, : len(row)] = row
        return t


def copy_pages(k_pool, v_pool, src, dst, k_scales=None, v_scales=None):
    """Whole-page copies src[i] -> dst[i] of K, V (and scales), in order.
    Returns new arrays; a pure copy of values."""
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    ks = None if k_scales is None else np.array(k_scales, copy=True)
    vs = None if v_scales is None else np.array(v_scales, copy=True)
    for s, d in zip(src, dst):
        k[d], v[d] = k[s], v[s]
        if ks is not None:
            ks[d], vs[d] = ks[s], vs[s]
    return k, v, ks, vs
