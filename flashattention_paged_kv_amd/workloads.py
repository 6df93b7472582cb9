"""Seeded synthetic inputs for paged attention workloads.

This module only draws random numbers and lays out page assignments; it holds
none of the attention arithmetic, and both the HIP path (benchmark, tests)
and the CPU oracle (tests) take their inputs from it.

Recipe (the same for every workload):
  * generator: numpy ``default_rng(SeedSequence([seed, stream, chunk]))``;
    streams: 0 = Q, 1 = K, 2 = V, 3 = context lengths, 4 = page permutation,
    5 = new-token K, 6 = new-token V.  ``chunk`` is the physical page index for
    pool-generated K/V (so a page's contents do not depend on how the pool is
    generated), 0 otherwise.
  * values: float32 N(0, 1); for bf16 workloads rounded to bf16 with
    round-to-nearest-even (torch's ``.to(torch.bfloat16)``).
  * page assignment: the pool holds exactly the pages the sequences need
    (plus ``spare_pages`` unused ones); physical pages are handed out by a
    random permutation, sequence after sequence, in logical order.  Unused
    block-table entries are -1.
  * decode context lengths: integers uniform on [ctx_lo, ctx_hi], both ends
    included.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_CTX, STREAM_PERM, STREAM_KNEW, STREAM_VNEW = range(7)

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, chunk]))


def normal(shape, dtype: str, seed: int, stream: int, chunk: int = 0) -> torch.Tensor:
    """float32 N(0,1) of ``shape`` as a CPU tensor of ``dtype`` ('f32' | 'bf16')."""
    x = rng(seed, stream, chunk).standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def _pool(num_pages: int, page_size: int, hkv: int, d: int, dtype: str, seed: int, stream: int,
          workers: int = 8) -> torch.Tensor:
    out = torch.empty((num_pages, page_size, hkv, d), dtype=_TORCH_DTYPES[dtype])

    def fill(n):
        out[n] = normal((page_size, hkv, d), dtype, seed, stream, chunk=n)

    if num_pages * page_size * hkv * d < (1 << 22):
        for n in range(num_pages):
            fill(n)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(num_pages)))
    return out


def page_assignment(pages_per_seq, max_pages: int, seed: int, spare_pages: int = 0):
    """Block table [B, max_pages] (int32, -1 = unused) handing out a random
    permutation of sum(pages_per_seq) + spare_pages physical pages."""
    total = int(sum(pages_per_seq)) + spare_pages
    perm = rng(seed, STREAM_PERM).permutation(total).astype(np.int32)
    table = np.full((len(pages_per_seq), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[off:off + n]
        off += n
    spare = perm[off:]
    return torch.from_numpy(table), total, torch.from_numpy(spare.copy())


@dataclass(frozen=True)
class PrefillWorkload:
    """Causal prefill of ``seq_lens`` prompts whose K/V are appended into pages."""
    name: str
    seq_lens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str = "bf16"
    seed: int = 0
    causal: bool = True
    window_left: int = -1
    spare_pages: int = 0

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step for ``batch`` sequences with random context lengths."""
    name: str
    batch: int
    ctx_lo: int
    ctx_hi: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str = "bf16"      # 'f32' | 'bf16' | 'i8' (int8 is made from bf16 pages)
    seed: int = 0
    window_left: int = -1
    spare_pages: int = 0
    ctx_lens: tuple = field(default=())   # explicit lengths override the random draw
    # Layered cache: the first `full_tokens` positions of each sequence sit in
    # a separate bf16 cache (pages of `full_page_size`), the rest in the
    # kv_dtype cache.  0: one cache.
    full_tokens: int = 0
    full_page_size: int = 16

    @property
    def q_dtype(self) -> str:
        return "f32" if self.kv_dtype == "f32" else "bf16"

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def prefill_inputs(w: PrefillWorkload) -> dict:
    """Dense Q/K/V for every prompt plus the page assignment of the cache the
    prompts' K/V are appended into (the pool itself starts as NaN)."""
    total = int(sum(w.seq_lens))
    q = normal((total, w.num_q_heads, w.head_dim), w.dtype, w.seed, STREAM_Q)
    k = normal((total, w.num_kv_heads, w.head_dim), w.dtype, w.seed, STREAM_K)
    v = normal((total, w.num_kv_heads, w.head_dim), w.dtype, w.seed, STREAM_V)
    pages = [-(-n // w.page_size) for n in w.seq_lens]
    max_pages = max(pages) if pages else 1
    table, num_pages, spare = page_assignment(pages, max_pages, w.seed, w.spare_pages)
    cu = torch.zeros(w.batch + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(w.seq_lens, dtype=torch.int32), 0)
    return dict(q=q, k=k, v=v, block_table=table, num_pages=num_pages, spare_pages=spare,
                cu_q=cu, ctx_lens=torch.tensor(w.seq_lens, dtype=torch.int32),
                start_pos=torch.zeros(w.batch, dtype=torch.int32))


def decode_ctx_lens(w: DecodeWorkload) -> np.ndarray:
    if w.ctx_lens:
        return np.asarray(w.ctx_lens, dtype=np.int64)
    return rng(w.seed, STREAM_CTX).integers(w.ctx_lo, w.ctx_hi, size=w.batch, endpoint=True)


def decode_inputs(w: DecodeWorkload) -> dict:
    """Query [B, Hq, D], a pre-filled K/V pool (bf16 or f32 pages; int8 pools
    are quantised from these by the caller), the page assignment, and the new
    token's K/V [B, Hkv, D] that the decode step appends at ctx_b - 1."""
    ctx = decode_ctx_lens(w)
    pages = [int(-(-int(c) // w.page_size)) for c in ctx]
    table, num_pages, spare = page_assignment(pages, max(pages), w.seed, w.spare_pages)
    src = "bf16" if w.kv_dtype == "i8" else w.kv_dtype
    k_pool = _pool(num_pages, w.page_size, w.num_kv_heads, w.head_dim, src, w.seed, STREAM_K)
    v_pool = _pool(num_pages, w.page_size, w.num_kv_heads, w.head_dim, src, w.seed, STREAM_V)
    q = normal((w.batch, w.num_q_heads, w.head_dim), w.q_dtype, w.seed, STREAM_Q)
    k_new = normal((w.batch, w.num_kv_heads, w.head_dim), src, w.seed, STREAM_KNEW)
    v_new = normal((w.batch, w.num_kv_heads, w.head_dim), src, w.seed, STREAM_VNEW)
    ctx_t = torch.from_numpy(ctx.astype(np.int32))
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, num_pages=num_pages,
                spare_pages=spare, ctx_lens=ctx_t, k_new=k_new, v_new=v_new,
                start_pos=(ctx_t - 1).to(torch.int32),
                cu_new=torch.arange(w.batch + 1, dtype=torch.int32))


def layered_full_inputs(w: DecodeWorkload) -> dict:
    """The full-precision part of a layered workload: bf16 pools holding
    min(full_tokens, ctx_b) positions of each sequence, its page assignment
    and those lengths."""
    ctx = decode_ctx_lens(w)
    lens = np.minimum(ctx, w.full_tokens)
    pages = [max(1, int(-(-int(n) // w.full_page_size))) for n in lens]
    table, num_pages, _ = page_assignment(pages, max(pages), w.seed + 1000, 0)
    shape = (num_pages, w.full_page_size, w.num_kv_heads, w.head_dim)
    return dict(k_pool=normal(shape, "bf16", w.seed, STREAM_K, chunk=1),
                v_pool=normal(shape, "bf16", w.seed, STREAM_V, chunk=1), block_table=table,
                lens=torch.from_numpy(lens.astype(np.int32)))


def tail_slots(block_table: torch.Tensor, ctx_lens, page_size: int):
    """(physical page, first unused slot) of each sequence's last page, as the
    page assignment above laid them out; used to poison slots no valid token
    occupies."""
    out = []
    for b, c in enumerate(ctx_lens):
        c = int(c)
        n = -(-c // page_size)
        used = c - (n - 1) * page_size
        if used < page_size:
            out.append((int(block_table[b, n - 1]), used))
    return out


# ---- the named workloads -------------------------------------------------

TINY_FP32 = PrefillWorkload("tiny_fp32_prefill_128_p16", (128,), 1, 1, 64, 16, "f32", seed=0)
TINY_FP32_DECODE_STEPS = 16   # then 16 single-token decode steps at t = 128 .. 143
LLAMA7B_PREFILL = PrefillWorkload("llama2_7b_causal_prefill_L2048_h32_d128_p256", (2048,), 32, 32,
                                  128, 256, "bf16", seed=2)
LLAMA70B_DECODE = DecodeWorkload("llama2_70b_gqa_decode_B64_hq64_hkv8_d128_ctx512-8192_p256",
                                 64, 512, 8192, 64, 8, 128, 256, "bf16", seed=3)
LONG_PREFILL = PrefillWorkload("long_causal_prefill_L32768_h32_d128_p256", (32768,), 32, 32,
                               128, 256, "bf16", seed=4)
LONG_PREFILL_WINDOW = PrefillWorkload("long_window128_prefill_L32768_h32_d128_p256", (32768,), 32, 32,
                                      128, 256, "bf16", seed=4, window_left=128)
DECODE_128K_INT8 = DecodeWorkload("int8_decode_B16_hq64_hkv8_d128_ctx64k-128k_p256",
                                  16, 65536, 131072, 64, 8, 128, 256, "i8", seed=5)

# The 128k int8 decode with each sequence's first 128 tokens kept in bf16.
DECODE_128K_LAYERED = DecodeWorkload("layered_decode_B16_hq64_hkv8_d128_ctx64k-128k_first128_bf16_rest_int8",
                                     16, 65536, 131072, 64, 8, 128, 256, "i8", seed=5, full_tokens=128,
                                     full_page_size=16)

WORKLOADS = {w.name: w for w in (TINY_FP32, LLAMA7B_PREFILL, LLAMA70B_DECODE, LONG_PREFILL,
                                 LONG_PREFILL_WINDOW, DECODE_128K_INT8, DECODE_128K_LAYERED)}
