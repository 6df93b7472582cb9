"""Shared set-up for the GPU parity tests: run a workload through the HIP
library and through the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a tensor as an integer array (exact comparison incl. NaN)."""
    t = t.detach().cpu().contiguous()
    view = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.int8: torch.int8}[t.dtype]
    return t.view(view).numpy()


def check_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str) -> dict:
    g = f64(gpu)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    stats = dict(max=float(err.max()) if err.size else 0.0, mean=float(err.mean()) if err.size else 0.0)
    say(f"  {what}: max|d|={stats['max']:.3e} mean|d|={stats['mean']:.3e}")
    if dtype == "f32":
        assert stats["max"] <= F32_MAX_ABS, f"{what}: {stats}"
    else:
        assert stats["max"] <= BF16_MAX_ABS and stats["mean"] <= BF16_MEAN_ABS, f"{what}: {stats}"
    return stats


def nan_pool(num_pages, page_size, hkv, d, dtype, device="cuda"):
    t = torch.empty((num_pages, page_size, hkv, d), dtype=dtype, device=device)
    t.fill_(float("nan"))
    return t


class PrefillRun:
    """Append a prefill workload's K/V into NaN-filled pages and run prefill
    on the GPU; keeps what the oracle needs.  fused=True: no separate append;
    run() calls attn_prefill_paged_append, which writes the pages itself."""

    def __init__(self, w: wl.PrefillWorkload, ctx_extra=None, fused: bool = False):
        inp = wl.prefill_inputs(w)
        self.w, self.inp = w, inp
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        dev = "cuda"
        self.k_pool = nan_pool(inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim, tdt)
        self.v_pool = nan_pool(inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim, tdt)
        self.cache = ops.KVCache(self.k_pool, self.v_pool)
        self.bt = inp["block_table"].to(dev)
        self.cu = inp["cu_q"].to(dev)
        self.ctx = inp["ctx_lens"].to(dev)
        self.fused = fused
        if fused:
            self.k, self.v = inp["k"].to(dev), inp["v"].to(dev)
        else:
            ops.kv_cache_append(self.cache, inp["k"].to(dev), inp["v"].to(dev), self.bt, inp["start_pos"].to(dev),
                                self.cu, max_new=max(w.seq_lens))
        self.q = inp["q"].to(dev)

    def run(self, return_lse=True):
        if self.fused:
            return ops.attn_prefill_paged_append(self.q, self.k, self.v, self.cu, self.cache, self.bt, self.ctx,
                                                 max_q_len=max(self.w.seq_lens), softmax_scale=self.w.softmax_scale,
                                                 causal=self.w.causal, window_left=self.w.window_left,
                                                 return_lse=return_lse)
        return ops.attn_prefill_paged(self.q, self.cu, self.cache, self.bt, self.ctx, max_q_len=max(self.w.seq_lens),
                                      softmax_scale=self.w.softmax_scale, causal=self.w.causal,
                                      window_left=self.w.window_left, return_lse=return_lse)

    def pages_match_oracle_append(self) -> bool:
        """The K and V pools, bit for bit, against the oracle's append of every
        row into NaN pages."""
        w, inp = self.w, self.inp
        nan_bits = bits(torch.full(tuple(self.k_pool.shape), float("nan"), dtype=self.k_pool.dtype))
        ek, ev = oracle.append_pages(nan_bits, nan_bits.copy(), bits(inp["k"]), bits(inp["v"]),
                                     inp["block_table"].numpy(), inp["start_pos"].numpy(), inp["cu_q"].numpy(),
                                     w.page_size)
        return np.array_equal(bits(self.k_pool), ek) and np.array_equal(bits(self.v_pool), ev)

    def oracle_pools(self):
        """The pools as the oracle's own append makes them (from NaN pages)."""
        w, inp = self.w, self.inp
        shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
        kp = np.full(shape, np.nan)
        vp = np.full(shape, np.nan)
        return oracle.append_pages(kp, vp, f64(inp["k"]), f64(inp["v"]), inp["block_table"].numpy(),
                                   inp["start_pos"].numpy(), inp["cu_q"].numpy(), w.page_size)

    def oracle(self, rows=None):
        """Oracle output for all rows, or for selected (sequence, row) pairs."""
        w, inp = self.w, self.inp
        kp, vp = self.oracle_pools()
        q = f64(inp["q"])
        bt = inp["block_table"].numpy()
        if rows is None:
            return oracle.attention_paged(q, inp["cu_q"].numpy(), kp, vp, bt, inp["ctx_lens"].numpy(),
                                          w.page_size, w.softmax_scale, w.causal, w.window_left)
        # each sampled row as its own one-query problem at its own position
        cu = inp["cu_q"].numpy()
        qs, ctxs, tables = [], [], []
        for b, r in rows:
            qs.append(q[cu[b] + r])
            ctxs.append(r + 1 if w.causal else inp["ctx_lens"][b].item())
            tables.append(bt[b])
        assert w.causal, "row sampling assumes causal rows"
        return oracle.attention_paged(np.stack(qs), np.arange(len(rows) + 1), kp, vp, np.stack(tables),
                                      np.array(ctxs), w.page_size, w.softmax_scale, True, w.window_left)


class DecodeRun:
    """Pre-filled pool (+ poisoned tails), append of the new token, decode."""

    def __init__(self, w: wl.DecodeWorkload, poison=True):
        inp = wl.decode_inputs(w)
        self.w, self.inp = w, inp
        dev = "cuda"
        k_pool, v_pool = inp["k_pool"], inp["v_pool"]
        if poison and w.kv_dtype != "i8":
            k_pool, v_pool = k_pool.clone(), v_pool.clone()
            for page, used in wl.tail_slots(inp["block_table"], inp["ctx_lens"], w.page_size):
                k_pool[page, used:] = float("nan")
                v_pool[page, used:] = float("nan")
            for page in inp["spare_pages"].tolist():
                k_pool[page] = float("nan")
                v_pool[page] = float("nan")
        self.k_src, self.v_src = k_pool, v_pool      # CPU, bf16 / f32
        self.bt = inp["block_table"].to(dev)
        self.ctx = inp["ctx_lens"].to(dev)
        self.q = inp["q"].to(dev)
        kd, vd = k_pool.to(dev), v_pool.to(dev)
        if w.kv_dtype == "i8":
            # append the new token into the bf16 pages, then quantise whole pages
            bf = ops.KVCache(kd, vd)
            ops.kv_cache_append(bf, inp["k_new"].to(dev), inp["v_new"].to(dev), self.bt, inp["start_pos"].to(dev),
                                inp["cu_new"].to(dev), max_new=1)
            kc, ks = ops.kv_pages_quantize_int8(kd)
            vc, vsc = ops.kv_pages_quantize_int8(vd)
            if poison:
                for page, used in wl.tail_slots(inp["block_table"], inp["ctx_lens"], w.page_size):
                    kc[page, used:] = -128
                    vc[page, used:] = -128
                for page in inp["spare_pages"].tolist():
                    kc[page] = -128
                    vc[page] = -128
            del kd, vd
            self.cache = ops.KVCache(kc, vc, ks, vsc)
        else:
            self.cache = ops.KVCache(kd, vd)
            ops.kv_cache_append(self.cache, inp["k_new"].to(dev), inp["v_new"].to(dev), self.bt,
                                inp["start_pos"].to(dev), inp["cu_new"].to(dev), max_new=1)

    def run(self, return_lse=True, workspace=None):
        return ops.attn_decode_paged(self.q, self.cache, self.bt, self.ctx, softmax_scale=self.w.softmax_scale,
                                     window_left=self.w.window_left, workspace=workspace, return_lse=return_lse)

    def oracle(self, seqs=None):
        """Oracle decode for all sequences or a subset (list of indices)."""
        w, inp = self.w, self.inp
        seqs = list(range(w.batch)) if seqs is None else list(seqs)
        bt = inp["block_table"].numpy()
        ctx = inp["ctx_lens"].numpy()
        # only the pages these sequences use, gathered into a compact pool
        used = sorted({int(p) for b in seqs for p in bt[b][: -(-int(ctx[b]) // w.page_size)]})
        remap = {p: i for i, p in enumerate(used)}
        tables = np.array([[remap.get(int(p), -1) for p in bt[b]] for b in seqs])
        kp = self.k_src[used].clone()
        vp = self.v_src[used].clone()
        # the appended token, by the oracle's own append
        start = inp["start_pos"].numpy()[seqs]
        kn = inp["k_new"][seqs]
        vn = inp["v_new"][seqs]
        kp_b, vp_b = bits(kp), bits(vp)
        kp_b, vp_b = oracle.append_pages(kp_b, vp_b, bits(kn), bits(vn), tables, start,
                                         np.arange(len(seqs) + 1), w.page_size)
        view = {np.int16: torch.bfloat16, np.int32: torch.float32}[kp_b.dtype.type]
        kp = torch.from_numpy(kp_b).view(view)
        vp = torch.from_numpy(vp_b).view(view)
        kw = {}
        if w.kv_dtype == "i8":
            kc, ks = oracle.quantize_int8_pages(kp.float().numpy())
            vc, vs = oracle.quantize_int8_pages(vp.float().numpy())
            kpool, vpool, kw = kc, vc, dict(k_scales=ks, v_scales=vs)
        else:
            kpool, vpool = f64(kp), f64(vp)
        q = f64(self.inp["q"][seqs])
        return oracle.decode_paged(q, kpool, vpool, tables, ctx[seqs], w.page_size, w.softmax_scale,
                                   w.window_left, **kw), used
