"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload NAME]

One step is one pass of the hot path over one batch of synthetic input.  The
headline (``value``) is the prompt step of the largest single-GPU prefill
configuration: a 32768-token causal prompt (32 heads, D=128, bf16) whose K/V
are appended into 256-token pages with a permuted block table and attended
over causally, by ``attn_prefill_paged_append`` (at this length the library
runs the append kernel and then the prefill kernel; the prefill kernel is the
dominant one and carries ``roofline``).  Beside it, under ``workloads``:
  * the 2048-token Llama-2-7B-shaped prompt step (append fused into the
    prefill kernel at this length);
  * the 32768-token prompt with a 128-key left window (below the ridge point:
    HBM-bound, timed with a cold cache);
  * the Llama-2-70B-shaped GQA decode step (64 sequences, 64 query heads over
    8 KV heads, contexts uniform in [512, 8192], bf16 pages): the new token's
    append, then attn_decode_paged;
  * the 128k-context int8 decode (16 sequences, contexts uniform in
    [65536, 131072], int8 pages with one fp32 scale per (page, KV head)).

Prefill throughput is TFLOP/s of algorithmic work (4 * D * Hq per visible
(query, key) pair); decode throughput is KV-read GB/s (each valid K/V element
once per KV head, plus the int8 scales of the pages touched).  Inputs are
resident in HBM before timing.  Kernel times come from HIP events on the
stream the library launches on (torch's current stream): warm timings run
back to back; cold timings read a 1 GiB buffer (untimed) before every rep
so that neither L2 nor the 256 MB MALL holds the inputs, and report the
mean, median and min over the reps.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from flashattention_paged_kv_amd import ops  # noqa: E402
from flashattention_paged_kv_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (dual issue) x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
FLUSH_BYTES = 1 << 30         # read before each cold rep (> L2 + MALL)

HEADLINE = wl.LONG_PREFILL
PAGE_COPY = "page_copy_512_pages_p256_hkv8_d128_bf16"
BACKWARD = "backward_causal_L2048_h32_d128_p256_bf16"


def causal_pairs(n: int, window_left: int = -1) -> int:
    """Visible (query, key) pairs of an n-token causal prompt, closed form:
    row i sees min(i + 1, window_left + 1) keys."""
    if window_left < 0:
        return n * (n + 1) // 2
    w1 = window_left + 1
    full = min(n, w1)
    return full * (full + 1) // 2 + (n - full) * w1


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs (scaled by
    the copy calibration), only while the kernel's sources are unchanged
    since they were taken; else None."""
    from flashattention_paged_kv_amd.profiling import source_hash
    try:
        t = json.load(open(TRAFFIC_FILE))[f"{kernel}:{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != source_hash(kernel):
        return None
    return round(t["hbm_bytes_per_launch"])


class _Flush:
    """A 1 GiB device buffer read (summed) before each cold rep: it evicts the
    inputs from L2 and the MALL and leaves only clean lines behind (a
    writing flush would leave 1 GiB of dirty lines whose write-back then
    competes with the timed kernel's reads)."""

    def __init__(self):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.acc = torch.zeros((), dtype=torch.int64, device="cuda")

    def __call__(self):
        torch.sum(self.buf, dim=0, dtype=torch.int64, out=self.acc)


_FLUSH = None


def _flush():
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = _Flush()
    return _FLUSH


def _settle(fn, warmup: int, min_s: float = 0.2):
    """Untimed warm-up: `warmup` calls, then calls until `min_s` seconds of
    work have run (so the clocks have settled before the timed region)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()


def time_warm(fn, reps: int, warmup: int) -> dict:
    """`reps` back-to-back calls bracketed by one pair of HIP events (mean =
    span / reps), then `reps` more with an event pair around each call
    (median and min per call), in ms."""
    _settle(fn, warmup)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return dict(mean_ms=s.elapsed_time(e) / reps, median_ms=statistics.median(per), min_ms=min(per), reps=reps)


def time_cold(fn, reps: int, warmup: int) -> dict:
    """Each rep: read 1 GiB (untimed), then one call between HIP events;
    mean, median and min per call, in ms."""
    flush = _flush()
    _settle(fn, warmup)
    per = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    return dict(mean_ms=statistics.fmean(per), median_ms=statistics.median(per), min_ms=min(per), reps=reps)


def _r(d: dict) -> dict:
    return {k: (round(v, 5) if isinstance(v, float) else v) for k, v in d.items()}


class ClockSampler:
    """Samples the GPU's current shader (sclk) and memory (mclk) clock levels
    from the amdgpu sysfs files of the device torch runs on, every 20 ms in a
    thread, while a timed region runs.  Reports null where the files are not
    readable."""

    def __init__(self):
        self.path = None
        try:
            p = torch.cuda.get_device_properties(0)
            cand = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            if os.path.exists(os.path.join(cand, "pp_dpm_sclk")):
                self.path = cand
        except Exception:
            self.path = None
        self.samples = {"sclk": [], "mclk": []}
        self._stop = threading.Event()
        self._t = None

    @staticmethod
    def _current_mhz(path: str):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    tok = line.split(":", 1)[1].strip().split()[0].lower()
                    return float(tok.replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k in ("sclk", "mclk"):
                v = self._current_mhz(os.path.join(self.path, f"pp_dpm_{k}"))
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(0.02)

    def __enter__(self):
        if self.path:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t is not None:
            self._t.join()

    def summary(self) -> dict:
        out = {"source": self.path and (self.path + "/pp_dpm_{sclk,mclk}")}
        for k, v in self.samples.items():
            out[k + "_mhz"] = (dict(min=min(v), median=statistics.median(v), max=max(v), samples=len(v))
                               if v else None)
        return out


def bench_prefill(w: wl.PrefillWorkload, steps: int, warmup: int, cold: bool = False,
                  sampler: ClockSampler | None = None) -> dict:
    """The prompt step (attn_prefill_paged_append) and the prefill kernel alone
    (attn_prefill_paged) on one workload.  cold=True (HBM-bound shapes) times
    both with L2 and the MALL flushed (a 1 GiB read) before every rep."""
    dev = torch.device("cuda")
    inp = wl.prefill_inputs(w)
    tdt = torch.bfloat16
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    cache = ops.KVCache(torch.zeros(shape, dtype=tdt, device=dev), torch.zeros(shape, dtype=tdt, device=dev))
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    bt, cu, ctx = (inp[n].to(dev) for n in ("block_table", "cu_q", "ctx_lens"))
    out = torch.empty_like(q)
    max_len = max(w.seq_lens)
    del inp

    def prefill():
        ops.attn_prefill_paged(q, cu, cache, bt, ctx, max_q_len=max_len, softmax_scale=w.softmax_scale,
                               causal=w.causal, window_left=w.window_left, out=out)

    def step():
        ops.attn_prefill_paged_append(q, k, v, cu, cache, bt, ctx, max_q_len=max_len, softmax_scale=w.softmax_scale,
                                      causal=w.causal, window_left=w.window_left, out=out)

    timer = time_cold if cold else time_warm
    t_step = timer(step, steps, warmup)
    if sampler is not None:
        with sampler:
            t_attn = timer(prefill, steps, warmup)
    else:
        t_attn = timer(prefill, steps, warmup)
    fused = ops.prefill_append_is_fused(cache, w.causal, w.window_left, max_len)
    # The dominant kernel: the step itself when it is one fused launch, else
    # the prefill kernel (the step is then the append kernel + it).
    t_kernel = t_step if fused else t_attn
    pairs = sum(causal_pairs(n, w.window_left) for n in w.seq_lens)
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    kv_bytes = 2 * sum(w.seq_lens) * w.num_kv_heads * w.head_dim * 2
    # Algorithmic HBM bytes: Q and O once per query row, K and V once per key.
    io_bytes = 2 * sum(w.seq_lens) * w.num_q_heads * w.head_dim * 2 + kv_bytes
    hbm_bound = flops / io_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

    def roof(ms, kernel):
        if hbm_bound:   # below the ridge point (a short window): bytes bound it
            gbs = io_bytes / (ms * 1e-3) / 1e9
            r = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                     frac=round(gbs / PEAK_HBM_GBS, 4))
        else:
            tf = flops / (ms * 1e-3) / 1e12
            r = dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(tf / PEAK_BF16_TFLOPS, 4))
        r["traffic"] = _traffic(kernel, w.name)
        return r

    kname = "prefill_bf16_kernel_fused" if fused else "prefill_bf16_kernel"
    return dict(workload=w.name, fused=fused, timing="cold" if cold else "warm",
                step=_r(t_step), prefill_kernel=_r(t_attn), flops=flops, io_bytes=io_bytes,
                tflops_step=flops / (t_step["mean_ms"] * 1e-3) / 1e12,
                roofline=roof(t_kernel["mean_ms"], kname),
                prefill_kernel_roofline=roof(t_attn["mean_ms"], "prefill_bf16_kernel"),
                config=dict(batch=w.batch, seq_len=max_len, num_q_heads=w.num_q_heads,
                            num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                            causal=w.causal, window_left=w.window_left))


def bench_decode(w: wl.DecodeWorkload, steps: int, warmup: int) -> dict:
    """The decode step (bf16: the new token's append, then attn_decode_paged;
    int8: attn_decode_paged over pages quantised once) timed cold (headline)
    and warm, and the decode call alone (split + merge kernels)."""
    dev = torch.device("cuda")
    inp = wl.decode_inputs(w)
    bt, ctx, start, cun = (inp[n].to(dev) for n in ("block_table", "ctx_lens", "start_pos", "cu_new"))
    q, k_new, v_new = (inp[n].to(dev) for n in ("q", "k_new", "v_new"))
    kd, vd = inp["k_pool"].to(dev), inp["v_pool"].to(dev)
    ctx_np = inp["ctx_lens"].numpy().astype(np.int64)
    del inp
    if w.kv_dtype == "i8":
        ops.kv_cache_append(ops.KVCache(kd, vd), k_new, v_new, bt, start, cun, max_new=1)
        kc, ks = ops.kv_pages_quantize_int8(kd)
        vc, vs = ops.kv_pages_quantize_int8(vd)
        del kd, vd
        cache = ops.KVCache(kc, vc, ks, vs)
        append = None
    else:
        cache = ops.KVCache(kd, vd)

        def append():
            ops.kv_cache_append(cache, k_new, v_new, bt, start, cun, max_new=1)
    nbytes = ops.decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, bt.shape[1],
                                        w.page_size)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def decode():
        ops.attn_decode_paged(q, cache, bt, ctx, softmax_scale=w.softmax_scale, window_left=w.window_left,
                              out=out, workspace=ws)

    def step():
        if append is not None:
            append()
        decode()

    reps = max(steps, 100) if w.batch >= 64 else max(steps, 20)
    cold_step = time_cold(step, reps, warmup)
    cold = time_cold(decode, reps, warmup)
    warm = time_warm(decode, reps, warmup)
    esz = 1 if w.kv_dtype == "i8" else 2
    kv_bytes = int(2 * ctx_np.sum() * w.num_kv_heads * w.head_dim * esz)
    if w.kv_dtype == "i8":
        kv_bytes += int(2 * sum(-(-int(c) // w.page_size) for c in ctx_np) * w.num_kv_heads * 4)
    gbs = lambda ms: kv_bytes / (ms * 1e-3) / 1e9
    return dict(workload=w.name, metric="decode KV-read GB/s", value=round(gbs(cold_step["median_ms"]), 1),
                unit="GB/s", timing="cold (1 GiB read before each rep); value from the step's median",
                step_cold=_r(cold_step), decode_cold=_r(cold), decode_warm=_r(warm), kv_bytes=kv_bytes,
                sum_ctx=int(ctx_np.sum()),
                step=("kv_cache_append + attn_decode_paged" if append is not None else "attn_decode_paged"),
                roofline=dict(bound="hbm", achieved=round(gbs(cold["mean_ms"]), 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs(cold["mean_ms"]) / PEAK_HBM_GBS, 4),
                              traffic=_traffic("decode_split_kernel", w.name)),
                warm_roofline_frac=round(gbs(warm["mean_ms"]) / PEAK_HBM_GBS, 4),
                config=dict(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                            head_dim=w.head_dim, page_size=w.page_size, kv_dtype=w.kv_dtype,
                            ctx_range=[w.ctx_lo, w.ctx_hi]))


def bench_layered(w: wl.DecodeWorkload, steps: int, warmup: int) -> dict:
    """Decode over a layered cache: the first w.full_tokens positions of each
    sequence in a bf16 cache, the rest in an int8 cache (quantised pages)."""
    dev = torch.device("cuda")
    inp = wl.decode_inputs(w)
    full = wl.layered_full_inputs(w)
    q = inp["q"].to(dev)
    kc, ks = ops.kv_pages_quantize_int8(inp["k_pool"].to(dev))
    vc, vs = ops.kv_pages_quantize_int8(inp["v_pool"].to(dev))
    lo = ops.KVCache(kc, vc, ks, vs)
    hi = ops.KVCache(full["k_pool"].to(dev), full["v_pool"].to(dev))
    ctx_np = inp["ctx_lens"].numpy().astype(np.int64)
    len_hi = full["lens"].numpy().astype(np.int64)
    len_lo = ctx_np - len_hi
    bt_hi, bt_lo = full["block_table"].to(dev), inp["block_table"].to(dev)
    lh, ll = full["lens"].to(dev), torch.from_numpy(len_lo.astype(np.int32)).to(dev)
    ws = torch.empty(ops.decode_layered_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def decode():
        ops.attn_decode_paged_layered(q, hi, bt_hi, lh, lo, bt_lo, ll, softmax_scale=w.softmax_scale, out=out,
                                      workspace=ws)

    cold = time_cold(decode, max(steps, 20), warmup)
    row = w.num_kv_heads * w.head_dim
    kv_bytes = int(2 * len_hi.sum() * row * 2 + 2 * len_lo.sum() * row
                   + 2 * sum(-(-int(c) // w.page_size) for c in len_lo) * w.num_kv_heads * 4)
    gbs = kv_bytes / (cold["mean_ms"] * 1e-3) / 1e9
    return dict(workload=w.name, decode_cold=_r(cold), kv_bytes=kv_bytes, sum_ctx=int(ctx_np.sum()),
                full_tokens=w.full_tokens,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None))


def bench_backward(steps: int, warmup: int) -> dict:
    """attn_backward_paged on the L=2048 causal prefill shape (32 heads, D=128,
    bf16, pages of 256): forward once for out / lse, then time the backward.
    Algorithmic FLOPs: the five products of the gradient chain (recompute
    q.K^T, dO.V^T, P^T.dO, dS^T.q, dS.K), 2.5x the forward's 4*D per pair."""
    w = wl.LLAMA7B_PREFILL
    dev = torch.device("cuda")
    inp = wl.prefill_inputs(w)
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    cache = ops.KVCache(torch.zeros(shape, dtype=torch.bfloat16, device=dev),
                        torch.zeros(shape, dtype=torch.bfloat16, device=dev))
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    bt, cu, ctx, start = (inp[n].to(dev) for n in ("block_table", "cu_q", "ctx_lens", "start_pos"))
    L = max(w.seq_lens)
    ops.kv_cache_append(cache, k, v, bt, start, cu, max_new=L)
    out, lse = ops.attn_prefill_paged(q, cu, cache, bt, ctx, max_q_len=L, return_lse=True)
    d_out = wl.normal(tuple(q.shape), "bf16", w.seed, wl.STREAM_KNEW).to(dev)
    dk = torch.zeros(shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(shape, dtype=torch.float32, device=dev)
    ws = torch.empty(ops.load_library().attn_backward_workspace_bytes(q.shape[0], w.num_q_heads), dtype=torch.uint8,
                     device=dev)
    fn = lambda: ops.attn_backward_paged(q, cu, cache, bt, ctx, out, lse, d_out, max_q_len=L, max_ctx=L, dk=dk, dv=dv,
                                         workspace=ws)
    t = time_warm(fn, steps, warmup)
    pairs = sum(causal_pairs(n, w.window_left) for n in w.seq_lens)
    flops = 10 * w.head_dim * w.num_q_heads * pairs
    tf = flops / (t["mean_ms"] * 1e-3) / 1e12
    # bf16 caches run the dQ and dK/dV products on MFMA (fp32 caches on the
    # vector ALUs, whose peak is PEAK_FP32_VALU_TFLOPS).
    return dict(workload=BACKWARD, backward=_r(t), flops=flops, tflops=tf,
                roofline=dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(tf / PEAK_BF16_TFLOPS, 4), traffic=None))


def bench_page_copy(steps: int, warmup: int) -> dict:
    """kv_cache_copy_pages (the device half of copy-on-write) over 512 page
    pairs of 256 tokens x 8 KV heads x 128 dims, bf16: each copy reads and
    writes one K and one V page (2 x 512 KiB)."""
    dev = torch.device("cuda")
    n, P, hkv, d = 512, 256, 8, 128
    shape = (2 * n, P, hkv, d)
    cache = ops.KVCache(torch.randn(shape, device=dev).to(torch.bfloat16), torch.randn(shape, device=dev).to(torch.bfloat16))
    perm = torch.randperm(2 * n, generator=torch.Generator().manual_seed(9)).to(torch.int32)
    src, dst = perm[:n].to(dev), perm[n:].to(dev)
    t = time_cold(lambda: ops.kv_cache_copy_pages(cache, src, dst), max(steps, 20), warmup)
    nbytes = 2 * 2 * n * P * hkv * d * 2     # K and V, read and written
    gbs = nbytes / (t["mean_ms"] * 1e-3) / 1e9
    return dict(workload=PAGE_COPY, copy_cold=_r(t), bytes=nbytes,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None))


def cpu_baseline(w: wl.PrefillWorkload, budget_s: float = 15.0) -> dict:
    """The CPU oracle (float64 numpy) on a bounded sample of the prefill
    workload: the whole prompt's append into pages, then blocks of 256
    consecutive query rows of head 0 (each block at its own causal
    positions, spread over the prompt) until about `budget_s` seconds have
    run; TFLOP/s of the algorithmic work of the rows done."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    inp = wl.prefill_inputs(w)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    L = max(w.seq_lens)
    bt = inp["block_table"].numpy()
    blk = 256
    starts = list(range(0, L, blk))
    order = starts[::2] + starts[1::2]   # spread over the prompt first, then the rest
    pairs, rows, heads, t_append, t_attn = 0, 0, 0, 0.0, 0.0
    shape = (inp["num_pages"], w.page_size, 1, w.head_dim)
    for h in range(w.num_q_heads):
        if t_attn >= budget_s:
            break
        t0 = time.perf_counter()
        g = h // (w.num_q_heads // w.num_kv_heads)
        kp, vp = oracle.append_pages(np.zeros(shape), np.zeros(shape), f64(inp["k"][:, g:g + 1]),
                                     f64(inp["v"][:, g:g + 1]), bt, inp["start_pos"].numpy(), inp["cu_q"].numpy(),
                                     w.page_size)
        q = f64(inp["q"][:, h:h + 1])
        t1 = time.perf_counter()
        t_append += t1 - t0
        for r0 in order:
            if t_attn + (time.perf_counter() - t1) >= budget_s:
                break
            r1 = min(L, r0 + blk)
            oracle.attention_paged(q[r0:r1], np.array([0, r1 - r0]), kp, vp, bt, np.array([r1]), w.page_size,
                                   w.softmax_scale, w.causal, w.window_left)
            pairs += oracle.visible_pairs(r1 - r0, r1, w.causal, w.window_left)
            rows += r1 - r0
        t_attn += time.perf_counter() - t1
        heads += 1
    flops = 4 * w.head_dim * pairs
    return dict(value=round(flops / t_attn / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{w.name}: {rows} query rows (blocks of {blk} at their causal positions, spread over the "
                       f"prompt) over {heads} of {w.num_q_heads} heads, {pairs} visible pairs in {t_attn:.1f} s "
                       f"of float64 numpy (BLAS threads {blas_threads}); each head's append into pages took "
                       f"{t_append:.1f} s more in all")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=None, help="bench a single named workload instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run device copies of BYTES bytes (the known-size kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library runs on a single device (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": max(1, args.steps)}), flush=True)
        return 0
    ops.load_library()

    if args.workload == BACKWARD:
        print(json.dumps(bench_backward(args.steps, args.warmup)), flush=True)
        return 0
    if args.workload == PAGE_COPY:
        print(json.dumps(bench_page_copy(args.steps, args.warmup)), flush=True)
        return 0
    if args.workload:
        w = wl.WORKLOADS[args.workload]
        if isinstance(w, wl.PrefillWorkload):
            r = bench_prefill(w, args.steps, args.warmup, cold=w.window_left >= 0)
        elif w.full_tokens:
            r = bench_layered(w, args.steps, args.warmup)
        else:
            r = bench_decode(w, args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return 0

    sampler = ClockSampler()
    head = bench_prefill(HEADLINE, args.steps, args.warmup, sampler=sampler)
    print(f"[bench] {HEADLINE.name}: step {head['step']['mean_ms']:.3f} ms", file=sys.stderr, flush=True)
    others = {}
    for w, fn in ((wl.LLAMA7B_PREFILL, lambda w: bench_prefill(w, max(args.steps, 100), args.warmup)),
                  (wl.LONG_PREFILL_WINDOW, lambda w: bench_prefill(w, args.steps, args.warmup, cold=True)),
                  (wl.LLAMA70B_DECODE, lambda w: bench_decode(w, args.steps, args.warmup)),
                  (wl.DECODE_128K_INT8, lambda w: bench_decode(w, args.steps, args.warmup))):
        r = fn(w)
        others[w.name] = r
        print(f"[bench] {w.name}: done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    line = {
        "metric": "prefill TFLOP/s & decode KV-read GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(head["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step"]["mean_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, permuted page tables)",
        "config": dict(workload=HEADLINE.name, **head["config"],
                       step="attn_prefill_paged_append" + (" (append fused into the prefill kernel)" if head["fused"]
                                                            else " (append kernel, then the prefill kernel)")),
        "roofline": head["roofline"],
        "step_ms": head["step"],
        "prefill_kernel_ms": head["prefill_kernel"],
        "clocks": sampler.summary(),
        "workloads": {
            name: ({k: r[k] for k in ("timing", "fused", "step", "prefill_kernel", "roofline", "prefill_kernel_roofline")}
                   | {"tflops_step": round(r["tflops_step"], 2)})
            if "prefill_kernel" in r else
            {k: r[k] for k in ("metric", "value", "unit", "timing", "step", "step_cold", "decode_cold", "decode_warm",
                               "kv_bytes", "sum_ctx", "roofline", "warm_roofline_frac")}
            for name, r in others.items()
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(HEADLINE)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
