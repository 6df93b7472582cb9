"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the hot path over one batch of synthetic input:
  * prefill step (the headline workload): a 2048-token Llama-2-7B-shaped
    prompt (32 heads, D=128, bf16) appended into 256-token pages with a
    permuted block table and attended over causally, by
    attn_prefill_paged_append (the append fused into the prefill kernel; the
    two separate calls, kv_cache_append then attn_prefill_paged, are timed
    beside it);
  * decode step (reported beside it): kv_cache_append of one new token for
    each of 64 Llama-2-70B-shaped GQA sequences (64 q heads, 8 KV heads,
    contexts uniform in [512, 8192]) and attn_decode_paged over their pages.

``value`` is prefill TFLOP/s over the whole prefill step (algorithmic FLOPs:
4 * D * Hq per visible (query, key) pair); the decode object gives KV-read
GB/s (each valid K/V element once per KV head).  Inputs are resident in HBM
before timing.  Kernel durations for the roofline objects come from HIP
events around back-to-back launches on the stream the library launches on
(torch's current stream).  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from flashattention_paged_kv_amd import ops  # noqa: E402
from flashattention_paged_kv_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def causal_pairs(n: int, window_left: int = -1) -> int:
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


def _time_loop(fn, steps: int, warmup: int, min_warm_s: float = 0.2) -> float:
    """Average ms per call of fn() over `steps` back-to-back calls.  The
    untimed warm-up runs `warmup` calls and then keeps calling until at least
    `min_warm_s` seconds of work have run, so the clocks have settled before
    the timed region (a 50-call loop of a 60 us kernel is over in 3 ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def bench_prefill(w: wl.PrefillWorkload, steps: int, warmup: int) -> dict:
    dev = torch.device("cuda")
    inp = wl.prefill_inputs(w)
    tdt = torch.bfloat16
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    cache = ops.KVCache(torch.zeros(shape, dtype=tdt, device=dev), torch.zeros(shape, dtype=tdt, device=dev))
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    bt, cu, ctx, start = (inp[n].to(dev) for n in ("block_table", "cu_q", "ctx_lens", "start_pos"))
    out = torch.empty_like(q)
    max_len = max(w.seq_lens)

    def append():
        ops.kv_cache_append(cache, k, v, bt, start, cu, max_new=max_len)

    def prefill():
        ops.attn_prefill_paged(q, cu, cache, bt, ctx, max_q_len=max_len, softmax_scale=w.softmax_scale,
                               causal=w.causal, window_left=w.window_left, out=out)

    def separate():
        append()
        prefill()

    def step():  # the append fused into the prefill kernel: one launch
        ops.attn_prefill_paged_append(q, k, v, cu, cache, bt, ctx, max_q_len=max_len, softmax_scale=w.softmax_scale,
                                      causal=w.causal, window_left=w.window_left, out=out)

    ms_step = _time_loop(step, steps, warmup)
    ms_separate = _time_loop(separate, steps, warmup)
    ms_attn_only = _time_loop(prefill, steps, warmup)
    # The dominant kernel: the step itself when it is one fused launch, else
    # the attention kernel (the step is then the append kernel + it).
    fused = ops.prefill_append_is_fused(cache, w.causal, w.window_left, max_len)
    ms_kernel = ms_step if fused else ms_attn_only
    pairs = sum(causal_pairs(n, w.window_left) for n in w.seq_lens)
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    kv_bytes = 2 * sum(w.seq_lens) * w.num_kv_heads * w.head_dim * 2
    # Algorithmic HBM bytes: Q and O once per query row, K and V once per key.
    io_bytes = 2 * sum(w.seq_lens) * w.num_q_heads * w.head_dim * 2 + kv_bytes
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    if flops / io_bytes >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    else:  # below the ridge point (a short window): bytes bound it
        gbs = io_bytes / (ms_kernel * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4))
    roof["traffic"] = _traffic("prefill_bf16_kernel_fused" if fused else "prefill_bf16_kernel", w.name)
    # The same for attention alone (attn_prefill_paged, no append), for reference.
    attn = flops / (ms_attn_only * 1e-3) / 1e12
    roof_attn = dict(bound=roof["bound"], achieved=round(attn, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(attn / PEAK_BF16_TFLOPS, 4), traffic=_traffic("prefill_bf16_kernel", w.name))
    if roof["bound"] == "hbm":
        gbs = io_bytes / (ms_attn_only * 1e-3) / 1e9
        roof_attn.update(achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4))
    return dict(workload=w.name, fused=fused, ms_per_step=ms_step, ms_prefill_kernel=ms_kernel,
                ms_separate_calls=ms_separate,
                ms_attention_only=ms_attn_only, flops=flops,
                tflops_step=flops / (ms_step * 1e-3) / 1e12, tflops_kernel=achieved, kv_bytes=kv_bytes,
                io_bytes=io_bytes, roofline=roof, attention_only_roofline=roof_attn)


def bench_decode(w: wl.DecodeWorkload, steps: int, warmup: int) -> dict:
    dev = torch.device("cuda")
    inp = wl.decode_inputs(w)
    bt, ctx, start, cun = (inp[n].to(dev) for n in ("block_table", "ctx_lens", "start_pos", "cu_new"))
    q, k_new, v_new = (inp[n].to(dev) for n in ("q", "k_new", "v_new"))
    kd, vd = inp["k_pool"].to(dev), inp["v_pool"].to(dev)
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

    ms_step = _time_loop(step, steps, warmup)
    ms_kernel = _time_loop(decode, steps, warmup)
    ctx_np = inp["ctx_lens"].numpy().astype(np.int64)
    esz = 1 if w.kv_dtype == "i8" else 2
    kv_bytes = int(2 * ctx_np.sum() * w.num_kv_heads * w.head_dim * esz)
    if w.kv_dtype == "i8":
        kv_bytes += int(2 * sum(-(-int(c) // w.page_size) for c in ctx_np) * w.num_kv_heads * 4)
    gbs = kv_bytes / (ms_kernel * 1e-3) / 1e9
    return dict(workload=w.name, ms_per_step=ms_step, ms_decode_kernels=ms_kernel, kv_bytes=kv_bytes,
                gbs_step=kv_bytes / (ms_step * 1e-3) / 1e9, gbs_kernel=gbs, sum_ctx=int(ctx_np.sum()),
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4),
                              traffic=_traffic("decode_split_kernel", w.name)))


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

    ms = _time_loop(decode, steps, warmup)
    row = w.num_kv_heads * w.head_dim
    kv_bytes = int(2 * len_hi.sum() * row * 2 + 2 * len_lo.sum() * row
                   + 2 * sum(-(-int(c) // w.page_size) for c in len_lo) * w.num_kv_heads * 4)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    return dict(workload=w.name, ms_decode_kernels=ms, kv_bytes=kv_bytes, gbs_kernel=gbs,
                sum_ctx=int(ctx_np.sum()), full_tokens=w.full_tokens,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None))


PAGE_COPY = "page_copy_512_pages_p256_hkv8_d128_bf16"
BACKWARD = "backward_causal_L2048_h32_d128_p256_bf16"
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (dual issue) x 2.4 GHz


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
    ms = _time_loop(fn, steps, warmup)
    pairs = sum(causal_pairs(n, w.window_left) for n in w.seq_lens)
    flops = 10 * w.head_dim * w.num_q_heads * pairs
    tf = flops / (ms * 1e-3) / 1e12
    # bf16 caches run the dQ and dK/dV products on MFMA (fp32 caches on the
    # vector ALUs, whose peak is PEAK_FP32_VALU_TFLOPS).
    return dict(workload=BACKWARD, ms_backward_kernels=ms, flops=flops, tflops=tf,
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
    ms = _time_loop(lambda: ops.kv_cache_copy_pages(cache, src, dst), steps, warmup)
    nbytes = 2 * 2 * n * P * hkv * d * 2     # K and V, read and written
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(workload=PAGE_COPY, ms_copy_kernel=ms, bytes=nbytes,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None))


def cpu_baseline(w: wl.PrefillWorkload, budget_s: float = 15.0) -> dict:
    """The CPU oracle (float64 numpy) on a bounded sample of the prefill
    workload: the whole prompt's append, then as many heads of the causal
    attention as fit in about `budget_s` seconds (heads are independent)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    inp = wl.prefill_inputs(w)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    t0 = time.perf_counter()
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    kp, vp = oracle.append_pages(np.zeros(shape), np.zeros(shape), f64(inp["k"]), f64(inp["v"]),
                                 inp["block_table"].numpy(), inp["start_pos"].numpy(), inp["cu_q"].numpy(),
                                 w.page_size)
    q = f64(inp["q"])
    heads = 0
    while heads < w.num_q_heads and time.perf_counter() - t0 < budget_s:
        h = heads
        oracle.attention_paged(q[:, h:h + 1], inp["cu_q"].numpy(), kp[:, :, h:h + 1], vp[:, :, h:h + 1],
                               inp["block_table"].numpy(), inp["ctx_lens"].numpy(), w.page_size,
                               w.softmax_scale, w.causal, w.window_left)
        heads += 1
    dt = time.perf_counter() - t0
    pairs = sum(causal_pairs(n, w.window_left) for n in w.seq_lens)
    flops = 4 * w.head_dim * heads * pairs
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{w.name}: append of all {sum(w.seq_lens)} tokens + causal attention of {heads} of "
                       f"{w.num_q_heads} heads ({dt:.1f} s, float64 numpy)")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
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
            r = bench_prefill(w, args.steps, args.warmup)
        elif w.full_tokens:
            r = bench_layered(w, args.steps, args.warmup)
        else:
            r = bench_decode(w, args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return 0

    pre = bench_prefill(wl.LLAMA7B_PREFILL, args.steps, args.warmup)
    dec = bench_decode(wl.LLAMA70B_DECODE, args.steps, args.warmup)
    line = {
        "metric": "prefill TFLOP/s & decode KV-read GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(pre["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, permuted page tables)",
        "config": {"workload": pre["workload"], "batch": 1, "seq_len": 2048, "num_q_heads": 32,
                   "num_kv_heads": 32, "head_dim": 128, "page_size": 256, "causal": True,
                   "step": "attn_prefill_paged_append" + (" (append fused into the prefill kernel)" if pre["fused"]
                                                            else " (append kernel, then the prefill)")},
        "roofline": pre["roofline"],
        "prefill_kernel_ms": round(pre["ms_prefill_kernel"], 5),
        "separate_calls_ms": round(pre["ms_separate_calls"], 5),
        "attention_only_kernel_ms": round(pre["ms_attention_only"], 5),
        "attention_only_roofline": pre["attention_only_roofline"],
        "decode": {"metric": "decode KV-read GB/s", "value": round(dec["gbs_step"], 1), "unit": "GB/s",
                   "ms_per_step": round(dec["ms_per_step"], 5), "kernel_ms": round(dec["ms_decode_kernels"], 5),
                   "kv_bytes": dec["kv_bytes"], "sum_ctx": dec["sum_ctx"],
                   "config": {"workload": dec["workload"], "step": "kv_cache_append + attn_decode_paged"},
                   "roofline": dec["roofline"]},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl.LLAMA7B_PREFILL)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
