"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times.  The 32k-row prompts are checked on every
row of two heads (the heads are independent with Hq = Hkv, so the oracle
works on pools sliced to them); the 128k decodes on all 16 sequences, one
sequence's pages at a time."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import DecodeRun, PrefillRun, check_close, f64, say

pytestmark = pytest.mark.gpu


def _dense_heads_check(run, heads):
    """Every row of one long causal sequence against the oracle, for two
    heads (MHA: heads are independent, so the pools are sliced to them),
    output and lse."""
    w = run.w
    assert w.num_q_heads == w.num_kv_heads and w.batch == 1
    out, lse = run.run(return_lse=True)
    torch.cuda.synchronize()
    inp = run.inp
    kp = np.full((inp["num_pages"], w.page_size, len(heads), w.head_dim), np.nan)
    vp = np.full_like(kp, np.nan)
    kp, vp = oracle.append_pages(kp, vp, f64(inp["k"][:, heads]), f64(inp["v"][:, heads]),
                                 inp["block_table"].numpy(), [0], inp["cu_q"].numpy(), w.page_size)
    for i, h in enumerate(heads):
        ref, ref_lse = oracle.attention_paged(f64(inp["q"][:, h:h + 1]), inp["cu_q"].numpy(), kp[:, :, i:i + 1],
                                              vp[:, :, i:i + 1], inp["block_table"].numpy(), inp["ctx_lens"].numpy(),
                                              w.page_size, w.softmax_scale, True, w.window_left)
        check_close(out[:, h:h + 1], ref, "bf16", f"all {ref.shape[0]} rows of head {h}")
        err = np.abs(f64(lse[:, h:h + 1]) - ref_lse).max()
        say(f"  head {h} lse max|d|={err:.3e}")
        assert err <= 1e-3


def test_llama7b_prefill_2048_full_oracle():
    w = wl.LLAMA7B_PREFILL
    say(f"full size: {w.name}")
    run = PrefillRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
    ref, ref_lse = run.oracle()
    check_close(out, ref, "bf16", "all rows, all heads")
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3


def test_llama7b_prompt_step_2048_fused_full_oracle():
    """The step the benchmark times: attn_prefill_paged_append (one fused
    kernel at this length) writes the pages and attends; every output and
    every page slot against the oracle."""
    w = wl.LLAMA7B_PREFILL
    say(f"full size, fused append: {w.name}")
    run = PrefillRun(w, fused=True)
    assert ops.prefill_append_is_fused(run.cache, w.causal, w.window_left, max(w.seq_lens))
    out, lse = run.run()
    torch.cuda.synchronize()
    assert run.pages_match_oracle_append(), "pages differ from the oracle's append"
    ref, ref_lse = run.oracle()
    check_close(out, ref, "bf16", "all rows, all heads")
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3


def test_llama70b_gqa_decode_full_oracle():
    w = wl.LLAMA70B_DECODE
    say(f"full size: {w.name}")
    run = DecodeRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
    (ref, ref_lse), _ = run.oracle()
    check_close(out, ref, "bf16", "all sequences, all heads")
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w,heads", [(wl.LONG_PREFILL, [0, 31]), (wl.LONG_PREFILL_WINDOW, [5, 22])],
                         ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_long_prefill_32k_every_row_of_two_heads(w, heads):
    say(f"full size: {w.name}, heads {heads}")
    run = PrefillRun(w)
    _dense_heads_check(run, heads)


@pytest.mark.timeout(900)
def test_long_window_prompt_step_32k_fused_every_row_of_two_heads():
    """The 128-key-window step at 32k rows as the benchmark times it (the
    fused kernel): every row of two heads against the oracle, every page slot
    bit for bit."""
    w = wl.LONG_PREFILL_WINDOW
    say(f"full size, fused append: {w.name}")
    run = PrefillRun(w, fused=True)
    assert ops.prefill_append_is_fused(run.cache, w.causal, w.window_left, max(w.seq_lens))
    _dense_heads_check(run, [13, 30])
    assert run.pages_match_oracle_append(), "pages differ from the oracle's append"


@pytest.mark.timeout(900)
def test_int8_decode_128k_all_sequences():
    """All 16 sequences of the 128k int8 decode, each against the oracle on
    a compact pool of its own pages (quantised by the oracle itself)."""
    w = wl.DECODE_128K_INT8
    say(f"full size: {w.name}")
    run = DecodeRun(w)
    out, lse = run.run(return_lse=True)
    torch.cuda.synchronize()
    ctx = run.inp["ctx_lens"].numpy()
    errs = []
    for b in range(w.batch):
        (ref, ref_lse), _ = run.oracle([b])
        errs.append(check_close(out[[b]], ref, "bf16", f"sequence {b} (ctx {int(ctx[b])})"))
        assert np.abs(f64(lse[[b]]) - ref_lse).max() <= 1e-3
    say(f"  all sequences: max|d|={max(e['max'] for e in errs):.3e} "
        f"mean|d|={np.mean([e['mean'] for e in errs]):.3e}")


@pytest.mark.timeout(900)
def test_layered_decode_128k_all_sequences():
    """The layered bench workload at full size (first 128 tokens bf16, the
    rest int8), in the launch configuration the bench times; every one of the
    16 sequences against the oracle, which quantises that sequence's int8
    pages itself."""
    w = wl.DECODE_128K_LAYERED
    say(f"full size: {w.name}")
    inp, full = wl.decode_inputs(w), wl.layered_full_inputs(w)
    kc, ks = ops.kv_pages_quantize_int8(inp["k_pool"].cuda())
    vc, vs = ops.kv_pages_quantize_int8(inp["v_pool"].cuda())
    ctx = inp["ctx_lens"].numpy().astype(np.int64)
    len_hi = full["lens"].numpy().astype(np.int64)
    len_lo = (ctx - len_hi).astype(np.int32)
    out = ops.attn_decode_paged_layered(inp["q"].cuda(), ops.KVCache(full["k_pool"].cuda(), full["v_pool"].cuda()),
                                        full["block_table"].cuda(), full["lens"].cuda(), ops.KVCache(kc, vc, ks, vs),
                                        inp["block_table"].cuda(), torch.from_numpy(len_lo).cuda())
    torch.cuda.synchronize()
    del kc, vc
    bt = inp["block_table"].numpy()
    hi_k, hi_v = f64(full["k_pool"]), f64(full["v_pool"])
    for b in range(w.batch):
        used = [int(p) for p in bt[b][: -(-int(len_lo[b]) // w.page_size)]]
        remap = {p: i for i, p in enumerate(used)}
        k8, k8s = oracle.quantize_int8_pages(f64(inp["k_pool"][used]))
        v8, v8s = oracle.quantize_int8_pages(f64(inp["v_pool"][used]))
        lo = dict(k=k8, v=v8, k_scales=k8s, v_scales=v8s, page_size=w.page_size, lens=len_lo[[b]],
                  block_table=np.array([[remap.get(int(p), 0) for p in bt[b]]]))
        hi = dict(k=hi_k, v=hi_v, page_size=w.full_page_size, lens=len_hi[[b]],
                  block_table=full["block_table"].numpy()[[b]])
        ref, _ = oracle.decode_layered(f64(inp["q"][[b]]), hi, lo)
        check_close(out[[b]], ref, "bf16", f"sequence {b} (ctx {int(ctx[b])})")


def test_backward_2048_sampled_heads():
    """The backward bench configuration (L=2048 causal, 32 heads, D=128, bf16,
    pages of 256) at full size; with Hq = Hkv the heads are independent, so
    the oracle differentiates three sampled heads."""
    w = wl.LLAMA7B_PREFILL
    say(f"full size backward: {w.name}")
    inp = wl.prefill_inputs(w)
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    cache = ops.KVCache(torch.zeros(shape, dtype=torch.bfloat16).cuda(), torch.zeros(shape, dtype=torch.bfloat16).cuda())
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    bt, cu, ctx, st = (inp[n].cuda() for n in ("block_table", "cu_q", "ctx_lens", "start_pos"))
    L = max(w.seq_lens)
    ops.kv_cache_append(cache, k, v, bt, st, cu, max_new=L)
    out, lse = ops.attn_prefill_paged(q, cu, cache, bt, ctx, max_q_len=L, return_lse=True)
    d_out = wl.normal(tuple(q.shape), "bf16", w.seed, wl.STREAM_KNEW)
    dq, dk, dv = ops.attn_backward_paged(q, cu, cache, bt, ctx, out, lse, d_out.cuda(), max_q_len=L, max_ctx=L)
    torch.cuda.synchronize()
    btn = inp["block_table"].numpy()
    t = np.arange(L)
    phys, slot = btn[0][t // w.page_size], t % w.page_size
    for h in (0, 13, 31):
        sl = slice(h, h + 1)
        rdq, rdk, rdv = oracle.attention_backward_paged(
            f64(inp["q"][:, sl]), inp["cu_q"].numpy(), _dense_pages(inp["k"][:, sl], w.page_size),
            _dense_pages(inp["v"][:, sl], w.page_size),
            _identity_table(L, w.page_size), inp["ctx_lens"].numpy(), w.page_size, f64(d_out[:, sl]))
        got_q = dq[:, sl].cpu().numpy()
        got_k = dk.cpu().numpy()[phys, slot][:, sl]
        got_v = dv.cpu().numpy()[phys, slot][:, sl]
        ref_k = rdk.reshape(L, 1, w.head_dim)
        ref_v = rdv.reshape(L, 1, w.head_dim)
        for what, got, ref in (("dq", got_q, rdq), ("dk", got_k, ref_k), ("dv", got_v, ref_v)):
            scale = max(1.0, float(np.abs(ref).max()))
            err = np.abs(got.astype(np.float64) - ref)
            say(f"  head {h} {what}: max|ref|={np.abs(ref).max():.3e} max|d|={err.max():.3e} mean|d|={err.mean():.3e}")
            assert err.max() <= 2e-2 * scale and err.mean() <= 2e-3 * scale, (h, what)


def _dense_pages(rows, page_size):
    """Rows [L, 1, D] laid out as consecutive pages [L / P, P, 1, D] (float64)."""
    x = f64(rows)
    return x.reshape(-1, page_size, x.shape[1], x.shape[2])


def _identity_table(n_tokens, page_size):
    return np.arange(n_tokens // page_size, dtype=np.int64)[None, :]
