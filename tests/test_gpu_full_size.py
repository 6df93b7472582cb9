"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration the benchmark times.  Where the oracle cannot do every output
in seconds it checks sampled rows (prefill) or sampled sequences (int8
decode), always all heads of a sampled row or a fixed head subset."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import DecodeRun, PrefillRun, check_close, f64, say

pytestmark = pytest.mark.gpu


def _sampled_rows_check(run, rows, heads):
    """Oracle rows of one long causal sequence, for a subset of heads (MHA:
    heads are independent, so the pools are sliced to those heads)."""
    w = run.w
    assert w.num_q_heads == w.num_kv_heads and w.batch == 1
    out = run.run(return_lse=False)
    torch.cuda.synchronize()
    inp = run.inp
    kp = np.full((inp["num_pages"], w.page_size, len(heads), w.head_dim), np.nan)
    vp = np.full_like(kp, np.nan)
    kp, vp = oracle.append_pages(kp, vp, f64(inp["k"][:, heads]), f64(inp["v"][:, heads]),
                                 inp["block_table"].numpy(), [0], inp["cu_q"].numpy(), w.page_size)
    q = f64(inp["q"][rows][:, heads])
    table = np.repeat(inp["block_table"].numpy(), len(rows), axis=0)
    ref, _ = oracle.attention_paged(q, np.arange(len(rows) + 1), kp, vp, table, np.array(rows) + 1, w.page_size,
                                    w.softmax_scale, True, w.window_left)
    got = out[torch.tensor(rows)][:, heads]
    return check_close(got, ref, "bf16", f"{len(rows)} rows x {len(heads)} heads")


def test_llama7b_prefill_2048_full_oracle():
    w = wl.LLAMA7B_PREFILL
    say(f"full size: {w.name}")
    run = PrefillRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
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


ROWS_32K = [0, 1, 63, 64, 127, 128, 129, 1000, 4095, 4096, 8191, 12345, 16384, 20000, 24575, 30000, 32766, 32767]


@pytest.mark.parametrize("w", [wl.LONG_PREFILL, wl.LONG_PREFILL_WINDOW], ids=lambda w: w.name)
def test_long_prefill_32k_sampled_rows(w):
    say(f"full size: {w.name}")
    run = PrefillRun(w)
    _sampled_rows_check(run, ROWS_32K, [0, 13, 31])


def test_int8_decode_128k_sampled_sequences():
    w = wl.DECODE_128K_INT8
    say(f"full size: {w.name}")
    run = DecodeRun(w)
    out = run.run(return_lse=False)
    torch.cuda.synchronize()
    ctx = run.inp["ctx_lens"].numpy()
    seqs = [int(np.argmin(ctx)), int(np.argmax(ctx)), 7]
    (ref, _), _ = run.oracle(seqs)
    check_close(out[seqs], ref, "bf16", f"sequences {seqs} (ctx {ctx[seqs].tolist()})")
