"""attn_decode_paged_noalloc (the decode entry point that allocates nothing,
its split partials in the library's own per-GPU scratch array) against
attn_decode_paged with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, each bit for bit equal to the
workspace call's output and lse and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import DecodeRun, bits, check_close, f64, say

pytestmark = pytest.mark.gpu


def _both(run):
    w = run.w
    out_ws, lse_ws = run.run(return_lse=True)
    out = torch.empty_like(run.q)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    ops.attn_decode_paged_noalloc(run.q, run.cache, run.bt, run.ctx, out, lse, softmax_scale=w.softmax_scale,
                                  window_left=w.window_left)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out, lse


def test_noalloc_decode_matches_the_workspace_call_twice():
    big = wl.LLAMA70B_DECODE
    say(f"noalloc decode, call 1: {big.name}")
    run1 = DecodeRun(big)
    need = ops.decode_workspace_bytes(big.batch, big.num_q_heads, big.num_kv_heads, big.head_dim,
                                      run1.bt.shape[1], big.page_size)
    assert need <= ops.NOALLOC_SCRATCH_BYTES
    out_ws, lse_ws, out, lse = _both(run1)
    assert np.array_equal(bits(out), bits(out_ws)) and np.array_equal(bits(lse), bits(lse_ws))
    seqs = [0, 17, 63]
    (ref, _), _ = run1.oracle(seqs)
    check_close(out[seqs], ref, "bf16", f"call 1, sequences {seqs}")
    del run1

    small = wl.DecodeWorkload("noalloc_small", 5, 0, 0, 16, 2, 128, 16, "i8", seed=81,
                              ctx_lens=(1, 33, 700, 4000, 2500))
    say(f"noalloc decode, call 2 (smaller): {small.name}")
    run2 = DecodeRun(small)
    out_ws, lse_ws, out, lse = _both(run2)
    assert np.array_equal(bits(out), bits(out_ws)) and np.array_equal(bits(lse), bits(lse_ws))
    (ref, ref_lse), _ = run2.oracle()
    check_close(out, ref, "bf16", "call 2, all sequences")
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3
