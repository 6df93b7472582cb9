"""GPU parity of attn_prefill_paged_append (the new rows' K/V written into
their pages and attended over in one call) against the CPU oracle's append
followed by its attention, on seeded inputs: fresh prompts, chunks after a
cached prefix whose first new position falls on a key-tile boundary, inside a
tile and inside a query tile, windows, no mask, GQA and MHA, D = 64 / 128,
and the caches that always take the two-launch route (16-key pages, fp32);
each with the route forced to the fused kernel, forced to two launches, and
left to the library.  Pools start as NaN, so a slot written twice, missed or
written out of place shows up in the bit-exact page comparison."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import bits, check_close, f64, nan_pool, say

pytestmark = pytest.mark.gpu

# (workload over the whole sequences, cached prefix length per sequence)
CASES = [
    (wl.PrefillWorkload("fresh_d128_g4_p256", (1200, 300, 77), 8, 2, 128, 256, "bf16", seed=61), (0, 0, 0)),
    # prefixes of 128 (tile-aligned), 64 (inside a query tile), 100 (inside a
    # key tile) and 1 token; 64-key pages
    (wl.PrefillWorkload("chunks_d128_g4_p64", (700, 520, 333, 129), 8, 2, 128, 64, "bf16", seed=62),
     (128, 64, 100, 1)),
    (wl.PrefillWorkload("chunks_d64_mha_p128", (513, 260, 64), 4, 4, 64, 128, "bf16", seed=63), (37, 250, 63)),
    (wl.PrefillWorkload("chunk_g8_p256", (1030,), 8, 1, 128, 256, "bf16", seed=64), (511,)),
    (wl.PrefillWorkload("window128_runs", (1500, 400), 4, 2, 128, 64, "bf16", seed=65, window_left=128), (0, 200)),
    (wl.PrefillWorkload("window0_chunk", (300,), 4, 2, 128, 64, "bf16", seed=66, window_left=0), (90,)),
    # 12 query heads in groups of 3 (the window's head-fastest order), one
    # fresh prompt and one chunk after a prefix inside a key tile
    (wl.PrefillWorkload("window64_h12_g3", (900, 400), 12, 4, 128, 64, "bf16", seed=72, window_left=64), (0, 130)),
    (wl.PrefillWorkload("noncausal_runs", (1100, 300), 2, 1, 128, 256, "bf16", seed=67, causal=False), (0, 70)),
    # a sequence with no new rows in the batch (its whole context cached)
    (wl.PrefillWorkload("empty_chunk_in_batch", (300, 200, 130), 8, 2, 128, 64, "bf16", seed=70), (0, 200, 64)),
    (wl.PrefillWorkload("two_launch_p16", (300, 77), 8, 2, 128, 16, "bf16", seed=68), (0, 33)),
    (wl.PrefillWorkload("two_launch_f32", (128, 45), 2, 1, 64, 64, "f32", seed=69), (0, 17)),
]


def _split(inp, w, prefix):
    """Rows of the cached prefixes and rows of the new chunks, as ragged
    batches (cu arrays) over the same sequences."""
    cu = inp["cu_q"].tolist()
    pre_rows, new_rows, cu_pre, cu_new = [], [], [0], [0]
    for b, (n, s) in enumerate(zip(w.seq_lens, prefix)):
        pre_rows += range(cu[b], cu[b] + s)
        new_rows += range(cu[b] + s, cu[b] + n)
        cu_pre.append(cu_pre[-1] + s)
        cu_new.append(cu_new[-1] + n - s)
    idx = lambda r: torch.tensor(r, dtype=torch.long)
    return idx(pre_rows), idx(new_rows), torch.tensor(cu_pre, dtype=torch.int32), torch.tensor(cu_new, dtype=torch.int32)


def _pools_with_prefix(w, inp, pre, cu_pre, prefix):
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    kp = nan_pool(inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim, tdt)
    vp = nan_pool(inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim, tdt)
    cache = ops.KVCache(kp, vp)
    if max(prefix) > 0:
        ops.kv_cache_append(cache, inp["k"][pre].cuda(), inp["v"][pre].cuda(), inp["block_table"].cuda(),
                            torch.zeros(w.batch, dtype=torch.int32).cuda(), cu_pre.cuda(), max_new=max(prefix))
    return cache, kp, vp


@pytest.mark.parametrize("route", ["fused", "separate", "auto"])
@pytest.mark.parametrize("w,prefix", CASES, ids=[c[0].name for c in CASES])
def test_prefill_append_matches_oracle(w, prefix, route, monkeypatch):
    """route: the library's choice between its fused kernel and two launches,
    forced either way (both must give the same result), or left to it."""
    if route == "auto":
        monkeypatch.delenv("PAGEDATTN_PREFILL_APPEND_ROUTE", raising=False)
    else:
        monkeypatch.setenv("PAGEDATTN_PREFILL_APPEND_ROUTE", route)
    say(f"prefill_append {w.name} route={route} lens={w.seq_lens} prefix={prefix}")
    inp = wl.prefill_inputs(w)
    pre, new, cu_pre, cu_new = _split(inp, w, prefix)
    q_new, k_new, v_new = inp["q"][new], inp["k"][new], inp["v"][new]
    bt, ctx = inp["block_table"].cuda(), inp["ctx_lens"].cuda()
    max_q = max(n - s for n, s in zip(w.seq_lens, prefix))

    cache, kp, vp = _pools_with_prefix(w, inp, pre, cu_pre, prefix)
    out, lse = ops.attn_prefill_paged_append(q_new.cuda(), k_new.cuda(), v_new.cuda(), cu_new.cuda(), cache, bt, ctx,
                                             max_q_len=max_q, softmax_scale=w.softmax_scale, causal=w.causal,
                                             window_left=w.window_left, return_lse=True)
    torch.cuda.synchronize()

    # Pages: the oracle's scatter of every row of every sequence into NaN pages.
    shape = (inp["num_pages"], w.page_size, w.num_kv_heads, w.head_dim)
    nan_bits = bits(torch.full(shape, float("nan"), dtype=kp.dtype))
    ek, ev = oracle.append_pages(nan_bits, nan_bits.copy(), bits(inp["k"]), bits(inp["v"]),
                                 inp["block_table"].numpy(), inp["start_pos"].numpy(), inp["cu_q"].numpy(),
                                 w.page_size)
    assert np.array_equal(bits(kp), ek), "K pages differ from the oracle's append"
    assert np.array_equal(bits(vp), ev), "V pages differ from the oracle's append"

    # Output: the oracle's attention of the new rows over the whole context.
    view = torch.float32 if w.dtype == "f32" else torch.bfloat16
    kp64 = torch.from_numpy(ek).view(view).double().numpy()
    vp64 = torch.from_numpy(ev).view(view).double().numpy()
    ref, ref_lse = oracle.attention_paged(f64(q_new), cu_new.numpy(), kp64, vp64, inp["block_table"].numpy(),
                                          inp["ctx_lens"].numpy(), w.page_size, w.softmax_scale, w.causal,
                                          w.window_left)
    check_close(out, ref, w.dtype, "out")
    err = np.abs(f64(lse) - ref_lse).max()
    say(f"  lse max|d|={err:.3e}")
    assert err <= (1e-4 if w.dtype == "f32" else 1e-3)

    # The separate calls (append at ctx - q_len, then prefill) give the same bits.
    cache2, _, _ = _pools_with_prefix(w, inp, pre, cu_pre, prefix)
    start = torch.tensor(prefix, dtype=torch.int32).cuda()
    ops.kv_cache_append(cache2, k_new.cuda(), v_new.cuda(), bt, start, cu_new.cuda(), max_new=max_q)
    out2, lse2 = ops.attn_prefill_paged(q_new.cuda(), cu_new.cuda(), cache2, bt, ctx, max_q_len=max_q,
                                        softmax_scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                                        return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(out2)), "fused and separate calls differ"
    assert np.array_equal(bits(lse), bits(lse2))


@pytest.mark.parametrize("run_tiles", [3, 8])
@pytest.mark.parametrize("w,prefix", [c for c in CASES if c[0].name in ("window128_runs", "noncausal_runs",
                                                                         "window64_h12_g3")],
                         ids=lambda c: getattr(c, "name", None))
def test_prefill_append_run_lengths(w, prefix, run_tiles, monkeypatch):
    """The fused kernel in run mode with longer runs than the grid size picks
    for these small inputs: same pages and output as the oracle."""
    monkeypatch.setenv("PAGEDATTN_PREFILL_RUN_TILES", str(run_tiles))
    test_prefill_append_matches_oracle(w, prefix, "fused", monkeypatch)


def _random_cases(n, seed=71):
    """Seeded random shapes: batch 1-4, prompt lengths 1-700, cached prefixes
    of any length (0 .. the whole sequence), causal / windowed / unmasked,
    GQA groups 1-8, D 64 / 128, pages of 64 / 128 / 256 keys."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        batch = int(rng.integers(1, 5))
        lens = tuple(int(x) for x in rng.integers(1, 701, size=batch))
        prefix = tuple(int(rng.integers(0, L + 1)) for L in lens)
        hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        page = int(rng.choice([64, 128, 256]))
        mode = i % 3  # causal, windowed, unmasked in turn
        causal = mode != 2
        window = int(rng.integers(0, 300)) if mode == 1 else -1
        w = wl.PrefillWorkload(f"random{i}", lens, hkv * group, hkv, d, page, "bf16", seed=100 + i, causal=causal,
                               window_left=window)
        cases.append((w, prefix))
    return cases


RANDOM_CASES = _random_cases(9)


@pytest.mark.parametrize("route", ["fused", "separate"])
@pytest.mark.parametrize("w,prefix", RANDOM_CASES, ids=[c[0].name for c in RANDOM_CASES])
def test_prefill_append_random_shapes(w, prefix, route, monkeypatch):
    """Random ragged batches, prefixes, masks, groups and page sizes, on both
    routes: pages bit-exact, outputs within tolerance of the oracle, and the
    same bits as the two separate calls."""
    test_prefill_append_matches_oracle(w, prefix, route, monkeypatch)
