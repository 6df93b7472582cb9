"""GPU parity of every entry point against the CPU oracle, on small seeded
inputs that still span several tiles, pages and splits with ragged tails,
plus the invariants the pages fix (cached decode = recompute, page shuffles)
and edge cases (lengths around page and tile boundaries, windows 0/1/127/128,
GQA group sizes 1/8/16, poisoned slots past the end of each sequence)."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_paged_kv_amd import ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import DecodeRun, PrefillRun, bits, check_close, f64, nan_pool, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("page_size", [16, 256])
def test_append_is_a_bitwise_scatter(dtype, page_size):
    w = wl.PrefillWorkload("append", (300, 77, 1, 256), 4, 2, 128, page_size, dtype, seed=11, spare_pages=3)
    say(f"append dtype={dtype} P={page_size}")
    inp = wl.prefill_inputs(w)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kp = nan_pool(inp["num_pages"], page_size, 2, 128, tdt)
    vp = nan_pool(inp["num_pages"], page_size, 2, 128, tdt)
    before_k, before_v = bits(kp), bits(vp)
    ops.kv_cache_append(ops.KVCache(kp, vp), inp["k"].cuda(), inp["v"].cuda(), inp["block_table"].cuda(),
                        inp["start_pos"].cuda(), inp["cu_q"].cuda(), max_new=300)
    torch.cuda.synchronize()
    ek, ev = oracle.append_pages(before_k, before_v, bits(inp["k"]), bits(inp["v"]), inp["block_table"].numpy(),
                                 inp["start_pos"].numpy(), inp["cu_q"].numpy(), page_size)
    assert np.array_equal(bits(kp), ek) and np.array_equal(bits(vp), ev)


@pytest.mark.parametrize("page_size,d", [(16, 128), (256, 128), (32, 64)])
def test_int8_quantiser_is_bit_exact(page_size, d):
    say(f"quantise P={page_size} D={d}")
    x = wl.normal((7, page_size, 3, d), "bf16", 21, 1)
    x[2, :, 1, :] = 0.0                      # an all-zero group
    x[4, 3, 0, 5] = 40.0                     # an outlier
    codes, scales = ops.kv_pages_quantize_int8(x.cuda())
    torch.cuda.synchronize()
    ec, es = oracle.quantize_int8_pages(x.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), ec)
    assert np.array_equal(bits(scales), es.view(np.int32))


PREFILL_CASES = [
    wl.PrefillWorkload("bf16_d128_g4_p16", (300, 77, 1, 128, 129), 8, 2, 128, 16, "bf16", seed=31, spare_pages=2),
    wl.PrefillWorkload("bf16_d64_mha_p256", (513,), 4, 4, 64, 256, "bf16", seed=32),
    wl.PrefillWorkload("bf16_d128_g8_win0", (200, 31), 8, 1, 128, 64, "bf16", seed=33, window_left=0),
    wl.PrefillWorkload("bf16_d128_g8_win1", (200, 31), 8, 1, 128, 64, "bf16", seed=33, window_left=1),
    wl.PrefillWorkload("bf16_d128_g8_win127", (400, 31), 8, 1, 128, 64, "bf16", seed=33, window_left=127),
    wl.PrefillWorkload("bf16_d128_g8_win128", (400, 129), 8, 1, 128, 64, "bf16", seed=33, window_left=128),
    wl.PrefillWorkload("bf16_d128_win_big", (300,), 2, 2, 128, 16, "bf16", seed=34, window_left=5000),
    wl.PrefillWorkload("bf16_noncausal", (100, 65), 2, 2, 128, 16, "bf16", seed=35, causal=False),
    # Several runs of 8 query tiles per sequence (windowed and unmasked
    # prefill split work that way), with partial last runs.
    wl.PrefillWorkload("bf16_win200_runs", (1500, 1030), 4, 2, 128, 64, "bf16", seed=39, window_left=200),
    wl.PrefillWorkload("bf16_noncausal_runs", (1100,), 2, 1, 128, 256, "bf16", seed=40, causal=False),
    # A window orders its workgroups query-head-fastest: 12 heads (groups of
    # 3, not a power of two), two sequences of several query tiles.
    wl.PrefillWorkload("bf16_h12_g3_win64", (1400, 520), 12, 4, 128, 64, "bf16", seed=42, window_left=64),
    wl.PrefillWorkload("f32_d64_p16", (128, 45), 2, 1, 64, 16, "f32", seed=36),
    wl.PrefillWorkload("f32_d128_win3", (70,), 2, 2, 128, 32, "f32", seed=37, window_left=3),
    # fp32 on its MFMA kernel (32-row blocks, 32-key steps): ragged rows over
    # several blocks, GQA 4:1, 64-key pages, unmasked and with a window that
    # starts inside a key step
    wl.PrefillWorkload("f32_d128_g4_noncausal", (97, 200, 1), 8, 2, 128, 64, "f32", seed=38, causal=False),
    wl.PrefillWorkload("f32_d64_win45", (161, 33), 4, 1, 64, 16, "f32", seed=41, window_left=45),
]


@pytest.mark.parametrize("w", PREFILL_CASES, ids=lambda w: w.name)
def test_prefill_matches_oracle(w):
    say(f"prefill {w}")
    run = PrefillRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
    ref, ref_lse = run.oracle()
    check_close(out, ref, w.dtype, "out")
    err = np.abs(f64(lse) - ref_lse).max()
    say(f"  lse max|d|={err:.3e}")
    assert err <= (1e-4 if w.dtype == "f32" else 1e-3)


def _random_prefill_cases(n, seed=81):
    """Seeded random shapes for the prefill alone: batch 1-3, lengths
    1-1500, GQA groups 1-4 over 1-3 KV heads (head counts that are not
    powers of two included), causal / windowed / unmasked in turn, D = 128,
    64- and 256-key pages."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        batch = int(rng.integers(1, 4))
        lens = tuple(int(x) for x in rng.integers(1, 1501, size=batch))
        hkv = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 3, 4]))
        mode = i % 3
        cases.append(wl.PrefillWorkload(f"random_prefill{i}", lens, hkv * group, hkv, 128, int(rng.choice([64, 256])),
                                        "bf16", seed=200 + i, causal=mode != 2,
                                        window_left=int(rng.integers(0, 400)) if mode == 1 else -1))
    return cases


@pytest.mark.parametrize("w", _random_prefill_cases(12), ids=lambda w: w.name)
def test_prefill_random_shapes(w):
    """Random ragged batches, head counts, masks and page sizes."""
    test_prefill_matches_oracle(w)


RUN_MODE_CASES = [w for w in PREFILL_CASES if w.name in ("bf16_win200_runs", "bf16_noncausal_runs",
                                                           "bf16_d128_g8_win128", "bf16_h12_g3_win64")]


@pytest.mark.parametrize("run_tiles", [2, 3, 8])
@pytest.mark.parametrize("w", RUN_MODE_CASES, ids=lambda w: w.name)
def test_prefill_run_lengths_match_oracle(w, run_tiles, monkeypatch):
    """Windowed and unmasked prefill give each workgroup a run of query
    tiles, as many as the grid allows (one on inputs this small); forced run
    lengths cover longer runs, partial last runs and the engines' split."""
    monkeypatch.setenv("PAGEDATTN_PREFILL_RUN_TILES", str(run_tiles))
    say(f"prefill {w.name} run_tiles={run_tiles}")
    run = PrefillRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
    ref, ref_lse = run.oracle()
    check_close(out, ref, w.dtype, "out")
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3


def test_chunked_prefill_rows_at_the_end_of_a_context():
    """q_len < ctx: the queries are the last rows of a longer cached context
    (bottom-right causal alignment)."""
    w = wl.PrefillWorkload("chunk", (700, 260), 8, 2, 128, 16, "bf16", seed=38)
    say("chunked prefill")
    run = PrefillRun(w)
    q_lens = [130, 1]
    cu = [0]
    rows = []
    for b, (n, ql) in enumerate(zip(w.seq_lens, q_lens)):
        start = int(run.inp["cu_q"][b])
        rows.append(run.inp["q"][start + n - ql:start + n])
        cu.append(cu[-1] + ql)
    q = torch.cat(rows)
    cu_t = torch.tensor(cu, dtype=torch.int32)
    out = ops.attn_prefill_paged(q.cuda(), cu_t.cuda(), run.cache, run.bt, run.ctx, max_q_len=max(q_lens))
    kp, vp = run.oracle_pools()
    ref, _ = oracle.attention_paged(f64(q), cu, kp, vp, run.inp["block_table"].numpy(), run.inp["ctx_lens"].numpy(),
                                    w.page_size)
    check_close(out, ref, "bf16", "chunked out")


DECODE_CASES = [
    wl.DecodeWorkload("bf16_g8_p16_edges", 10, 0, 0, 16, 2, 128, 16, "bf16", seed=41, spare_pages=2,
                      ctx_lens=(1, 15, 16, 17, 255, 256, 257, 1000, 3000, 5000)),
    wl.DecodeWorkload("bf16_g8_p256", 6, 1, 3000, 64, 8, 128, 256, "bf16", seed=42),
    wl.DecodeWorkload("bf16_d64_g1_p32", 5, 1, 2000, 4, 4, 64, 32, "bf16", seed=43),
    wl.DecodeWorkload("bf16_g16", 3, 1, 1500, 16, 1, 128, 64, "bf16", seed=44),
    wl.DecodeWorkload("bf16_win0", 4, 1, 900, 16, 2, 128, 16, "bf16", seed=45, window_left=0),
    wl.DecodeWorkload("bf16_win1", 4, 1, 900, 16, 2, 128, 16, "bf16", seed=45, window_left=1),
    wl.DecodeWorkload("bf16_win127", 4, 1, 900, 16, 2, 128, 16, "bf16", seed=45, window_left=127),
    wl.DecodeWorkload("bf16_win128", 4, 1, 900, 16, 2, 128, 256, "bf16", seed=45, window_left=128),
    wl.DecodeWorkload("i8_g4_p16", 7, 0, 0, 8, 2, 128, 16, "i8", seed=46, spare_pages=2,
                      ctx_lens=(1, 16, 17, 33, 300, 2049, 4100)),
    wl.DecodeWorkload("i8_g8_p256_win200", 4, 1, 3000, 64, 8, 128, 256, "i8", seed=47, window_left=200),
    wl.DecodeWorkload("i8_d64", 3, 1, 2500, 8, 1, 64, 128, "i8", seed=48),
    wl.DecodeWorkload("f32_d64", 3, 1, 500, 1, 1, 64, 16, "f32", seed=49),
    wl.DecodeWorkload("f32_d128_g2_win9", 3, 1, 300, 4, 2, 128, 32, "f32", seed=50, window_left=9),
]


@pytest.mark.parametrize("w", DECODE_CASES, ids=lambda w: w.name)
def test_decode_matches_oracle(w):
    say(f"decode {w.name} ctx={wl.decode_ctx_lens(w).tolist()}")
    run = DecodeRun(w)
    out, lse = run.run()
    torch.cuda.synchronize()
    (ref, ref_lse), _ = run.oracle()
    check_close(out, ref, "f32" if w.kv_dtype == "f32" else "bf16", "out")
    err = np.abs(f64(lse) - ref_lse).max()
    say(f"  lse max|d|={err:.3e}")
    assert err <= (1e-4 if w.kv_dtype == "f32" else 1e-3)


def test_tiny_fp32_prefill_then_16_decode_steps():
    """fp32, 1 head, D=64, 128-token causal prefill then 16 single-token
    decode steps appending to a cache of 16-token pages with a permuted block
    table; every step against the oracle at 1e-4."""
    base = wl.TINY_FP32
    n_total = 128 + wl.TINY_FP32_DECODE_STEPS
    w = wl.PrefillWorkload(base.name, (n_total,), 1, 1, 64, 16, "f32", seed=base.seed)
    say("tiny fp32 prefill + 16 decode steps")
    inp = wl.prefill_inputs(w)
    dev = "cuda"
    kp = nan_pool(inp["num_pages"], 16, 1, 64, torch.float32)
    vp = nan_pool(inp["num_pages"], 16, 1, 64, torch.float32)
    cache = ops.KVCache(kp, vp)
    bt = inp["block_table"].to(dev)
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    ops.kv_cache_append(cache, k[:128], v[:128], bt, i32([0]), i32([0, 128]))
    out = ops.attn_prefill_paged(q[:128], i32([0, 128]), cache, bt, i32([128]), max_q_len=128)
    dec = []
    for t in range(128, n_total):
        ops.kv_cache_append(cache, k[t:t + 1], v[t:t + 1], bt, i32([t]), i32([0, 1]))
        dec.append(ops.attn_decode_paged(q[t:t + 1], cache, bt, i32([t + 1])))
    torch.cuda.synchronize()
    kpo, vpo = oracle.append_pages(np.full(kp.shape, np.nan), np.full(vp.shape, np.nan), f64(inp["k"]),
                                   f64(inp["v"]), inp["block_table"].numpy(), [0], [0, n_total], 16)
    ref, _ = oracle.attention_paged(f64(inp["q"]), [0, n_total], kpo, vpo, inp["block_table"].numpy(), [n_total], 16)
    check_close(out, ref[:128], "f32", "prefill")
    check_close(torch.cat(dec), ref[128:], "f32", "decode steps")


def test_decode_equals_last_prefill_row():
    w = wl.PrefillWorkload("dec_eq_pre", (300,), 8, 2, 128, 16, "bf16", seed=51)
    say("decode == last prefill row")
    run = PrefillRun(w)
    out = run.run(return_lse=False)
    dec = ops.attn_decode_paged(run.q[-1:].contiguous(), run.cache, run.bt, run.ctx)
    torch.cuda.synchronize()
    d = (dec[0].double() - out[-1].double()).abs().max().item()
    say(f"  max|decode - prefill row| = {d:.3e}")
    assert d <= 2e-2


def _shuffle(pool, bt, seed):
    n = pool.shape[0]
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(n)).to(pool.device)
    new = torch.empty_like(pool)
    new[perm] = pool                         # old page i -> new page perm[i]
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    return new, bt2


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_decode_page_shuffle_is_bitwise_identical(kv):
    w = wl.DecodeWorkload("shuffle", 5, 1, 3000, 16, 2, 128, 16, kv, seed=52)
    say(f"decode page shuffle {kv}")
    run = DecodeRun(w)
    out1 = run.run(return_lse=False)
    c = run.cache
    k2, bt2 = _shuffle(c.k_pages, run.bt, 1)
    v2, _ = _shuffle(c.v_pages, run.bt, 1)
    ks2 = vs2 = None
    if kv == "i8":
        ks2, _ = _shuffle(c.k_scales, run.bt, 1)
        vs2, _ = _shuffle(c.v_scales, run.bt, 1)
    out2 = ops.attn_decode_paged(run.q, ops.KVCache(k2, v2, ks2, vs2), bt2, run.ctx)
    out3 = run.run(return_lse=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out1), bits(out2))
    assert np.array_equal(bits(out1), bits(out3))      # run-to-run determinism


def test_prefill_page_shuffle_is_bitwise_identical():
    w = wl.PrefillWorkload("pshuffle", (333, 64), 8, 2, 128, 16, "bf16", seed=53)
    say("prefill page shuffle")
    run = PrefillRun(w)
    out1 = run.run(return_lse=False)
    k2, bt2 = _shuffle(run.k_pool, run.bt, 2)
    v2, _ = _shuffle(run.v_pool, run.bt, 2)
    out2 = ops.attn_prefill_paged(run.q, run.cu, ops.KVCache(k2, v2), bt2, run.ctx, max_q_len=333)
    out3 = run.run(return_lse=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out1), bits(out2))
    assert np.array_equal(bits(out1), bits(out3))


@pytest.mark.parametrize("wgs", ["1", "7", "64", "5000"])
def test_decode_other_grid_sizes_match_oracle(monkeypatch, wgs):
    """The balanced decode partition cuts the (sequence, KV head, tile) list
    into as many equal ranges as there are workgroups; any grid size must
    give the same attention within tolerance (pieces, partial slots and the
    merge all move with it)."""
    w = wl.DecodeWorkload("grids", 5, 0, 0, 16, 2, 128, 16, "bf16", seed=54,
                          ctx_lens=(1, 33, 700, 4000, 2500))
    run = DecodeRun(w)
    base = run.run(return_lse=False)
    monkeypatch.setenv("PAGEDATTN_DECODE_WGS", wgs)
    say(f"decode with {wgs} workgroups")
    other = run.run(return_lse=False)
    torch.cuda.synchronize()
    (ref, _), _ = run.oracle()
    check_close(other, ref, "bf16", f"{wgs} workgroups")
    assert (other.double() - base.double()).abs().max().item() <= 2e-2


def test_shared_prefix_pages_match_oracle():
    """Two sequences whose block tables share the physical pages of a common
    prefix (the refcounted prefix sharing of "Flash Attention与Paged KV Cache
    优化大模型计算效率" section 3.2's page table, one page set read by two
    logical sequences): the prefix is appended once, each sequence appends its
    own suffix into private pages, and chunked prefill of the suffixes plus a
    decode step of each sequence must match the oracle on the same tables."""
    P, hq, hkv, d, seed = 16, 8, 2, 128, 60
    n_pre, n_a, n_b = 160, 70, 45                      # prefix = 10 whole pages
    pre_pages, a_pages, b_pages = n_pre // P, -(-n_a // P), -(-n_b // P)
    n_pages = pre_pages + a_pages + b_pages + 2        # two spare pages
    perm = wl.rng(seed, wl.STREAM_PERM).permutation(n_pages).astype(np.int32)
    shared, own_a = perm[:pre_pages], perm[pre_pages:pre_pages + a_pages]
    own_b = perm[pre_pages + a_pages:pre_pages + a_pages + b_pages]
    width = pre_pages + max(a_pages, b_pages)
    bt = np.full((2, width), -1, dtype=np.int32)
    bt[0, :pre_pages + a_pages] = np.concatenate([shared, own_a])
    bt[1, :pre_pages + b_pages] = np.concatenate([shared, own_b])
    k_all = wl.normal((n_pre + n_a + n_b, hkv, d), "bf16", seed, wl.STREAM_K)
    v_all = wl.normal((n_pre + n_a + n_b, hkv, d), "bf16", seed, wl.STREAM_V)
    q = wl.normal((n_a + n_b, hq, d), "bf16", seed, wl.STREAM_Q)
    q_dec = wl.normal((2, hq, d), "bf16", seed + 1, wl.STREAM_Q)
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32)).cuda()
    say("shared prefix pages")
    kp = nan_pool(n_pages, P, hkv, d, torch.bfloat16)
    vp = nan_pool(n_pages, P, hkv, d, torch.bfloat16)
    cache = ops.KVCache(kp, vp)
    # prefix once (through sequence 0's table), then both suffixes
    ops.kv_cache_append(cache, k_all[:n_pre].cuda(), v_all[:n_pre].cuda(), i32(bt[:1]), i32([0]), i32([0, n_pre]),
                        max_new=n_pre)
    shared_before = bits(kp[torch.from_numpy(shared).long().cuda()])
    ops.kv_cache_append(cache, k_all[n_pre:].cuda(), v_all[n_pre:].cuda(), i32(bt), i32([n_pre, n_pre]),
                        i32([0, n_a, n_a + n_b]), max_new=max(n_a, n_b))
    assert np.array_equal(shared_before, bits(kp[torch.from_numpy(shared).long().cuda()]))
    ctx = [n_pre + n_a, n_pre + n_b]
    out = ops.attn_prefill_paged(q.cuda(), i32([0, n_a, n_a + n_b]), cache, i32(bt), i32(ctx), max_q_len=n_a)
    dec = ops.attn_decode_paged(q_dec.cuda(), cache, i32(bt), i32(ctx))
    torch.cuda.synchronize()
    # the oracle replays the same appends on NaN pools
    shape = (n_pages, P, hkv, d)
    okp, ovp = oracle.append_pages(np.full(shape, np.nan), np.full(shape, np.nan), f64(k_all[:n_pre]),
                                   f64(v_all[:n_pre]), bt[:1], [0], [0, n_pre], P)
    okp, ovp = oracle.append_pages(okp, ovp, f64(k_all[n_pre:]), f64(v_all[n_pre:]), bt, [n_pre, n_pre],
                                   [0, n_a, n_a + n_b], P)
    ref, _ = oracle.attention_paged(f64(q), [0, n_a, n_a + n_b], okp, ovp, bt, ctx, P)
    check_close(out, ref, "bf16", "prefill of both suffixes")
    ref_dec, _ = oracle.decode_paged(f64(q_dec), okp, ovp, bt, ctx, P)
    check_close(dec, ref_dec, "bf16", "decode of both sequences")


def test_int8_append_is_bit_exact_then_decodes():
    """Appends into an int8 cache requantise each touched (page, KV head)
    group over its valid slots; codes and scales must equal the oracle's bit
    for bit after several ragged rounds (starting mid-page, crossing pages),
    and decode over the result must match the oracle's dequantised cache."""
    P, hq, hkv, d, seed = 16, 8, 2, 128, 61
    start0 = [0, 37, 16, 5]                       # lengths before the first append
    rounds = [[5, 20, 1, 11], [1, 1, 1, 0], [40, 3, 0, 12]]
    final = [s + sum(r[b] for r in rounds) for b, s in enumerate(start0)]
    pages = [-(-n // P) for n in final]
    n_pages = sum(pages) + 2
    perm = wl.rng(seed, wl.STREAM_PERM).permutation(n_pages).astype(np.int32)
    bt = np.full((4, max(pages)), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[at:at + n]
        at += n
    say("int8 append")
    pool_k = wl.normal((n_pages, P, hkv, d), "bf16", seed, wl.STREAM_K)
    pool_v = wl.normal((n_pages, P, hkv, d), "bf16", seed, wl.STREAM_V)
    kc, ks = ops.kv_pages_quantize_int8(pool_k.cuda())
    vc, vs = ops.kv_pages_quantize_int8(pool_v.cuda())
    cache = ops.KVCache(kc, vc, ks, vs)
    ok, oks = oracle.quantize_int8_pages(f64(pool_k))
    ov, ovs = oracle.quantize_int8_pages(f64(pool_v))
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32)).cuda()
    starts = list(start0)
    for i, n_new in enumerate(rounds):
        cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        k_new = wl.normal((int(cu[-1]), hkv, d), "bf16", seed + 10 + i, wl.STREAM_KNEW)
        v_new = wl.normal((int(cu[-1]), hkv, d), "bf16", seed + 10 + i, wl.STREAM_VNEW)
        ops.kv_cache_append(cache, k_new.cuda(), v_new.cuda(), i32(bt), i32(starts), i32(cu), max_new=max(n_new))
        ok, oks = oracle.append_int8_pages(ok, oks, f64(k_new), bt, starts, cu, P)
        ov, ovs = oracle.append_int8_pages(ov, ovs, f64(v_new), bt, starts, cu, P)
        starts = [s + n for s, n in zip(starts, n_new)]
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), ok) and np.array_equal(vc.cpu().numpy(), ov)
    assert np.array_equal(ks.cpu().numpy(), oks) and np.array_equal(vs.cpu().numpy(), ovs)
    q = wl.normal((4, hq, d), "bf16", seed, wl.STREAM_Q)
    out = ops.attn_decode_paged(q.cuda(), cache, i32(bt), i32(final))
    torch.cuda.synchronize()
    ref, _ = oracle.decode_paged(f64(q), ok, ov, bt, final, P, k_scales=oks, v_scales=ovs)
    check_close(out, ref, "bf16", "decode after int8 appends")


def _layered_part(lens, page_size, hkv, d, seed, stream0, int8, pad=None):
    """Pools and a permuted block table holding `lens` positions per sequence
    (int8 parts quantised by the oracle on the CPU).  pad=None: every
    sequence holds at least one page and unused entries are 0; else unused
    entries are `pad` and a sequence without keys holds no page (as a page
    pool's table has them)."""
    pages = [(-(-n // page_size)) if pad is not None else max(1, -(-n // page_size)) for n in lens]
    n_pages = sum(pages) + 1
    perm = wl.rng(seed, wl.STREAM_PERM, stream0).permutation(n_pages).astype(np.int32)
    bt = np.full((len(lens), max(1, max(pages))), 0 if pad is None else pad, dtype=np.int32)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[at:at + n]
        at += n
    k = wl.normal((n_pages, page_size, hkv, d), "bf16", seed, wl.STREAM_K, stream0)
    v = wl.normal((n_pages, page_size, hkv, d), "bf16", seed, wl.STREAM_V, stream0)
    part = dict(block_table=bt, lens=np.asarray(lens, dtype=np.int32), page_size=page_size)
    if int8:
        kc, ks = oracle.quantize_int8_pages(f64(k))
        vc, vs = oracle.quantize_int8_pages(f64(v))
        part.update(k=kc, v=vc, k_scales=ks, v_scales=vs)
        cache = ops.KVCache(torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
                            torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda())
    else:
        part.update(k=f64(k), v=f64(v))
        cache = ops.KVCache(k.cuda(), v.cuda())
    return part, cache


@pytest.mark.parametrize("F,p_hi,p_lo,lo_int8,hq,hkv", [
    (128, 16, 256, True, 64, 8), (64, 64, 16, False, 8, 2), (32, 16, 64, True, 16, 1),
])
def test_layered_decode_matches_oracle(F, p_hi, p_lo, lo_int8, hq, hkv):
    """First F positions of each sequence in a bf16 cache, the rest in a
    second cache (int8 or bf16, other page size); lengths around F, a single
    key and a sequence without keys."""
    d, seed = 128, 71
    ctx = [1, F - 1, F, F + 1, 700, 2049, 0]
    say(f"layered decode F={F} P_hi={p_hi} P_lo={p_lo} int8={lo_int8} hq={hq} hkv={hkv}")
    hi, c_hi = _layered_part([min(F, n) for n in ctx], p_hi, hkv, d, seed, 0, False)
    lo, c_lo = _layered_part([max(0, n - F) for n in ctx], p_lo, hkv, d, seed, 1, lo_int8)
    q = wl.normal((len(ctx), hq, d), "bf16", seed, wl.STREAM_Q)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out, lse = ops.attn_decode_paged_layered(q.cuda(), c_hi, dev(hi["block_table"]), dev(hi["lens"]), c_lo,
                                             dev(lo["block_table"]), dev(lo["lens"]), return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_layered(f64(q), hi, lo)
    check_close(out[:-1], ref[:-1], "bf16", "layered out")
    assert torch.count_nonzero(out[-1]).item() == 0 and bool(torch.isneginf(lse[-1]).all())
    err = np.abs(f64(lse[:-1]) - ref_lse[:-1]).max()
    say(f"  lse max|d|={err:.3e}")
    assert err <= 1e-3


def test_decode_empty_context_gives_zero_output():
    """A sequence with ctx_lens = 0 has no keys: O = 0, lse = -inf, and the
    other sequences of the batch are unaffected."""
    P, hq, hkv, d, seed = 16, 8, 2, 128, 72
    ctx = [0, 37, 0, 300]
    say("decode with empty contexts")
    part, cache = _layered_part(ctx, P, hkv, d, seed, 0, False)
    q = wl.normal((len(ctx), hq, d), "bf16", seed, wl.STREAM_Q)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out, lse = ops.attn_decode_paged(q.cuda(), cache, dev(part["block_table"]), dev(part["lens"]), return_lse=True)
    torch.cuda.synchronize()
    # decode_layered with an empty second part is the plain decode (pinned),
    # and defines the no-key case.
    empty = dict(part, lens=np.zeros(len(ctx), dtype=np.int32))
    ref, ref_lse = oracle.decode_layered(f64(q), part, empty)
    check_close(out, ref, "bf16", "decode out")
    for b in (0, 2):
        assert torch.count_nonzero(out[b]).item() == 0 and bool(torch.isneginf(lse[b]).all())


@pytest.mark.parametrize("wgs", ["1", "7", "256"])
def test_decode_walk_over_empty_sequences(monkeypatch, wgs):
    """Regression: a split workgroup whose range of tiles runs over sequences
    without keys (here at the start of the batch, twice in a row and between
    long ones) moves on to the next sequence with keys; block tables padded
    with -1 as a page pool leaves them.  With 1 or 7 workgroups every range
    crosses the empty sequences."""
    P, hq, hkv, d, seed = 16, 8, 2, 128, 73
    ctx = [0, 300, 0, 0, 4000, 0, 2500, 0]
    part, cache = _layered_part(ctx, P, hkv, d, seed, 0, False, pad=-1)
    q = wl.normal((len(ctx), hq, d), "bf16", seed, wl.STREAM_Q)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    monkeypatch.setenv("PAGEDATTN_DECODE_WGS", wgs)
    say(f"decode over empty sequences, {wgs} workgroups, ctx {ctx}")
    out, lse = ops.attn_decode_paged(q.cuda(), cache, dev(part["block_table"]), dev(part["lens"]), return_lse=True)
    torch.cuda.synchronize()
    empty = dict(part, lens=np.zeros(len(ctx), dtype=np.int32))
    ref, ref_lse = oracle.decode_layered(f64(q), part, empty)
    check_close(out, ref, "bf16", "decode out")
    for b in (0, 2, 3, 5, 7):
        assert torch.count_nonzero(out[b]).item() == 0 and bool(torch.isneginf(lse[b]).all())


def test_layered_decode_int8_part_empty_among_64k_sequences():
    """Regression: the layered bench shape (first 128 positions bf16 in
    16-key pages, the rest int8 in 256-key pages, 64 query heads over 8 KV
    heads) with sequences of at most 128 tokens, whose int8 part is empty,
    among 64k-70k-token ones: thousands of int8 tiles over the default grid,
    so workgroups walk across the empty parts.  -1-padded block tables."""
    F, hq, hkv, d, seed = 128, 64, 8, 128, 74
    ctx = [65000, 100, 0, 70000, 128, 66000, 5]
    say(f"layered decode, int8 parts empty among 64k sequences, ctx {ctx}")
    hi, c_hi = _layered_part([min(F, n) for n in ctx], 16, hkv, d, seed, 0, False, pad=-1)
    lo, c_lo = _layered_part([max(0, n - F) for n in ctx], 256, hkv, d, seed, 1, True, pad=-1)
    q = wl.normal((len(ctx), hq, d), "bf16", seed, wl.STREAM_Q)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out, lse = ops.attn_decode_paged_layered(q.cuda(), c_hi, dev(hi["block_table"]), dev(hi["lens"]), c_lo,
                                             dev(lo["block_table"]), dev(lo["lens"]), return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_layered(f64(q), hi, lo)
    check_close(out[[0, 1, 3, 4, 5, 6]], ref[[0, 1, 3, 4, 5, 6]], "bf16", "layered out")
    assert torch.count_nonzero(out[2]).item() == 0 and bool(torch.isneginf(lse[2]).all())
    keep = [0, 1, 3, 4, 5, 6]
    err = np.abs(f64(lse[keep]) - ref_lse[keep]).max()
    say(f"  lse max|d|={err:.3e}")
    assert err <= 1e-3


@pytest.mark.parametrize("int8", [False, True])
def test_page_pool_prefix_sharing_with_copy_on_write(int8):
    """A 150-token prompt in sequence 0, forked whole into sequence 1 and at
    100 tokens into sequence 2; each then appends its own rows, so the pool
    hands out private copies of the shared partly filled pages
    (kv_cache_copy_pages) before the appends.  The device pools must equal
    the oracle's replay of the same steps (its model's tables, page copies
    and appends) bit for bit, and each sequence's decode must match the
    oracle over its own tokens."""
    from oracle import pages
    n_pages, P, hq, hkv, d, seed = 48, 16, 8, 2, 128, 81
    say(f"page pool with copy-on-write, int8={int8}")
    pool = ops.PagePool(n_pages, P, 3, 16)
    model = pages.PagePoolModel(n_pages, P, 3, 16)
    shape = (n_pages, P, hkv, d)
    if int8:
        kc, vc = torch.zeros(shape, dtype=torch.int8), torch.zeros(shape, dtype=torch.int8)
        ks, vs = torch.ones((n_pages, hkv)), torch.ones((n_pages, hkv))
        cache = ops.KVCache(kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda())
        ref = [kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy()]
    else:
        cache = ops.KVCache(torch.zeros(shape, dtype=torch.bfloat16).cuda(), torch.zeros(shape, dtype=torch.bfloat16).cuda())
        ref = [np.zeros(shape, dtype=np.int16), np.zeros(shape, dtype=np.int16), None, None]
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32)).cuda()

    def step(seq, rows_k, rows_v, fork=None):
        if fork is not None:
            pool.fork(*fork)
            model.fork(*fork)
            return
        start = model.lens[seq]
        new_len = start + rows_k.shape[0]
        copies = pool.extend(seq, new_len)
        want = model.extend(seq, new_len)
        assert copies == want
        table = model.block_table()
        assert np.array_equal(pool.block_table().numpy(), table)
        if copies:
            src, dst = [c[0] for c in copies], [c[1] for c in copies]
            ops.kv_cache_copy_pages(cache, i32(src), i32(dst))
            ref[0], ref[1], ref[2], ref[3] = pages.copy_pages(ref[0], ref[1], src, dst, ref[2], ref[3])
        row = table[seq:seq + 1]
        ops.kv_cache_append(cache, rows_k.cuda(), rows_v.cuda(), i32(row), i32([start]),
                            i32([0, rows_k.shape[0]]), max_new=rows_k.shape[0])
        if int8:
            ref[0], ref[2] = oracle.append_int8_pages(ref[0], ref[2], f64(rows_k), row, [start], [0, rows_k.shape[0]], P)
            ref[1], ref[3] = oracle.append_int8_pages(ref[1], ref[3], f64(rows_v), row, [start], [0, rows_k.shape[0]], P)
        else:
            ref[0], ref[1] = oracle.append_pages(ref[0], ref[1], bits(rows_k), bits(rows_v), row, [start],
                                                 [0, rows_k.shape[0]], P)

    rows = lambda n, c: (wl.normal((n, hkv, d), "bf16", seed, wl.STREAM_KNEW, c),
                         wl.normal((n, hkv, d), "bf16", seed, wl.STREAM_VNEW, c))
    step(0, *rows(150, 0))
    step(None, None, None, fork=(0, 1, 150))
    step(None, None, None, fork=(0, 2, 100))
    step(1, *rows(40, 1))
    step(2, *rows(37, 2))
    step(0, *rows(5, 3))
    torch.cuda.synchronize()
    if int8:
        assert np.array_equal(cache.k_pages.cpu().numpy(), ref[0]) and np.array_equal(cache.v_pages.cpu().numpy(), ref[1])
        assert np.array_equal(cache.k_scales.cpu().numpy(), ref[2]) and np.array_equal(cache.v_scales.cpu().numpy(), ref[3])
    else:
        assert np.array_equal(bits(cache.k_pages), ref[0]) and np.array_equal(bits(cache.v_pages), ref[1])
    lens = model.lens
    assert lens == [155, 190, 137] and pool.lens().tolist() == lens
    q = wl.normal((3, hq, d), "bf16", seed, wl.STREAM_Q)
    out = ops.attn_decode_paged(q.cuda(), cache, i32(model.block_table()), i32(lens))
    torch.cuda.synchronize()
    if int8:
        want, _ = oracle.decode_paged(f64(q), ref[0], ref[1], model.block_table(), lens, P, k_scales=ref[2], v_scales=ref[3])
    else:
        kf = torch.from_numpy(ref[0]).view(torch.bfloat16).float().numpy()
        vf = torch.from_numpy(ref[1]).view(torch.bfloat16).float().numpy()
        want, _ = oracle.decode_paged(f64(q), kf, vf, model.block_table(), lens, P)
    check_close(out, want, "bf16", "decode over shared and copied pages")


BACKWARD_CASES = [
    # name, q_lens, ctx_lens, hq, hkv, d, P, dtype, causal, window
    ("bf16_chunked_gqa", (300, 77), (300, 200), 8, 2, 128, 16, "bf16", True, -1),
    ("bf16_window64", (257,), (257,), 4, 4, 128, 64, "bf16", True, 64),
    ("bf16_unmasked_d64", (130,), (130,), 4, 1, 64, 32, "bf16", False, -1),
    ("f32_d64", (100, 33), (100, 60), 4, 2, 64, 16, "f32", True, -1),
    # groups of 3, a window over chunks after a cached prefix, a window of
    # zero (each row sees its own key only), D = 64 on 256-key pages, and an
    # unmasked chunk
    ("bf16_g3_chunked_window100", (190, 333), (400, 333), 6, 2, 128, 64, "bf16", True, 100),
    ("bf16_window0", (129,), (129,), 2, 1, 128, 64, "bf16", True, 0),
    ("bf16_d64_gqa_p256", (520,), (520,), 8, 2, 64, 256, "bf16", True, -1),
    ("bf16_unmasked_chunked", (150, 40), (300, 90), 4, 2, 128, 32, "bf16", False, -1),
]


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=lambda c: c[0])
def test_backward_matches_oracle(case):
    """Gradients of the paged attention: the GPU forward's out and lse feed
    the GPU backward; the oracle differentiates the definition in float64
    from q, K, V and dO alone.  Gradient pages start as NaN, so every cached
    position must be written and no other slot touched."""
    name, q_lens, ctx, hq, hkv, d, P, dtype, causal, window = case
    say(f"backward {name}")
    seed = 91
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    pages = [-(-c // P) for c in ctx]
    n_pages = sum(pages) + 2
    perm = wl.rng(seed, wl.STREAM_PERM).permutation(n_pages).astype(np.int32)
    bt = np.zeros((len(ctx), max(pages)), dtype=np.int32)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[at:at + n]
        at += n
    kpool = wl.normal((n_pages, P, hkv, d), dtype, seed, wl.STREAM_K)
    vpool = wl.normal((n_pages, P, hkv, d), dtype, seed, wl.STREAM_V)
    q = wl.normal((int(cu[-1]), hq, d), dtype, seed, wl.STREAM_Q)
    dout = wl.normal((int(cu[-1]), hq, d), dtype, seed, wl.STREAM_KNEW)
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32)).cuda()
    cache = ops.KVCache(kpool.cuda(), vpool.cuda())
    out, lse = ops.attn_prefill_paged(q.cuda(), i32(cu), cache, i32(bt), i32(ctx), max_q_len=max(q_lens),
                                      causal=causal, window_left=window, return_lse=True)
    dk0 = torch.full((n_pages, P, hkv, d), float("nan"), device="cuda")
    dv0 = torch.full((n_pages, P, hkv, d), float("nan"), device="cuda")
    dq, dk, dv = ops.attn_backward_paged(q.cuda(), i32(cu), cache, i32(bt), i32(ctx), out, lse, dout.cuda(),
                                         max_q_len=max(q_lens), max_ctx=max(ctx), causal=causal,
                                         window_left=window, dk=dk0, dv=dv0)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward_paged(f64(q), cu, f64(kpool), f64(vpool), bt, ctx, P, f64(dout),
                                                    causal=causal, window_left=window)
    used = np.zeros((n_pages, P), dtype=bool)
    for b, c in enumerate(ctx):
        for t in range(c):
            used[bt[b, t // P], t % P] = True
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.isfinite(gk[used]).all() and np.isfinite(gv[used]).all(), "a cached position was not written"
    assert np.isnan(gk[~used]).all() and np.isnan(gv[~used]).all(), "a slot outside the cache was written"
    # bf16: O (rounded to bf16 by the forward) enters through D = dO . O, and
    # q, K, V, dO are bf16; errors scale with the gradient's own size.
    tol_max, tol_mean = (1e-4, 1e-5) if dtype == "f32" else (2e-2, 2e-3)
    for what, got, ref in (("dq", dq.cpu().numpy(), rdq), ("dk", gk[used], rdk[used]), ("dv", gv[used], rdv[used])):
        scale = max(1.0, float(np.abs(ref).max()))
        err = np.abs(got.astype(np.float64) - ref)
        say(f"  {what}: max|ref|={np.abs(ref).max():.3e} max|d|={err.max():.3e} mean|d|={err.mean():.3e}")
        assert err.max() <= tol_max * scale and err.mean() <= tol_mean * scale, what
