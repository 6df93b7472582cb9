"""Pins of the CPU oracle against things other than itself: a hand-derived
closed form, torch's CPU scaled_dot_product_attention (float64), pure-Python
brute force, and invariants the pages fix (cached decode = recompute, page
shuffles, GQA as repeated heads, online softmax = two-pass softmax)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_case import Case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(case, b):
    ks, vs = case.dense(b)
    q0 = int(case.cu_q[b])
    g = case.hq // case.hkv
    outs = np.zeros((case.q_lens[b], case.hq, case.d))
    lses = np.zeros((case.q_lens[b], case.hq))
    for h in range(case.hq):
        kh = [row[h // g] for row in ks]
        vh = [row[h // g] for row in vs]
        qrows = [case.q[q0 + i, h].tolist() for i in range(case.q_lens[b])]
        o, l = oracle.brute_force_attention(qrows, kh, vh, case.scale, case.visible(b))
        outs[:, h, :] = np.array(o)
        lses[:, h] = np.array(l)
    return outs, lses


def test_closed_form_example():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_example.json")))
    q = np.array(g["q"]).reshape(1, 1, 1)
    k_pool = np.array(g["keys"]).reshape(1, 2, 1, 1)
    v_pool = np.array(g["values"]).reshape(1, 2, 1, 1)
    out, lse = oracle.attention_paged(q, [0, 1], k_pool, v_pool, [[0]], [2], 2,
                                      softmax_scale=g["softmax_scale"], causal=False)
    assert abs(out[0, 0, 0] - g["expected_out"]) < 1e-15
    assert abs(lse[0, 0] - g["expected_lse"]) < 1e-15
    # the same with the query placed as the last token of a causal prefix
    out2, _ = oracle.attention_paged(q, [0, 1], k_pool, v_pool, [[0]], [2], 2,
                                     softmax_scale=1.0, causal=True)
    assert abs(out2[0, 0, 0] - 0.75) < 1e-15


CASES = [
    dict(seed=1, hq=4, hkv=2, d=8, page_size=4, seqs=[(7, 7), (13, 13)]),
    dict(seed=2, hq=6, hkv=1, d=5, page_size=2, seqs=[(9, 9)], window_left=3),
    dict(seed=3, hq=3, hkv=3, d=4, page_size=8, seqs=[(5, 21), (1, 11), (4, 4)]),      # chunked + decode rows
    dict(seed=4, hq=8, hkv=2, d=16, page_size=4, seqs=[(11, 11)], causal=False),
    dict(seed=5, hq=2, hkv=1, d=3, page_size=4, seqs=[(6, 17)], window_left=0),
    dict(seed=6, hq=4, hkv=4, d=6, page_size=16, seqs=[(1, 1), (20, 20)], window_left=5, scale=0.3),
]


@pytest.mark.parametrize("kw", CASES)
def test_oracle_matches_brute_force(kw):
    case = Case(**kw)
    out, lse = oracle.attention_paged(*case.oracle_args(), softmax_scale=case.scale,
                                      causal=case.causal, window_left=case.window_left)
    for b in range(len(case.q_lens)):
        bo, bl = _brute(case, b)
        q0, q1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        np.testing.assert_allclose(out[q0:q1], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[q0:q1], bl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,causal,window", [(4, 4, True, -1), (8, 2, True, -1), (6, 3, False, -1),
                                                  (4, 2, True, 4)])
def test_oracle_matches_torch_sdpa(hq, hkv, causal, window):
    """Identity paging, one sequence: torch's CPU SDPA in float64 (GQA via
    enable_gqa, which shares KV head h // G)."""
    r = np.random.default_rng(7)
    L, d, P = 37, 16, 8
    q = r.standard_normal((L, hq, d))
    k = r.standard_normal((L, hkv, d))
    v = r.standard_normal((L, hkv, d))
    n = -(-L // P)
    k_pool = np.zeros((n, P, hkv, d))
    v_pool = np.zeros((n, P, hkv, d))
    k_pool.reshape(n * P, hkv, d)[:L] = k
    v_pool.reshape(n * P, hkv, d)[:L] = v
    out, _ = oracle.attention_paged(q, [0, L], k_pool, v_pool, [list(range(n))], [L], P,
                                    causal=causal, window_left=window)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    if window >= 0:
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        mask = (j <= i) & (i - j <= window)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_causal_row0_and_zero_query():
    case = Case(seed=11, hq=2, hkv=2, d=4, page_size=4, seqs=[(10, 10)])
    out, _ = oracle.attention_paged(*case.oracle_args())
    ks, vs = case.dense(0)
    vs = np.array(vs)
    assert np.array_equal(out[0], vs[0])          # row 0 sees only key 0: weight exactly 1
    case.q[:] = 0.0                                # all scores 0: uniform weights
    out, _ = oracle.attention_paged(*case.oracle_args())
    for i in range(10):
        np.testing.assert_allclose(out[i], vs[:i + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_window_special_cases():
    case = Case(seed=12, hq=2, hkv=1, d=4, page_size=4, seqs=[(12, 12)])
    ks, vs = case.dense(0)
    vs = np.array(vs)
    out0, _ = oracle.attention_paged(*case.oracle_args(), window_left=0)
    for i in range(12):
        assert np.array_equal(out0[i, 0], vs[i, 0]) and np.array_equal(out0[i, 1], vs[i, 0])
    full, _ = oracle.attention_paged(*case.oracle_args(), window_left=-1)
    wide, _ = oracle.attention_paged(*case.oracle_args(), window_left=11)
    assert np.array_equal(full, wide)
    vis = oracle.visible_mask(12, 12, True, 3)
    assert list(vis.sum(axis=1)) == [min(i + 1, 4) for i in range(12)]


def test_constant_v_and_normalisation():
    case = Case(seed=13, hq=4, hkv=2, d=8, page_size=4, seqs=[(9, 9), (3, 14)])
    row = np.arange(8.0) - 3.5
    case.v_pool[:] = row
    out, lse = oracle.attention_paged(*case.oracle_args())
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-14)
    # sum_j exp(s_ij - lse_i) = 1, with s_ij from brute-force dot products
    for b in range(2):
        ks, _ = case.dense(b)
        q0 = int(case.cu_q[b])
        for i in range(case.q_lens[b]):
            for h in range(case.hq):
                tot = math.fsum(
                    math.exp(case.scale * math.fsum(a * c for a, c in zip(case.q[q0 + i, h], ks[j][h // 2]))
                             - lse[q0 + i, h])
                    for j in range(int(case.ctx_lens[b])) if case.visible(b)(i, j))
                assert abs(tot - 1.0) < 1e-12


def test_gqa_equals_repeated_mha():
    case = Case(seed=14, hq=8, hkv=2, d=8, page_size=4, seqs=[(10, 10), (2, 7)])
    out, lse = oracle.attention_paged(*case.oracle_args())
    kr = np.repeat(case.k_pool, 4, axis=2)   # repeat_interleave on the head dim
    vr = np.repeat(case.v_pool, 4, axis=2)
    out2, lse2 = oracle.attention_paged(case.q, case.cu_q, kr, vr, case.block_table, case.ctx_lens,
                                        case.page_size)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_page_permutation_is_bitwise_invariant():
    case = Case(seed=15, hq=4, hkv=2, d=8, page_size=4, seqs=[(13, 13), (5, 9)])
    out, lse = oracle.attention_paged(*case.oracle_args(), window_left=6)
    perm = np.random.default_rng(0).permutation(case.num_pages)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    k2 = case.k_pool[perm]          # new physical page n holds old page perm[n]
    v2 = case.v_pool[perm]
    bt2 = np.where(case.block_table >= 0, inv[np.maximum(case.block_table, 0)], -1)
    out2, lse2 = oracle.attention_paged(case.q, case.cu_q, k2, v2, bt2, case.ctx_lens, case.page_size,
                                        window_left=6)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_page_size_invariance():
    r = np.random.default_rng(16)
    L, hq, hkv, d = 19, 4, 2, 8
    q = r.standard_normal((L, hq, d))
    k = r.standard_normal((L, hkv, d))
    v = r.standard_normal((L, hkv, d))
    outs = []
    for P in (1, 4, 32):
        n = -(-L // P)
        kp = np.full((n, P, hkv, d), np.nan)
        vp = np.full((n, P, hkv, d), np.nan)    # slots past the end stay NaN: never read
        kp.reshape(n * P, hkv, d)[:L] = k
        vp.reshape(n * P, hkv, d)[:L] = v
        outs.append(oracle.attention_paged(q, [0, L], kp, vp, [list(range(n))], [L], P)[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert np.isfinite(outs[0]).all()


def test_decode_equals_prefill_row():
    """A cached decode at position t equals row t of causal prefill over t+1 tokens."""
    case = Case(seed=17, hq=4, hkv=2, d=8, page_size=4, seqs=[(15, 15)])
    full, full_lse = oracle.attention_paged(*case.oracle_args())
    for t in (0, 3, 4, 14):
        dec, dec_lse = oracle.decode_paged(case.q[t:t + 1], case.k_pool, case.v_pool, case.block_table,
                                           [t + 1], case.page_size)
        np.testing.assert_allclose(dec[0], full[t], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dec_lse[0], full_lse[t], rtol=0, atol=1e-13)


@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_online_softmax_equals_two_pass(block):
    case = Case(seed=18, hq=1, hkv=1, d=8, page_size=4, seqs=[(40, 40)], window_left=9)
    out, lse = oracle.attention_paged(*case.oracle_args(), window_left=9)
    ks, vs = case.dense(0)
    k = np.array(ks)[:, 0]
    v = np.array(vs)[:, 0]
    vis = oracle.visible_mask(40, 40, True, 9)
    o2, l2 = oracle.online_softmax_attention(case.q[:, 0], k, v, case.scale, vis, block)
    np.testing.assert_allclose(o2, out[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse[:, 0], rtol=0, atol=1e-12)


def test_split_merge_equals_unsplit():
    case = Case(seed=19, hq=1, hkv=1, d=8, page_size=4, seqs=[(1, 50)])
    out, lse = oracle.decode_paged(case.q, case.k_pool, case.v_pool, case.block_table, case.ctx_lens, 4)
    ks, vs = case.dense(0)
    vis = np.ones((1, 50), dtype=bool)
    for bounds in ([0, 50], [0, 16, 32, 48, 50], [0, 1, 2, 49, 50], [0, 25, 25, 50]):
        parts = oracle.split_partials(case.q[:, 0], np.array(ks)[:, 0], np.array(vs)[:, 0], case.scale,
                                      vis, bounds)
        o, l = oracle.merge_partials(parts)
        np.testing.assert_allclose(o, out[:, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lse[:, 0], rtol=0, atol=1e-12)


def test_empty_key_ranges_are_neutral():
    """A split that sees no key (m = -inf, l = 0) must not change the merge,
    and a row with no visible key gives out = 0, lse = -inf."""
    r = np.random.default_rng(20)
    q = r.standard_normal((3, 4))
    k = r.standard_normal((10, 4))
    v = r.standard_normal((10, 4))
    vis = np.ones((3, 10), dtype=bool)
    vis[1, :] = False
    vis[2, :5] = False
    o, l = oracle.online_softmax_attention(q, k, v, 0.5, vis, 4)
    assert np.array_equal(o[1], np.zeros(4)) and l[1] == -np.inf
    parts = oracle.split_partials(q, k, v, 0.5, vis, [0, 5, 10])
    o2, l2 = oracle.merge_partials(parts)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    assert l2[1] == -np.inf and np.isfinite(l2[[0, 2]]).all()
