"""Pins of oracle.decode_layered (the layered cache of "大模型推理优化：KV Cache与
FlashAttention实战" section 2.2: a sequence's first tokens in one cache at full
precision, the rest in a second, int8 cache with group scales):

  * splitting one cache's positions between two caches (any page sizes and
    tables) gives the same attention as the whole cache;
  * an empty part reduces to the plain decode of the other part;
  * int8 codes are read back as code * scale of their physical page, checked
    against brute force over values rebuilt by a per-element loop;
  * a sequence with no keys gets out = 0, lse = -inf."""
import math

import numpy as np

import oracle


def _perm_pool(rng, n_pages, page_size, hkv, d, lens):
    """Random pool and a permuted block table with ceil(len / P) pages per sequence."""
    pool_k = rng.standard_normal((n_pages, page_size, hkv, d))
    pool_v = rng.standard_normal((n_pages, page_size, hkv, d))
    per = [max(1, -(-n // page_size)) for n in lens]
    perm = rng.permutation(n_pages)
    bt = np.zeros((len(lens), max(per)), dtype=np.int64)
    at = 0
    for b, n in enumerate(per):
        bt[b, :n] = perm[at:at + n]
        at += n
    assert at <= n_pages
    return pool_k, pool_v, bt


def test_layered_split_equals_whole_cache():
    rng = np.random.default_rng(7)
    hq, hkv, d, P, F, P_lo = 4, 2, 16, 16, 32, 64
    ctx = [5, 32, 40, 130]
    kw, vw, btw = _perm_pool(rng, 20, P, hkv, d, ctx)
    q = rng.standard_normal((len(ctx), hq, d))
    ref, ref_lse = oracle.decode_paged(q, kw, vw, btw, ctx, P)
    lens_lo = [max(0, n - F) for n in ctx]
    lo_k = np.full((8, P_lo, hkv, d), np.nan)
    lo_v = np.full((8, P_lo, hkv, d), np.nan)
    bt_lo = np.array([[5, 2], [7, 0], [1, 3], [6, 4]])
    for b, n in enumerate(ctx):                 # positions F.. of the whole cache, moved by hand
        for pos in range(F, n):
            i = pos - F
            src = kw[btw[b, pos // P], pos % P], vw[btw[b, pos // P], pos % P]
            lo_k[bt_lo[b, i // P_lo], i % P_lo], lo_v[bt_lo[b, i // P_lo], i % P_lo] = src
    hi = dict(k=kw, v=vw, block_table=btw, lens=[min(F, n) for n in ctx], page_size=P)
    lo = dict(k=lo_k, v=lo_v, block_table=bt_lo, lens=lens_lo, page_size=P_lo)
    out, lse = oracle.decode_layered(q, hi, lo)
    assert np.allclose(out, ref, atol=1e-12, rtol=0) and np.allclose(lse, ref_lse, atol=1e-12, rtol=0)


def _int8_part(rng, n_pages, page_size, hkv, d, lens):
    codes_k = rng.integers(-127, 128, size=(n_pages, page_size, hkv, d)).astype(np.int8)
    codes_v = rng.integers(-127, 128, size=(n_pages, page_size, hkv, d)).astype(np.int8)
    ks = rng.uniform(0.001, 0.05, size=(n_pages, hkv)).astype(np.float32)
    vs = rng.uniform(0.001, 0.05, size=(n_pages, hkv)).astype(np.float32)
    _, _, bt = _perm_pool(rng, n_pages, page_size, hkv, d, lens)
    return dict(k=codes_k, v=codes_v, k_scales=ks, v_scales=vs, block_table=bt, lens=lens, page_size=page_size)


def test_layered_with_an_empty_part_is_the_plain_decode():
    rng = np.random.default_rng(8)
    hq, hkv, d = 6, 3, 16
    lens = [9, 40, 1]
    kw, vw, bt = _perm_pool(rng, 6, 16, hkv, d, lens)
    q = rng.standard_normal((3, hq, d))
    hi = dict(k=kw, v=vw, block_table=bt, lens=lens, page_size=16)
    lo = _int8_part(rng, 4, 32, hkv, d, lens)
    none = [0, 0, 0]
    out, lse = oracle.decode_layered(q, hi, dict(lo, lens=none))
    ref, ref_lse = oracle.decode_paged(q, kw, vw, bt, lens, 16)
    assert np.allclose(out, ref, atol=1e-12, rtol=0) and np.allclose(lse, ref_lse, atol=1e-12, rtol=0)
    out, lse = oracle.decode_layered(q, dict(hi, lens=none), lo)
    ref, ref_lse = oracle.decode_paged(q, lo["k"], lo["v"], lo["block_table"], lens, 32,
                                       k_scales=lo["k_scales"], v_scales=lo["v_scales"])
    assert np.allclose(out, ref, atol=1e-12, rtol=0) and np.allclose(lse, ref_lse, atol=1e-12, rtol=0)


def test_layered_int8_part_matches_brute_force():
    rng = np.random.default_rng(9)
    hq, hkv, d = 2, 1, 8
    hi_lens, lo_lens = [3, 0, 4], [5, 7, 0]
    kw, vw, bt = _perm_pool(rng, 4, 4, hkv, d, hi_lens)
    hi = dict(k=kw, v=vw, block_table=bt, lens=hi_lens, page_size=4)
    lo = _int8_part(rng, 6, 4, hkv, d, lo_lens)
    q = rng.standard_normal((3, hq, d))
    out, lse = oracle.decode_layered(q, hi, lo)
    for b in range(3):
        keys, vals = [], []
        for pos in range(hi_lens[b]):
            keys.append([float(x) for x in kw[bt[b, pos // 4], pos % 4, 0]])
            vals.append([float(x) for x in vw[bt[b, pos // 4], pos % 4, 0]])
        for pos in range(lo_lens[b]):
            page, slot = lo["block_table"][b, pos // 4], pos % 4
            keys.append([float(c) * float(lo["k_scales"][page, 0]) for c in lo["k"][page, slot, 0]])
            vals.append([float(c) * float(lo["v_scales"][page, 0]) for c in lo["v"][page, slot, 0]])
        for h in range(hq):
            o, l = oracle.brute_force_attention([q[b, h]], keys, vals, 1 / math.sqrt(d), lambda i, j: True)
            assert np.allclose(out[b, h], o[0], atol=1e-12, rtol=0)
            assert math.isclose(lse[b, h], l[0], abs_tol=1e-12)


def test_layered_sequence_without_keys():
    rng = np.random.default_rng(10)
    kw, vw, bt = _perm_pool(rng, 2, 16, 1, 8, [4, 0])
    hi = dict(k=kw, v=vw, block_table=bt, lens=[4, 0], page_size=16)
    lo = dict(k=kw, v=vw, block_table=bt, lens=[0, 0], page_size=16)
    out, lse = oracle.decode_layered(rng.standard_normal((2, 2, 8)), hi, lo)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1])) and np.all(np.isfinite(lse[0]))
