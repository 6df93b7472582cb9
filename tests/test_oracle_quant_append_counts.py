"""Pins of the oracle's int8 group quantiser, cache append and work counters."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_values(shape, seed):
    """float32 values that are exactly bf16 (low 16 bits cleared, rounded)."""
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32)


def test_int8_quantiser_bounds_and_roundtrip():
    x = _bf16_values((5, 16, 3, 8), 1)
    codes, scales = oracle.quantize_int8_pages(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float32 and scales.shape == (5, 3)
    assert codes.min() >= -127 and codes.max() <= 127          # -128 never produced
    xh = oracle.dequantize_int8_pages(codes, scales)
    err = np.abs(xh - x.astype(np.float64))
    assert (err <= scales.astype(np.float64)[:, None, :, None] / 2 * (1 + 1e-6)).all()
    # the largest magnitude of each group lands on +-127
    for n in range(5):
        for h in range(3):
            g = x[n, :, h, :]
            idx = np.unravel_index(np.abs(g).argmax(), g.shape)
            assert abs(int(codes[n, idx[0], h, idx[1]])) == 127
    # requantising the dequantised values with the same scales returns the codes
    y = (xh.astype(np.float32) / scales[:, None, :, None]).astype(np.float32)
    assert np.array_equal(np.rint(np.clip(y, -128, 127)).astype(np.int8), codes)


def test_int8_quantiser_matches_per_element_fp32_loop():
    """Element by element, in float32 scalar arithmetic: scale = absmax / 127,
    code = round-half-even(clamp(x / scale))."""
    x = _bf16_values((2, 4, 2, 4), 2)
    x[1, :, 1, :] = 0.0                     # an all-zero group: scale 1, codes 0
    codes, scales = oracle.quantize_int8_pages(x)
    for n in range(2):
        for h in range(2):
            am = np.float32(0.0)
            for s in range(4):
                for d in range(4):
                    am = max(am, np.float32(abs(x[n, s, h, d])))
            sc = np.float32(am / np.float32(127.0)) if am != 0 else np.float32(1.0)
            assert scales[n, h] == sc
            for s in range(4):
                for d in range(4):
                    y = np.float32(x[n, s, h, d] / sc)
                    y = min(max(y, np.float32(-128)), np.float32(127))
                    c = int(round(float(y)))        # Python round = half-to-even
                    assert codes[n, s, h, d] == c


def test_int8_dequantiser_matches_per_element_loop():
    """code * scale of the code's own (page, KV head) group, element by
    element, on a pool whose four axes all differ in length (a broadcast
    over the wrong axis cannot line up) and whose scales all differ."""
    r = np.random.default_rng(11)
    N, P, H, D = 3, 5, 2, 7
    codes = r.integers(-127, 128, size=(N, P, H, D)).astype(np.int8)
    scales = (r.random((N, H)) + 0.5).astype(np.float32)
    got = oracle.dequantize_int8_pages(codes, scales)
    assert got.shape == (N, P, H, D) and got.dtype == np.float64
    for n in range(N):
        for p in range(P):
            for h in range(H):
                for d in range(D):
                    assert got[n, p, h, d] == float(int(codes[n, p, h, d])) * float(scales[n, h])


def test_int8_half_way_rounds_to_even():
    # absmax 127 -> scale 1 exactly; 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    x = np.zeros((1, 1, 1, 4), dtype=np.float32)
    x[0, 0, 0, :] = [127.0, 2.5, 3.5, -2.5]
    codes, scales = oracle.quantize_int8_pages(x)
    assert scales[0, 0] == 1.0
    assert codes[0, 0, 0].tolist() == [127, 2, 4, -2]


def test_append_scatter_matches_loop_and_leaves_other_slots():
    r = np.random.default_rng(3)
    P, hkv, d = 4, 2, 3
    k_pool = r.integers(-1000, 1000, (6, P, hkv, d)).astype(np.int16)   # raw 16-bit words
    v_pool = r.integers(-1000, 1000, (6, P, hkv, d)).astype(np.int16)
    table = np.array([[4, 1, 3], [0, 5, -1]])
    start = [2, 3]
    n_new = [7, 2]
    cu = [0, 7, 9]
    k_new = r.integers(-1000, 1000, (9, hkv, d)).astype(np.int16)
    v_new = r.integers(-1000, 1000, (9, hkv, d)).astype(np.int16)
    k2, v2 = oracle.append_pages(k_pool, v_pool, k_new, v_new, table, start, cu, P)
    expect_k = k_pool.copy()
    expect_v = v_pool.copy()
    written = set()
    for b in range(2):
        for rr in range(n_new[b]):
            pos = start[b] + rr
            page, slot = table[b][pos // P], pos % P
            expect_k[page, slot] = k_new[cu[b] + rr]
            expect_v[page, slot] = v_new[cu[b] + rr]
            written.add((page, slot))
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    assert k2.dtype == np.int16
    for page in range(6):
        for slot in range(P):
            if (page, slot) not in written:
                assert np.array_equal(k2[page, slot], k_pool[page, slot])
    # sequence 0 positions 2..8: pages 4 (slots 2,3), 1 (0..3), 3 (slot 0)
    assert (4, 2) in written and (3, 0) in written and (3, 1) not in written


def test_counts_match_the_pages_examples():
    g = json.load(open(os.path.join(GOLDEN, "page_counts.json")))
    n = g["pair_count"]["tokens"]
    with_self = oracle.visible_pairs(n, n, causal=True)
    assert with_self - n == g["pair_count"]["pairs_excluding_self"]
    assert with_self == n * (n + 1) // 2
    kb = g["kv_bytes_per_token"]
    assert oracle.kv_bytes_per_token(kb["num_layers"], kb["d_k"], kb["d_v"],
                                     kb["bytes_per_value"]) == kb["bytes_per_token"]
    gq = g["gqa_kv_saving"]
    assert 1 - gq["num_groups"] / gq["num_q_heads"] == gq["kv_fraction_saved"]


def test_counts_match_mask_and_workload_figures():
    for q_len, ctx, causal, w in [(7, 7, True, -1), (3, 10, True, 2), (5, 5, False, -1), (9, 9, True, 0)]:
        assert oracle.visible_pairs(q_len, ctx, causal, w) == int(oracle.visible_mask(q_len, ctx, causal, w).sum())
    # Llama-2-7B-shaped causal prefill, L = 2048, 32 heads, D = 128
    assert oracle.attention_flops(oracle.visible_pairs(2048, 2048), 128, 32) == 34_376_515_584
    # 32k prefill with a 128-token left window: sum_i min(i + 1, 129)
    assert oracle.visible_pairs(32768, 32768, True, 128) == 4_218_816
    assert oracle.kv_read_bytes([10, 300], 8, 128, 2) == 2 * 310 * 8 * 128 * 2
    assert oracle.kv_read_bytes([10, 300], 8, 128, 1, 4, 256) == 2 * 310 * 8 * 128 + 2 * 3 * 8 * 4


def test_bench_pair_counter_is_the_oracle_count():
    """The benchmark's closed-form pair count (which prices its FLOPs) equals
    the oracle's row-by-row count for the prefill workloads it times."""
    import bench
    for n, w in [(2048, -1), (32768, -1), (32768, 128), (128, -1), (1, -1), (1, 128), (129, 128), (130, 128),
                 (1000, 0), (64, 127)]:
        assert bench.causal_pairs(n, w) == oracle.visible_pairs(n, n, True, w), (n, w)


def _rows_bf16(n, hkv, d, seed, mag=1.0):
    return _bf16_values((n, hkv, d), seed) * np.float32(mag)


def test_int8_append_of_a_whole_page_is_the_page_quantiser():
    """P rows appended at a page boundary into a page holding garbage codes:
    the page's codes and scales are those of the whole-page quantiser."""
    P, hkv, d = 16, 2, 8
    r = np.random.default_rng(5)
    codes = r.integers(-128, 128, (3, P, hkv, d)).astype(np.int8)
    scales = r.random((3, hkv)).astype(np.float32) + np.float32(0.5)
    rows = _rows_bf16(P, hkv, d, 6, mag=3.0)
    table = np.array([[2, 0]])
    c2, s2 = oracle.append_int8_pages(codes, scales, rows, table, [0], [0, P], P)
    qc, qs = oracle.quantize_int8_pages(rows[None])
    assert np.array_equal(c2[2], qc[0]) and np.array_equal(s2[2], qs[0])
    assert np.array_equal(c2[:2], codes[:2]) and np.array_equal(s2[:2], scales[:2])   # other pages untouched


def test_int8_append_with_smaller_rows_keeps_scale_and_old_codes():
    P, hkv, d = 16, 2, 8
    codes = np.zeros((1, P, hkv, d), np.int8)
    scales = np.ones((1, hkv), np.float32)
    first = _rows_bf16(5, hkv, d, 7, mag=4.0)
    c1, s1 = oracle.append_int8_pages(codes, scales, first, np.array([[0]]), [0], [0, 5], P)
    small = _rows_bf16(6, hkv, d, 8, mag=0.01)
    c2, s2 = oracle.append_int8_pages(c1, s1, small, np.array([[0]]), [5], [0, 6], P)
    assert np.array_equal(s2, s1)
    assert np.array_equal(c2[0, :5], c1[0, :5])
    assert np.array_equal(c2[0, 11:], codes[0, 11:])      # slots past the end untouched


def test_int8_append_error_bound_on_old_and_new_rows():
    """After one append: new rows within half a step of the new scale, old
    rows (requantised from their codes) within one step."""
    P, hkv, d = 32, 3, 16
    codes = np.zeros((2, P, hkv, d), np.int8)
    scales = np.ones((2, hkv), np.float32)
    x_old = _rows_bf16(40, hkv, d, 9, mag=1.0)
    c1, s1 = oracle.append_int8_pages(codes, scales, x_old, np.array([[1, 0]]), [0], [0, 40], P)
    x_new = _rows_bf16(17, hkv, d, 10, mag=2.5)          # larger: the second page's scale grows
    c2, s2 = oracle.append_int8_pages(c1, s1, x_new, np.array([[1, 0]]), [40], [0, 17], P)
    allx = np.concatenate([x_old, x_new]).astype(np.float64)
    deq = oracle.dequantize_int8_pages(c2, s2)
    for pos in range(57):
        phys, slot = [1, 0][pos // P], pos % P
        err = np.abs(deq[phys, slot] - allx[pos])
        step = s2[phys].astype(np.float64)
        bound = (0.5 if pos >= 40 else 1.0) * step * (1 + 1e-5)
        assert (err <= bound[:, None]).all(), (pos, err.max(), step)
    # the scale of a group is its largest valid magnitude over 127
    assert abs(float(s2[0, 0]) * 127 - np.abs(np.concatenate([c1[0, :8, 0] * s1[0, 0], x_new[:, 0]])).max()) \
        <= 1e-5 * float(s2[0, 0]) * 127


def test_int8_append_matches_scalar_loop():
    """Element by element in float32 scalars, on a tiny ragged case with two
    sequences, a page crossing and a partly filled first page."""
    P, hkv, d = 4, 2, 3
    r = np.random.default_rng(11)
    codes = r.integers(-127, 128, (5, P, hkv, d)).astype(np.int8)
    scales = (r.random((5, hkv)) + 0.1).astype(np.float32)
    table = np.array([[3, 1, 4], [0, 2, -1]])
    start, cu = [2, 1], [0, 5, 7]
    rows = _rows_bf16(7, hkv, d, 12, mag=2.0)
    c2, s2 = oracle.append_int8_pages(codes, scales, rows, table, start, cu, P)
    ec, es = codes.copy(), scales.copy()
    for b in range(2):
        n = cu[b + 1] - cu[b]
        pages = sorted({(start[b] + i) // P for i in range(n)})
        for lp in pages:
            phys = table[b, lp]
            for h in range(hkv):
                vals = {}
                for slot in range(P):
                    pos = lp * P + slot
                    if pos < start[b]:
                        vals[slot] = [np.float32(np.float32(ec[phys, slot, h, k]) * es[phys, h]) for k in range(d)]
                    elif pos < start[b] + n:
                        vals[slot] = [np.float32(rows[cu[b] + pos - start[b], h, k]) for k in range(d)]
                am = np.float32(0)
                for v in vals.values():
                    for e in v:
                        am = max(am, np.float32(abs(e)))
                sc = np.float32(am / np.float32(127)) if am != 0 else np.float32(1)
                for slot, v in vals.items():
                    for k, e in enumerate(v):
                        y = min(max(np.float32(e / sc), np.float32(-128)), np.float32(127))
                        ec[phys, slot, h, k] = int(round(float(y)))
                es[phys, h] = sc
    assert np.array_equal(c2, ec) and np.array_equal(s2, es)
