"""The debug build (libpagedattn_debug.so: the same kernels with device-side
range checks of the device-resident integers) on one GPU: it gives the
release build's results on valid inputs, and reports PA_ERR_DEVICE_ASSERT
with what was out of range for a block-table entry past the pool, a context
longer than the block-table row and an append past the row, after which the
next valid call succeeds.

The bad inputs are laid out so that every access stays inside memory the
test allocated even without the checks: the pools and tables are views of
larger buffers whose extra pages and entries are valid, so the out-of-range
value still names real memory.  Only the status tells whether it was seen."""
import os

import numpy as np
import pytest
import torch

from flashattention_paged_kv_amd import build, ops
from flashattention_paged_kv_amd import workloads as wl
from gpu_cases import bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not os.path.exists(build.DEBUG_OUT), reason="debug build missing")]


@pytest.fixture
def debug_lib(monkeypatch):
    lib = ops.open_library(build.DEBUG_OUT)
    assert lib.pa_device_checks() == 1
    monkeypatch.setattr(ops, "_lib", lib)
    return lib


def _cache(n_pages, spare, P, hkv, d, seed):
    """bf16 pools of n_pages pages that are views of n_pages + spare pages."""
    k = wl.normal((n_pages + spare, P, hkv, d), "bf16", seed, wl.STREAM_K).cuda()
    v = wl.normal((n_pages + spare, P, hkv, d), "bf16", seed, wl.STREAM_V).cuda()
    return ops.KVCache(k[:n_pages], v[:n_pages])


def test_release_build_has_no_device_checks():
    assert ops.load_library().pa_device_checks() == 0


def test_debug_build_matches_release_on_valid_inputs(debug_lib, monkeypatch):
    P, hq, hkv, d, seed = 16, 8, 2, 128, 91
    ctx = torch.tensor([300, 37, 1000], dtype=torch.int32)
    pages = [-(-int(c) // P) for c in ctx]
    table, n, _ = wl.page_assignment(pages, max(pages), seed)
    cache = _cache(n, 0, P, hkv, d, seed)
    q = wl.normal((3, hq, d), "bf16", seed, wl.STREAM_Q).cuda()
    bt, c = table.cuda(), ctx.cuda()
    say("debug build: decode on valid inputs")
    out_dbg = ops.attn_decode_paged(q, cache, bt, c)
    qp = wl.normal((37, hq, d), "bf16", seed, wl.STREAM_KNEW).cuda()
    cu = torch.tensor([0, 0, 37, 37], dtype=torch.int32).cuda()
    pre_dbg = ops.attn_prefill_paged(qp, cu, cache, bt, c, max_q_len=37)
    torch.cuda.synchronize()
    monkeypatch.setattr(ops, "_lib", ops.open_library(ops.LIB_PATH))
    out_rel = ops.attn_decode_paged(q, cache, bt, c)
    pre_rel = ops.attn_prefill_paged(qp, cu, cache, bt, c, max_q_len=37)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_dbg), bits(out_rel))
    assert np.array_equal(bits(pre_dbg), bits(pre_rel))


def test_block_table_entry_past_the_pool_is_reported(debug_lib):
    P, hq, hkv, d, seed = 16, 8, 2, 128, 92
    cache = _cache(8, 4, P, hkv, d, seed)            # 8 pages declared, 12 allocated
    bt = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 8]], dtype=torch.int32).cuda()   # 8: one past the pool
    ctx = torch.tensor([64, 64], dtype=torch.int32).cuda()
    q = wl.normal((2, hq, d), "bf16", seed, wl.STREAM_Q).cuda()
    say("debug build: decode with a block-table entry past the pool")
    with pytest.raises(ops.PagedAttnError) as e:
        ops.attn_decode_paged(q, cache, bt, ctx)
    assert e.value.status == 6 and "page id 8 of sequence 1 outside [0, 7]" in e.value.detail, e.value.detail
    # the fault record was cleared: a valid call succeeds afterwards
    bt_ok = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7]], dtype=torch.int32).cuda()
    ops.attn_decode_paged(q, cache, bt_ok, ctx)
    torch.cuda.synchronize()


def test_context_longer_than_the_table_row_is_reported(debug_lib):
    P, hq, hkv, d, seed = 16, 4, 4, 64, 93
    cache = _cache(12, 0, P, hkv, d, seed)
    flat = torch.arange(12, dtype=torch.int32).cuda()
    bt = flat[:8].view(1, 8)                        # row of 8 entries (128 keys); the buffer holds 12
    ctx = torch.tensor([150], dtype=torch.int32).cuda()   # needs 10 entries
    q = wl.normal((16, hq, d), "bf16", seed, wl.STREAM_Q).cuda()   # the last 16 positions
    cu = torch.tensor([0, 16], dtype=torch.int32).cuda()
    say("debug build: prefill with a context longer than its block-table row")
    with pytest.raises(ops.PagedAttnError) as e:
        ops.attn_prefill_paged(q, cu, cache, bt, ctx, max_q_len=16)
    assert e.value.status == 6 and "context length 150 of sequence 0 outside [16, 128]" in e.value.detail, \
        e.value.detail


def test_append_past_the_table_row_is_reported(debug_lib):
    P, hkv, d, seed = 16, 2, 64, 94
    cache = _cache(6, 0, P, hkv, d, seed)
    flat = torch.arange(6, dtype=torch.int32).cuda()
    bt = flat[:4].view(1, 4)                        # 64 positions; the buffer holds 6 valid entries
    k = wl.normal((8, hkv, d), "bf16", seed, wl.STREAM_KNEW).cuda()
    start = torch.tensor([60], dtype=torch.int32).cuda()    # rows land at 60..67: past position 63
    cu = torch.tensor([0, 8], dtype=torch.int32).cuda()
    say("debug build: append past the block-table row")
    with pytest.raises(ops.PagedAttnError) as e:
        ops.kv_cache_append(cache, k, k, bt, start, cu, max_new=8)
    assert e.value.status == 6 and "append start position 60 of sequence 0 outside [0, 56]" in e.value.detail, \
        e.value.detail
