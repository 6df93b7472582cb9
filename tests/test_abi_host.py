"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments with the documented status codes before enqueuing any
work (so these run without a GPU: no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

from flashattention_paged_kv_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="library not built")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its checks first


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:pa_status|size_t|const char \*|int32_t|void)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declarations_are_exported():
    names = _declared_functions()
    assert set(names) == set(ops.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
    lib = ops.load_library()
    for n in names:
        assert hasattr(lib, n)
    assert lib.pa_abi_version() == 1


def test_status_strings():
    lib = ops.load_library()
    assert lib.pa_status_string(0) == b"ok"
    for s in range(1, 6):
        assert lib.pa_status_string(s) not in (b"ok", b"unknown status")
    assert lib.pa_status_string(99) == b"unknown status"


def _cache(**kw):
    c = dict(k_pages=0x1000, v_pages=0x2000, k_scales=None, v_scales=None, num_pages=4, page_size=16,
             num_kv_heads=2, head_dim=128, dtype=ops.PA_BF16)
    c.update(kw)
    return ops._Cache(**c)


def _prefill(cache, **kw):
    lib = ops.load_library()
    a = dict(q=FAKE, cu_q=FAKE, block_table=FAKE, max_pages=4, ctx=FAKE, batch=1, max_q_len=8, hq=4,
             scale=0.1, causal=1, window=-1, out=FAKE, lse=None)
    a.update(kw)
    return lib.attn_prefill_paged(a["q"], a["cu_q"], ctypes.byref(cache), a["block_table"], a["max_pages"],
                                  a["ctx"], a["batch"], a["max_q_len"], a["hq"], a["scale"], a["causal"],
                                  a["window"], a["out"], a["lse"], None)


def _decode(cache, **kw):
    lib = ops.load_library()
    a = dict(q=FAKE, block_table=FAKE, max_pages=4, ctx=FAKE, batch=2, hq=4, scale=0.1, window=-1, out=FAKE,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.attn_decode_paged(a["q"], ctypes.byref(cache), a["block_table"], a["max_pages"], a["ctx"],
                                 a["batch"], a["hq"], a["scale"], a["window"], a["out"], None, a["ws"],
                                 a["ws_bytes"], None)


def _detail():
    return ops.load_library().pa_last_error_detail().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2), (dict(page_size=24), 2), (dict(page_size=512), 2), (dict(page_size=8), 2),
    (dict(dtype=7), 2), (dict(dtype=ops.PA_I8), 2), (dict(k_pages=None), 1), (dict(num_pages=0), 1),
    (dict(num_kv_heads=0), 1),
])
def test_prefill_rejects_bad_cache(kw, status):
    assert _prefill(_cache(**kw)) == status
    assert _detail() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3), 1), (dict(hq=0), 1), (dict(scale=0.0), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(scale=-1.0), 1), (dict(causal=2), 1), (dict(q=None), 1),
    (dict(cu_q=None), 1), (dict(out=None), 1), (dict(block_table=None), 1), (dict(max_pages=0), 1),
    (dict(batch=-1), 1),
])
def test_prefill_rejects_bad_args(kw, status):
    assert _prefill(_cache(), **kw) == status


def test_prefill_empty_batch_is_ok_without_work():
    assert _prefill(_cache(), batch=0, q=None, out=None) == 0
    assert _prefill(_cache(), max_q_len=0) == 0


def _prefill_append(cache, **kw):
    lib = ops.load_library()
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, cu_q=FAKE, block_table=FAKE, max_pages=4, ctx=FAKE, batch=1,
             max_q_len=8, hq=4, scale=0.1, causal=1, window=-1, out=FAKE, lse=None)
    a.update(kw)
    return lib.attn_prefill_paged_append(a["q"], a["k_new"], a["v_new"], a["cu_q"], ctypes.byref(cache),
                                         a["block_table"], a["max_pages"], a["ctx"], a["batch"], a["max_q_len"],
                                         a["hq"], a["scale"], a["causal"], a["window"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), 1), (dict(v_new=None), 1), (dict(hq=3), 1), (dict(scale=0.0), 1), (dict(causal=2), 1),
    (dict(q=None), 1), (dict(out=None), 1), (dict(max_pages=0), 1), (dict(batch=-1), 1),
])
def test_prefill_append_rejects_bad_args(kw, status):
    assert _prefill_append(_cache(), **kw) == status
    assert _detail() != ""


def test_prefill_append_rejects_bad_cache_and_allows_empty():
    assert _prefill_append(_cache(dtype=ops.PA_I8)) == 2
    assert _prefill_append(_cache(head_dim=96)) == 2
    assert _prefill_append(_cache(), batch=0, q=None, out=None, k_new=None, v_new=None) == 0
    assert _prefill_append(_cache(), max_q_len=0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3), 1), (dict(scale=0.0), 1), (dict(q=None), 1), (dict(ws=None), 4), (dict(ws_bytes=16), 4),
    (dict(hq=2 * 17), 2),
])
def test_decode_rejects_bad_args(kw, status):
    assert _decode(_cache(), **kw) == status


def test_decode_int8_needs_scales():
    assert _decode(_cache(dtype=ops.PA_I8)) == 1
    assert "scales" in _detail()


def test_workspace_size_query():
    lib = ops.load_library()
    n = lib.attn_decode_workspace_bytes(64, 64, 8, 128, 32, 256)
    assert n >= 64 * 64 * (128 + 2) * 4          # at least one split per (sequence, head)
    assert n % 4 == 0
    assert lib.attn_decode_workspace_bytes(0, 64, 8, 128, 32, 256) == 0
    assert lib.attn_decode_workspace_bytes(4, 64, 8, 128, 32, 100) == 0
    # a workspace one byte short of the query is rejected
    assert _decode(_cache(num_kv_heads=2, page_size=16), batch=2, hq=4, max_pages=4,
                   ws_bytes=lib.attn_decode_workspace_bytes(2, 4, 2, 128, 4, 16) - 1) == 4


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    """attn_decode_paged_noalloc checks the scratch its sizes need against
    the library's fixed array before anything else happens (no device
    call), and runs attn_decode_paged's own checks otherwise."""
    lib = ops.load_library()
    cap = ops.NOALLOC_SCRATCH_BYTES
    # 1024 sequences x 64 query heads over 8 KV heads need ~ 34 MB > 32 MiB
    need = lib.attn_decode_workspace_bytes(1024, 64, 8, 128, 32, 256)
    assert need > cap
    c = _cache(num_kv_heads=8, page_size=256)
    st = lib.attn_decode_paged_noalloc(FAKE, ctypes.byref(c), FAKE, 32, FAKE, 1024, 64, 0.1, -1, FAKE, None, None)
    assert st == 4 and b"scratch" in lib.pa_last_error_detail()
    # ordinary argument errors are attn_decode_paged's
    assert lib.attn_decode_paged_noalloc(FAKE, ctypes.byref(c), FAKE, 32, FAKE, 4, 60, 0.1, -1, FAKE, None,
                                         None) == 1
    assert lib.attn_decode_paged_noalloc(FAKE, ctypes.byref(c), FAKE, 32, FAKE, 4, 64, 0.0, -1, FAKE, None,
                                         None) == 1
    assert lib.attn_decode_paged_noalloc(FAKE, ctypes.byref(_cache(head_dim=96)), FAKE, 32, FAKE, 4, 64, 0.1, -1,
                                         FAKE, None, None) == 2
    assert lib.attn_decode_paged_noalloc(FAKE, ctypes.byref(c), FAKE, 32, FAKE, 0, 64, 0.1, -1, None, None,
                                         None) == 0


def test_append_rejects_bad_args():
    lib = ops.load_library()
    c = _cache(dtype=ops.PA_I8)                       # int8 cache without scales
    assert lib.kv_cache_append(ctypes.byref(c), FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 1, None) == 1
    c = _cache()
    assert lib.kv_cache_append(ctypes.byref(c), None, FAKE, FAKE, 4, FAKE, FAKE, 1, 1, None) == 1
    assert lib.kv_cache_append(ctypes.byref(c), FAKE, FAKE, FAKE, 4, FAKE, FAKE, -1, 1, None) == 1
    assert lib.kv_cache_append(ctypes.byref(c), None, None, None, 4, None, None, 0, 0, None) == 0
    assert lib.kv_cache_append(None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 1, None) == 1


def test_quantize_rejects_bad_args():
    lib = ops.load_library()
    assert lib.kv_pages_quantize_int8(None, FAKE, FAKE, 1, 16, 1, 128, None) == 1
    assert lib.kv_pages_quantize_int8(FAKE, FAKE, FAKE, 1, 16, 1, 80, None) == 2
    assert lib.kv_pages_quantize_int8(FAKE, FAKE, FAKE, 1, 48, 1, 128, None) == 2
    assert lib.kv_pages_quantize_int8(FAKE, FAKE, FAKE, 0, 16, 1, 128, None) == 0


def _layered(hi, lo, **kw):
    lib = ops.load_library()
    a = dict(q=FAKE, bt_hi=FAKE, mp_hi=4, len_hi=FAKE, bt_lo=FAKE, mp_lo=4, len_lo=FAKE, batch=2, hq=4, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.attn_decode_paged_layered(a["q"], ctypes.byref(hi), a["bt_hi"], a["mp_hi"], a["len_hi"],
                                         ctypes.byref(lo), a["bt_lo"], a["mp_lo"], a["len_lo"], a["batch"],
                                         a["hq"], a["scale"], a["out"], None, a["ws"], a["ws_bytes"], None)


def _i8_cache(**kw):
    c = dict(dtype=ops.PA_I8, k_scales=0x3000, v_scales=0x4000, page_size=256)
    c.update(kw)
    return _cache(**c)


@pytest.mark.parametrize("hi_kw,lo_kw,kw,status", [
    (dict(), dict(), dict(hq=3), 1),                         # heads not a multiple of Hkv
    (dict(), dict(num_kv_heads=4), dict(), 1),               # caches disagree on heads
    (dict(), dict(head_dim=64), dict(), 1),                  # caches disagree on head_dim
    (dict(dtype=ops.PA_F32), dict(), dict(), 2),             # fp32 is not a layered dtype
    (dict(), dict(k_scales=None), dict(), 1),                # int8 without scales
    (dict(), dict(), dict(len_lo=None), 1),
    (dict(), dict(), dict(mp_lo=0), 1),
    (dict(), dict(), dict(ws=None), 4),
    (dict(), dict(), dict(ws_bytes=1024), 4),
    (dict(), dict(), dict(hq=2 * 17), 2),
    (dict(), dict(), dict(batch=-1), 1),
])
def test_layered_decode_rejects_bad_args(hi_kw, lo_kw, kw, status):
    assert _layered(_cache(**hi_kw), _i8_cache(**lo_kw), **kw) == status
    assert _detail() != ""


def test_layered_decode_workspace_and_empty_batch():
    lib = ops.load_library()
    n = lib.attn_decode_layered_workspace_bytes(16, 64, 8, 128)
    assert n >= 2 * lib.attn_decode_workspace_bytes(16, 64, 8, 128, 4, 16) and n % 256 == 0
    assert lib.attn_decode_layered_workspace_bytes(0, 64, 8, 128) == 0
    assert _layered(_cache(), _i8_cache(), batch=0, q=None, out=None) == 0
    # one byte short of the query for these sizes is rejected (no work enqueued)
    need = lib.attn_decode_layered_workspace_bytes(2, 4, 2, 128)
    assert _layered(_cache(), _i8_cache(), batch=2, hq=4, ws_bytes=need - 1) == 4


def _backward(cache, **kw):
    lib = ops.load_library()
    a = dict(q=FAKE, cu_q=FAKE, block_table=FAKE, max_pages=4, ctx=FAKE, batch=1, total_q=8, max_q_len=8,
             max_ctx=8, hq=4, scale=0.1, causal=1, window=-1, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE,
             dv=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.attn_backward_paged(a["q"], a["cu_q"], ctypes.byref(cache), a["block_table"], a["max_pages"],
                                   a["ctx"], a["batch"], a["total_q"], a["max_q_len"], a["max_ctx"], a["hq"],
                                   a["scale"], a["causal"], a["window"], a["out"], a["lse"], a["dout"], a["dq"],
                                   a["dk"], a["dv"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("cache_kw,kw,status", [
    (dict(dtype=ops.PA_I8, k_scales=0x3000, v_scales=0x4000), dict(), 2),
    (dict(), dict(hq=3), 1), (dict(), dict(scale=0.0), 1), (dict(), dict(causal=3), 1),
    (dict(), dict(dk=None), 1), (dict(), dict(lse=None), 1), (dict(), dict(ws=None), 4),
    (dict(), dict(ws_bytes=8 * 4 * 4 - 1), 4), (dict(), dict(batch=-1), 1), (dict(), dict(max_pages=0), 1),
])
def test_backward_rejects_bad_args(cache_kw, kw, status):
    assert _backward(_cache(**cache_kw), **kw) == status
    assert _detail() != ""


def test_backward_empty_and_workspace_query():
    lib = ops.load_library()
    assert lib.attn_backward_workspace_bytes(8, 4) == 8 * 4 * 4
    assert lib.attn_backward_workspace_bytes(8, 0) == 0
    assert _backward(_cache(), batch=0, q=None) == 0
    assert _backward(_cache(), total_q=0, q=None) == 0


def test_prefill_append_route_query(monkeypatch):
    """The host query says which route attn_prefill_paged_append takes: one
    fused kernel only for bf16 caches with pages of >= 64 keys, at the
    lengths where it is measured faster, unless the environment forces it."""
    lib = ops.load_library()
    monkeypatch.delenv("PAGEDATTN_PREFILL_APPEND_ROUTE", raising=False)
    bf = _cache(page_size=256)
    q = lambda c, causal, win, n: lib.attn_prefill_append_is_fused(ctypes.byref(c), causal, win, n)
    assert q(bf, 1, -1, 2048) == 1 and q(bf, 1, -1, 6144) == 1 and q(bf, 1, -1, 6145) == 0
    assert q(bf, 1, -1, 32768) == 0
    assert q(bf, 1, 128, 1024) == 1 and q(bf, 1, 128, 32768) == 1 and q(bf, 0, -1, 8192) == 1
    assert q(_cache(page_size=16), 1, -1, 2048) == 0
    assert q(_cache(page_size=64, dtype=ops.PA_F32), 1, -1, 2048) == 0
    assert lib.attn_prefill_append_is_fused(None, 1, -1, 2048) == 0
    monkeypatch.setenv("PAGEDATTN_PREFILL_APPEND_ROUTE", "fused")
    assert q(bf, 1, -1, 32768) == 1 and q(_cache(page_size=16), 1, -1, 2048) == 0
    monkeypatch.setenv("PAGEDATTN_PREFILL_APPEND_ROUTE", "separate")
    assert q(bf, 1, -1, 2048) == 0
