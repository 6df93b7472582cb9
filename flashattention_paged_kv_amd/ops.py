"""Python binding of libpagedattn.so (ctypes).  Argument marshalling only:
tensors are checked for device, dtype and contiguity, outputs are allocated
with torch, and every computation runs in the library's HIP kernels on the
current torch stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

The entry points keep the library's names: ``kv_cache_append``,
``kv_pages_quantize_int8``, ``attn_prefill_paged``, ``attn_decode_paged``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDATTN_LIB selects another build of the library (e.g. the host-sanitizer
# build, libpagedattn_hostsan.so); by default the one built in place.
LIB_PATH = os.environ.get("PAGEDATTN_LIB") or os.path.join(_HERE, "libpagedattn.so")

PA_F32, PA_BF16, PA_I8 = 0, 1, 2
_DTYPE_CODE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"pagedattn status {status}: {detail}")
        self.status = status
        self.detail = detail


class _Cache(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None

EXPORTED = ("kv_cache_append", "kv_pages_quantize_int8", "attn_prefill_paged", "attn_prefill_paged_append",
            "attn_prefill_append_is_fused",
            "attn_decode_workspace_bytes",
            "attn_decode_paged", "attn_decode_paged_noalloc", "attn_decode_layered_workspace_bytes", "attn_decode_paged_layered",
            "kv_cache_copy_pages", "attn_backward_workspace_bytes", "attn_backward_paged", "pa_pool_create", "pa_pool_destroy", "pa_pool_extend", "pa_pool_fork",
            "pa_pool_release", "pa_pool_export", "pa_pool_free_pages", "pa_pool_refcount",
            "pa_status_string", "pa_last_error_detail", "pa_abi_version", "pa_device_checks")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A build of the library at `path` with its argument types declared (not
    cached: e.g. the debug build beside the release one)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m flashattention_paged_kv_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    CP = ctypes.POINTER(_Cache)
    lib.kv_cache_append.argtypes = [CP, P, P, P, I32, P, P, I32, I32, P]
    lib.kv_pages_quantize_int8.argtypes = [P, P, P, I32, I32, I32, I32, P]
    lib.attn_prefill_paged.argtypes = [P, P, CP, P, I32, P, I32, I32, I32, F32, I32, I32, P, P, P]
    lib.attn_prefill_paged_append.argtypes = [P, P, P, P, CP, P, I32, P, I32, I32, I32, F32, I32, I32, P, P, P]
    lib.attn_prefill_append_is_fused.argtypes = [CP, I32, I32, I32]
    lib.attn_prefill_append_is_fused.restype = I32
    lib.attn_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.attn_decode_workspace_bytes.restype = SZ
    lib.attn_decode_paged.argtypes = [P, CP, P, I32, P, I32, I32, F32, I32, P, P, P, SZ, P]
    lib.attn_decode_paged_noalloc.argtypes = [P, CP, P, I32, P, I32, I32, F32, I32, P, P, P]
    lib.attn_decode_layered_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.attn_decode_layered_workspace_bytes.restype = SZ
    lib.attn_decode_paged_layered.argtypes = [P, CP, P, I32, P, CP, P, I32, P, I32, I32, F32, P, P, P, SZ, P]
    lib.kv_cache_copy_pages.argtypes = [CP, P, P, I32, P]
    lib.attn_backward_workspace_bytes.argtypes = [I32, I32]
    lib.attn_backward_workspace_bytes.restype = SZ
    lib.attn_backward_paged.argtypes = [P, P, CP, P, I32, P, I32, I32, I32, I32, I32, F32, I32, I32, P, P, P, P, P, P,
                                        P, SZ, P]
    PI = ctypes.POINTER(I32)
    lib.pa_pool_create.argtypes = [I32, I32, I32, I32, ctypes.POINTER(P)]
    lib.pa_pool_destroy.argtypes = [P]
    lib.pa_pool_destroy.restype = None
    lib.pa_pool_extend.argtypes = [P, I32, I32, PI, PI, I32, PI]
    lib.pa_pool_fork.argtypes = [P, I32, I32, I32]
    lib.pa_pool_release.argtypes = [P, I32]
    lib.pa_pool_export.argtypes = [P, PI, PI]
    lib.pa_pool_free_pages.argtypes = [P]
    lib.pa_pool_refcount.argtypes = [P, I32]
    for name in ("pa_pool_free_pages", "pa_pool_refcount"):
        getattr(lib, name).restype = I32
    for name in ("kv_cache_append", "kv_pages_quantize_int8", "attn_prefill_paged", "attn_decode_paged",
                 "attn_decode_paged_noalloc",
                 "attn_decode_paged_layered", "kv_cache_copy_pages", "attn_backward_paged", "pa_pool_create",
                 "pa_pool_extend",
                 "pa_pool_fork", "pa_pool_release", "pa_pool_export"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error_detail.argtypes = []
    lib.pa_last_error_detail.restype = ctypes.c_char_p
    lib.pa_abi_version.restype = I32
    lib.pa_device_checks.restype = I32
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise PagedAttnError(status, f"{lib.pa_status_string(status).decode()}: "
                                     f"{lib.pa_last_error_detail().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


@dataclass
class KVCache:
    """Caller-owned paged cache: pools [num_pages, page_size, Hkv, D] (float32,
    bfloat16, or int8 codes with float32 scales [num_pages, Hkv])."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    k_scales: Optional[torch.Tensor] = None
    v_scales: Optional[torch.Tensor] = None

    @property
    def num_pages(self) -> int:
        return self.k_pages.shape[0]

    @property
    def page_size(self) -> int:
        return self.k_pages.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.k_pages.shape[2]

    @property
    def head_dim(self) -> int:
        return self.k_pages.shape[3]

    @property
    def dtype(self) -> torch.dtype:
        return self.k_pages.dtype

    def _struct(self) -> _Cache:
        _dev(self.k_pages, "k_pages")
        _dev(self.v_pages, "v_pages", self.k_pages.dtype)
        if self.k_pages.dim() != 4 or self.v_pages.shape != self.k_pages.shape:
            raise ValueError("k_pages / v_pages must be [num_pages, page_size, num_kv_heads, head_dim]")
        if self.k_pages.dtype not in _DTYPE_CODE:
            raise ValueError(f"unsupported cache dtype {self.k_pages.dtype}")
        for s in (self.k_scales, self.v_scales):
            if s is not None:
                _dev(s, "scales", torch.float32)
        return _Cache(self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                      None if self.k_scales is None else self.k_scales.data_ptr(),
                      None if self.v_scales is None else self.v_scales.data_ptr(),
                      self.num_pages, self.page_size, self.num_kv_heads, self.head_dim,
                      _DTYPE_CODE[self.k_pages.dtype])


def kv_cache_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, block_table: torch.Tensor,
                    start_pos: torch.Tensor, cu_new: torch.Tensor, max_new: Optional[int] = None) -> None:
    """Write rows of k_new / v_new [total_new, Hkv, D] into their page slots
    (bfloat16 rows for an int8 cache, which requantises the touched pages)."""
    lib = load_library()
    cs = cache._struct()
    row_dtype = torch.bfloat16 if cache.dtype == torch.int8 else cache.dtype
    _dev(k_new, "k_new", row_dtype)
    _dev(v_new, "v_new", row_dtype)
    _dev(block_table, "block_table", torch.int32)
    _dev(start_pos, "start_pos", torch.int32)
    _dev(cu_new, "cu_new", torch.int32)
    batch = start_pos.shape[0]
    max_new = k_new.shape[0] if max_new is None else max_new
    _check(lib.kv_cache_append(ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(block_table),
                               block_table.shape[1], _ptr(start_pos), _ptr(cu_new), batch, max_new, _stream()))


def kv_pages_quantize_int8(src: torch.Tensor, codes: Optional[torch.Tensor] = None,
                           scales: Optional[torch.Tensor] = None):
    """bf16 pages [N, P, Hkv, D] -> (int8 codes, fp32 scales [N, Hkv])."""
    lib = load_library()
    _dev(src, "src", torch.bfloat16)
    n, p, hkv, d = src.shape
    codes = torch.empty(src.shape, dtype=torch.int8, device=src.device) if codes is None else codes
    scales = torch.empty((n, hkv), dtype=torch.float32, device=src.device) if scales is None else scales
    _dev(codes, "codes", torch.int8)
    _dev(scales, "scales", torch.float32)
    _check(lib.kv_pages_quantize_int8(_ptr(src), _ptr(codes), _ptr(scales), n, p, hkv, d, _stream()))
    return codes, scales


def attn_prefill_paged(q: torch.Tensor, cu_q: torch.Tensor, cache: KVCache, block_table: torch.Tensor,
                       ctx_lens: torch.Tensor, max_q_len: Optional[int] = None,
                       softmax_scale: Optional[float] = None, causal: bool = True, window_left: int = -1,
                       out: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Attention of q [total_q, Hq, D] (ragged by cu_q) against the paged
    cache.  Returns out (and lse [total_q, Hq] if asked)."""
    lib = load_library()
    cs = cache._struct()
    _dev(q, "q")
    _dev(cu_q, "cu_q", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    _dev(ctx_lens, "ctx_lens", torch.int32)
    total_q, hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    max_q_len = total_q if max_q_len is None else max_q_len
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_prefill_paged(_ptr(q), _ptr(cu_q), ctypes.byref(cs), _ptr(block_table), block_table.shape[1],
                                  _ptr(ctx_lens), ctx_lens.shape[0], max_q_len, hq, scale, int(bool(causal)),
                                  int(window_left), _ptr(out), _ptr(lse), _stream()))
    return (out, lse) if return_lse else out


def attn_prefill_paged_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cu_q: torch.Tensor,
                              cache: KVCache, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                              max_q_len: Optional[int] = None, softmax_scale: Optional[float] = None,
                              causal: bool = True, window_left: int = -1, out: Optional[torch.Tensor] = None,
                              return_lse: bool = False):
    """Append the queries' own K/V rows k_new / v_new [total_q, Hkv, D] at
    positions ctx_lens[b] - q_len_b + i, then attend q over the whole
    context: kv_cache_append followed by attn_prefill_paged, in one kernel
    for bf16 caches with pages of 64 keys or more."""
    lib = load_library()
    cs = cache._struct()
    _dev(q, "q")
    _dev(k_new, "k_new", cache.dtype)
    _dev(v_new, "v_new", cache.dtype)
    _dev(cu_q, "cu_q", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    _dev(ctx_lens, "ctx_lens", torch.int32)
    total_q, hq, d = q.shape
    if k_new.shape != (total_q, cache.num_kv_heads, d) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new / v_new must be [{total_q}, {cache.num_kv_heads}, {d}]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    max_q_len = total_q if max_q_len is None else max_q_len
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_prefill_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_q), ctypes.byref(cs),
                                         _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), ctx_lens.shape[0],
                                         max_q_len, hq, scale, int(bool(causal)), int(window_left), _ptr(out),
                                         _ptr(lse), _stream()))
    return (out, lse) if return_lse else out


def prefill_append_is_fused(cache: KVCache, causal: bool = True, window_left: int = -1,
                            max_q_len: int = 1) -> bool:
    """Whether attn_prefill_paged_append runs as one fused kernel for these
    arguments (else: the append kernel, then the prefill)."""
    return bool(load_library().attn_prefill_append_is_fused(ctypes.byref(cache._struct()), int(bool(causal)),
                                                            int(window_left), int(max_q_len)))


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_pages_per_seq: int, page_size: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                          max_pages_per_seq, page_size))


def attn_decode_paged(q: torch.Tensor, cache: KVCache, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                      softmax_scale: Optional[float] = None, window_left: int = -1,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      return_lse: bool = False):
    """One query per sequence, q [B, Hq, D], against its ctx_lens[b] cached
    keys.  ``workspace`` (uint8, at least decode_workspace_bytes(...)) is
    allocated if not given."""
    lib = load_library()
    cs = cache._struct()
    _dev(q, "q")
    _dev(block_table, "block_table", torch.int32)
    _dev(ctx_lens, "ctx_lens", torch.int32)
    batch, hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if workspace is None:
        nbytes = decode_workspace_bytes(batch, hq, cache.num_kv_heads, d, block_table.shape[1], cache.page_size)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_decode_paged(_ptr(q), ctypes.byref(cs), _ptr(block_table), block_table.shape[1],
                                 _ptr(ctx_lens), batch, hq, scale, int(window_left), _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 32 << 20   # PA_NOALLOC_SCRATCH_BYTES of the header


def attn_decode_paged_noalloc(q: torch.Tensor, cache: KVCache, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                              out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                              softmax_scale: Optional[float] = None, window_left: int = -1) -> torch.Tensor:
    """attn_decode_paged with the library's own scratch instead of a
    workspace: the call allocates nothing (the caller passes ``out`` and,
    optionally, ``lse`` [B, Hq] float32).  Calls on one GPU share the
    scratch, so overlapping calls race."""
    lib = load_library()
    cs = cache._struct()
    _dev(q, "q")
    _dev(block_table, "block_table", torch.int32)
    _dev(ctx_lens, "ctx_lens", torch.int32)
    _dev(out, "out", q.dtype)
    batch, hq, d = q.shape
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if tuple(lse.shape) != (batch, hq):
            raise ValueError(f"lse must be [{batch}, {hq}]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_decode_paged_noalloc(_ptr(q), ctypes.byref(cs), _ptr(block_table), block_table.shape[1],
                                         _ptr(ctx_lens), batch, hq, scale, int(window_left), _ptr(out), _ptr(lse),
                                         _stream()))
    return out


def decode_layered_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    return int(load_library().attn_decode_layered_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim))


def attn_decode_paged_layered(q: torch.Tensor, cache_hi: KVCache, block_table_hi: torch.Tensor,
                              len_hi: torch.Tensor, cache_lo: KVCache, block_table_lo: torch.Tensor,
                              len_lo: torch.Tensor, softmax_scale: Optional[float] = None,
                              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              return_lse: bool = False):
    """One query per sequence, q [B, Hq, D], against len_hi[b] keys of cache_hi
    followed by len_lo[b] keys of cache_lo (e.g. the first tokens in bf16, the
    rest int8).  ``workspace`` is allocated if not given."""
    lib = load_library()
    cs_hi, cs_lo = cache_hi._struct(), cache_lo._struct()
    _dev(q, "q")
    for t, name in ((block_table_hi, "block_table_hi"), (len_hi, "len_hi"), (block_table_lo, "block_table_lo"),
                    (len_lo, "len_lo")):
        _dev(t, name, torch.int32)
    batch, hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if workspace is None:
        nbytes = decode_layered_workspace_bytes(batch, hq, cache_hi.num_kv_heads, d)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_decode_paged_layered(_ptr(q), ctypes.byref(cs_hi), _ptr(block_table_hi), block_table_hi.shape[1],
                                         _ptr(len_hi), ctypes.byref(cs_lo), _ptr(block_table_lo),
                                         block_table_lo.shape[1], _ptr(len_lo), batch, hq, scale, _ptr(out),
                                         _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream()))
    return (out, lse) if return_lse else out


def kv_cache_copy_pages(cache: KVCache, src_pages: torch.Tensor, dst_pages: torch.Tensor) -> None:
    """Copy whole pages src_pages[i] -> dst_pages[i] of the cache (K, V and
    int8 scales) on the current stream."""
    lib = load_library()
    cs = cache._struct()
    _dev(src_pages, "src_pages", torch.int32)
    _dev(dst_pages, "dst_pages", torch.int32)
    if src_pages.numel() != dst_pages.numel():
        raise ValueError("src_pages and dst_pages must have the same length")
    _check(lib.kv_cache_copy_pages(ctypes.byref(cs), _ptr(src_pages), _ptr(dst_pages), src_pages.numel(),
                                   _stream()))


class PagePool:
    """Host page pool of the library (native): block-table rows, shared
    pages with reference counts, copy-on-write of a shared partly filled
    page.  Host-only; ``block_table()`` gives the table to upload."""

    def __init__(self, num_pages: int, page_size: int, max_seqs: int, max_pages_per_seq: int):
        self._lib = load_library()
        self._h = ctypes.c_void_p()
        _check(self._lib.pa_pool_create(num_pages, page_size, max_seqs, max_pages_per_seq, ctypes.byref(self._h)))
        self.num_pages, self.page_size = num_pages, page_size
        self.max_seqs, self.max_pages_per_seq = max_seqs, max_pages_per_seq

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_pool_destroy(h)
            self._h = None

    def extend(self, seq: int, new_len: int):
        """Grow `seq` to `new_len` tokens; returns the (src, dst) page pairs to
        copy before appending (empty unless a shared page was replaced)."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_pool_extend(self._h, seq, new_len, ctypes.byref(src), ctypes.byref(dst), 1,
                                        ctypes.byref(n)))
        return [(src.value, dst.value)] if n.value else []

    def fork(self, parent: int, child: int, n_tokens: int) -> None:
        _check(self._lib.pa_pool_fork(self._h, parent, child, n_tokens))

    def release(self, seq: int) -> None:
        _check(self._lib.pa_pool_release(self._h, seq))

    def block_table(self) -> torch.Tensor:
        t = torch.empty((self.max_seqs, self.max_pages_per_seq), dtype=torch.int32)
        _check(self._lib.pa_pool_export(self._h, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32)), None))
        return t

    def lens(self) -> torch.Tensor:
        t = torch.empty(self.max_seqs, dtype=torch.int32)
        _check(self._lib.pa_pool_export(self._h, None, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))))
        return t

    def free_pages(self) -> int:
        return int(self._lib.pa_pool_free_pages(self._h))

    def refcount(self, page: int) -> int:
        return int(self._lib.pa_pool_refcount(self._h, page))


def attn_backward_paged(q: torch.Tensor, cu_q: torch.Tensor, cache: KVCache, block_table: torch.Tensor,
                        ctx_lens: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, d_out: torch.Tensor,
                        max_q_len: Optional[int] = None, max_ctx: Optional[int] = None,
                        softmax_scale: Optional[float] = None, causal: bool = True, window_left: int = -1,
                        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk_pages, dv_pages), fp32, of attn_prefill_paged's output
    for upstream gradient d_out; out and lse are the forward's.  dk / dv
    (fp32, pool-shaped) are allocated zero-filled if not given; only the slots
    of cached positions are written."""
    lib = load_library()
    cs = cache._struct()
    for t, name in ((q, "q"), (out, "out"), (d_out, "d_out")):
        _dev(t, name, cache.dtype)
    _dev(lse, "lse", torch.float32)
    for t, name in ((cu_q, "cu_q"), (block_table, "block_table"), (ctx_lens, "ctx_lens")):
        _dev(t, name, torch.int32)
    total_q, hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    max_q_len = total_q if max_q_len is None else max_q_len
    max_ctx = int(ctx_lens.max().item()) if max_ctx is None else max_ctx
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    shape = tuple(cache.k_pages.shape)
    dk = torch.zeros(shape, dtype=torch.float32, device=q.device) if dk is None else _dev(dk, "dk", torch.float32)
    dv = torch.zeros(shape, dtype=torch.float32, device=q.device) if dv is None else _dev(dv, "dv", torch.float32)
    if workspace is None:
        workspace = torch.empty(max(lib.attn_backward_workspace_bytes(total_q, hq), 1), dtype=torch.uint8,
                                device=q.device)
    _dev(workspace, "workspace")
    _check(lib.attn_backward_paged(_ptr(q), _ptr(cu_q), ctypes.byref(cs), _ptr(block_table), block_table.shape[1],
                                   _ptr(ctx_lens), ctx_lens.shape[0], total_q, max_q_len, max_ctx, hq, scale,
                                   int(bool(causal)), int(window_left), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream()))
    return dq, dk, dv
