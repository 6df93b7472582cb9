// C ABI of libpagedattn.so: argument checks, dispatch and launch.  Every
// check that the host can make is made before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/pagedattn.h"
#include "pa_internal.h"

namespace {

thread_local char g_detail[512] = "";

pa_status fail(pa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status fail(pa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return st;
}

pa_status ok() {
  g_detail[0] = '\0';
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The status of a call whose kernels have been enqueued on `s`.  Debug
// builds (PA_DEVICE_CHECKS=1) wait for them and report the first
// device-resident integer they found out of range (PA_ERR_DEVICE_ASSERT);
// release builds return at once.
pa_status launched(hipError_t e, hipStream_t s, const char *what) {
  if (e != hipSuccess) return hip_status(e, what);
#if PA_DEVICE_CHECKS
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_status(e, what);
  static const char *const kSite[] = {"-", "page id", "context length", "query count", "new-row count",
                                      "append start position", "row offset"};
  hipError_t (*const readers[])(pa::DeviceFault *) = {pa::take_fault_append, pa::take_fault_prefill,
                                                      pa::take_fault_decode, pa::take_fault_backward,
                                                      pa::take_fault_page_pool};
  for (auto read : readers) {
    pa::DeviceFault f = {};
    if ((e = read(&f)) != hipSuccess) return hip_status(e, what);
    if (f.flag != 0) {
      const int site = f.site >= 0 && f.site <= 6 ? f.site : 0;
      return fail(PA_ERR_DEVICE_ASSERT, "%s: device check: %s %d of sequence %d outside [%d, %d]", what,
                  kSite[site], f.value, f.batch, f.lo, f.hi);
    }
  }
#else
  (void)s;
#endif
  return ok();
}

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

// Checks shared by every call that reads a cache.
pa_status check_cache(const pa_kv_cache *c, bool need_scales_if_i8) {
  if (c == nullptr) return fail(PA_ERR_INVALID_ARG, "cache is NULL");
  if (c->k_pages == nullptr || c->v_pages == nullptr) return fail(PA_ERR_INVALID_ARG, "cache pages are NULL");
  if (c->num_pages <= 0) return fail(PA_ERR_INVALID_ARG, "num_pages must be > 0 (got %d)", c->num_pages);
  if (c->num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", c->num_kv_heads);
  if (c->dtype != PA_F32 && c->dtype != PA_BF16 && c->dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED, "unknown cache dtype %d", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  const int lp = log2_exact(c->page_size);
  if (lp < 4 || lp > 8) return fail(PA_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 256] (got %d)", c->page_size);
  if (c->dtype == PA_I8 && need_scales_if_i8 && (c->k_scales == nullptr || c->v_scales == nullptr))
    return fail(PA_ERR_INVALID_ARG, "int8 cache needs k_scales and v_scales");
  return PA_OK;
}

pa::CacheView view_of(const pa_kv_cache *c) {
  pa::CacheView v;
  v.k = c->k_pages;
  v.v = c->v_pages;
  v.k_scales = c->k_scales;
  v.v_scales = c->v_scales;
  v.num_pages = c->num_pages;
  v.page_size = c->page_size;
  v.log2_page = log2_exact(c->page_size);
  v.num_kv_heads = c->num_kv_heads;
  v.head_dim = c->head_dim;
  v.dtype = c->dtype;
  return v;
}

pa_status check_scale(float s) {
  if (!(s > 0.f) || !isfinite(s)) return fail(PA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return PA_OK;
}

// Decode workspace: partial (O, m, l) for batch * Hkv / hpw + nwg slots of
// hpw KV heads x G query heads each, then batch + 1 int32 prefix sums.
size_t decode_ws_bytes(int batch, int hq, int hkv, int d, int nwg) {
  const size_t heads = (size_t)batch * hkv + (size_t)nwg * pa::decode_heads_per_wg(hkv);
  const size_t g = (size_t)(hq / hkv);
  return heads * g * ((size_t)d + 2) * sizeof(float) + ((size_t)batch + 1) * sizeof(int32_t);
}

size_t round_up_256(size_t n) { return (n + 255) & ~(size_t)255; }

// Split/merge arguments of one decode over `cache`, with its workspace at
// `workspace` (decode_ws_bytes(...) bytes).
pa::DecodeArgs decode_args(const void *q, const pa_kv_cache *cache, const int32_t *block_table, int32_t max_pages,
                           const int32_t *ctx_lens, int32_t batch, int32_t num_q_heads, float softmax_scale,
                           int32_t window_left, void *out, float *lse, void *workspace, int nwg) {
  pa::DecodeArgs a;
  const int group = num_q_heads / cache->num_kv_heads;
  a.q = q;
  a.c = view_of(cache);
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.ctx_lens = ctx_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.group = group;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.out = out;
  a.lse = lse;
  const int hpw = pa::decode_heads_per_wg(cache->num_kv_heads);
  const size_t slots_g = ((size_t)batch * cache->num_kv_heads + (size_t)nwg * hpw) * group;
  a.ws_o = (float *)workspace;
  a.ws_ml = a.ws_o + slots_g * cache->head_dim;
  a.ws_prefix = (int32_t *)(a.ws_ml + slots_g * 2);
  a.nwg = nwg;
  a.hpw = hpw;
  return a;
}

}  // namespace

namespace pa {
// Status reporting for the host-side parts outside this file.
pa_status report(pa_status st, const char *msg) {
  if (st == PA_OK) return ok();
  return fail(st, "%s", msg);
}
}  // namespace pa

// Checks shared by the prefill entry points; fills *a.  *empty: nothing to
// compute (batch or max_q_len is 0).
static pa_status prefill_args(const void *q, const int32_t *cu_q, const pa_kv_cache *cache, const int32_t *block_table,
                       int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch, int32_t max_q_len,
                       int32_t num_q_heads, float softmax_scale, int32_t causal, int32_t window_left, void *out,
                       float *lse, pa::PrefillArgs *a, bool *empty) {
  pa_status st = check_cache(cache, false);
  if (st != PA_OK) return st;
  if (cache->dtype == PA_I8) return fail(PA_ERR_UNSUPPORTED, "prefill over an int8 cache is not supported");
  if (batch < 0 || max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "batch and max_q_len must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, cache->num_kv_heads);
  if ((st = check_scale(softmax_scale)) != PA_OK) return st;
  if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
  *empty = batch == 0 || max_q_len == 0;
  if (*empty) return ok();
  if (q == nullptr || cu_q == nullptr || block_table == nullptr || ctx_lens == nullptr || out == nullptr)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_pages_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  a->q = q;
  a->cu_q = cu_q;
  a->c = view_of(cache);
  a->block_table = block_table;
  a->max_pages = max_pages_per_seq;
  a->ctx_lens = ctx_lens;
  a->batch = batch;
  a->max_q_len = max_q_len;
  a->num_q_heads = num_q_heads;
  a->group = num_q_heads / cache->num_kv_heads;
  a->scale_log2 = softmax_scale * 1.4426950408889634f;
  a->causal = causal;
  a->window_left = window_left < 0 ? -1 : window_left;
  a->out = out;
  a->lse = lse;
  a->k_new = nullptr;
  a->v_new = nullptr;
  return ok();
}

// attn_prefill_paged_append on a bf16 cache with pages of >= 64 keys: one
// fused kernel, or the append kernel and then the prefill.  Same result
// either way; the choice follows measured times on MI355X (L = 1k..32k, 32
// heads, D = 128): with a causal mask and no window (pairs of query tiles)
// the fused kernel wins up to about 6k query rows and is level or behind
// beyond (its page stores cost more than the separate copy); with a window
// or no mask (runs of query tiles) it is level or ahead at every length.
// PAGEDATTN_PREFILL_APPEND_ROUTE=fused|separate in the environment forces a
// route (tests use it to cover both kernels at small sizes).
static bool prefill_append_fused(int32_t causal, int32_t window_left, int32_t max_q_len) {
  const char *route = getenv("PAGEDATTN_PREFILL_APPEND_ROUTE");
  if (route != nullptr && strcmp(route, "fused") == 0) return true;
  if (route != nullptr && strcmp(route, "separate") == 0) return false;
  const bool pairs = causal != 0 && window_left < 0;
  return pairs ? max_q_len <= 6144 : true;
}

// Host checks of a single-token decode (attn_decode_paged and its variant
// without a workspace), before anything touches the device.  PA_OK with
// batch == 0: nothing to do.
static pa_status decode_check_args(const void *q, const pa_kv_cache *cache, const int32_t *block_table,
                                   int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch,
                                   int32_t num_q_heads, float softmax_scale, const void *out) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, cache->num_kv_heads);
  const int group = num_q_heads / cache->num_kv_heads;
  if (cache->dtype != PA_F32 && group > 16)
    return fail(PA_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)", group);
  if ((st = check_scale(softmax_scale)) != PA_OK) return st;
  if (batch == 0) return ok();
  if (q == nullptr || block_table == nullptr || ctx_lens == nullptr || out == nullptr)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_pages_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  return ok();
}

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

int32_t pa_device_checks(void) { return PA_DEVICE_CHECKS; }

const char *pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_OUT_OF_PAGES: return "not enough free pages in the pool";
    case PA_ERR_DEVICE_ASSERT: return "a device-side check failed (debug build)";
  }
  return "unknown status";
}

const char *pa_last_error_detail(void) { return g_detail; }

pa_status kv_cache_append(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                          const int32_t *block_table, int32_t max_pages_per_seq, const int32_t *start_pos,
                          const int32_t *cu_new, int32_t batch, int32_t max_new, void *stream) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (batch < 0 || max_new < 0) return fail(PA_ERR_INVALID_ARG, "batch and max_new must be >= 0");
  if (batch == 0 || max_new == 0) return ok();
  if (k_new == nullptr || v_new == nullptr || block_table == nullptr || start_pos == nullptr || cu_new == nullptr)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_pages_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  if (cache->dtype == PA_I8) {
    pa::AppendI8Args a;
    a.k_codes = (int8_t *)cache->k_pages;
    a.v_codes = (int8_t *)cache->v_pages;
    a.k_scales = cache->k_scales;
    a.v_scales = cache->v_scales;
    a.k_new = (const uint16_t *)k_new;
    a.v_new = (const uint16_t *)v_new;
    a.block_table = block_table;
    a.max_pages = max_pages_per_seq;
    a.start_pos = start_pos;
    a.cu_new = cu_new;
    a.batch = batch;
    a.max_new = max_new;
    a.page_size = cache->page_size;
    a.log2_page = log2_exact(cache->page_size);
    a.num_kv_heads = cache->num_kv_heads;
    a.head_dim = cache->head_dim;
    a.num_pages = cache->num_pages;
    return launched(pa::launch_append_i8(a, (hipStream_t)stream), (hipStream_t)stream, "kv_cache_append");
  }
  pa::AppendArgs a;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.max_pages = max_pages_per_seq;
  a.start_pos = start_pos;
  a.ctx_lens = nullptr;
  a.cu_new = cu_new;
  a.batch = batch;
  a.max_new = max_new;
  a.page_size = cache->page_size;
  a.log2_page = log2_exact(cache->page_size);
  a.row_bytes = cache->num_kv_heads * cache->head_dim * (cache->dtype == PA_F32 ? 4 : 2);
  a.num_pages = cache->num_pages;
  return launched(pa::launch_append(a, (hipStream_t)stream), (hipStream_t)stream, "kv_cache_append");
}

pa_status kv_pages_quantize_int8(const void *src, int8_t *codes, float *scales, int32_t num_pages,
                                 int32_t page_size, int32_t num_kv_heads, int32_t head_dim, void *stream) {
  if (src == nullptr || codes == nullptr || scales == nullptr) return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (num_pages < 0 || num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "bad num_pages / num_kv_heads");
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int lp = log2_exact(page_size);
  if (lp < 4 || lp > 8) return fail(PA_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 256]");
  if (num_pages == 0) return ok();
  pa::QuantArgs a;
  a.src = (const uint16_t *)src;
  a.codes = codes;
  a.scales = scales;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  return launched(pa::launch_quantize(a, (hipStream_t)stream), (hipStream_t)stream, "kv_pages_quantize_int8");
}

pa_status attn_prefill_paged(const void *q, const int32_t *cu_q, const pa_kv_cache *cache,
                             const int32_t *block_table, int32_t max_pages_per_seq, const int32_t *ctx_lens,
                             int32_t batch, int32_t max_q_len, int32_t num_q_heads, float softmax_scale,
                             int32_t causal, int32_t window_left, void *out, float *lse, void *stream) {
  pa::PrefillArgs a;
  bool empty = false;
  pa_status st = prefill_args(q, cu_q, cache, block_table, max_pages_per_seq, ctx_lens, batch, max_q_len, num_q_heads,
                              softmax_scale, causal, window_left, out, lse, &a, &empty);
  if (st != PA_OK || empty) return st;
  return launched(pa::launch_prefill(a, (hipStream_t)stream), (hipStream_t)stream, "attn_prefill_paged");
}

int32_t attn_prefill_append_is_fused(const pa_kv_cache *cache, int32_t causal, int32_t window_left,
                                     int32_t max_q_len) {
  return cache != nullptr && cache->dtype == PA_BF16 && cache->page_size >= 64 &&
         prefill_append_fused(causal, window_left, max_q_len);
}

pa_status attn_prefill_paged_append(const void *q, const void *k_new, const void *v_new, const int32_t *cu_q,
                                    const pa_kv_cache *cache, const int32_t *block_table, int32_t max_pages_per_seq,
                                    const int32_t *ctx_lens, int32_t batch, int32_t max_q_len, int32_t num_q_heads,
                                    float softmax_scale, int32_t causal, int32_t window_left, void *out, float *lse,
                                    void *stream) {
  pa::PrefillArgs a;
  bool empty = false;
  pa_status st = prefill_args(q, cu_q, cache, block_table, max_pages_per_seq, ctx_lens, batch, max_q_len, num_q_heads,
                              softmax_scale, causal, window_left, out, lse, &a, &empty);
  if (st != PA_OK) return st;
  if (!empty && (k_new == nullptr || v_new == nullptr)) return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (empty) return ok();
  const hipStream_t s = (hipStream_t)stream;
  if (attn_prefill_append_is_fused(cache, causal, window_left, max_q_len)) {
    a.k_new = k_new;
    a.v_new = v_new;
    return launched(pa::launch_prefill(a, s), s, "attn_prefill_paged_append");
  }
  // Other caches (fp32, or pages smaller than a key tile), and the lengths
  // where two launches are faster: the append kernel (start = ctx_lens[b] -
  // q_len_b) and then the prefill, on the same stream.
  pa::AppendArgs ap;
  ap.k_pages = cache->k_pages;
  ap.v_pages = cache->v_pages;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.block_table = block_table;
  ap.max_pages = max_pages_per_seq;
  ap.start_pos = nullptr;
  ap.ctx_lens = ctx_lens;
  ap.cu_new = cu_q;
  ap.batch = batch;
  ap.max_new = max_q_len;
  ap.page_size = cache->page_size;
  ap.log2_page = log2_exact(cache->page_size);
  ap.row_bytes = cache->num_kv_heads * cache->head_dim * (cache->dtype == PA_F32 ? 4 : 2);
  ap.num_pages = cache->num_pages;
  if ((st = launched(pa::launch_append(ap, s), s, "attn_prefill_paged_append (append)")) != PA_OK) return st;
  return launched(pa::launch_prefill(a, s), s, "attn_prefill_paged_append");
}

pa_status kv_cache_copy_pages(const pa_kv_cache *cache, const int32_t *src_pages, const int32_t *dst_pages,
                              int32_t n, void *stream) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (src_pages == nullptr || dst_pages == nullptr) return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (n > 65535) return fail(PA_ERR_INVALID_ARG, "at most 65535 pages per call (got %d)", n);
  const size_t esz = cache->dtype == PA_F32 ? 4 : cache->dtype == PA_BF16 ? 2 : 1;
  const size_t page_bytes = (size_t)cache->page_size * cache->num_kv_heads * cache->head_dim * esz;
  const bool i8 = cache->dtype == PA_I8;
  return launched(pa::launch_copy_pages(cache->k_pages, cache->v_pages, i8 ? cache->k_scales : nullptr,
                                          i8 ? cache->v_scales : nullptr, cache->num_kv_heads, src_pages, dst_pages,
                                          n, page_bytes, cache->num_pages, (hipStream_t)stream),
                  (hipStream_t)stream,
                    "kv_cache_copy_pages");
}

size_t attn_backward_workspace_bytes(int32_t total_q, int32_t num_q_heads) {
  if (total_q < 0 || num_q_heads <= 0) return 0;
  return (size_t)total_q * num_q_heads * sizeof(float);
}

pa_status attn_backward_paged(const void *q, const int32_t *cu_q, const pa_kv_cache *cache, const int32_t *block_table,
                              int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch, int32_t total_q,
                              int32_t max_q_len, int32_t max_ctx, int32_t num_q_heads, float softmax_scale,
                              int32_t causal, int32_t window_left, const void *out, const float *lse,
                              const void *d_out, float *dq, float *dk_pages, float *dv_pages, void *workspace,
                              size_t workspace_bytes, void *stream) {
  pa_status st = check_cache(cache, false);
  if (st != PA_OK) return st;
  if (cache->dtype == PA_I8) return fail(PA_ERR_UNSUPPORTED, "the backward pass takes bf16 or fp32 caches");
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_ctx < 0)
    return fail(PA_ERR_INVALID_ARG, "batch, total_q, max_q_len and max_ctx must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, cache->num_kv_heads);
  if ((st = check_scale(softmax_scale)) != PA_OK) return st;
  if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (q == nullptr || cu_q == nullptr || block_table == nullptr || ctx_lens == nullptr || out == nullptr ||
      lse == nullptr || d_out == nullptr || dq == nullptr || dk_pages == nullptr || dv_pages == nullptr)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_pages_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq must be > 0");
  if (max_q_len > 65535 * 64 || batch > 65535) return fail(PA_ERR_INVALID_ARG, "batch or max_q_len too large");
  const size_t need = attn_backward_workspace_bytes(total_q, num_q_heads);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "backward needs %zu workspace bytes (got %zu)", need, workspace_bytes);
  pa::BackwardArgs a;
  a.q = q;
  a.cu_q = cu_q;
  a.c = view_of(cache);
  a.block_table = block_table;
  a.max_pages = max_pages_per_seq;
  a.ctx_lens = ctx_lens;
  a.batch = batch;
  a.max_q_len = max_q_len;
  a.max_ctx = max_ctx;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.group = num_q_heads / cache->num_kv_heads;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.window_left = window_left < 0 ? -1 : window_left;
  a.out = out;
  a.lse = lse;
  a.d_out = d_out;
  a.dq = dq;
  a.dk = dk_pages;
  a.dv = dv_pages;
  a.delta = (float *)workspace;
  return launched(pa::launch_backward(a, (hipStream_t)stream), (hipStream_t)stream, "attn_backward_paged");
}

size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_pages_per_seq, int32_t page_size) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_pages_per_seq <= 0 ||
      log2_exact(page_size) < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int nwg = pa::decode_grid_size();
  if (nwg <= 0) return 0;
  return decode_ws_bytes(batch, num_q_heads, num_kv_heads, head_dim, nwg);
}

pa_status attn_decode_paged(const void *q, const pa_kv_cache *cache, const int32_t *block_table,
                            int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch, int32_t num_q_heads,
                            float softmax_scale, int32_t window_left, void *out, float *lse, void *workspace,
                            size_t workspace_bytes, void *stream) {
  pa_status st = decode_check_args(q, cache, block_table, max_pages_per_seq, ctx_lens, batch, num_q_heads,
                                   softmax_scale, out);
  if (st != PA_OK || batch == 0) return st;
  const int group = num_q_heads / cache->num_kv_heads;

  if (cache->dtype == PA_F32) {
    pa::PrefillArgs a;
    a.q = q;
    a.cu_q = nullptr;  // one query per sequence
    a.c = view_of(cache);
    a.block_table = block_table;
    a.max_pages = max_pages_per_seq;
    a.ctx_lens = ctx_lens;
    a.batch = batch;
    a.max_q_len = 1;
    a.num_q_heads = num_q_heads;
    a.group = group;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.causal = 1;
    a.window_left = window_left < 0 ? -1 : window_left;
    a.out = out;
    a.lse = lse;
    return launched(pa::launch_prefill(a, (hipStream_t)stream), (hipStream_t)stream, "attn_decode_paged");
  }

  const int nwg = pa::decode_grid_size();
  if (nwg <= 0) return fail(PA_ERR_HIP, "cannot query the current device");
  const size_t need = decode_ws_bytes(batch, num_q_heads, cache->num_kv_heads, cache->head_dim, nwg);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "decode needs %zu workspace bytes (got %zu)", need, workspace_bytes);
  const pa::DecodeArgs a = decode_args(q, cache, block_table, max_pages_per_seq, ctx_lens, batch, num_q_heads,
                                       softmax_scale, window_left, out, lse, workspace, nwg);
  return launched(pa::launch_decode(a, (hipStream_t)stream), (hipStream_t)stream, "attn_decode_paged");
}

pa_status attn_decode_paged_noalloc(const void *q, const pa_kv_cache *cache, const int32_t *block_table,
                                    int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch,
                                    int32_t num_q_heads, float softmax_scale, int32_t window_left, void *out,
                                    float *lse, void *stream) {
  pa_status st = decode_check_args(q, cache, block_table, max_pages_per_seq, ctx_lens, batch, num_q_heads,
                                   softmax_scale, out);
  if (st != PA_OK || batch == 0) return st;
  if (cache->dtype == PA_F32)  // fp32 caches decode without partials (no scratch)
    return attn_decode_paged(q, cache, block_table, max_pages_per_seq, ctx_lens, batch, num_q_heads, softmax_scale,
                             window_left, out, lse, nullptr, 0, stream);
  const size_t cap = pa::noalloc_scratch_bytes();
  const size_t need = attn_decode_workspace_bytes(batch, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                                  max_pages_per_seq, cache->page_size);
  if (need > cap)
    return fail(PA_ERR_WORKSPACE,
                "attn_decode_paged_noalloc: batch %d with %d query heads over %d KV heads needs %zu bytes of "
                "scratch, more than the %zu the library holds (use attn_decode_paged with a workspace)",
                batch, num_q_heads, cache->num_kv_heads, need, cap);
  void *ws = nullptr;
  if ((st = hip_status(pa::noalloc_scratch(&ws), "attn_decode_paged_noalloc scratch address")) != PA_OK) return st;
  return attn_decode_paged(q, cache, block_table, max_pages_per_seq, ctx_lens, batch, num_q_heads, softmax_scale,
                           window_left, out, lse, ws, cap, stream);
}

size_t attn_decode_layered_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int nwg = pa::decode_grid_size();
  if (nwg <= 0) return 0;
  return 2 * round_up_256(decode_ws_bytes(batch, num_q_heads, num_kv_heads, head_dim, nwg));
}

pa_status attn_decode_paged_layered(const void *q, const pa_kv_cache *cache_hi, const int32_t *block_table_hi,
                                    int32_t max_pages_hi, const int32_t *len_hi, const pa_kv_cache *cache_lo,
                                    const int32_t *block_table_lo, int32_t max_pages_lo, const int32_t *len_lo,
                                    int32_t batch, int32_t num_q_heads, float softmax_scale, void *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  pa_status st = check_cache(cache_hi, true);
  if (st != PA_OK) return st;
  if ((st = check_cache(cache_lo, true)) != PA_OK) return st;
  if (cache_hi->dtype == PA_F32 || cache_lo->dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "layered decode takes bf16 or int8 caches");
  if (cache_hi->num_kv_heads != cache_lo->num_kv_heads || cache_hi->head_dim != cache_lo->head_dim)
    return fail(PA_ERR_INVALID_ARG, "the two caches must have the same num_kv_heads and head_dim");
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % cache_hi->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, cache_hi->num_kv_heads);
  if (num_q_heads / cache_hi->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)",
                num_q_heads / cache_hi->num_kv_heads);
  if ((st = check_scale(softmax_scale)) != PA_OK) return st;
  if (batch == 0) return ok();
  if (q == nullptr || block_table_hi == nullptr || len_hi == nullptr || block_table_lo == nullptr ||
      len_lo == nullptr || out == nullptr)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer argument");
  if (max_pages_hi <= 0 || max_pages_lo <= 0) return fail(PA_ERR_INVALID_ARG, "max_pages_* must be > 0");
  const int nwg = pa::decode_grid_size();
  if (nwg <= 0) return fail(PA_ERR_HIP, "cannot query the current device");
  const size_t part = round_up_256(decode_ws_bytes(batch, num_q_heads, cache_hi->num_kv_heads, cache_hi->head_dim, nwg));
  if (workspace == nullptr || workspace_bytes < 2 * part)
    return fail(PA_ERR_WORKSPACE, "layered decode needs %zu workspace bytes (got %zu)", 2 * part, workspace_bytes);
  const pa::DecodeArgs hi = decode_args(q, cache_hi, block_table_hi, max_pages_hi, len_hi, batch, num_q_heads,
                                        softmax_scale, -1, out, lse, workspace, nwg);
  const pa::DecodeArgs lo = decode_args(q, cache_lo, block_table_lo, max_pages_lo, len_lo, batch, num_q_heads,
                                        softmax_scale, -1, out, lse, (char *)workspace + part, nwg);
  return launched(pa::launch_decode_layered(hi, lo, (hipStream_t)stream), (hipStream_t)stream, "attn_decode_paged_layered");
}

}  // extern "C"
