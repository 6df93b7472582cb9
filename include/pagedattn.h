/*
 * pagedattn.h - C ABI of libpagedattn.so: exact scaled-dot-product attention
 * read from a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes, with the web pages it follows (cited by title
 * and section):
 *   - "大模型推理优化：KV Cache与FlashAttention实战" (LLM inference optimisation:
 *     KV Cache and FlashAttention in practice), section 2.1: a query attends to
 *     every cached key up to and including its own position, with weights
 *     softmax(q.K^T / sqrt(d)) applied to V; section 5.1: the attention call
 *     takes a softmax scale (default 1/sqrt(d)), a causal flag and a local
 *     window.
 *   - "Flash Attention与Paged KV Cache优化大模型计算效率" (Flash Attention and
 *     Paged KV Cache), section 2.1: tiles of Q/K/V are processed on chip;
 *     section 3.2: the cache is cut into fixed-size pages found through a
 *     page table (logical page -> physical page), each page holding
 *     (page_size, d_model) values; section 4.1: the prompt goes through
 *     FlashAttention, generation reads the paged cache.
 *   - "大模型推理优化实战：KV Cache + Flash Attention，让 Token 生成快 3 倍"
 *     (3x faster token generation), "KV Cache" section: new K/V are appended
 *     to the cache before the query attends; "Flash Attention" section: the
 *     online softmax (running max, running sum, rescaling) makes the tiled
 *     result exactly the plain one.
 *   - "LLM推理系统优化：KV缓存管理与动态批处理技术" (KV-cache management and
 *     dynamic batching), section 2.1: grouped-query attention, query head h
 *     reads KV head h / (Hq / Hkv); section 3.1: paged KV blocks (256 tokens
 *     per block); section 3.2: symmetric abs-max group quantisation.
 *
 * Conventions shared by every entry point:
 *   - Memory: every pointer argument is a DEVICE pointer (caller-owned,
 *     e.g. a torch tensor's data_ptr) unless stated otherwise.  The library
 *     allocates and frees no device memory; decode's split partials live in
 *     the caller's workspace.
 *   - Layout: a KV pool is [num_pages, page_size, num_kv_heads, head_dim],
 *     row-major (token-major pages, d_model = num_kv_heads * head_dim).  K and
 *     V have separate pools.  A block table is int32 [batch, max_pages_per_seq]:
 *     entry [b][n] is the physical page holding tokens [n*P, (n+1)*P) of
 *     sequence b.  Token t of sequence b is slot t % P of page
 *     block_table[b][t / P].
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Every call only enqueues work on it: no host sync.
 *   - Errors: calls return pa_status and never abort.  Arguments the host can
 *     check are checked before any work is enqueued (PA_ERR_INVALID_ARG,
 *     PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE); a failed launch returns
 *     PA_ERR_HIP.  Device-resident integers (block-table entries, lengths,
 *     prefix sums) are not validated in release builds: out-of-range values
 *     are undefined behaviour.  A debug build (pa_device_checks() == 1)
 *     checks each of them on the device against the range the entry point
 *     documents, keeps every access inside the caller's buffers, waits for
 *     its kernels at the end of each call and returns PA_ERR_DEVICE_ASSERT
 *     for the first violation (what, which sequence, value and range in
 *     pa_last_error_detail(); the outputs are then undefined).
 *     pa_last_error_detail() gives a message for the last failure on the
 *     calling thread.
 *   - Thread safety: no global mutable state apart from a per-thread error
 *     string and a once-initialised device-property cache.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad scale, ...      */
  PA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, page_size, dtype  */
  PA_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed        */
  PA_ERR_WORKSPACE = 4,   /* decode workspace missing or too small             */
  PA_ERR_OUT_OF_PAGES = 5, /* a page pool has too few free pages (no change)   */
  PA_ERR_DEVICE_ASSERT = 6 /* debug builds: a device-side range check failed   */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,  /* float32 K/V pages, float32 queries and outputs                */
  PA_BF16 = 1, /* bfloat16 K/V pages, bfloat16 queries and outputs              */
  PA_I8 = 2    /* int8 K/V codes with fp32 scales; bfloat16 queries and outputs */
} pa_dtype;

/* A paged KV cache.  The struct itself is read on the host during the call
 * only; the pointers inside are device pointers owned by the caller.
 *   k_pages, v_pages : [num_pages, page_size, num_kv_heads, head_dim] of dtype
 *   k_scales, v_scales: PA_I8 only, fp32 [num_pages, num_kv_heads]; the value
 *                       of code c in page n, head g is c * scales[n][g]
 *                       (NULL for other dtypes)
 *   page_size        : a power of two in [16, 256]
 *   head_dim         : 64 or 128                                              */
typedef struct pa_kv_cache {
  void *k_pages;
  void *v_pages;
  float *k_scales;
  float *v_scales;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* a pa_dtype */
} pa_kv_cache;

/* kv_cache_append - write new K/V rows into their page slots.
 * Source: the KV-cache growth step ("KV Cache" section of the 3x-faster page:
 * the cache grows by appending the new tokens' K/V) through the page table
 * (section 3.2 of the Flash Attention + Paged KV Cache page).
 *   k_new, v_new : [cu_new[batch], num_kv_heads, head_dim], cache dtype
 *                  (bfloat16 rows for a PA_I8 cache)
 *   block_table  : int32 [batch, max_pages_per_seq]; pages must already be
 *                  assigned for every written position
 *   start_pos    : int32 [batch], length of sequence b before this append
 *   cu_new       : int32 [batch + 1], prefix sums of new-token counts
 *   max_new      : host int, an upper bound on cu_new[b+1] - cu_new[b]
 * Row r of sequence b lands at position start_pos[b] + r.  A bit copy for
 * PA_F32 / PA_BF16 caches.  For a PA_I8 cache (k_scales, v_scales needed)
 * each (page, KV head) group that receives rows is requantised with the
 * group quantiser of section 3.2 of the KV-cache management page over its
 * valid slots (positions before the sequence's new end; old slots entering
 * as code * old scale): scale = largest magnitude / 127 (1 if 0), code =
 * round-half-even(clamp(value / scale, -128, 127)), in float32.  A whole
 * page appended at once into an empty page gets exactly the codes of
 * kv_pages_quantize_int8.  Pages shared with another sequence must not be
 * appended to (the caller copies them first).  Errors: PA_ERR_INVALID_ARG
 * for NULL pointers, negative sizes or an int8 cache without scales. */
pa_status kv_cache_append(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                          const int32_t *block_table, int32_t max_pages_per_seq,
                          const int32_t *start_pos, const int32_t *cu_new, int32_t batch,
                          int32_t max_new, void *stream);

/* kv_pages_quantize_int8 - symmetric abs-max int8 quantisation of whole pages.
 * Source: section 3.2 (group quantisation) of the KV-cache management page,
 * with bits = 8 and one group per (physical page, KV head): P x D values.
 *   src     : bf16 [num_pages, page_size, num_kv_heads, head_dim]
 *   codes   : int8, same shape (output)
 *   scales  : fp32 [num_pages, num_kv_heads] (output)
 * scale = absmax / 127 in fp32 (1 when absmax is 0); code =
 * round-half-even(clamp(x / scale, -128, 127)), divisions in IEEE fp32.
 * Call once per pool (K and V separately). */
pa_status kv_pages_quantize_int8(const void *src, int8_t *codes, float *scales, int32_t num_pages,
                                 int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                 void *stream);

/* attn_prefill_paged - causal (optionally windowed) attention of ragged query
 * rows against the paged cache, FlashAttention-style (tiles + online
 * softmax).  Sources: section 2.1 of the KV Cache + FlashAttention page
 * (definition), its section 5.1 (scale, causal, window), section 2.1 of the
 * Flash Attention + Paged KV Cache page (tiling), the online-softmax section
 * of the 3x-faster page, section 2.1 of the KV-cache management page (GQA).
 *   q          : [cu_q[batch], num_q_heads, head_dim]; bf16 for PA_BF16
 *                caches, fp32 for PA_F32 caches (PA_I8: unsupported)
 *   cu_q       : int32 [batch + 1], prefix sums of query counts
 *   ctx_lens   : int32 [batch], keys of sequence b INCLUDING its queries;
 *                query row i of sequence b sits at position
 *                ctx_lens[b] - q_len_b + i (bottom-right alignment)
 *   max_q_len  : host int, upper bound on q_len_b (sizes the grid)
 *   softmax_scale: > 0 and finite (callers pass 1/sqrt(head_dim) by default)
 *   causal     : 0 or 1
 *   window_left: < 0 for no window; else key j is visible to the query at
 *                position p only if p - j <= window_left
 *   out        : [cu_q[batch], num_q_heads, head_dim], dtype of q
 *   lse        : fp32 [cu_q[batch], num_q_heads] natural-log log-sum-exp of the
 *                scaled scores, or NULL
 * num_q_heads must be a multiple of cache->num_kv_heads.
 * Arithmetic: bf16 caches on bf16 MFMA (P rounded to bf16 as the P.V
 * operand), fp32 caches on fp32 MFMA; accumulation and softmax in fp32. */
pa_status attn_prefill_paged(const void *q, const int32_t *cu_q, const pa_kv_cache *cache,
                             const int32_t *block_table, int32_t max_pages_per_seq,
                             const int32_t *ctx_lens, int32_t batch, int32_t max_q_len,
                             int32_t num_q_heads, float softmax_scale, int32_t causal,
                             int32_t window_left, void *out, float *lse, void *stream);

/* attn_prefill_paged_append - kv_cache_append of the queries' own K/V rows
 * followed by attn_prefill_paged over the grown context, in one pass: the
 * prompt step of "大模型推理优化实战：KV Cache + Flash Attention" (KV Cache
 * section: the new tokens' keys and values join the cache, then the queries
 * attend over everything cached), with the paging of section 3.2 of the
 * Flash Attention + Paged KV Cache page.  The result (out, lse and the page
 * contents) is the same as calling kv_cache_append(cache, k_new, v_new,
 * block_table, max_pages_per_seq, start_pos, cu_q, batch, max_q_len) with
 * start_pos[b] = ctx_lens[b] - q_len_b and then attn_prefill_paged with the
 * remaining arguments.
 *   k_new, v_new : [cu_q[batch], num_kv_heads, head_dim], cache element type
 *                (bf16 or fp32); row cu_q[b] + i is the key / value at
 *                position ctx_lens[b] - q_len_b + i (the position of query
 *                row i)
 *   all other arguments: as attn_prefill_paged
 * bf16 caches with page_size >= 64 run, at the lengths where it is faster
 * (attn_prefill_append_is_fused), as one kernel that reads the new keys
 * from k_new / v_new and writes them into their page slots; otherwise the
 * append kernel and then the prefill run on the same stream.  The slots of the new positions must not be read by
 * another sequence of the same call (they are written during it).  int8
 * caches: PA_ERR_UNSUPPORTED (as for attn_prefill_paged). */
pa_status attn_prefill_paged_append(const void *q, const void *k_new, const void *v_new,
                                    const int32_t *cu_q, const pa_kv_cache *cache,
                                    const int32_t *block_table, int32_t max_pages_per_seq,
                                    const int32_t *ctx_lens, int32_t batch, int32_t max_q_len,
                                    int32_t num_q_heads, float softmax_scale, int32_t causal,
                                    int32_t window_left, void *out, float *lse, void *stream);

/* attn_prefill_append_is_fused - HOST function: 1 if attn_prefill_paged_append
 * with this cache and these arguments runs as one fused kernel, 0 if it runs
 * the append kernel and then the prefill (same result either way).  The
 * fused kernel needs a bf16 cache with page_size >= 64; beyond that the
 * choice follows measured times (causal without a window: up to 6144 query
 * rows; a window or no mask: always), and the environment variable
 * PAGEDATTN_PREFILL_APPEND_ROUTE=fused or =separate overrides it.  NULL cache: 0. */
int32_t attn_prefill_append_is_fused(const pa_kv_cache *cache, int32_t causal, int32_t window_left,
                                     int32_t max_q_len);

/* attn_decode_workspace_bytes - HOST function: bytes of workspace that
 * attn_decode_paged needs for these sizes (an upper bound; 0 on bad input). */
size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_pages_per_seq, int32_t page_size);

/* attn_decode_paged - one query token per sequence against its whole paged
 * context, split over the context (split-K) and merged by a second kernel.
 * Sources: as attn_prefill_paged, with q_len = 1; the split merge uses the
 * same running-max / running-sum rescaling as the online softmax.
 *   q        : [batch, num_q_heads, head_dim]; fp32 for PA_F32, else bf16
 *   ctx_lens : int32 [batch] keys per sequence INCLUDING the new token (>= 1;
 *              a sequence with 0 keys gets O = 0 and lse = -inf)
 *   window_left: as for prefill (the query sits at position ctx_lens[b] - 1)
 *   out      : [batch, num_q_heads, head_dim], dtype of q
 *   lse      : fp32 [batch, num_q_heads] or NULL
 *   workspace: device scratch of at least attn_decode_workspace_bytes(...)
 *              bytes for the same sizes; its contents are undefined after
 *              the call; calls that share a workspace on different streams
 *              race. */
pa_status attn_decode_paged(const void *q, const pa_kv_cache *cache, const int32_t *block_table,
                            int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch,
                            int32_t num_q_heads, float softmax_scale, int32_t window_left, void *out,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* attn_decode_paged_noalloc - attn_decode_paged without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * split partials go to a scratch array the library holds on each GPU
 * (PA_NOALLOC_SCRATCH_BYTES, reserved from the first use of the library on
 * that GPU until the process ends); the call allocates nothing.  Arguments,
 * result and errors are those of attn_decode_paged, plus PA_ERR_WORKSPACE
 * when attn_decode_workspace_bytes(...) of these sizes exceeds
 * PA_NOALLOC_SCRATCH_BYTES.  Every call on one GPU shares that GPU's array
 * (which keeps the last call's contents; nothing in it needs to start at
 * zero): calls that overlap on one GPU, from several streams or threads,
 * race and must be serialised by the caller. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status attn_decode_paged_noalloc(const void *q, const pa_kv_cache *cache, const int32_t *block_table,
                                    int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch,
                                    int32_t num_q_heads, float softmax_scale, int32_t window_left, void *out,
                                    float *lse, void *stream);

/* attn_decode_layered_workspace_bytes - HOST function: workspace bytes that
 * attn_decode_paged_layered needs for these sizes (0 on bad input). */
size_t attn_decode_layered_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim);

/* attn_decode_paged_layered - single-token decode over a context held in two
 * caches: the first len_hi[b] positions of sequence b in cache_hi (through
 * block_table_hi) and the next len_lo[b] positions in cache_lo (through
 * block_table_lo).  This is the layered cache of "大模型推理优化：KV Cache与
 * FlashAttention实战" section 2.2: the first tokens of a sequence (128
 * there) kept at full precision, later ones int8 with group scales
 * ("LLM推理系统优化：KV缓存管理与动态批处理技术" section 3.2).  The result is exactly the attention of the query over all
 * len_hi[b] + len_lo[b] keys (no mask: the query is the last position).
 *   q, out, lse : as attn_decode_paged
 *   cache_hi, cache_lo : bf16 or int8 caches (with scales), same
 *              num_kv_heads and head_dim; page sizes may differ
 *   len_hi, len_lo : int32 [batch] device arrays, >= 0 each (a sequence
 *              with no keys at all gets O = 0, lse = -inf)
 *   workspace: at least attn_decode_layered_workspace_bytes(...) bytes;
 *              contents undefined after the call
 * Errors: PA_ERR_UNSUPPORTED for an fp32 cache or more than 16 query heads
 * per KV head, PA_ERR_INVALID_ARG for mismatched caches, NULL pointers or
 * bad sizes, PA_ERR_WORKSPACE when the workspace is missing or too small. */
pa_status attn_decode_paged_layered(const void *q, const pa_kv_cache *cache_hi, const int32_t *block_table_hi,
                                    int32_t max_pages_hi, const int32_t *len_hi, const pa_kv_cache *cache_lo,
                                    const int32_t *block_table_lo, int32_t max_pages_lo, const int32_t *len_lo,
                                    int32_t batch, int32_t num_q_heads, float softmax_scale, void *out,
                                    float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* attn_backward_workspace_bytes - HOST function: workspace bytes of
 * attn_backward_paged (total_q * num_q_heads floats; 0 on bad input). */
size_t attn_backward_workspace_bytes(int32_t total_q, int32_t num_q_heads);

/* attn_backward_paged - gradients of attn_prefill_paged's output with
 * respect to q and to the cached K and V, from the forward's out and lse.
 * Source: recomputation in the backward pass ("大模型推理优化：KV Cache与
 * FlashAttention实战" section 3.1; "Flash Attention与Paged KV Cache优化大模型
 * 计算效率" section 2.1): the probabilities are rebuilt from q, K and lse
 * instead of being stored, and differentiated through softmax and the two
 * products.  Same arguments, masks and GQA map as attn_prefill_paged, plus:
 *   total_q, max_ctx : host ints, cu_q[batch] and max over b of ctx_lens[b]
 *   out, lse         : the forward output and log-sum-exp (natural log)
 *   d_out            : [total_q, num_q_heads, head_dim] upstream gradient
 *   q, out, d_out    : bf16 for a PA_BF16 cache, fp32 for PA_F32
 *   dq               : fp32 [total_q, num_q_heads, head_dim]
 *   dk_pages, dv_pages: fp32 [num_pages, page_size, num_kv_heads, head_dim];
 *                      the slot of every cached position 0..ctx_lens[b]-1 of
 *                      every sequence is written (gradients of the GQA
 *                      group's query heads summed), other slots untouched.
 *                      Sequences must not share physical pages here.
 *   workspace        : at least attn_backward_workspace_bytes(...) bytes
 * Arithmetic: bf16 caches run every product on bf16 MFMA with fp32
 * accumulation (P and dS rounded to bf16 as operands); fp32 caches run in
 * fp32 on the vector ALUs.  PA_ERR_UNSUPPORTED for an int8 cache. */
pa_status attn_backward_paged(const void *q, const int32_t *cu_q, const pa_kv_cache *cache, const int32_t *block_table,
                              int32_t max_pages_per_seq, const int32_t *ctx_lens, int32_t batch, int32_t total_q,
                              int32_t max_q_len, int32_t max_ctx, int32_t num_q_heads, float softmax_scale,
                              int32_t causal, int32_t window_left, const void *out, const float *lse,
                              const void *d_out, float *dq, float *dk_pages, float *dv_pages, void *workspace,
                              size_t workspace_bytes, void *stream);

/* kv_cache_copy_pages - copy whole pages src_pages[i] -> dst_pages[i]
 * (K, V and, for PA_I8, the pages' scales): the device half of a page pool's
 * copy-on-write (below).
 *   src_pages, dst_pages : int32 [n] device arrays of physical page ids
 *                          (not validated; dst pages must not be src pages)
 *   n                    : host int, 0 <= n <= 65535 */
pa_status kv_cache_copy_pages(const pa_kv_cache *cache, const int32_t *src_pages, const int32_t *dst_pages,
                              int32_t n, void *stream);

/* Page pool - HOST bookkeeping of a cache's physical pages: which pages each
 * sequence holds (its block-table row) and how many sequences hold each
 * page.  Sources: the page table of "Flash Attention与Paged KV Cache优化大模型
 * 计算效率" section 3.2 (allocate a page per logical page; releasing a
 * sequence also clears its table entries, that page's section 5), and the
 * shared prompt pages with reference counts of "大模型推理优化：KV Cache与
 * FlashAttention实战" section 4.1 and "LLM推理系统优化：KV缓存管理与动态批处理
 * 技术" section 3.1.  Free pages are taken lowest id first.  Every function
 * below runs on the host only, touches no device memory and serialises
 * calls on one pool with a lock; the caller uploads the exported table. */
typedef struct pa_page_pool pa_page_pool;

/* Pool of num_pages pages of page_size tokens for sequences 0..max_seqs-1 of
 * at most max_pages_per_seq pages each; *pool receives the handle. */
pa_status pa_pool_create(int32_t num_pages, int32_t page_size, int32_t max_seqs, int32_t max_pages_per_seq,
                         pa_page_pool **pool);
void pa_pool_destroy(pa_page_pool *pool);

/* Grow sequence seq to new_len tokens (before its rows [len, new_len) are
 * appended), taking fresh pages as needed.  If the page that receives
 * position len is partly filled and held by other sequences too, seq gets a
 * fresh page in its place and the pair (shared page, fresh page) is written
 * to copy_src[0] / copy_dst[0] with *n_copies = 1: copy it on the device
 * (kv_cache_copy_pages) before appending.  PA_ERR_OUT_OF_PAGES leaves the
 * pool unchanged. */
pa_status pa_pool_extend(pa_page_pool *pool, int32_t seq, int32_t new_len, int32_t *copy_src, int32_t *copy_dst,
                         int32_t copy_cap, int32_t *n_copies);

/* Let the empty sequence child share the pages that hold the first n_tokens
 * (1 <= n_tokens <= parent length) of parent: a shared prompt. */
pa_status pa_pool_fork(pa_page_pool *pool, int32_t parent, int32_t child, int32_t n_tokens);

/* Drop seq's hold on its pages (a page is free once no sequence holds it)
 * and clear its table row (entries -1, length 0). */
pa_status pa_pool_release(pa_page_pool *pool, int32_t seq);

/* Copy the block table, int32 [max_seqs, max_pages_per_seq] (-1 unused),
 * and/or the lengths, int32 [max_seqs], into HOST buffers (NULL skips). */
pa_status pa_pool_export(pa_page_pool *pool, int32_t *block_table, int32_t *lens);

/* Free pages, and the number of sequences holding a page (-1 on bad input). */
int32_t pa_pool_free_pages(pa_page_pool *pool);
int32_t pa_pool_refcount(pa_page_pool *pool, int32_t page);

/* Static description of a status code (a pa_status value, passed as an int
 * so that any value is well defined; others give "unknown status"). */
const char *pa_status_string(int32_t status);

/* Message of the last failure on the calling thread ("" if none). */
const char *pa_last_error_detail(void);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

/* 1 for a debug build with device-side checks of block-table entries,
 * lengths and prefix sums (synchronous calls, PA_ERR_DEVICE_ASSERT), 0 for
 * a release build. */
int32_t pa_device_checks(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
