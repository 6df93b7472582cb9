// Host-side argument bundles and kernel launchers shared by the library's
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Debug builds (PA_DEVICE_CHECKS=1) check, on the device, every
// device-resident integer a kernel reads against the range its entry point
// documents; the first violation in a source file is kept in that file's
// fault record, which the host reads after the launch.  Release builds
// compile the checks away.
#ifndef PA_DEVICE_CHECKS
#define PA_DEVICE_CHECKS 0
#endif

// What was out of range.
enum CheckSite : int {
  kSiteNone = 0,
  kSitePageId = 1,     // a block-table entry (or a page id to copy) outside [0, num_pages)
  kSiteCtxLen = 2,     // a context length outside [q_len, max_pages_per_seq * page_size]
  kSiteQueryLen = 3,   // a query count (prefix-sum difference) outside [0, max_q_len]
  kSiteNewLen = 4,     // a new-row count outside [0, max_new]
  kSiteStartPos = 5,   // an append's first position outside [0, max_pages_per_seq * page_size - rows]
  kSiteRowOffset = 6,  // a prefix sum (first row of a sequence) below 0
};

struct DeviceFault {
  int flag;   // 0: nothing recorded
  int site;   // a CheckSite
  int value;  // the value read
  int lo, hi; // the range it had to lie in
  int batch;  // the sequence (or page pair) it belongs to
};

// A paged cache as the kernels see it.
struct CacheView {
  const void *k;
  const void *v;
  const float *k_scales;
  const float *v_scales;
  int num_pages;
  int page_size;
  int log2_page;
  int num_kv_heads;
  int head_dim;
  int dtype;  // pa_dtype
};

struct AppendArgs {
  void *k_pages;
  void *v_pages;
  const void *k_new;
  const void *v_new;
  const int32_t *block_table;
  int max_pages;
  const int32_t *start_pos;  // NULL: start = ctx_lens[b] - (new rows of b)
  const int32_t *ctx_lens;   // used only when start_pos is NULL
  const int32_t *cu_new;
  int batch;
  int max_new;
  int page_size;
  int log2_page;
  int row_bytes;  // num_kv_heads * head_dim * element size
  int num_pages;  // pages of the pools (device checks only)
};

// Append into an int8 cache: bf16 rows in, codes and scales requantised
// per touched (page, KV head) group.
struct AppendI8Args {
  int8_t *k_codes;
  int8_t *v_codes;
  float *k_scales;
  float *v_scales;
  const uint16_t *k_new;  // bf16 bits [total_new, num_kv_heads, head_dim]
  const uint16_t *v_new;
  const int32_t *block_table;
  int max_pages;
  const int32_t *start_pos;
  const int32_t *cu_new;
  int batch;
  int max_new;
  int page_size;
  int log2_page;
  int num_kv_heads;
  int head_dim;
  int num_pages;  // pages of the pools (device checks only)
};

struct QuantArgs {
  const uint16_t *src;
  int8_t *codes;
  float *scales;
  int num_pages;
  int page_size;
  int num_kv_heads;
  int head_dim;
};

struct PrefillArgs {
  const void *q;
  const int32_t *cu_q;
  CacheView c;
  const int32_t *block_table;
  int max_pages;
  const int32_t *ctx_lens;
  int batch;
  int max_q_len;
  int num_q_heads;
  int group;           // num_q_heads / num_kv_heads
  float scale_log2;    // softmax_scale * log2(e)
  int causal;
  int window_left;
  void *out;
  float *lse;
  // Fused append (bf16 caches with page_size >= 64): the K/V rows of the
  // queries themselves, [cu_q[batch], num_kv_heads, head_dim], positions
  // ctx_lens[b] - q_len_b + i.  The kernel reads these keys from here and
  // writes them into their page slots (c.k / c.v).  NULL: no append.
  const void *k_new;
  const void *v_new;
  int run_tiles;  // set by the launcher: query tiles per run-mode workgroup
};

struct DecodeArgs {
  const void *q;
  CacheView c;
  const int32_t *block_table;
  int max_pages;
  const int32_t *ctx_lens;
  int batch;
  int num_q_heads;
  int group;
  float scale_log2;
  int window_left;
  void *out;
  float *lse;
  float *ws_o;         // [slots, G, head_dim] partial outputs (unnormalised)
  float *ws_ml;        // [slots, G, 2] partial (max in log2 units, sum)
  int32_t *ws_prefix;  // [batch + 1] tiles per KV head before sequence b; total last
  int nwg;             // workgroups launched
  int hpw;             // KV heads per split workgroup; slots = batch * Hkv / hpw + nwg, hpw heads each
};

// Backward pass: gradients of the attention of ragged query rows against a
// paged cache (bf16 or fp32), fp32 outputs.
struct BackwardArgs {
  const void *q;             // [total_q, num_q_heads, head_dim], cache element type
  const int32_t *cu_q;
  CacheView c;
  const int32_t *block_table;
  int max_pages;
  const int32_t *ctx_lens;
  int batch;
  int max_q_len;
  int max_ctx;
  int total_q;
  int num_q_heads;
  int group;
  float scale;
  float scale_log2;
  int causal;
  int window_left;
  const void *out;           // forward output O, like q
  const float *lse;          // forward log-sum-exp (natural log) [total_q, num_q_heads]
  const void *d_out;         // upstream gradient dO, like q
  float *dq;                 // [total_q, num_q_heads, head_dim]
  float *dk;                 // [num_pages, page_size, num_kv_heads, head_dim]
  float *dv;
  float *delta;              // workspace [total_q, num_q_heads]: dO . O
};

// Compute units of the current device (256 on an MI355X; also the answer
// when no device can be queried), cached per device.
int device_cu_count();
// Decode grid size (workgroups) on the current device, used by both the
// workspace query and the call.
int decode_grid_size();
// KV heads a decode split workgroup handles together: the largest power of
// two <= 8 that divides hkv (its waves then read whole contiguous rows of
// those heads).
inline int decode_heads_per_wg(int hkv) {
  int h = 8;
  while (hkv % h != 0) h >>= 1;
  return h;
}

// Decode scratch held by the library itself (a device array per GPU, for
// the entry point that allocates nothing): its size, and its address on the
// current device (taken once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_quantize(const QuantArgs &a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
// Two split launches over disjoint key sets of the same sequences (the
// caches may differ in dtype and page size), then one merge of both.
hipError_t launch_decode_layered(const DecodeArgs &a, const DecodeArgs &a2, hipStream_t s);
hipError_t launch_append_i8(const AppendI8Args &a, hipStream_t s);
hipError_t launch_backward(const BackwardArgs &a, hipStream_t s);
// Copy whole pages src[i] -> dst[i] (K, V and, when given, their scales).
hipError_t launch_copy_pages(void *k, void *v, float *k_scales, float *v_scales, int num_kv_heads,
                             const int32_t *src, const int32_t *dst, int n, size_t page_bytes, int num_pages,
                             hipStream_t s);

#if PA_DEVICE_CHECKS
// Each kernel source file's fault record: copied to *f and cleared (if a
// fault was recorded).  Call after the launches have completed.
hipError_t take_fault_append(DeviceFault *f);
hipError_t take_fault_prefill(DeviceFault *f);
hipError_t take_fault_decode(DeviceFault *f);
hipError_t take_fault_backward(DeviceFault *f);
hipError_t take_fault_page_pool(DeviceFault *f);
#endif

}  // namespace pa
