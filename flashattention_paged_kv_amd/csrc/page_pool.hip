// Host page pool and the device page copy it asks for.
//
// The cache is cut into fixed-size physical pages; each sequence owns a row
// of the page table mapping its logical pages to physical ones ("Flash
// Attention与Paged KV Cache优化大模型计算效率" section 3.2); releasing a
// sequence must also clear its table entries (that page's section 5: pages
// freed without clearing their table entries leaked memory).  Requests with
// the same prompt share its KV pages, with reference counts deciding when a
// page is free again ("大模型推理优化：KV Cache与FlashAttention实战" section 4.1,
// zero-copy sharing; "LLM推理系统优化：KV缓存管理与动态批处理技术" section 3.1,
// shared system-prompt blocks).
//
// A sequence about to write into a page that other sequences also hold
// (only possible for a partly filled last page) first gets a private copy of
// it: the pool swaps in a fresh page and reports the (old, new) pair, and
// the caller copies that page on the device before appending.
//
// Free pages are handed out lowest id first, so a sequence of calls always
// produces the same tables.
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "../../include/pagedattn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
pa_status report(pa_status st, const char *msg);
}  // namespace pa

struct pa_page_pool {
  int32_t num_pages;
  int32_t page_size;
  int32_t max_seqs;
  int32_t max_pages;
  std::vector<int32_t> refcount;  // [num_pages]
  std::set<int32_t> free_pages;   // ids with refcount 0
  std::vector<int32_t> table;     // [max_seqs * max_pages], -1 unused
  std::vector<int32_t> lens;      // [max_seqs] tokens
  std::mutex mu;

  int32_t pages_of(int32_t n_tokens) const { return (n_tokens + page_size - 1) / page_size; }
  int32_t *row(int32_t seq) { return table.data() + (size_t)seq * max_pages; }
  int32_t take_lowest() {
    const int32_t p = *free_pages.begin();
    free_pages.erase(free_pages.begin());
    refcount[p] = 1;
    return p;
  }
  void drop(int32_t p) {
    if (--refcount[p] == 0) free_pages.insert(p);
  }
};

namespace {

pa_status bad(const char *msg) { return pa::report(PA_ERR_INVALID_ARG, msg); }

pa_status check_seq(const pa_page_pool *pool, int32_t seq) {
  if (pool == nullptr) return bad("pool is NULL");
  if (seq < 0 || seq >= pool->max_seqs) return bad("sequence index out of range");
  return PA_OK;
}

// One workgroup copies a slice of one page pair: K and V rows as 16-byte
// chunks, and (int8 caches) the page's per-head scales.
__global__ __launch_bounds__(256) void copy_pages_kernel(uint4 *k, uint4 *v, float *k_scales, float *v_scales,
                                                         int num_kv_heads, const int32_t *src_pages,
                                                         const int32_t *dst_pages, size_t page_chunks,
                                                         int num_pages) {
  const int i = blockIdx.y;
  const int sp = pa::checked(src_pages[i], 0, num_pages - 1, pa::kSitePageId, i);
  const int dp = pa::checked(dst_pages[i], 0, num_pages - 1, pa::kSitePageId, i);
  const size_t src = (size_t)sp * page_chunks;
  const size_t dst = (size_t)dp * page_chunks;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < page_chunks; e += (size_t)gridDim.x * blockDim.x) {
    k[dst + e] = k[src + e];
    v[dst + e] = v[src + e];
  }
  if (k_scales != nullptr && blockIdx.x == 0 && (int)threadIdx.x < num_kv_heads) {
    const size_t h = threadIdx.x;
    k_scales[(size_t)dp * num_kv_heads + h] = k_scales[(size_t)sp * num_kv_heads + h];
    v_scales[(size_t)dp * num_kv_heads + h] = v_scales[(size_t)sp * num_kv_heads + h];
  }
}

}  // namespace

namespace pa {

PA_DEFINE_FAULT_READER(take_fault_page_pool)

hipError_t launch_copy_pages(void *k, void *v, float *k_scales, float *v_scales, int num_kv_heads,
                             const int32_t *src, const int32_t *dst, int n, size_t page_bytes, int num_pages,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t chunks = page_bytes / 16;
  const int gx = (int)((chunks + 255) / 256 < 16 ? (chunks + 255) / 256 : 16);
  hipLaunchKernelGGL(copy_pages_kernel, dim3(gx, n), dim3(256), 0, s, (uint4 *)k, (uint4 *)v, k_scales, v_scales,
                     num_kv_heads, src, dst, chunks, num_pages);
  return hipGetLastError();
}

}  // namespace pa

extern "C" {

pa_status pa_pool_create(int32_t num_pages, int32_t page_size, int32_t max_seqs, int32_t max_pages_per_seq,
                         pa_page_pool **pool) {
  if (pool == nullptr) return bad("pool is NULL");
  *pool = nullptr;
  if (num_pages <= 0 || page_size <= 0 || max_seqs <= 0 || max_pages_per_seq <= 0)
    return bad("num_pages, page_size, max_seqs and max_pages_per_seq must be > 0");
  pa_page_pool *p = new (std::nothrow) pa_page_pool();
  if (p == nullptr) return pa::report(PA_ERR_INVALID_ARG, "out of host memory");
  p->num_pages = num_pages;
  p->page_size = page_size;
  p->max_seqs = max_seqs;
  p->max_pages = max_pages_per_seq;
  p->refcount.assign(num_pages, 0);
  for (int32_t i = 0; i < num_pages; ++i) p->free_pages.insert(p->free_pages.end(), i);
  p->table.assign((size_t)max_seqs * max_pages_per_seq, -1);
  p->lens.assign(max_seqs, 0);
  *pool = p;
  return pa::report(PA_OK, "");
}

void pa_pool_destroy(pa_page_pool *pool) { delete pool; }

pa_status pa_pool_extend(pa_page_pool *pool, int32_t seq, int32_t new_len, int32_t *copy_src, int32_t *copy_dst,
                         int32_t copy_cap, int32_t *n_copies) {
  pa_status st = check_seq(pool, seq);
  if (st != PA_OK) return st;
  if (n_copies == nullptr) return bad("n_copies is NULL");
  std::lock_guard<std::mutex> lock(pool->mu);
  *n_copies = 0;
  const int32_t len = pool->lens[seq];
  if (new_len < len) return bad("new_len is below the sequence's length");
  const int32_t have = pool->pages_of(len);
  const int32_t need = pool->pages_of(new_len);
  if (need > pool->max_pages) return bad("new_len needs more pages than max_pages_per_seq");
  int32_t *row = pool->row(seq);
  const bool cow = new_len > len && len % pool->page_size != 0 && pool->refcount[row[have - 1]] > 1;
  if (cow && (copy_src == nullptr || copy_dst == nullptr || copy_cap < 1))
    return bad("a shared page must be copied: copy_src / copy_dst with room for one pair are needed");
  const size_t fresh = (size_t)(need - have) + (cow ? 1 : 0);
  if (fresh > pool->free_pages.size()) return pa::report(PA_ERR_OUT_OF_PAGES, "not enough free pages");
  if (cow) {
    const int32_t old = row[have - 1];
    const int32_t mine = pool->take_lowest();
    pool->drop(old);
    row[have - 1] = mine;
    copy_src[0] = old;
    copy_dst[0] = mine;
    *n_copies = 1;
  }
  for (int32_t i = have; i < need; ++i) row[i] = pool->take_lowest();
  pool->lens[seq] = new_len;
  return pa::report(PA_OK, "");
}

pa_status pa_pool_fork(pa_page_pool *pool, int32_t parent, int32_t child, int32_t n_tokens) {
  pa_status st = check_seq(pool, parent);
  if (st != PA_OK) return st;
  if ((st = check_seq(pool, child)) != PA_OK) return st;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (parent == child) return bad("parent and child must differ");
  if (pool->lens[child] != 0) return bad("the child sequence must be empty");
  if (n_tokens <= 0 || n_tokens > pool->lens[parent]) return bad("n_tokens must be in [1, parent length]");
  const int32_t n = pool->pages_of(n_tokens);
  const int32_t *from = pool->row(parent);
  int32_t *to = pool->row(child);
  for (int32_t i = 0; i < n; ++i) {
    to[i] = from[i];
    ++pool->refcount[from[i]];
  }
  pool->lens[child] = n_tokens;
  return pa::report(PA_OK, "");
}

pa_status pa_pool_release(pa_page_pool *pool, int32_t seq) {
  pa_status st = check_seq(pool, seq);
  if (st != PA_OK) return st;
  std::lock_guard<std::mutex> lock(pool->mu);
  int32_t *row = pool->row(seq);
  const int32_t n = pool->pages_of(pool->lens[seq]);
  for (int32_t i = 0; i < n; ++i) {
    pool->drop(row[i]);
    row[i] = -1;
  }
  pool->lens[seq] = 0;
  return pa::report(PA_OK, "");
}

pa_status pa_pool_export(pa_page_pool *pool, int32_t *block_table, int32_t *lens) {
  if (pool == nullptr) return bad("pool is NULL");
  if (block_table == nullptr && lens == nullptr) return bad("nothing to export into");
  std::lock_guard<std::mutex> lock(pool->mu);
  if (block_table != nullptr)
    for (size_t i = 0; i < pool->table.size(); ++i) block_table[i] = pool->table[i];
  if (lens != nullptr)
    for (int32_t i = 0; i < pool->max_seqs; ++i) lens[i] = pool->lens[i];
  return pa::report(PA_OK, "");
}

int32_t pa_pool_free_pages(pa_page_pool *pool) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return (int32_t)pool->free_pages.size();
}

int32_t pa_pool_refcount(pa_page_pool *pool, int32_t page) {
  if (pool == nullptr || page < 0 || page >= pool->num_pages) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return pool->refcount[page];
}

}  // extern "C"
