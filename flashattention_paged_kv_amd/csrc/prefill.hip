// Causal / sliding-window prefill over a paged KV cache, bf16 on MFMA.
//
// Method: the attention definition of "大模型推理优化：KV Cache与FlashAttention
// 实战" section 2.1 (query at position p sees keys 0..p) with the scale /
// causal / window arguments of its section 5.1; computed tile by tile as in
// "Flash Attention与Paged KV Cache优化大模型计算效率" section 2.1 (Q/K/V blocks
// kept on chip) with the online softmax of "大模型推理优化实战：KV Cache + Flash
// Attention" (Flash Attention section: running max m, running sum l, rescale
// by exp(m - m_new), divide by l once at the end); K/V are read from pages
// through the block table (section 3.2 of the Flash Attention + Paged KV page),
// query head h reading KV head h / G ("LLM推理系统优化：KV缓存管理与动态批处理
// 技术" section 2.1).
//
// Work split.  Query rows are cut into 128-row tiles; a tile's work is the
// list of 64-key tiles it can see.  Under a causal mask without a window, one
// workgroup of 8 waves takes the pair of query tiles (p, n-1-p) of one
// (sequence, query head): their key-tile counts add up to the same total for
// every p, so all workgroups carry equal work.  With a window or without a
// mask every query tile has about the same work, and a workgroup takes a run
// of consecutive query tiles instead (up to 8: fewer, longer workgroups,
// while the grid keeps one per CU).  The
// workgroup is two engines of 4 waves that each take half of the pair's key
// tiles: engine 0 all of the earlier tile and the top of the later one,
// engine 1 the bottom of the later one, both ascending, so that the two
// engines read the same key tile at the same step while both are in the
// shared prefix.  The query tile split between them is merged in LDS at the
// end with the same rescaling algebra as the online softmax, each engine
// merging and storing half of the head dimensions.  Each engine has its own
// double-buffered K/V tiles in LDS and loads the next key tile into
// registers a whole step ahead; its first query tile's Q arrives with its
// first K/V tile, staged in the free LDS buffer.  Workgroup
// ids are remapped so that the pairs of one query head run on the same XCD
// (shared L2) and stream its K/V tiles together.
//
// Per key tile a wave (32 query rows) runs a GEMM phase and a softmax phase,
// each ended by a workgroup barrier, with engine 1 one phase behind engine
// 0 so that on every SIMD one wave's softmax (VALU) overlaps the other
// wave's MFMAs.  The GEMM phase computes O^T += V^T . P^T of the previous
// tile (V^T read transposed from LDS by ds_read_b64_tr_b16, P^T from
// registers) and S^T = K . Q^T of this tile, both with
// v_mfma_f32_32x32x16_bf16 (keys on M, the wave's rows on N, Q^T in
// registers).  The softmax phase applies the mask and the online softmax on
// the S^T registers (one query per lane column) and rounds P^T to bf16.
// exp is exp2 with log2(e) folded into the scale.  The exponent reference
// of a row (m) is a maximum the row had earlier and may lag its true
// maximum: a tile's probabilities are first taken against it, and only if
// some lane's partial row sum leaves [0, 4096] (a probability above 4096,
// or a row without a reference yet) does the wave compute the rows' maxima
// (one cross-lane max), move the references up, rescale O and l and take
// the probabilities again.  O and l share the reference, so the result is
// the same attention; probabilities stay <= 4096.
//
// The FUSED instantiation is the prompt step with the append inside (KV
// Cache section of "大模型推理优化实战：KV Cache + Flash Attention": the new
// tokens' K/V join the cache, then the queries attend over all of it):
// tiles of new keys are read from the new rows themselves, and each new row
// is written to its page slot once, by the item of its own position (see
// the kernel's comment).
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_rowwise_f32(const PrefillArgs &a, hipStream_t s);

constexpr int kPfRows = 128;         // query rows per query tile (4 waves x 32)
constexpr int kPfKeys = 64;          // keys per key tile
constexpr int kPfEngineThreads = 256;
constexpr float kPfSumCap = 4096.f;  // largest partial row sum (so probability) the reference may give
constexpr int kPfRun = 8;            // most query tiles per workgroup in run mode (a.run_tiles <= this)

template <int D>
struct PfCfg {
  static constexpr int kKRow = 2 * D + 16;   // staged K row bytes (bank spread for b128 reads)
  static constexpr int kVRow = 2 * D + 64;   // staged V row bytes (bank spread for transpose reads)
  static constexpr int kCpr = D / 8;         // 16-byte chunks per row
  static constexpr int kNs = D / 16;         // QK k-steps
  static constexpr int kNdb = D / 32;        // O^T 32-dim blocks
  static constexpr int kKBuf = kPfKeys * kKRow;
  static constexpr int kVBuf = kPfKeys * kVRow;
  static constexpr int kEngine = 2 * (kKBuf + kVBuf);                   // two K/V buffers
  static constexpr int kLoads = kPfKeys * kCpr / kPfEngineThreads;      // per thread per tile, K and V each
};

// BIG_PAGE: page_size >= 64, so each 64-key tile lies in one page.
// FUSED (with BIG_PAGE): the queries' own K/V rows arrive in a.k_new /
// a.v_new; keys at positions >= ctx - q_len are read from there, and each
// such row is written into its page slot once, by the item (query tile, key
// tile) of that position in a workgroup of the first query head of its KV
// group.  No key the launch reads from a page is written by it.
// block_table is a.block_table, passed again as a restrict pointer so that
// uniform page-id reads are scalar loads.
template <int D, bool BIG_PAGE, bool RUNS, bool FUSED>
__global__ __launch_bounds__(512, 2) void prefill_bf16_kernel(PrefillArgs a, const int32_t *__restrict__ block_table) {
  static_assert(!FUSED || BIG_PAGE, "the fused append needs whole key tiles inside one page");
  using C = PfCfg<D>;
  __shared__ __align__(16) unsigned char smem[2 * C::kEngine];
  // kDirect: K/V tiles go from global memory straight into LDS (16-byte
  // buffer loads with the LDS as destination) instead of through registers;
  // their rows are then unpadded (2D bytes) and XOR-swizzled in 16-byte
  // chunks (see lane_dt).  Pages smaller than a tile, and head
  // dimension 64, keep the register path.
  constexpr bool kDirect = BIG_PAGE && D == 128;
  constexpr int kKRowL = kDirect ? 2 * D : C::kKRow;  // LDS row pitch of staged K
  constexpr int kVRowL = kDirect ? 2 * D : C::kVRow;  // and of staged V
  constexpr int kKBufL = kPfKeys * kKRowL;
  constexpr int kVBufL = kPfKeys * kVRowL;
  static_assert(2 * (kKBufL + kVBufL) + (kDirect ? 4 * 1024 : 0) <= C::kEngine,
                "an engine's two K/V buffers (and, direct, its waves' scratch) must fit its LDS share");

  const int eng = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);  // 0: forward, 1: backward
  const int tid = threadIdx.x & (kPfEngineThreads - 1);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);             // wave inside the engine
  const int col = lane & 31;
  const int g = lane >> 5;
  const int gam = lane >> 4;
  const int tp = lane & 15;

  // Everything the prologue needs from memory (sequence bounds, context
  // length and, in pair mode, the page of key tile 0, which is every
  // engine's first tile there: causal, no window) is read first, in one
  // round trip; readfirstlane keeps these values, and every tile decision
  // derived from them, in scalar registers, and keeps the loads above the
  // branches below.
  const int b = blockIdx.z;
  const int q0_raw = __builtin_amdgcn_readfirstlane(a.cu_q[b]);
  const int q_end = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]);
  const int ctx_raw = __builtin_amdgcn_readfirstlane(a.ctx_lens[b]);
  const int pg0_raw = RUNS ? 0 : __builtin_amdgcn_readfirstlane(block_table[(size_t)b * a.max_pages]);
  // Debug builds: the ranges the entry point documents (no-ops otherwise);
  // q_len is also bounded by the keys the block-table row can address, so
  // that a context in [q_len, that bound] exists to stand in for a bad one.
  const int max_keys = a.max_pages << a.c.log2_page;
  const int q0 = checked(q0_raw, 0, 0x7fffffff, kSiteRowOffset, b);
  const int q_len = checked(q_end - q0, 0, min(a.max_q_len, max_keys), kSiteQueryLen, b);
  const int ctx = checked(ctx_raw, q_len, max_keys, kSiteCtxLen, b);
  const int pg0 = RUNS || q_len == 0 ? pg0_raw : checked(pg0_raw, 0, a.c.num_pages - 1, kSitePageId, b);
  const int grid_x = gridDim.x, grid_y = gridDim.y;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2): consecutive ids are remapped so that the pairs of one query head run
  // on one XCD and stream that head's K/V tiles together.
  int pair = blockIdx.x;  // pair mode: the pair index; run mode: the run index
  int h = blockIdx.y;
  if (RUNS && a.window_left >= 0) {
    // A window reads each key tile about once, at the memory's pace: here
    // the query head varies fastest, so that the workgroups running together
    // read every head's part of the same cache rows (whole rows of all KV
    // heads instead of scattered 256-byte pieces of them).
    const int k = blockIdx.x + grid_x * blockIdx.y;
    h = k % grid_y;
    pair = k / grid_y;
  } else if ((grid_y & 7) == 0) {
    const int k = blockIdx.x + grid_x * blockIdx.y;  // id inside this sequence
    const int k8 = k >> 3;
    h = (k & 7) + 8 * (k8 / grid_x);
    pair = k8 % grid_x;
  }
  const int n_qt = (q_len + kPfRows - 1) / kPfRows;
  if (RUNS ? pair * a.run_tiles >= n_qt : pair >= (n_qt + 1) / 2) return;  // uniform
  const int off = ctx - q_len;
  const int hk = h / a.group;
  const int W = a.window_left;
  const int causal = a.causal;

  // Visible key tiles [lo, hi) of query tile qt.
  auto tile_range = [=](int qt, int &lo, int &hi) __attribute__((always_inline)) {
    const int p_first = off + qt * kPfRows;
    const int p_last = off + min(qt * kPfRows + kPfRows - 1, q_len - 1);
    const int k_lo = W >= 0 ? max(0, p_first - W) : 0;
    const int k_hi = causal ? min(p_last + 1, ctx) : ctx;
    lo = k_lo / kPfKeys;
    hi = (k_hi + kPfKeys - 1) / kPfKeys;
  };
  // The workgroup's items (query tile, key tile) are split between the
  // engines, half each, as runs of consecutive key tiles of one query tile:
  // run j of this engine covers its items [st[j], st[j+1]) with query tile
  // rq[j] and first key tile rk[j].  Whichever query tile the split falls in
  // (if any) is the last one both engines work on; it is merged at the end.
  constexpr int kRuns = RUNS ? kPfRun : 2;
  int st[kRuns], rq[kRuns], rk[kRuns];
  int total, half, n1;
  bool shared;
  if constexpr (!RUNS) {
    // Pair mode (causal, no window): query tiles (p, n-1-p), whose key-tile
    // counts add up to the same total for every p.  With na <= nb (always
    // under a causal mask, tile qa being the earlier one): engine 0 takes all
    // of qa, then the top of qb's tiles; engine 1 takes the bottom of qb's
    // tiles.  Both ascend, so (both ranges starting at key 0) the engines
    // read the same key tile at the same step.  Otherwise (na > nb, or the
    // middle tile of an odd count, nb = 0): engine 0 takes the bottom of qa;
    // engine 1 takes all of qb, then the top of qa.
    const int qa = pair;
    const int qb = n_qt - 1 - pair;  // == qa for the middle tile of an odd count
    int lo_a, hi_a, lo_b = 0, hi_b = 0;
    tile_range(qa, lo_a, hi_a);
    if (qb != qa) tile_range(qb, lo_b, hi_b);
    const int na = hi_a - lo_a;
    const int nb = hi_b - lo_b;
    total = na + nb;
    half = (total + 1) / 2;
    n1 = total - half;
    shared = half != na;
    st[0] = 0;
    if (na <= nb) {
      if (eng == 0) {
        rq[0] = qa, rk[0] = lo_a, st[1] = na, rq[1] = qb, rk[1] = lo_b + n1;
      } else {
        rq[0] = qb, rk[0] = lo_b, st[1] = n1, rq[1] = qb, rk[1] = lo_b + n1;
      }
    } else {
      if (eng == 0) {
        rq[0] = qa, rk[0] = lo_a, st[1] = half, rq[1] = qa, rk[1] = lo_a + half;
      } else {
        rq[0] = qb, rk[0] = lo_b, st[1] = nb, rq[1] = qa, rk[1] = lo_a + half;
      }
    }
  } else {
    // Run mode (a window, or no causal mask: about the same work for every
    // query tile): a.run_tiles (<= kPfRun) consecutive query tiles.  Engine
    // 0 takes the first half of their items in order; engine 1 takes the
    // second half with its query tiles in reverse order, so that the tile
    // holding the split comes last for both.
    const int rt = a.run_tiles;
    const int q_begin = pair * rt;
    int lo[kPfRun], cum[kPfRun + 1];
    cum[0] = 0;
#pragma unroll
    for (int r = 0; r < kPfRun; ++r) {
      int l = 0, hh = 0;
      if (r < rt && q_begin + r < n_qt) tile_range(q_begin + r, l, hh);
      lo[r] = l;
      cum[r + 1] = cum[r] + (hh - l);
    }
    total = cum[kPfRun];
    half = (total + 1) / 2;
    n1 = total - half;
    shared = false;
#pragma unroll
    for (int r = 1; r < kPfRun; ++r) shared |= cum[r] == half;
    shared = !shared && half > 0 && half < total;
    if (eng == 0) {
#pragma unroll
      for (int r = 0; r < kPfRun; ++r) {
        st[r] = min(cum[r], half);
        rq[r] = q_begin + r;
        rk[r] = lo[r];
      }
    } else {
      // Engine 1 also walks each query tile's key tiles downward (rk: the
      // highest), so that consecutive query tiles of a window meet the key
      // tiles they share as neighbouring items (see `resident`).
      int at = 0;
#pragma unroll
      for (int j = 0; j < kPfRun; ++j) {
        const int r = kPfRun - 1 - j;
        const int first = max(cum[r], half);
        st[j] = at;
        rq[j] = q_begin + r;
        rk[j] = lo[r] + (cum[r + 1] - cum[r]) - 1;
        at += max(0, cum[r + 1] - first);
      }
    }
  }
  const int n_mine = eng == 0 ? half : n1;
  // my_item(t): run j applies when t >= st[j] (runs in increasing start
  // order, empty ones telescoping away).  Written as sums of "value or zero"
  // offsets between consecutive runs, kept in scalar registers.
  // Run j's key tile at item t is rk[j] + ks (t - st[j]), ks = 1 (upward)
  // or -1 (downward: engine 1 in run mode).
  const int ks = (RUNS && eng == 1) ? -1 : 1;
  int dst[kRuns], ddq[kRuns], ddk[kRuns];
  const int q_base = __builtin_amdgcn_readfirstlane(rq[0]);
  const int k_base = __builtin_amdgcn_readfirstlane(rk[0] - ks * st[0]);
#pragma unroll
  for (int j = 1; j < kRuns; ++j) {
    dst[j] = __builtin_amdgcn_readfirstlane(st[j]);
    ddq[j] = __builtin_amdgcn_readfirstlane(rq[j] - rq[j - 1]);
    ddk[j] = __builtin_amdgcn_readfirstlane((rk[j] - ks * st[j]) - (rk[j - 1] - ks * st[j - 1]));
  }
  auto my_item = [=](int t, int &qt, int &kt) __attribute__((always_inline)) {
    int q = q_base, k = ks * t + k_base;
#pragma unroll
    for (int j = 1; j < kRuns; ++j) {
      const bool in = t >= dst[j];
      q += in ? ddq[j] : 0;
      k += in ? ddk[j] : 0;
    }
    qt = q;
    kt = k;
  };

  unsigned char *ebase = smem + eng * C::kEngine;
  const int P = a.c.page_size;
  const int lp = a.c.log2_page;
  const size_t row_bytes = (size_t)a.c.num_kv_heads * D * 2;
  const char *kbase = (const char *)a.c.k + (size_t)hk * D * 2;
  const char *vbase = (const char *)a.c.v + (size_t)hk * D * 2;
  const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
  // Fused append: key position k >= off is row q0 + k - off of k_new / v_new.
  const char *knew = FUSED ? (const char *)a.k_new + ((size_t)q0 * a.c.num_kv_heads + hk) * D * 2 : nullptr;
  const char *vnew = FUSED ? (const char *)a.v_new + ((size_t)q0 * a.c.num_kv_heads + hk) * D * 2 : nullptr;
  // Of the query heads sharing KV head hk, the first writes its new rows.
  const bool kv_writer = h % a.group == 0;
  // A pointer the same for every lane, said so (a buffer descriptor built
  // from a pointer the compiler takes as per-lane becomes a loop over its
  // distinct values).
  auto uniform_ptr = [](const char *p) __attribute__((always_inline)) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    return (const char *)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
  };

  // Prefetch of one key tile, K and V separately: thread `tid` moves chunks
  // tid + 256 i, i.e. row tid / kCpr + i * kRowsPerPass, chunk tid % kCpr.
  // BIG_PAGE (P >= 64): the tile sits in one page (one scalar page-id load)
  // and is read through a buffer descriptor whose range ends at the last key
  // of the context, so rows at or beyond ctx read as zeros (their slots may
  // hold anything; they are masked).  Otherwise each row looks its page up.
  constexpr int kRowsPerPass = kPfEngineThreads / C::kCpr;
  const int lrow = tid / C::kCpr;
  const int lch = tid % C::kCpr;
  const uint32_t lane_goff = (uint32_t)lrow * (uint32_t)row_bytes + lch * 16;
  // Byte offset of key tile kt inside the K (or V) pool (BIG_PAGE: one
  // page), from the block-table entry of its page.
  auto page_off = [&](int entry, int kt) __attribute__((always_inline)) {
    const int key0 = kt * kPfKeys;
    const int page = checked(entry, 0, a.c.num_pages - 1, kSitePageId, b);
    return ((size_t)page * P + (key0 & (P - 1))) * row_bytes;
  };
  auto tile_page_off = [&](int kt) __attribute__((always_inline)) {
    return page_off(block_table[(size_t)b * a.max_pages + ((kt * kPfKeys) >> lp)], kt);
  };
  // res: the tile is already resident in its LDS buffers (see `resident`):
  // the same loads are issued through a descriptor of length 0, so they
  // move no data (and return zeros) but keep the count of loads in flight
  // the same on every path.
  auto load_half = [&](int kt, size_t tile_off, const char *base, const char *nbase, uint4 *dst, bool res)
      __attribute__((always_inline)) {
    const int key0 = kt * kPfKeys;
    if constexpr (BIG_PAGE) {
      // Fused: a tile of new keys only comes from the new rows; a tile that
      // also holds cached keys comes from its page, and its new rows are
      // replaced once the loads have landed (fix_new_rows).
      const char *tb = base + tile_off;
      if constexpr (FUSED) {
        if (key0 >= off) tb = nbase + (size_t)(key0 - off) * row_bytes;
        tb = uniform_ptr(tb);
      }
      const uint32_t span = res ? 0u : (uint32_t)(min(kPfKeys, ctx - key0) * row_bytes);
      const __amdgpu_buffer_rsrc_t r = make_rsrc(tb, span);
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i)
        dst[i] = buf_load16(r, lane_goff + (uint32_t)(i * kRowsPerPass) * (uint32_t)row_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        const int key = key0 + lrow + i * kRowsPerPass;
        dst[i] = make_uint4(0, 0, 0, 0);
        if (!res && key < ctx) {
          const int page = checked(bt[key >> lp], 0, a.c.num_pages - 1, kSitePageId, b);
          const size_t ro = ((size_t)page * P + (key & (P - 1))) * row_bytes + lch * 16;
          dst[i] = *reinterpret_cast<const uint4 *>(base + ro);
        }
      }
    }
  };
  const uint32_t lane_koff = (uint32_t)lrow * C::kKRow + lch * 16;
  const uint32_t lane_voff = (uint32_t)lrow * C::kVRow + lch * 16;
  auto kbuf = [&](int buf) __attribute__((always_inline)) { return ebase + buf * (kKBufL + kVBufL); };
  auto vbuf = [&](int buf) __attribute__((always_inline)) { return ebase + buf * (kKBufL + kVBufL) + kKBufL; };
  // Direct path: wave w's loads of a tile fill its 16 rows 16 w .. 16 w + 15
  // (4 KiB), load i the rows 16 w + 4 i .. +3 (lane l: row 16 w + 4 i + l /
  // 16, physical chunk l % 16).  The four loads share one LDS base (so one
  // M0 value) and differ in the instruction offset 1024 i, which the
  // hardware adds to the LDS address and to the memory offset alike (also
  // in the range check); each lane's memory offset is passed less that.
  // The lane loads the logical chunk that the swizzle puts there, from its
  // row in the page.  K: chunk c of row r sits at chunk c ^ (r % 16), so
  // the 16 rows an MFMA operand read touches at one logical chunk fall in 16
  // different bank groups.  V: chunk c of row r sits at c ^ 2 (r % 4), so
  // the four rows a transposed read takes two adjacent chunks from fall in
  // four different 32-byte bank groups.  lane_dt(v, i): the lane's offset
  // inside a tile for load i, of K (v false: four registers, as its chunk
  // depends on i) or V (one register plus a uniform step).
  const int drow = 16 * w + (lane >> 4);  // the lane's row in load 0; load i: drow + 4 i
  // (Four named values, not an array: a local array used inside these
  // lambdas keeps the host compilation pass from emitting the kernel.)
  auto dk_of = [&](int i) __attribute__((always_inline)) {
    const int r = drow + 4 * i;
    return (uint32_t)r * (uint32_t)row_bytes + (uint32_t)(((lane & 15) ^ (r & 15)) * 16);
  };
  const uint32_t dk0 = dk_of(0), dk1 = dk_of(1), dk2 = dk_of(2), dk3 = dk_of(3);
  const uint32_t dv0 = (uint32_t)drow * (uint32_t)row_bytes + (uint32_t)(((lane & 15) ^ ((drow & 3) << 1)) * 16);
  auto lane_dt = [&](bool v, int i) __attribute__((always_inline)) {
    return v ? dv0 + (uint32_t)(4 * i) * (uint32_t)row_bytes : i == 0 ? dk0 : i == 1 ? dk1 : i == 2 ? dk2 : dk3;
  };
  // Tile kt (its page offset tile_off) of the pool at `base` into the LDS
  // buffer `dst`: four 16-byte loads per lane, through a descriptor whose
  // range ends at the context's last key (rows past it arrive as zeros).
  // res: the tile is resident already (see `resident`); the same loads then
  // go through a descriptor of length 0 (no memory traffic) into this
  // wave's 1 KiB of scratch LDS beyond the engine's buffers, so the count of
  // loads in flight is the same on every path.
  // Fused: a tile of new keys comes from the new rows at nbase; the one tile
  // that holds both cached and new keys (when the first new position is not
  // a multiple of 64) takes each row from where it is, every lane loading
  // through one of two descriptors, so each LDS slot is written once.  mx
  // (std::bool_constant): whether this copy of the loops handles such a
  // tile at all.
  auto issue_direct = [&](auto mx, int kt, size_t tile_off, const char *base, const char *nbase, unsigned char *dst,
                          bool is_v, bool res) __attribute__((always_inline)) {
    if constexpr (kDirect) {
      static_assert(!kDirect || C::kLoads == 4, "the direct path issues four loads per lane and tile");
      const int key0 = kt * kPfKeys;
      const uint32_t span = res ? 0u : (uint32_t)(min(kPfKeys, ctx - key0) * row_bytes);
      const char *tb = base + tile_off;
      bool mixed = false;
      if constexpr (FUSED) {
        if (key0 >= off) tb = uniform_ptr(nbase + (size_t)(key0 - off) * row_bytes);
        if constexpr (decltype(mx)::value) mixed = !res && key0 < off && key0 + kPfKeys > off;
      }
      const __amdgpu_buffer_rsrc_t r = make_rsrc(tb, span);
      unsigned char *dw = dst + 16 * w * kKRowL;  // this wave's 4 KiB of the buffer
      // The resident case takes no branch of its own: a branch around the
      // loads leaves the compiler a path that it thinks issues none (it cannot
      // tell that one side always runs), and then it no longer takes the
      // previous step's Q loads as landed at the end of the phase and waits
      // for every load in flight before the next QK product.  (The fused
      // append's tile of both cached and new keys, whose lanes choose
      // between two descriptors in branches, does that: it is loaded only in
      // a copy of the loops of its own, for sequences whose cached part does
      // not end on a 64-key boundary.)
      if (FUSED && mixed) {
        // New rows from nbase (row index key - off), the rest from the page.
        // (The distinct asm markers keep the two loads apart: merged into
        // one, its descriptor would be chosen per lane.)
        const __amdgpu_buffer_rsrc_t rn = make_rsrc(uniform_ptr(nbase), (uint32_t)(min(kPfKeys, ctx - off) * row_bytes));
        const uint32_t new_off = (uint32_t)((key0 - off) * (int)row_bytes);
#define PA_LD_MIXED(I)                                                                         \
  {                                                                                            \
    const uint32_t vo = lane_dt(is_v, I) - 1024 * (I);                                         \
    if (key0 + drow + 4 * (I) < off) {                                                         \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PA_LDS void *)dw, 16, vo, 0, 1024 * (I), 0); \
      __asm__ volatile("; cached rows" ::: "memory");                                          \
    } else {                                                                                   \
      const uint32_t vn = vo + new_off;                                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rn, (PA_LDS void *)dw, 16, vn, 0, 1024 * (I), 0); \
      __asm__ volatile("; new rows" ::: "memory");                                             \
    }                                                                                          \
  }
        PA_LD_MIXED(0)
        PA_LD_MIXED(1)
        PA_LD_MIXED(2)
        PA_LD_MIXED(3)
#undef PA_LD_MIXED
      } else {
        // A resident tile: the same loads through the descriptor of length 0
        // land in this wave's 1 KiB of scratch LDS (LDS base moved back by
        // the instruction offset, so all four write the same 1 KiB).
        unsigned char *scratch = ebase + 2 * (kKBufL + kVBufL) + w * 1024;
#define PA_LD(I)                                                                               \
  {                                                                                            \
    const uint32_t vo = lane_dt(is_v, I) - 1024 * (I);                                         \
    unsigned char *d = res ? scratch - 1024 * (I) : dw;                                        \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PA_LDS void *)d, 16, vo, 0, 1024 * (I), 0);   \
  }
        PA_LD(0)
        PA_LD(1)
        PA_LD(2)
        PA_LD(3)
#undef PA_LD
      }
    }
  };
  // Fused append, direct path: item (qt, kt)'s tile is in the LDS buffer
  // `src` (K or V), each wave's rows put there by its own loads; `entry` is
  // the block-table entry of the tile's page.  The rows that are new and
  // belong to the item's query tile go to their page slots: every lane
  // stores the 16 bytes it loaded at the page offset it would have read
  // them from.  The stores go through a descriptor that ends at the last
  // such row, so the hardware's range check drops the rows past it; a row
  // before the first gets the descriptor's length as its offset, out of
  // range the same way.  No lane branches, and only the 32-bit lane offsets
  // the loads use.  (The rows are read from LDS as bf16 vectors, like the
  // QK operands: read as integers, they made the compiler wait for every
  // load in flight first.)  The caller runs this before the wave's next
  // loads into `src`.
  auto write_back = [&](int qt, int kt, int entry, const unsigned char *src, char *pool, bool is_v)
      __attribute__((always_inline)) {
    if constexpr (FUSED && kDirect) {
      const int key0 = kt * kPfKeys;
      const int w_lo = max(key0, off + qt * kPfRows);
      const int w_hi = min(min(key0 + kPfKeys, off + qt * kPfRows + kPfRows), ctx);
      if (kv_writer && w_lo < w_hi) {
        // (Said uniform: the compiler computes w_hi on the vector unit, and a
        // descriptor it takes as per-lane becomes a loop over its values.)
        const uint32_t span =
            (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(w_hi - key0) * (uint32_t)row_bytes));
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(uniform_ptr(pool + (size_t)hk * D * 2 + page_off(entry, kt)), span);
        const int lo = w_lo - key0;
        bf16x8 x[C::kLoads];
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i)
          x[i] = *reinterpret_cast<const bf16x8 *>(src + (16 * w + 4 * i) * kKRowL + lane * 16);
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
          const uint32_t vo = drow + 4 * i >= lo ? lane_dt(is_v, i) : span;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[i]), r, (int)vo, 0, 0);
        }
      }
    }
  };
  // Direct path, reading side: the byte offset inside a row of this lane's
  // K operand chunk for k-step s (logical chunk 2 s + g, swizzled by the row
  // col % 16), and the offset of its transposed V read for output block db
  // from the first of the 16-row group (row g * 4 + tp / 4, logical chunk
  // 4 db + 2 (gam % 2) + (tp % 4) / 2, swizzled by the row % 4 = tp / 4,
  // plus the 8-byte half (tp % 2)).
  uint32_t kd_off[C::kNs], vd_off[C::kNdb];
#pragma unroll
  for (int s2 = 0; s2 < C::kNs; ++s2) kd_off[s2] = (uint32_t)((((2 * s2 + g) ^ (col & 15)) & 15) * 16);
#pragma unroll
  for (int db = 0; db < C::kNdb; ++db)
    vd_off[db] = (uint32_t)((g * 4 + (tp >> 2)) * kVRowL +
                            (((4 * db + 2 * (gam & 1) + ((tp & 3) >> 1)) ^ ((tp >> 2) << 1)) & 15) * 16 + 8 * (tp & 1));
  auto store_k = [&](int buf, const uint4 *src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      *reinterpret_cast<uint4 *>(kbuf(buf) + lane_koff + i * kRowsPerPass * C::kKRow) = src[i];
  };
  auto store_v = [&](int buf, const uint4 *src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      *reinterpret_cast<uint4 *>(vbuf(buf) + lane_voff + i * kRowsPerPass * C::kVRow) = src[i];
  };
  uint4 pk[C::kLoads], pv[C::kLoads];  // K / V of a tile in flight
  size_t pk_off = 0;  // BIG_PAGE: tile_page_off of the tile in pk / pv
  auto load_tile = [&](int kt, bool res) __attribute__((always_inline)) {
    if (!res) pk_off = BIG_PAGE ? tile_page_off(kt) : 0;
    load_half(kt, pk_off, kbase, knew, pk, res);
    load_half(kt, pk_off, vbase, vnew, pv, res);
  };
  // Fused append, tile kt holding both cached and new keys (only the first
  // new position's tile): once its page loads have landed in pk / pv, the
  // rows of new positions are read again from the new rows.  Rare (one tile
  // per sequence, and only when that position is not a multiple of 64), so
  // these loads are waited for at once, outside the prefetch pipeline.
  auto fix_new_rows = [&](int kt) __attribute__((always_inline)) {
    if constexpr (FUSED) {
      const int key0 = kt * kPfKeys;
      if (key0 < off && key0 + kPfKeys > off) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
          const int key = key0 + lrow + i * kRowsPerPass;
          if (key >= off && key < ctx) {
            const size_t o = (size_t)(key - off) * row_bytes + lch * 16;
            pk[i] = *reinterpret_cast<const uint4 *>(knew + o);
            pv[i] = *reinterpret_cast<const uint4 *>(vnew + o);
          }
        }
      }
    }
  };
  // Fused append: whether item (qt, kt) writes new rows into their pages
  // (rows that are new and belong to the item's query tile, in a workgroup
  // of the first query head of the KV group).
  auto writes_new_qk = [&](int qt, int kt) __attribute__((always_inline)) {
    if constexpr (FUSED) {
      const int key0 = kt * kPfKeys;
      return kv_writer && max(key0, off + qt * kPfRows) < min(min(key0 + kPfKeys, off + qt * kPfRows + kPfRows), ctx);
    }
    return false;
  };
  auto writes_new = [&](int idx) __attribute__((always_inline)) {
    int qt, kt;
    my_item(idx, qt, kt);
    return writes_new_qk(qt, kt);
  };
  // Item t (t >= 2) finds its key tile still in its LDS buffers when item
  // t - 2, the previous user of buffers t % 2, had the same key tile (same
  // sequence and KV head: the same data).  Consecutive query tiles of a
  // window share two key tiles, which the items meet this way (engine 0
  // walking keys upward, engine 1 downward), so each tile is read from
  // memory about once per run instead of once per query tile.  Fused, on the
  // register path: an item that writes new rows needs its tile in registers
  // and always loads (the direct path writes them from LDS).
  auto resident = [&](int t) __attribute__((always_inline)) {
    if (!RUNS || t < 2) return false;  // pair mode: query tiles share no key-tile pairs
    int qa_, ka_, qb_, kb_;
    my_item(t, qa_, ka_);
    my_item(t - 2, qb_, kb_);
    return ka_ == kb_ && (kDirect || !writes_new(t));
  };
  // Fused append: the tile of item idx is in pk / pv; write the rows that
  // are new and belong to the item's query tile into their page slots.
  auto write_new = [&](int idx) __attribute__((always_inline)) {
    if constexpr (FUSED) {
      int qt, kt;
      my_item(idx, qt, kt);
      const int key0 = kt * kPfKeys;
      const int w_lo = max(key0, off + qt * kPfRows);
      const int w_hi = min(min(key0 + kPfKeys, off + qt * kPfRows + kPfRows), ctx);
      if (kv_writer && w_lo < w_hi) {
        char *kd = (char *)a.c.k + (size_t)hk * D * 2 + pk_off + lane_goff;
        char *vd = (char *)a.c.v + (size_t)hk * D * 2 + pk_off + lane_goff;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
          const int key = key0 + lrow + i * kRowsPerPass;
          if (key >= w_lo && key < w_hi) {
            *reinterpret_cast<uint4 *>(kd + (size_t)(i * kRowsPerPass) * row_bytes) = pk[i];
            *reinterpret_cast<uint4 *>(vd + (size_t)(i * kRowsPerPass) * row_bytes) = pv[i];
          }
        }
      }
    }
  };
  // Per-wave state.  qt_q: the query tile whose Q^T is in bq; qt_o: the
  // query tile that (m, lsum, o) belong to.
  int qt_q = -1, qt_o = -1;
  bf16x8 bq[C::kNs];
  float m = -INFINITY;  // exponent reference of this lane's row (log2 units)
  float lsum = 0.f;     // this lane's half of the row sum
  f32x16 o[C::kNdb];
  f32x16 sacc[2];       // S^T of a tile between its GEMM and softmax phases
  bf16x8 bp[4];         // P^T of a tile between its softmax phase and the next GEMM phase

  // Q^T of query tile qt into bq (waited for where it is first used).
  auto load_q_async = [&](int qt) __attribute__((always_inline)) {
    const int qrow = qt * kPfRows + w * 32 + col;
    const __bf16 *qp = (const __bf16 *)a.q + ((size_t)(q0 + min(qrow, q_len - 1)) * a.num_q_heads + h) * D;
#pragma unroll
    for (int s = 0; s < C::kNs; ++s)
      bq[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 16 * s + 8 * g));
  };
  auto reset_o = [&]() __attribute__((always_inline)) {
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  };
  // Normalise and store this wave's rows of query tile qt.
  // Normalise and store 32-dim blocks [db0, db1) of this wave's rows of
  // query tile qt.  Lanes l and l + 32 hold the two 4-dim halves of each
  // 8-dim group; a permlane32 swap gives each lane one whole group, so every
  // store writes 16 contiguous bytes.
  auto finish_part = [&](int qt, float m_row, float l_half, const f32x16 *acc, auto DB0, auto DB1, bool with_lse)
      __attribute__((always_inline)) {
    constexpr int db0 = decltype(DB0)::value, db1 = decltype(DB1)::value;
    const int qrow = qt * kPfRows + w * 32 + col;
    const float ltot = l_half + __shfl_xor(l_half, 32, 64);
    const float inv = 1.f / ltot;
    uint16_t *orow = (uint16_t *)a.out + ((size_t)(q0 + min(qrow, q_len - 1)) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db) {
      if (db < db0 || db >= db1) continue;
#pragma unroll
      for (int jp = 0; jp < 4; jp += 2) {
        uint32_t x[2], y[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int ia = 4 * jp + 2 * hlf, ib = 4 * (jp + 1) + 2 * hlf;
          const uint32_t va = pack_bf16x2(acc[db][ia] * inv, acc[db][ia + 1] * inv);
          const uint32_t vb = pack_bf16x2(acc[db][ib] * inv, acc[db][ib + 1] * inv);
          const auto r = __builtin_amdgcn_permlane32_swap(va, vb, false, false);
          x[hlf] = r[0];
          y[hlf] = r[1];
        }
        if (qrow < q_len)
          *reinterpret_cast<uint4 *>(orow + db * 32 + (jp + g) * 8) = make_uint4(x[0], x[1], y[0], y[1]);
      }
    }
    if (with_lse && a.lse != nullptr && g == 0 && qrow < q_len)
      a.lse[(size_t)(q0 + qrow) * a.num_q_heads + h] = (m_row + __log2f(ltot)) * kLn2;
  };
  auto finish = [&](int qt, float m_row, float l_half, const f32x16 *acc) __attribute__((always_inline)) {
    finish_part(qt, m_row, l_half, acc, std::integral_constant<int, 0>{}, std::integral_constant<int, C::kNdb>{}, true);
  };

  // S^T = K . Q^T for the two 32-key blocks of the tile in LDS buffer `buf`.
  // The K fragments are read kAhead MFMAs ahead of their use (a ring of
  // registers), so the LDS latency hides behind the MFMAs before them.
  // Consecutive MFMAs alternate between the two blocks' accumulators, so
  // none waits for the one just issued (a chain of eight on one
  // accumulator was measurably slower).
  auto qk_mfma = [&](int buf) __attribute__((always_inline)) {
    const unsigned char *ks = kbuf(buf);
    constexpr int kSteps = 2 * C::kNs;  // (key block, k-step) pairs
    constexpr int kAhead = 6;
    auto rd = [&](int u) __attribute__((always_inline)) {
      const int kb = u & 1, s = u >> 1;
      if constexpr (kDirect)  // logical chunk 2 s + g of row kb * 32 + col, swizzled by the row
        return *reinterpret_cast<const bf16x8 *>(ks + (kb * 32 + col) * kKRowL + kd_off[s]);
      else
        return *reinterpret_cast<const bf16x8 *>(ks + (kb * 32 + col) * C::kKRow + (16 * s + 8 * g) * 2);
    };
    bf16x8 ka[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) ka[u] = rd(u);
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int kb = u & 1, s = u >> 1;
      const bf16x8 cur = ka[u % kAhead];
      if (u + kAhead < kSteps) ka[u % kAhead] = rd(u + kAhead);
      sacc[kb] = mfma32(cur, bq[s], s == 0 ? f32x16{} : sacc[kb]);
      // Keep the product in this (GEMM) half-step: left alone, the compiler
      // sinks it to its first use after the barrier.
      if (s == C::kNs - 1) __asm__ volatile("" : "+v"(sacc[kb]));
      __builtin_amdgcn_sched_barrier(0);  // keep each read kAhead MFMAs ahead
    }
  };
  // O^T += V^T . P^T over four 16-key steps, V from LDS buffer `buf`.  The
  // V^T fragments of step t + 1 are read before the MFMAs of step t; those
  // of step 0 go out alone, so that its MFMAs wait for them only.
  auto read_v = [&](const unsigned char *vs, int t, bf16x8 *va) __attribute__((always_inline)) {
    const int r0 = (t >> 1) * 32 + (t & 1) * 16 + g * 4;
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db) {
      if constexpr (kDirect) {
        const unsigned char *p1 = vs + ((t >> 1) * 32 + (t & 1) * 16) * kVRowL + vd_off[db];
        va[db] = cat(lds_read_tr16(p1), lds_read_tr16(p1 + 8 * kVRowL));
      } else {
        const unsigned char *p1 = vs + (r0 + (tp >> 2)) * C::kVRow + (db * 32 + 16 * (gam & 1) + 4 * (tp & 3)) * 2;
        va[db] = cat(lds_read_tr16(p1), lds_read_tr16(p1 + 8 * C::kVRow));
      }
    }
  };
  auto pv_mfma = [&](int buf) __attribute__((always_inline)) {
    const unsigned char *vs = vbuf(buf);
    bf16x8 va[2][C::kNdb];
    read_v(vs, 0, va[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 1 < 4) read_v(vs, t + 1, va[(t + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // the next step's reads go out first
#pragma unroll
      for (int db = 0; db < C::kNdb; ++db) o[db] = mfma32(va[t & 1][db], bp[t], o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Mask and online softmax of tile (qt, kt) on sacc; P^T -> bp.
  auto softmax = [&](int qt, int kt, bool fresh) __attribute__((always_inline)) {
    const int key0 = kt * kPfKeys;
    const int pos = off + qt * kPfRows + w * 32 + col;
    const int p_first = off + qt * kPfRows;
    const int p_last = off + min(qt * kPfRows + kPfRows - 1, q_len - 1);
    // Mask (only tiles that cross a boundary; this lane's row sees keys
    // [klo, khi]) on the raw scores; the scale (> 0) is applied inside the
    // exponent, after the max.
    const bool edge = (causal && key0 + kPfKeys - 1 > p_first) || (W >= 0 && key0 < p_last - W) ||
                      (key0 + kPfKeys > ctx);
    if (edge) {
      // Bounds relative to this lane's first key, so that each element's
      // offset in the tile is a constant: visible iff lo <= offset <= hi.
      // The lane's visible offsets as a bit mask, one 32-bit word per 32-key
      // block (vm[kb] bit j: offset 32 kb + j); each element then takes one
      // sign-extending bit extract and one bit select (score or -inf).
      const int base = key0 + g * 4;
      const int hi = (causal ? min(pos, ctx - 1) : ctx - 1) - base;
      const int lo = (W >= 0 ? pos - W : 0) - base;
      uint32_t vm[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int h = hi - 32 * kb, l = lo - 32 * kb;
        const uint32_t le = h >= 31 ? 0xffffffffu : h < 0 ? 0u : (2u << h) - 1u;
        const uint32_t ge = l <= 0 ? 0xffffffffu : l >= 32 ? 0u : ~((1u << l) - 1u);
        vm[kb] = le & ge;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = (i >> 2) * 8 + (i & 3);  // offset inside the 32-key block
          const uint32_t keep = (uint32_t)((int32_t)(vm[kb] << (31 - c)) >> 31);
          // (Through a scalar: a bit cast of a vector element read element 0
          // with this compiler.)
          const float v = sacc[kb][i];
          sacc[kb][i] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, v) & keep) | (0xff800000u & ~keep));
        }
    }
    // P^T against reference nm = -m, rounded into bp; returns this lane's
    // partial row sum (its 32 of the row's 64 keys).
    auto exps = [&](float nm) __attribute__((always_inline)) {
      float ps[4];  // four partial sums, each started at its first term
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[kb][i], a.scale_log2, nm));
          if (kb == 0 && i < 4)
            ps[i] = p;
          else
            ps[i & 3] += p;
          bp[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
        }
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // First try the row's present reference: if every lane's partial sum is
    // at most the cap, every probability is too, and the reference stands.
    // A lane without a reference yet (m = -inf) gets +inf or NaN and fails.
    float part = fresh ? INFINITY : exps(m == -INFINITY ? INFINITY : -m);
    if (__any(!(part <= kPfSumCap))) {
      // Move every row's reference up to its maximum so far (a row whose
      // maximum did not grow keeps a factor of 1; one without a visible key
      // yet keeps m = -inf), rescale, and recompute.
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mx0 = fmaxf(mx0, sacc[0][i]);
        mx1 = fmaxf(mx1, sacc[1][i]);
      }
      const float mx = max_xor32(fmaxf(mx0, mx1)) * a.scale_log2;
      const float m_new = fmaxf(m, mx);
      const float corr = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      // Rows without a reference yet hold o = 0 and lsum = 0: the first
      // visible tile of a query tile rescales nothing.
      if (__any(m != -INFINITY)) {
        lsum *= corr;
#pragma unroll
        for (int db = 0; db < C::kNdb; ++db) o[db] *= corr;
      }
      m = m_new;
      part = exps(m == -INFINITY ? 0.f : -m);
    }
    lsum += part;
    // Materialise P in this (softmax) half-step, like S above.
#pragma unroll
    for (int t = 0; t < 4; ++t) __asm__ volatile("" : "+v"(bp[t]));
  };

  // Ping-pong schedule in half-steps (one workgroup barrier each).  For its
  // tile t an engine runs a GEMM phase G(t) = [QK of tile t, PV of tile t-1]
  // (MFMA; in that order, so the QK results the softmax reads first are done
  // while the PV products finish) and then a softmax phase S(t) (VALU);
  // after its last tile, G(n) = PV of tile n-1 alone.  Engine 1 runs one half-step behind engine 0, so on
  // every SIMD one wave's softmax overlaps the other wave's MFMAs.  Tile t
  // lives in LDS buffer t % 2.  Its K and V are loaded into registers at the
  // start of G(t-1) and stored at the end of S(t-1): a whole step of load
  // latency.  By then the buffer's previous tile t-2 has been read (its K by
  // G(t-2), its V by G(t-1)), and the next reads, G(t) for K and G(t+1) for
  // V, come after the next barrier.
  // The first query tile's Q is loaded with the first K/V tile (both
  // latencies overlap) and staged in LDS buffer 1, free until S(0) stores
  // tile 1 there; G(0) reads Q^T from it.
  constexpr int kQLoads = kPfRows * C::kCpr / kPfEngineThreads;
  static_assert(kPfRows * C::kKRow <= C::kKBuf + C::kVBuf, "Q tile must fit one K/V buffer");
  // Direct path barriers: a bare s_barrier (a workgroup fence would also
  // wait for every LDS-bound load in flight) with the waits it needs made
  // explicit; the empty asm statements keep the compiler from moving memory
  // accesses across it.  After a GEMM phase: this wave's LDS reads are done
  // (the buffers they read are reloaded in the next phase).  After a softmax
  // phase and after the prologue: every load but the last 8 (those of this
  // phase: the next-but-one K tile and the next V tile) has landed, and so
  // has the phase's block-table read (a scalar load still in flight would
  // make the compiler wait for all of the next phase's LDS reads before its
  // first MFMA, as it cannot count them apart).  (The compiler, which
  // cannot tell those 8 LDS writes from the next GEMM phase's LDS reads,
  // also waits for them before its first read: their latency hides behind
  // the softmax phase.)
  constexpr int kWaitLgkm0 = 0xC07F;  // vmcnt(63) expcnt(7) lgkmcnt(0)
  constexpr int kWaitVm8 = 0x0078;    // vmcnt(8) expcnt(7) lgkmcnt(0)
  auto bar_after_gemm = [&]() __attribute__((always_inline)) {
    if constexpr (kDirect) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };
  auto bar_after_loads = [&]() __attribute__((always_inline)) {
    if constexpr (kDirect) {
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };
  // Direct path: the items t - 1 .. t + 2 of this engine as (query tile,
  // key tile) pairs, kept from step to step (pair mode: clamped to the last
  // item, whose tile the loads past the end read again; run mode: past the
  // end they are never used).  Each step computes one new item: pair mode
  // from the two runs directly, run mode by walking (the next key tile of
  // the query tile, or the first of the next query tile in the engine's
  // direction), which costs a few scalar instructions where the run table
  // would cost dozens.  pg2: the block-table entry of item t + 2's page,
  // read a step before it is needed.  (ck, coff, cres): the K tile loaded
  // last, which is the next V tile.
  int wq_m1 = 0, wk_m1 = 0, wq0 = 0, wk0 = 0, wq1 = 0, wk1 = 0, wq2 = 0, wk2 = 0;
  int wlo = 0, whi = 0;  // run mode: the key-tile range of query tile wq2
  int pg2 = 0;
  // Fused: the block-table entries of items t - 1, t and t + 1, carried
  // along so that the write-back of items t and t - 1 reads no table.
  int pe_m1 = 0, pe0 = 0, pe1 = 0;
  int ck = 0;
  size_t coff = 0;
  bool cres = false;
  auto page_entry = [&](int kt, bool valid) __attribute__((always_inline)) {
    return block_table[(size_t)b * a.max_pages + (valid ? (kt * kPfKeys) >> lp : 0)];
  };
  auto advance = [&](int t) __attribute__((always_inline)) {  // window of step t -> step t + 1
    wq_m1 = wq0, wk_m1 = wk0, wq0 = wq1, wk0 = wk1, wq1 = wq2, wk1 = wk2;
    if constexpr (FUSED) pe_m1 = pe0, pe0 = pe1, pe1 = pg2;
    if constexpr (RUNS) {
      wk2 += ks;
      if (ks > 0 ? wk2 >= whi : wk2 < wlo) {
        wq2 += ks;
        tile_range(wq2, wlo, whi);
        wk2 = ks > 0 ? wlo : whi - 1;
      }
    } else {
      my_item(min(t + 3, n_mine - 1), wq2, wk2);
    }
    pg2 = page_entry(wk2, t + 3 < n_mine || !RUNS);
  };
  auto direct_prologue = [&](auto mx) __attribute__((always_inline)) {
    // Q^T of the first query tile straight into registers, then K(0), V(0)
    // and K(1) into LDS buffers 0, 0 and 1 (K(t + 2) and V(t + 1) follow in
    // softmax phase t, once the buffers' previous tiles have been read).
    if (kDirect && n_mine > 0) {
      my_item(0, wq0, wk0);
      my_item(min(1, n_mine - 1), wq1, wk1);
      my_item(min(2, n_mine - 1), wq2, wk2);
      if constexpr (RUNS) tile_range(wq2, wlo, whi);
      pg2 = page_entry(wk2, 2 < n_mine || !RUNS);
      if constexpr (FUSED) pe0 = page_entry(wk0, true), pe1 = page_entry(wk1, true);
      load_q_async(wq0);
      qt_q = wq0;
      const size_t off0 = (!RUNS && wk0 == 0) ? (size_t)pg0 * P * row_bytes : tile_page_off(wk0);
      issue_direct(mx, wk0, off0, kbase, knew, kbuf(0), false, false);
      issue_direct(mx, wk0, off0, vbase, vnew, vbuf(0), true, false);
      const bool r1 = RUNS && n_mine < 2;
      const size_t off1 = r1 ? 0 : tile_page_off(wk1);
      issue_direct(mx, wk1, off1, kbase, knew, kbuf(1), false, r1);
      ck = wk1, coff = off1, cres = r1;
    }
  };
  if (!kDirect && n_mine > 0) {
    int qt, kt;
    my_item(0, qt, kt);
    if (!RUNS && BIG_PAGE && kt == 0) {
      pk_off = (size_t)pg0 * P * row_bytes;
      load_half(kt, pk_off, kbase, knew, pk, false);
      load_half(kt, pk_off, vbase, vnew, pv, false);
    } else {
      load_tile(kt, false);
    }
    u32x4 qs[kQLoads];
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int row = min(qt * kPfRows + lrow + i * kRowsPerPass, q_len - 1);
      qs[i] = *reinterpret_cast<const u32x4 *>((const char *)a.q + ((size_t)(q0 + row) * a.num_q_heads + h) * D * 2 + lch * 16);
    }
    fix_new_rows(kt);
    store_k(0, pk);
    store_v(0, pv);
#pragma unroll
    for (int i = 0; i < kQLoads; ++i)
      *reinterpret_cast<u32x4 *>(kbuf(1) + (lrow + i * kRowsPerPass) * C::kKRow + lch * 16) = qs[i];
    write_new(0);
  }
  // Wave priorities: the GEMM wave's MFMAs are the critical path of each
  // half-step, so its instructions win issue slots over the other engine's
  // softmax on the same SIMD.
  auto gemm_phase = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    // Inside the loop the next tile's loads are unconditional (the last step
    // re-reads its own tile, never stored): the same loads are in flight on
    // every path, so the wait counts stay exact.
    if constexpr (!kDirect) {
      if (t < n_mine) {
        int qt, kt;
        my_item(min(t + 1, n_mine - 1), qt, kt);
        load_tile(kt, RUNS && (t + 1 >= n_mine || resident(t + 1)));
      }
    }
    if (t < n_mine) {
      int qt, kt;
      my_item(t, qt, kt);
      if (!kDirect && t == 0) {
#pragma unroll
        for (int s = 0; s < C::kNs; ++s)
          bq[s] = *reinterpret_cast<const bf16x8 *>(kbuf(1) + (w * 32 + col) * C::kKRow + (16 * s + 8 * g) * 2);
        qt_q = qt;
      }
      qk_mfma(t & 1);
    }
    if (t >= 1) pv_mfma((t - 1) & 1);
    // The next item's Q, if it starts a new query tile, is loaded once the
    // PV product is issued, so that the compiler's wait for the loads in
    // flight before the first V read (it cannot tell their LDS writes from
    // those reads) does not take in the Q loads as well.  It arrives during
    // the softmax phase, at whose end every load but that phase's has landed.
    if (t + 1 < n_mine) {
      int qn = wq1, kn;
      if constexpr (!kDirect) my_item(t + 1, qn, kn);
      if (qn != qt_q) {
        load_q_async(qn);
        qt_q = qn;
      }
    }
  };
  auto softmax_phase = [&](int t, auto mx) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    if constexpr (FUSED && !kDirect) {
      // The next tile's new rows go to their pages first, so that the whole
      // softmax hides the stores' completion: the memory counter drains in
      // order, and the wait for the next tile's loads at the end of the
      // phase includes them.
      if (t + 1 < n_mine && !resident(t + 1)) {
        int qn, kn;
        my_item(t + 1, qn, kn);
        fix_new_rows(kn);
        write_new(t + 1);
      }
    }
    int qt = wq0, kt = wk0;
    if constexpr (!kDirect) my_item(t, qt, kt);
    const bool fresh = qt != qt_o;
    if (fresh) {
      if (qt_o >= 0) finish(qt_o, m, lsum, o);
      reset_o();
      qt_o = qt;
    }
    if constexpr (kDirect) {
      // K buffer t % 2 (K(t), read in G(t)) takes K(t + 2); V buffer
      // (t + 1) % 2 (V(t - 1), read in G(t)) takes V(t + 1).  The softmax
      // wave issues them, off the GEMM wave's path.  A tile already
      // resident, or an index past the engine's last item, gets the same
      // loads with no data (see issue_direct), so every phase issues the
      // same number of loads.
      // Fused: first the new rows of K(t) and V(t - 1), the buffers' present
      // tiles, go from LDS to their pages (V(t - 1) landed before this
      // step's barrier; K(t) too).  The stores are issued before the loads,
      // so the wait for all but the last 8 memory operations at the end of
      // the phase still covers exactly the older loads.
      if constexpr (FUSED) {
        if (writes_new_qk(wq0, wk0)) write_back(wq0, wk0, pe0, kbuf(t & 1), (char *)a.c.k, false);
        if (t >= 1 && writes_new_qk(wq_m1, wk_m1))
          write_back(wq_m1, wk_m1, pe_m1, vbuf((t + 1) & 1), (char *)a.c.v, true);
      }
      // K(t + 2): resident when item t had the same key tile (run mode).
      // V(t + 1): the K tile of the previous step.
      const bool r2 = RUNS && (t + 2 >= n_mine || wk2 == wk0);
      const size_t off2 = r2 ? 0 : page_off(pg2, wk2);
      issue_direct(mx, wk2, off2, kbase, knew, kbuf(t & 1), false, r2);
      issue_direct(mx, ck, coff, vbase, vnew, vbuf((t + 1) & 1), true, cres);
      ck = wk2, coff = off2, cres = r2;
      advance(t);
    }
    softmax(qt, kt, fresh);
    if constexpr (!kDirect) {
      if (t + 1 < n_mine && !resident(t + 1)) {
        store_k((t + 1) & 1, pk);
        store_v((t + 1) & 1, pv);
      }
    }
  };
  // Fused, direct path: the last item's V rows, still in their buffer
  // (landed before the last GEMM phase, which read them), before the merge
  // reuses the buffers.
  auto last_write_back = [&]() __attribute__((always_inline)) {
    if constexpr (FUSED && kDirect)  // the window has moved on: item n_mine - 1 is its first
      if (n_mine > 0 && writes_new_qk(wq_m1, wk_m1))
        write_back(wq_m1, wk_m1, pe_m1, vbuf((n_mine - 1) & 1), (char *)a.c.v, true);
  };
  // The prologue and the loops of both engines, once per kind of sequence:
  // in the fused append, a sequence whose cached part does not end on a
  // 64-key boundary has a key tile of both cached and new keys, loaded
  // through per-lane branches (mx true); the copy for the others has none,
  // so that the compiler counts the loads in flight of every path exactly.
  auto run = [&](auto mx) __attribute__((always_inline)) {
    direct_prologue(mx);
    bar_after_loads();
    // Engine 0 passes 2 * half + 1 barriers in its loop, engine 1 one leading
    // barrier and 2 * n1 + 1 in its loop; the engine with fewer pads one at
    // the end (half - n1 is 0 or 1).  Each engine's loop is its own
    // straight-line code so that its registers keep one assignment.
    if (eng == 0) {
      for (int t = 0; t < n_mine; ++t) {
        gemm_phase(t);
        bar_after_gemm();
        softmax_phase(t, mx);
        bar_after_loads();
      }
      gemm_phase(n_mine);
      last_write_back();
      if constexpr (kDirect) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes the LDS
      __syncthreads();
      if (half == n1) __syncthreads();
    } else {
      bar_after_gemm();
      for (int t = 0; t < n_mine; ++t) {
        gemm_phase(t);
        bar_after_gemm();
        softmax_phase(t, mx);
        bar_after_loads();
      }
      gemm_phase(n_mine);
      last_write_back();
      if constexpr (kDirect) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes the LDS
      __syncthreads();
      if (half > n1) __syncthreads();
    }
  };
  if constexpr (FUSED && kDirect) {
    if (off % kPfKeys != 0)
      run(std::true_type{});
    else
      run(std::false_type{});
  } else {
    run(std::false_type{});
  }
  const int qt_cur = qt_o;

  // The query tile split between the engines (qb in the first case, qa in
  // the second; none if the split falls on the boundary, half == na) has a
  // partial result in each engine.  Each engine finishes half of its 32-dim
  // blocks (engine 0 the first half, engine 1 the second): it hands the
  // other half of its (O, m, l) to the other engine through LDS (the K/V
  // buffers are free now) and merges the half it receives.
  if (!shared) {
    if (qt_cur >= 0) finish(qt_cur, m, lsum, o);
    return;
  }
  constexpr int kHalfDb = C::kNdb / 2;
  constexpr int kMrgLane = 16 * kHalfDb + 4;
  static_assert(2 * 4 * 64 * kMrgLane * 4 <= 2 * C::kEngine, "merge area must fit the K/V buffers");
  float *mine_out = reinterpret_cast<float *>(smem) + (size_t)((eng * 4 + w) * 64 + lane) * kMrgLane;
  const float *other_in = reinterpret_cast<const float *>(smem) + (size_t)(((1 - eng) * 4 + w) * 64 + lane) * kMrgLane;
  auto merge = [&](auto E) __attribute__((always_inline)) {
    constexpr int e = decltype(E)::value;
    constexpr int give0 = e == 0 ? kHalfDb : 0;  // first block handed over
    constexpr int keep0 = e == 0 ? 0 : kHalfDb;  // first block finished here
#pragma unroll
    for (int d = 0; d < kHalfDb; ++d)
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<f32x4 *>(mine_out + 16 * d + i) =
            f32x4{o[give0 + d][i], o[give0 + d][i + 1], o[give0 + d][i + 2], o[give0 + d][i + 3]};
    mine_out[16 * kHalfDb] = m;
    mine_out[16 * kHalfDb + 1] = lsum;
    __syncthreads();
    const float m_other = other_in[16 * kHalfDb];
    const float l_other = other_in[16 * kHalfDb + 1];
    // (m0, l0) of engine 0, (m1, l1) of engine 1.
    const float m0 = e == 0 ? m : m_other, m1 = e == 0 ? m_other : m;
    const float l0 = e == 0 ? lsum : l_other, l1 = e == 0 ? l_other : lsum;
    const float mm = fmaxf(m0, m1);
    const float f0 = m0 == -INFINITY ? 0.f : fast_exp2(m0 - mm);
    const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int d = 0; d < kHalfDb; ++d)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const f32x4 vo = *reinterpret_cast<const f32x4 *>(other_in + 16 * d + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v0 = e == 0 ? o[keep0 + d][i + j] : vo[j];
          const float v1 = e == 0 ? vo[j] : o[keep0 + d][i + j];
          o[keep0 + d][i + j] = v1 * f1 + v0 * f0;
        }
      }
    finish_part(qt_cur, mm, l1 * f1 + l0 * f0, o, std::integral_constant<int, keep0>{},
                std::integral_constant<int, keep0 + kHalfDb>{}, e == 1);
  };
  if (eng == 0)
    merge(std::integral_constant<int, 0>{});
  else
    merge(std::integral_constant<int, 1>{});
}

// fp32 caches (the 1e-4 configuration): the same attention with fp32
// operands on v_mfma_f32_32x32x2_f32, one wave per 32 query rows of one
// head, K and V read from the pages straight into the operand registers (no
// LDS), the online softmax of the bf16 kernel in fp32 throughout (P is not
// rounded).  Operand layout of the 32x32x2 product: lane l gives A[l % 32][l
// / 32] and B[l / 32][l % 32]; accumulator element e of lane l is row 8 (e /
// 4) + 4 (l / 32) + e % 4, column l % 32.  So, with g = l / 32:
//   S^T = K . Q^T over D/2 steps, step s pairing dims s (g = 0) and D/2 + s
//   (g = 1): lane (g, c) gives K[key0 + c][g D/2 + s] and Q[row c][g D/2 + s];
//   element e of S^T is key key0 + 8 (e / 4) + 4 g + e % 4 of row c;
//   O^T += V^T . P^T over 16 steps, step s pairing the keys that the lanes'
//   own element s holds, so B is P element s of the lane itself and A is
//   V[key0 + 8 (s / 4) + 4 g + s % 4][32 db + c]: no exchange between lanes.
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int kHalf = D / 2;
  const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, col = lane & 31, g = lane >> 5;
  const int max_keys = a.max_pages << a.c.log2_page;
  const int q0 = checked(a.cu_q[b], 0, 0x7fffffff, kSiteRowOffset, b);
  const int q_len = checked(a.cu_q[b + 1] - q0, 0, min(a.max_q_len, max_keys), kSiteQueryLen, b);
  if (rb * 32 >= q_len) return;  // uniform
  const int ctx = checked(a.ctx_lens[b], q_len, max_keys, kSiteCtxLen, b);
  const int off = ctx - q_len;
  const int hk = h / a.group;
  const int W = a.window_left;
  const int row = rb * 32 + col;
  const int pos = off + min(row, q_len - 1);
  const int p_first = off + rb * 32, p_last = off + min(rb * 32 + 31, q_len - 1);
  const int k_lo = W >= 0 ? max(0, p_first - W) : 0;
  const int k_hi = a.causal ? min(p_last, ctx - 1) : ctx - 1;
  const int hi_r = a.causal ? min(pos, ctx - 1) : ctx - 1;  // this lane's row sees keys [lo_r, hi_r]
  const int lo_r = W >= 0 ? pos - W : 0;
  const float *kp = (const float *)a.c.k + (size_t)hk * D;
  const float *vp = (const float *)a.c.v + (size_t)hk * D;
  const size_t row_elems = (size_t)a.c.num_kv_heads * D;
  auto row_of = [&](int key) __attribute__((always_inline)) {  // element offset of key's row
    const int page = checked(a.block_table[(size_t)b * a.max_pages + (key >> a.c.log2_page)], 0, a.c.num_pages - 1,
                             kSitePageId, b);
    return ((size_t)page * a.c.page_size + (key & (a.c.page_size - 1))) * row_elems;
  };
  float qv[kHalf];
  {
    const float *qr = (const float *)a.q + ((size_t)(q0 + min(row, q_len - 1)) * a.num_q_heads + h) * D + g * kHalf;
#pragma unroll
    for (int s = 0; s < kHalf; s += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(qr + s);
      qv[s] = v.x, qv[s + 1] = v.y, qv[s + 2] = v.z, qv[s + 3] = v.w;
    }
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;  // l: this lane's half of the row sum
  for (int key0 = k_lo & ~31; key0 <= k_hi; key0 += 32) {
    // S^T of the 32 keys (rows past the context read the last key; masked).
    float kv[kHalf];
    {
      const float *kr = kp + row_of(min(key0 + col, ctx - 1)) + g * kHalf;
#pragma unroll
      for (int s = 0; s < kHalf; s += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(kr + s);
        kv[s] = v.x, kv[s + 1] = v.y, kv[s + 2] = v.z, kv[s + 3] = v.w;
      }
    }
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < kHalf; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[s], qv[s], sacc, 0, 0, 0);
    float x[16], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 8 * (e >> 2) + 4 * g + (e & 3);
      x[e] = (key >= lo_r && key <= hi_r) ? sacc[e] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    mx = max_xor32(mx);
    const float m_new = fmaxf(m, mx);
    const float corr = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
    l *= corr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= corr;
    m = m_new;
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = m == -INFINITY ? 0.f : fast_exp2(x[e] - m);
      l += p[e];
    }
    // O^T += V^T . P^T; step s takes the keys of the lanes' element s.
    size_t vrow[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) vrow[s] = row_of(min(key0 + 8 * (s >> 2) + 4 * g + (s & 3), ctx - 1)) + col;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int s = 0; s < 16; ++s)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[vrow[s] + 32 * db], p[s], o[db], 0, 0, 0);
  }
  const float ltot = l + __shfl_xor(l, 32, 64);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (row < q_len) {
    float *orow = (float *)a.out + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(orow + 32 * db + 8 * j + 4 * g) =
            make_float4(o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
    if (a.lse != nullptr && g == 0)
      a.lse[(size_t)(q0 + row) * a.num_q_heads + h] = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

static hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
  const dim3 grid((a.max_q_len + 31) / 32, a.num_q_heads, a.batch);
  if (a.c.head_dim == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// Query tiles per run-mode workgroup: as many as kPfRun (fewer, longer
// workgroups: a 128-key window at 8192 rows ran 121 us with 8 tiles against
// 132 us with 4) while the grid still has a workgroup per CU, down to one
// for short prompts (the same window at 1024 rows: 66 us with 8, 25 with 1).  PAGEDATTN_PREFILL_RUN_TILES (1..8) overrides it
// (tests use it to cover every run length on small inputs).
static int prefill_run_tiles(int n_qt, int heads, int batch) {
  if (const char *env = getenv("PAGEDATTN_PREFILL_RUN_TILES")) {
    const int v = atoi(env);
    if (v >= 1 && v <= kPfRun) return v;
  }
  const long long tiles = (long long)n_qt * heads * batch;
  return (int)std::min<long long>(kPfRun, std::max<long long>(1, tiles / device_cu_count()));
}

PA_DEFINE_FAULT_READER(take_fault_prefill)

hipError_t launch_prefill(const PrefillArgs &a_in, hipStream_t s) {
  if (a_in.batch == 0 || a_in.max_q_len == 0) return hipSuccess;
  // fp32: prefill on the fp32 MFMA; a single-token decode (no cu_q) keeps
  // the one-wave-per-row kernel (a 32-row block would be 1/32 used).
  if (a_in.c.dtype == 0) return a_in.cu_q != nullptr ? launch_prefill_f32(a_in, s) : launch_rowwise_f32(a_in, s);
  PrefillArgs a = a_in;
  const int n_qt = (a.max_q_len + kPfRows - 1) / kPfRows;
  // Causal without a window: pairs (p, n-1-p) balance the triangle.  A window
  // or no mask gives every query tile about the same work: runs of
  // run_tiles query tiles.
  const bool runs = !(a.causal && a.window_left < 0);
  a.run_tiles = runs ? prefill_run_tiles(n_qt, a.num_q_heads, a.batch) : 1;
  dim3 grid(runs ? (n_qt + a.run_tiles - 1) / a.run_tiles : (n_qt + 1) / 2, a.num_q_heads, a.batch);
  const dim3 block(2 * kPfEngineThreads);
  const bool big = a.c.page_size >= kPfKeys;
#define PA_PREFILL_LAUNCH(DD, BIG, RUN) \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, BIG, RUN, false>), grid, block, 0, s, a, a.block_table)
#define PA_PREFILL_FUSED(DD, RUN) \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, true, RUN, true>), grid, block, 0, s, a, a.block_table)
  if (a.k_new != nullptr) {
    // The fused append reads whole key tiles from one page (the caller
    // routes smaller pages through a separate append).
    if (!big) return hipErrorInvalidValue;
    if (a.c.head_dim == 64) {
      if (runs) PA_PREFILL_FUSED(64, true); else PA_PREFILL_FUSED(64, false);
    } else {
      if (runs) PA_PREFILL_FUSED(128, true); else PA_PREFILL_FUSED(128, false);
    }
    return hipGetLastError();
  }
  if (a.c.head_dim == 64) {
    if (runs) {
      if (big) PA_PREFILL_LAUNCH(64, true, true); else PA_PREFILL_LAUNCH(64, false, true);
    } else {
      if (big) PA_PREFILL_LAUNCH(64, true, false); else PA_PREFILL_LAUNCH(64, false, false);
    }
  } else {
    if (runs) {
      if (big) PA_PREFILL_LAUNCH(128, true, true); else PA_PREFILL_LAUNCH(128, false, true);
    } else {
      if (big) PA_PREFILL_LAUNCH(128, true, false); else PA_PREFILL_LAUNCH(128, false, false);
    }
  }
#undef PA_PREFILL_LAUNCH
#undef PA_PREFILL_FUSED
  return hipGetLastError();
}

}  // namespace pa
