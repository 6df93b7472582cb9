// Single-token decode over a paged KV cache: split-K kernel + merge kernel.
//
// Method: exact attention of one query per sequence against all cached keys
// ("大模型推理优化：KV Cache与FlashAttention实战" section 2.1; the new token's
// own K/V are in the cache, "大模型推理优化实战：KV Cache + Flash Attention" KV
// Cache section), read page by page through the block table ("Flash Attention
// 与Paged KV Cache优化大模型计算效率" section 3.2), with GQA sharing ("LLM推理
// 系统优化：KV缓存管理与动态批处理技术" section 2.1) and, for int8 caches, the
// per-(page, KV head) scales of that page's section 3.2.  The online softmax
// (running max, running sum, rescale by exp(m_old - m_new)) of the 3x-faster
// page's Flash Attention section is applied per wave, then across the waves of
// a workgroup, then across splits; all three merges are the same algebra.
//
// Work split (balanced for ragged context lengths): a split workgroup has 8
// waves and handles hpw KV heads together (the largest power of two <= 8
// dividing Hkv); wave w takes head w % hpw and every (8 / hpw)-th tile of
// it, so with 8 KV heads the workgroup reads whole contiguous token rows.
// The keys of every (sequence b, head group) pair form a segment of 32-key
// tiles; all segments laid end to end make one list of T tiles.  A fixed
// grid of N workgroups (one per CU) cuts the list into N equal ranges,
// [jT/N, (j+1)T/N) for workgroup j, so every workgroup streams the same
// number of bytes whatever the length mix.  A range is cut further at
// segment boundaries into pieces; for each piece the waves of each head
// merge their running (m, l, O) through LDS and write one partial per head
// to slot (segment + j), which is unique because both the segments and the
// ranges are in list order.  All G = Hq/Hkv query heads of a KV head are
// handled together so each K/V byte is read from HBM once.  The merge
// kernel finds the workgroups that touched a segment from the same
// arithmetic and combines their partials.
//
// Per 32-key tile a wave computes S^T = K . Q^T with v_mfma_f32_16x16x32_bf16
// (keys on the M side, query heads on the N side, zero-padded to 16), the
// online softmax on the S^T registers, then O^T += V^T . P^T with V staged
// through LDS and read back transposed by ds_read_b64_tr_b16 (ds_read_b64_tr_b8
// for int8, converted to exact bf16 integers).  Loads are 16-byte buffer
// loads from one page per 16-key block; the next tile is in flight while a
// tile is computed.
#include <math.h>
#include <stdlib.h>

#include <atomic>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kDecWaves = 8;
constexpr int kDecTile = 32;            // keys per wave iteration
constexpr int kDecWgsPerCu = 1;         // resident split workgroups per CU (register bound)

int device_cu_count() {
  // Without a queryable device (host-only use of the argument checks) the
  // count is that of an MI355X.
  constexpr int kDefaultCus = 256;
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCus;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = kDefaultCus;
    v = cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// kDecWgsPerCu workgroups per CU of the current device (the split kernel's
// occupancy, so the whole grid is resident at once).  PAGEDATTN_DECODE_WGS
// overrides it (tests use it to exercise other partitions of the same work).
int decode_grid_size() {
  if (const char *env = getenv("PAGEDATTN_DECODE_WGS")) {
    const int v = atoi(env);
    if (v >= 1 && v <= 65536) return v;
  }
  return kDecWgsPerCu * device_cu_count();
}

// Tiles of 32 keys that a decode query at position ctx - 1 reads: from the
// tile holding the first visible key to the tile holding the last (none for
// an empty context).
__device__ __forceinline__ int seg_tiles(int ctx, int window_left) {
  ctx = max(ctx, 0);
  const int lo = window_left >= 0 ? max(0, ctx - 1 - window_left) : 0;
  return (ctx + kDecTile - 1) / kDecTile - lo / kDecTile;
}

// ctx_lens[b] of a decode (checked in debug builds against [0, the keys its
// block-table row can address]).
__device__ __forceinline__ int ctx_len(const DecodeArgs &a, int b) {
  return checked(a.ctx_lens[b], 0, a.max_pages << a.c.log2_page, kSiteCtxLen, b);
}

// Workgroups that actually take tiles: at least kMinTilesPerWg tiles each.
// One: a small problem (a few short contexts) is spread over as many
// workgroups as it has tiles, so its time is about one tile's latency rather
// than a chain of them (each tile waits for its block-table entry, then its
// rows).
constexpr int kMinTilesPerWg = 1;
__device__ __forceinline__ int active_wgs(long long total, int launched) {
  const long long want = (total + kMinTilesPerWg - 1) / kMinTilesPerWg;
  return (int)max(1LL, min((long long)launched, want));
}

template <int D, bool I8>
struct DecodeCfg {
  static constexpr int kEsz = I8 ? 1 : 2;
  // A lane holds 2 keys of a tile (one per 16-key block kb) and, for each,
  // kChunks 16-byte pieces of the row: dims 32j + 8g .. +7 (bf16) or
  // 64j + 16g .. +15 (int8), j < kChunks, g = lane / 16.
  static constexpr int kChunks = I8 ? D / 64 : D / 32;
  static constexpr int kLoads = 2 * kChunks;               // per lane per tile, for K and for V
  static constexpr int kVRow = I8 ? D + 16 : 2 * D + 32;   // staged V row bytes (bank spread)
  static constexpr int kNdb = D / 16;                      // 16-dim output blocks
  static constexpr int kNst = D / 32;                      // 32-dim QK k-steps
  static constexpr int kStage = kDecWaves * kDecTile * kVRow;
  static constexpr int kMerge = kDecWaves * 16 * D * 4 + 2 * kDecWaves * 16 * 4;
  static constexpr int kSmem = kStage > kMerge ? kStage : kMerge;
};

template <int D, bool I8>
struct TileRegs {
  uint4 k[DecodeCfg<D, I8>::kLoads];
  uint4 v[DecodeCfg<D, I8>::kLoads];
};

// LDS row of tile key k (0..31) in the staged V tile.  bf16: row = key.
// int8: keys are permuted so that rows 8g .. 8g+7 hold the 8 keys whose
// probabilities lane group g carries (16kb + 4g + r, kb = 0..1, r = 0..3):
// one ds_read_b64_tr_b8 of 8 consecutive rows then gives a lane its V^T
// operand in that key order.
template <bool I8>
__device__ __forceinline__ int v_row(int k) {
  return I8 ? 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3) : k;
}

// NB: tiles in flight per wave (register buffers); WPC: resident workgroups
// per CU the register budget is sized for (the grid is WPC per CU).
template <int D, bool I8, int NB, int WPC>
__global__ __launch_bounds__(kDecWaves * 64, kDecWaves / 4 * WPC) void decode_split_kernel(DecodeArgs a,
                                                                         const int32_t *__restrict__ block_table,
                                                                         const float *__restrict__ k_scales,
                                                                         const float *__restrict__ v_scales) {
  using C = DecodeCfg<D, I8>;
  __shared__ __align__(16) unsigned char smem[C::kSmem];
  __shared__ int s_wave_sum[kDecWaves];
  __shared__ int s_first[2];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int j = blockIdx.x;
  const int hkv = a.c.num_kv_heads;
  const int hpw = a.hpw;            // KV heads per workgroup (a power of two dividing hkv, <= kDecWaves)
  const int ngr = hkv / hpw;        // head groups
  const int wph = kDecWaves / hpw;  // waves per head
  const int hh = w % hpw;           // this wave's head inside the group
  const int sub = w / hpw;          // and its share of that head's tiles
  const int W = a.window_left;

  // --- Plan: tiles per sequence (the same for every head group), their
  // prefix sums and the total, by a block scan over the batch.  Thread t
  // owns the sequences [t*per, (t+1)*per).
  const int per = (a.batch + blockDim.x - 1) / blockDim.x;
  const int b_lo = min(a.batch, (int)threadIdx.x * per);
  const int b_hi = min(a.batch, b_lo + per);
  int mine = 0;
  for (int bb = b_lo; bb < b_hi; ++bb) mine += seg_tiles(ctx_len(a, bb), W);
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave_sum[w] = incl;
  __syncthreads();
  int before = 0, per_group_total = 0;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) {
    const int v = s_wave_sum[i];
    before += i < w ? v : 0;
    per_group_total += v;
  }
  const int excl = before + incl - mine;  // per-group tiles of sequences < b_lo
  const long long total = (long long)ngr * per_group_total;
  const int nwg = active_wgs(total, a.nwg);
  if (j == 0) {
    // The merge kernel reads the per-sequence prefix sums from here.
    int acc = excl;
    for (int bb = b_lo; bb < b_hi; ++bb) {
      a.ws_prefix[bb] = acc;
      acc += seg_tiles(ctx_len(a, bb), W);
    }
    if (threadIdx.x == 0) a.ws_prefix[a.batch] = per_group_total;
  }
  if (j >= nwg || total == 0) return;  // uniform across the workgroup
  const long long start = (long long)j * total / nwg;
  const long long end = (long long)(j + 1) * total / nwg;
  // The thread whose sequences hold list position `start` finds it.
  if ((long long)ngr * excl <= start && start < (long long)ngr * (excl + mine)) {
    int acc = excl;
    for (int bb = b_lo; bb < b_hi; ++bb) {
      const int n = seg_tiles(ctx_len(a, bb), W);
      if (start < (long long)ngr * (acc + n)) {
        s_first[0] = bb;
        s_first[1] = acc;
        break;
      }
      acc += n;
    }
  }
  __syncthreads();

  const int G = a.group;
  const bool head_ok = r16 < G;
  const uint32_t row_bytes = (uint32_t)hkv * D * C::kEsz;
  const int lp = a.c.log2_page;
  const uint32_t page_bytes = row_bytes << lp;
  unsigned char *vs = smem + w * kDecTile * C::kVRow;

  int b = s_first[0];
  int nb = seg_tiles(ctx_len(a, b), W);
  const int r0 = (int)(start - (long long)ngr * s_first[1]);
  int hg = r0 / nb;
  int tloc = r0 - hg * nb;
  long long remaining = end - start;

  while (remaining > 0) {
    const int len = (int)min((long long)(nb - tloc), remaining);
    const int ctx = ctx_len(a, b);
    const int lo = W >= 0 ? max(0, ctx - 1 - W) : 0;
    const int t_first = lo / kDecTile + tloc;  // first tile of this piece
    const int k_begin = max(lo, t_first * kDecTile);
    const int k_end = min(ctx, (t_first + len) * kDecTile);
    const int n_w = (len - sub + wph - 1) / wph;  // this wave's tiles
    const int hk = hg * hpw + hh;
    const uint32_t head_off = (uint32_t)hk * D * C::kEsz;
    const int32_t *bt = block_table + (size_t)b * a.max_pages;

    // Q^T operand: lane (head column r16, k-group g), same dim order as K.
    const __bf16 *qrow = (const __bf16 *)a.q + ((size_t)b * a.num_q_heads + hk * G + (head_ok ? r16 : 0)) * D;
    bf16x8 bq[C::kNst];
#pragma unroll
    for (int st = 0; st < C::kNst; ++st) {
      const int dim = I8 ? 64 * (st >> 1) + 16 * g + 8 * (st & 1) : 32 * st + 8 * g;
      uint4 raw = head_ok ? *reinterpret_cast<const uint4 *>(qrow + dim) : make_uint4(0, 0, 0, 0);
      bq[st] = __builtin_bit_cast(bf16x8, raw);
    }

    // Addressing of the 16-key block kb of this wave's i-th tile.  Indices
    // past the wave's last tile re-read that tile (already in cache; the
    // registers are never consumed), so every load is unconditional and the
    // compiler's wait counts stay exact.  Keys outside [k_begin, k_end) read
    // the nearest valid row, which always lies in the block's own page
    // (clamped block start; P >= 16), so the page id is wave-uniform.  Loads
    // go through a buffer descriptor over that page (hardware range check;
    // also keeps the loads opaque to load merging across the loop).
    const int lo16 = k_begin & ~15;
    const int hi16 = (k_end - 1) & ~15;
    auto blk = [&](int i, int kb, const void *pool, uint32_t &off) {
      const int t = t_first + sub + wph * min(i, n_w - 1);
      const int bs = min(max(t * kDecTile + 16 * kb, lo16), hi16);
      const int key = min(max(t * kDecTile + 16 * kb + r16, k_begin), k_end - 1);
      const size_t pbase = (size_t)checked(bt[bs >> lp], 0, a.c.num_pages - 1, kSitePageId, b) * page_bytes + head_off;
      off = (uint32_t)(key & ((1 << lp) - 1)) * row_bytes + 16 * g;
      return make_rsrc((const char *)pool + pbase, page_bytes - head_off);
    };
    auto load_half = [&](int i, const void *pool, uint4 *dst) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t off;
        const __amdgpu_buffer_rsrc_t r = blk(i, kb, pool, off);
#pragma unroll
        for (int jj = 0; jj < C::kChunks; ++jj) dst[kb * C::kChunks + jj] = buf_load16(r, off + 64 * jj);
      }
    };

    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 o[C::kNdb];
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Register buffers recycled half by half: V(i) is staged to LDS and its
    // registers take V(i + NB); K(i) feeds the QK product and its
    // registers take K(i + NB).  NB tiles are in flight while a tile is
    // computed.  The loop runs a multiple of NB steps; a step past the
    // wave's last tile re-reads that tile and masks every key, which leaves
    // (m, l, O) exactly unchanged.
    auto step = [&](int i, TileRegs<D, I8> &R) {
      const int key0 = (t_first + sub + wph * i) * kDecTile;
      // Stage V rows for the transposed reads.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < C::kChunks; ++jj)
          *reinterpret_cast<uint4 *>(vs + v_row<I8>(16 * kb + r16) * C::kVRow + 64 * jj + 16 * g) =
              R.v[kb * C::kChunks + jj];
      load_half(i + NB, a.c.v, R.v);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the K wait

      // S^T = K . Q^T for the two 16-key blocks (keys on M, heads on N).
      f32x4 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < C::kNst; ++st) {
          bf16x8 ka;
          if constexpr (I8) {
            const uint4 raw = R.k[kb * C::kChunks + (st >> 1)];
            ka = (st & 1) ? i8x8_to_bf16x8(raw.z, raw.w) : i8x8_to_bf16x8(raw.x, raw.y);
          } else {
            ka = __builtin_bit_cast(bf16x8, R.k[kb * C::kChunks + st]);
          }
          sacc[kb] = mfma16(ka, bq[st], sacc[kb]);
        }
      }
      load_half(i + NB, a.c.k, R.k);
      __builtin_amdgcn_sched_barrier(0);

      // Scale (with the page's K scale for int8), mask, online softmax.
      float sl[2] = {a.scale_log2, a.scale_log2};
      float vsc[2] = {1.f, 1.f};
      if constexpr (I8) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int bs = min(max(key0 + 16 * kb, lo16), hi16);
          const int page = checked(bt[bs >> lp], 0, a.c.num_pages - 1, kSitePageId, b);
          sl[kb] *= k_scales[(size_t)page * hkv + hk];
          vsc[kb] = v_scales[(size_t)page * hkv + hk];
        }
      }
      float x[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 16 * kb + 4 * g + r;
          const bool vis = key >= k_begin && key < k_end;
          x[kb][r] = vis ? sacc[kb][r] * sl[kb] : -INFINITY;
          mx = fmaxf(mx, x[kb][r]);
        }
      mx = max_xor32(max_xor16(mx));
      const float m_new = fmaxf(m, mx);
      // Rescale only when some head's running max grew (otherwise the factor
      // is exp2(0) = 1 for every lane).
      if (__any(m_new > m)) {
        const float corr = fast_exp2(m - m_new);
        lsum *= corr;
#pragma unroll
        for (int db = 0; db < C::kNdb; ++db) o[db] *= corr;
        m = m_new;
      }
      // m is -inf only before the first visible key, and a wave's first
      // tile always holds one, so the exponents below are of finite numbers
      // or -inf (masked keys -> 0).
      float ps = 0.f;
      bf16x8 bp;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(x[kb][r] - m);
          ps += p;
          bp[kb * 4 + r] = (__bf16)(p * vsc[kb]);
        }
      lsum += ps;

      // O^T += V^T . P^T, V^T read transposed from the staged rows.
#pragma unroll
      for (int db = 0; db < C::kNdb; ++db) {
        bf16x8 va;
        if constexpr (I8) {
          const unsigned char *p1 = vs + (8 * g + (r16 >> 1)) * C::kVRow + db * 16 + 8 * (r16 & 1);
          const i32x2 raw = lds_read_tr8(p1);
          va = i8x8_to_bf16x8((uint32_t)raw[0], (uint32_t)raw[1]);
        } else {
          const unsigned char *p1 = vs + (4 * g + (r16 >> 2)) * C::kVRow + (db * 16 + 4 * (r16 & 3)) * 2;
          va = cat(lds_read_tr16(p1), lds_read_tr16(p1 + 16 * C::kVRow));
        }
        o[db] = mfma16(va, bp, o[db]);
      }
    };

    // The first loads are issued even by a wave without tiles, so the wait
    // counts are the same on every path.  Every piece holds at least one
    // tile (the walk below skips sequences without tiles), so k_begin <
    // k_end and the clamped rows and block indices lie inside the piece.
    // Issue order is pinned (sched_barrier) so that waiting for one tile
    // never waits for a later one.
    TileRegs<D, I8> R[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      load_half(u, a.c.v, R[u].v);
      __builtin_amdgcn_sched_barrier(0);
      load_half(u, a.c.k, R[u].k);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i = 0; i < n_w; i += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) step(i + u, R[u]);
    }
    lsum = sum_xor32(sum_xor16(lsum));

    // Merge the waves of each head (wph of them; a wave without tiles has
    // m = -inf, l = 0, O = 0 and drops out) through LDS and write this
    // piece's partial for each of the group's heads.
    __syncthreads();
    float *wo = reinterpret_cast<float *>(smem);
    float *wm = wo + kDecWaves * 16 * D;
    float *wl = wm + kDecWaves * 16;
    if (head_ok) {
#pragma unroll
      for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) wo[(w * 16 + r16) * D + db * 16 + 4 * g + r] = o[db][r];
      if (g == 0) {
        wm[w * 16 + r16] = m;
        wl[w * 16 + r16] = lsum;
      }
    }
    __syncthreads();
    const size_t slot = (size_t)b * ngr + hg + j;
    for (int e = threadIdx.x; e < hpw * G * D; e += blockDim.x) {
      const int eh = e / (G * D);
      const int rem = e - eh * G * D;
      const int c = rem / D;
      const int d = rem - c * D;
      float big_m = -INFINITY;
      for (int s = 0; s < wph; ++s) big_m = fmaxf(big_m, wm[(eh + hpw * s) * 16 + c]);
      float big_l = 0.f, acc = 0.f;
      for (int s = 0; s < wph; ++s) {
        const int ww = eh + hpw * s;
        const float mw = wm[ww * 16 + c];
        const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - big_m);
        big_l += wl[ww * 16 + c] * f;
        acc += wo[(ww * 16 + c) * D + d] * f;
      }
      const size_t idx = (slot * hpw + eh) * G + c;
      a.ws_o[idx * D + d] = acc;
      if (d == 0) {
        a.ws_ml[idx * 2] = big_m;
        a.ws_ml[idx * 2 + 1] = big_l;
      }
    }
    __syncthreads();  // the LDS is staged into again by the next piece
    remaining -= len;
    tloc = 0;
    if (++hg == ngr && remaining > 0) {
      // Next sequence with tiles: one exists, since tiles remain in this
      // range, so b stays below the batch.  Stepping onto a sequence
      // without tiles would form an empty piece (k_end = 0), whose clamped
      // block index would fall before the block-table row.
      hg = 0;
      do {
        ++b;
        nb = seg_tiles(ctx_len(a, b), W);
      } while (nb == 0);
    }
  }
}

// Running merge of the partials that the split kernel wrote with arguments
// `a` for (sequence b, KV head hk), query head c, dims d..d+3:
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M), accumulated
// in one pass with the same running rescale as the online softmax.  The
// workgroups that touched the head's segment (sequence, head group) are
// those whose list ranges contain its first and last tiles and every one in
// between.  A segment without tiles (empty context) adds nothing.
template <int D>
__device__ __forceinline__ void merge_partials(const DecodeArgs &a, int b, int hk, int c, int d, float &m, float &l,
                                               f32x4 &acc) {
  const int hkv = a.c.num_kv_heads;
  const int hpw = a.hpw;
  const int ngr = hkv / hpw;
  const int hg = hk / hpw;
  const int hh = hk - hg * hpw;
  const int G = a.group;
  const long long total = (long long)ngr * a.ws_prefix[a.batch];
  const int nb = seg_tiles(ctx_len(a, b), a.window_left);
  if (total == 0 || nb == 0) return;
  const int nwg = active_wgs(total, a.nwg);
  const long long f0 = (long long)ngr * a.ws_prefix[b] + (long long)hg * nb;
  const long long f1 = f0 + nb - 1;
  // Workgroup holding list position f: the largest j with j*total/nwg <= f.
  const int j_lo = (int)(((f0 + 1) * nwg - 1) / total);
  const int j_hi = (int)(((f1 + 1) * nwg - 1) / total);
  const size_t seg = (size_t)b * ngr + hg;
#pragma unroll 4
  for (int jj = j_lo; jj <= j_hi; ++jj) {
    const size_t idx = ((seg + jj) * hpw + hh) * G + c;
    const float2 ml = *reinterpret_cast<const float2 *>(a.ws_ml + idx * 2);
    const f32x4 ov = *reinterpret_cast<const f32x4 *>(a.ws_o + idx * D + d);
    const float m_new = fmaxf(m, ml.x);
    const float f_old = fast_exp2(m - m_new);  // 0 on the first piece
    const float f_new = fast_exp2(ml.x - m_new);
    l = l * f_old + ml.y * f_new;
    acc = acc * f_old + ov * f_new;
    m = m_new;
  }
}

// Merge kernel: one workgroup per (KV head, sequence) merges the partials of
// the split kernel (NP = 1), or of two split kernels over disjoint key sets
// of the same sequences (NP = 2, `a2`), and writes O = acc / L and
// lse = M + log2 L (natural log).  A sequence without keys gets O = 0 and
// lse = -inf.  A thread owns 4 consecutive dims of one query head.
template <int D, int NP>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a, DecodeArgs a2) {
  const int hk = blockIdx.x;
  const int b = blockIdx.y;
  const int G = a.group;
  for (int e = 4 * threadIdx.x; e < G * D; e += 4 * blockDim.x) {
    const int c = e / D;
    const int d = e - c * D;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    merge_partials<D>(a, b, hk, c, d, m, l, acc);
    if constexpr (NP == 2) merge_partials<D>(a2, b, hk, c, d, m, l, acc);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const uint32_t lo = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    const uint32_t hi = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    const size_t orow = ((size_t)b * a.num_q_heads + hk * G + c) * D;
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + orow + d) = make_uint2(lo, hi);
    if (a.lse != nullptr && d == 0)
      a.lse[(size_t)b * a.num_q_heads + hk * G + c] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// fp32 caches: one wave per (query row, head), keys one per lane, the same
// online softmax, fp32 FMA throughout.  Also serves fp32 prefill.
template <int D>
__global__ __launch_bounds__(64) void rowwise_f32_kernel(const float *q, const int32_t *cu_q, CacheView c,
                                                         const int32_t *block_table, int max_pages,
                                                         const int32_t *ctx_lens, int num_q_heads, int group,
                                                         float scale_log2, int causal, int window_left,
                                                         float *out, float *lse) {
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  // cu_q == nullptr: one query per sequence (decode), row b of q.
  const int q0 = cu_q != nullptr ? checked(cu_q[b], 0, 0x7fffffff, kSiteRowOffset, b) : b;
  const int q_len = cu_q != nullptr
                        ? checked(cu_q[b + 1] - q0, 0, min((int)gridDim.x, max_pages << c.log2_page), kSiteQueryLen, b)
                        : 1;
  if (row >= q_len) return;
  // prefill rows need their own positions in the context; a decode query
  // may have none (ctx 0: O = 0, lse = -inf)
  const int ctx = checked(ctx_lens[b], cu_q != nullptr ? q_len : 0, max_pages << c.log2_page, kSiteCtxLen, b);
  const int pos = ctx - q_len + row;
  const int hk = h / group;
  const int hi = causal ? pos : ctx - 1;                      // last visible key
  const int lo = window_left >= 0 ? max(0, pos - window_left) : 0;
  const int lane = threadIdx.x;
  const float *qv = q + ((size_t)(q0 + row) * num_q_heads + h) * D;
  const float *kp = (const float *)c.k;
  const float *vp = (const float *)c.v;
  const size_t row_elems = (size_t)c.num_kv_heads * D;
  const int P = c.page_size;
  auto row_off = [&](int key) {
    const int page = checked(block_table[(size_t)b * max_pages + (key >> c.log2_page)], 0, c.num_pages - 1,
                             kSitePageId, b);
    return ((size_t)page * P + (key & (P - 1))) * row_elems + (size_t)hk * D;
  };
  constexpr int kPer = D / 64;
  float o[kPer] = {};
  float m = -INFINITY, l = 0.f;
  for (int k0 = lo; k0 <= hi; k0 += 64) {
    const int key = k0 + lane;
    const bool ok = key <= hi;
    float x = -INFINITY;
    if (ok) {
      const float *kr = kp + row_off(key);
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
      x = s * scale_log2;
    }
    float mx = x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = wave_max_xor(mx, off);
    const float m_new = fmaxf(m, mx);
    const float corr = fast_exp2(m - m_new);
    const float p = ok ? fast_exp2(x - m_new) : 0.f;
    float ps = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 64);
    l = l * corr + ps;
    m = m_new;
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] *= corr;
    const int n = min(64, hi - k0 + 1);
    for (int j = 0; j < n; ++j) {
      const float pj = __shfl(p, j, 64);
      const float *vr = vp + row_off(k0 + j);
#pragma unroll
      for (int e = 0; e < kPer; ++e) o[e] = fmaf(pj, vr[lane + 64 * e], o[e]);
    }
  }
  // A row without visible keys (empty context) gets O = 0 and lse = -inf.
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *orow = out + ((size_t)(q0 + row) * num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[lane + 64 * e] = o[e] * inv;
  if (lse != nullptr && lane == 0)
    lse[(size_t)(q0 + row) * num_q_heads + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_rowwise_f32(const PrefillArgs &a, hipStream_t s) {
  dim3 grid(a.max_q_len, a.num_q_heads, a.batch);
  if (a.c.head_dim == 64)
    hipLaunchKernelGGL(rowwise_f32_kernel<64>, grid, dim3(64), 0, s, (const float *)a.q, a.cu_q, a.c,
                       a.block_table, a.max_pages, a.ctx_lens, a.num_q_heads, a.group, a.scale_log2,
                       a.causal, a.window_left, (float *)a.out, a.lse);
  else
    hipLaunchKernelGGL(rowwise_f32_kernel<128>, grid, dim3(64), 0, s, (const float *)a.q, a.cu_q, a.c,
                       a.block_table, a.max_pages, a.ctx_lens, a.num_q_heads, a.group, a.scale_log2,
                       a.causal, a.window_left, (float *)a.out, a.lse);
  return hipGetLastError();
}

template <int D, bool I8, int NB, int WPC>
static hipError_t launch_split_t(const DecodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<D, I8, NB, WPC>), dim3(a.nwg), dim3(kDecWaves * 64), 0, s, a, a.block_table,
                     a.c.k_scales, a.c.v_scales);
  return hipGetLastError();
}

// Tiles in flight per wave: 1 for bf16 (16 KB), 2 for int8 (8 KB each).
static hipError_t launch_split(const DecodeArgs &a, hipStream_t s) {
  const bool i8 = a.c.dtype == 2;
  if (a.c.head_dim == 64)
    return i8 ? launch_split_t<64, true, 2, kDecWgsPerCu>(a, s) : launch_split_t<64, false, 1, kDecWgsPerCu>(a, s);
  return i8 ? launch_split_t<128, true, 2, kDecWgsPerCu>(a, s) : launch_split_t<128, false, 1, kDecWgsPerCu>(a, s);
}

template <int NP>
static hipError_t launch_reduce(const DecodeArgs &a, const DecodeArgs &a2, hipStream_t s) {
  const dim3 grid(a.c.num_kv_heads, a.batch);
  if (a.c.head_dim == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<64, NP>), grid, dim3(256), 0, s, a, a2);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<128, NP>), grid, dim3(256), 0, s, a, a2);
  return hipGetLastError();
}

PA_DEFINE_FAULT_READER(take_fault_decode)

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipError_t e = launch_split(a, s);
  if (e != hipSuccess) return e;
  return launch_reduce<1>(a, a, s);
}

hipError_t launch_decode_layered(const DecodeArgs &a, const DecodeArgs &a2, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipError_t e = launch_split(a, s);
  if (e != hipSuccess) return e;
  e = launch_split(a2, s);
  if (e != hipSuccess) return e;
  return launch_reduce<2>(a, a2, s);
}

}  // namespace pa
