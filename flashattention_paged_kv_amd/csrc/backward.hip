// Backward pass of paged attention: dQ, dK, dV from Q, the paged K/V, the
// forward output O, its log-sum-exp and the upstream gradient dO.
//
// Method: the attention probabilities are not stored by the forward pass but
// recomputed here from Q, K and the saved log-sum-exp ("大模型推理优化：KV Cache
// 与FlashAttention实战" section 3.1 and "Flash Attention与Paged KV Cache优化大模型
// 计算效率" section 2.1: recomputation in the backward pass).  For one query
// row with scale s, probabilities p_j = exp(s q.k_j - lse), the derivative of
// o = sum_j p_j v_j gives
//   dV_j += p_j dO,   dp_j = dO . v_j,   ds_j = p_j (dp_j - dO . o),
//   dQ    = s sum_j ds_j k_j,   dK_j += s ds_j q,
// with the masks, GQA head map and page layout of the forward pass.
//
// Three kernels:
//   D = dO . O   : per (row, head); computed by the bf16 dQ kernel, by
//                  delta_kernel for fp32 caches;
//   dQ           : bf16 caches: dq_mfma_kernel (128 query rows per workgroup,
//                  K/V tiles staged in LDS, products on MFMA); fp32 caches:
//                  dq_kernel, one wave per (query row, head) on the vector
//                  ALUs;
//   dK / dV      : bf16: dkv_mfma_kernel (128 keys per workgroup, Q / dO
//                  tiles staged in LDS); fp32: dkv_kernel, one wave per (key
//                  position, KV head).  Each key's gradient is accumulated in
//                  one workgroup over all query rows and heads of its group
//                  and written once, so no atomics and no zero fill are
//                  needed.
// dS (like P in the forward pass) is rounded to bf16 before its MFMA.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p) {
  if constexpr (sizeof(T) == 2)
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
  else
    return *p;
}

// Eight consecutive elements (16 bytes of bf16, 32 of fp32) as floats.
template <typename T>
__device__ __forceinline__ void load8(const T *p, float *x) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  }
}

// Two dot products of one row pair (x.a, y.b) where a, b sit in LDS as
// floats (read by every lane at once) and x, y in memory.
template <int D, typename T>
__device__ __forceinline__ void dot2(const T *x, const T *y, const float *a, const float *b, float &sx, float &sy) {
#pragma unroll 4
  for (int c = 0; c < D; c += 8) {
    float xv[8], yv[8];
    load8(x + c, xv);
    load8(y + c, yv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sx = fmaf(xv[i], a[c + i], sx);
      sy = fmaf(yv[i], b[c + i], sy);
    }
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void delta_kernel(BackwardArgs a) {
  const int row = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T *o = (const T *)a.out;
  const T *dout = (const T *)a.d_out;
  for (int h = w; h < a.num_q_heads; h += 4) {
    const size_t base = ((size_t)row * a.num_q_heads + h) * D;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc = fmaf(ld(dout + base + lane + 64 * e), ld(o + base + lane + 64 * e), acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) a.delta[(size_t)row * a.num_q_heads + h] = acc;
  }
}

// acc += a . b on v_mfma_f32_32x32x16_bf16 with the accumulator held in the
// accumulation registers (AGPRs): the dK/dV kernel's long-lived dK and dV
// sums then leave the vector registers to the operands and the score blocks
// the softmax arithmetic reads.  Back-to-back products on one accumulator
// need no wait states; a VALU read of it does (see the reader).
__device__ __forceinline__ void mfma32_agpr(f32x16 &acc, bf16x8 a, bf16x8 b) {
  __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Device-resident integers of sequence b (checked in debug builds against
// the ranges the entry point documents).
__device__ __forceinline__ int bw_q0(const BackwardArgs &a, int b) {
  return checked(a.cu_q[b], 0, 0x7fffffff, kSiteRowOffset, b);
}
__device__ __forceinline__ int bw_qlen(const BackwardArgs &a, int b, int q0) {
  // also bounded by the context bound below, so a valid context exists
  const int hi = min(a.max_q_len, min(a.max_ctx, a.max_pages << a.c.log2_page));
  return checked(a.cu_q[b + 1] - q0, 0, hi, kSiteQueryLen, b);
}
__device__ __forceinline__ int bw_ctx(const BackwardArgs &a, int b, int q_len) {
  return checked(a.ctx_lens[b], q_len, min(a.max_ctx, a.max_pages << a.c.log2_page), kSiteCtxLen, b);
}
// Physical page of logical page n of sequence b.
__device__ __forceinline__ int bw_page(const BackwardArgs &a, int b, int n) {
  return checked(a.block_table[(size_t)b * a.max_pages + n], 0, a.c.num_pages - 1, kSitePageId, b);
}

// Row offset of token `key` of sequence b, KV head hk, in a pool.
__device__ __forceinline__ size_t key_row(const BackwardArgs &a, int b, int key, int hk, int D) {
  const int page = bw_page(a, b, key >> a.c.log2_page);
  return (((size_t)page * a.c.page_size + (key & (a.c.page_size - 1))) * a.c.num_kv_heads + hk) * D;
}

template <int D, typename T>
__global__ __launch_bounds__(64) void dq_kernel(BackwardArgs a) {
  const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int q0 = bw_q0(a, b);
  const int q_len = bw_qlen(a, b, q0);
  if (row >= q_len) return;
  const int ctx = bw_ctx(a, b, q_len);
  const int pos = ctx - q_len + row;
  const int hk = h / a.group;
  const int hi = a.causal ? min(pos, ctx - 1) : ctx - 1;
  const int lo = a.window_left >= 0 ? max(0, pos - a.window_left) : 0;
  const int lane = threadIdx.x;
  const size_t qrow = ((size_t)(q0 + row) * a.num_q_heads + h) * D;
  const T *qv = (const T *)a.q + qrow;
  const T *dov = (const T *)a.d_out + qrow;
  const T *kp = (const T *)a.c.k;
  const T *vp = (const T *)a.c.v;
  const float lse = a.lse[(size_t)(q0 + row) * a.num_q_heads + h];
  const float lse2 = lse * kLog2e;
  const float dlt = a.delta[(size_t)(q0 + row) * a.num_q_heads + h];
  __shared__ float qs[D], dos[D];
  for (int d = lane; d < D; d += 64) {
    qs[d] = ld(qv + d);
    dos[d] = ld(dov + d);
  }
  __syncthreads();
  constexpr int kPer = D / 64;
  float dq[kPer] = {};
  for (int k0 = lo; k0 <= hi && lse != -INFINITY; k0 += 64) {
    const int key = k0 + lane;
    const bool ok = key <= hi;
    float ds = 0.f;
    if (ok) {
      const size_t kr = key_row(a, b, key, hk, D);
      float s = 0.f, dp = 0.f;
      dot2<D>(kp + kr, vp + kr, qs, dos, s, dp);
      const float p = fast_exp2(s * a.scale_log2 - lse2);
      ds = p * (dp - dlt);
    }
    const int n = min(64, hi - k0 + 1);
    for (int j = 0; j < n; ++j) {
      const float dsj = __shfl(ds, j, 64);
      const size_t kr = key_row(a, b, k0 + j, hk, D);
#pragma unroll
      for (int e = 0; e < kPer; ++e) dq[e] = fmaf(dsj, ld(kp + kr + lane + 64 * e), dq[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) a.dq[qrow + lane + 64 * e] = dq[e] * a.scale;
}

template <int D, typename T>
__global__ __launch_bounds__(64) void dkv_kernel(BackwardArgs a) {
  const int key = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int q0 = bw_q0(a, b);
  const int q_len = bw_qlen(a, b, q0);
  const int ctx = bw_ctx(a, b, q_len);
  if (key >= ctx) return;
  const int off = ctx - q_len;  // position of query row 0
  // Rows whose position p sees this key: p >= key (causal), p - key <= W.
  int r_lo = 0, r_hi = q_len - 1;
  if (a.causal) r_lo = max(r_lo, key - off);
  if (a.window_left >= 0) r_hi = min(r_hi, key + a.window_left - off);
  const int lane = threadIdx.x;
  const size_t kr = key_row(a, b, key, hk, D);
  const T *kv = (const T *)a.c.k + kr;
  const T *vv = (const T *)a.c.v + kr;
  const T *qp = (const T *)a.q;
  const T *dop = (const T *)a.d_out;
  __shared__ float ks[D], vs[D];
  for (int d = lane; d < D; d += 64) {
    ks[d] = ld(kv + d);
    vs[d] = ld(vv + d);
  }
  __syncthreads();
  constexpr int kPer = D / 64;
  float dk[kPer] = {}, dv[kPer] = {};
  for (int g = 0; g < a.group; ++g) {
    const int h = hk * a.group + g;
    for (int r0 = r_lo; r0 <= r_hi; r0 += 64) {
      const int row = r0 + lane;
      float p = 0.f, ds = 0.f;
      if (row <= r_hi) {
        const size_t idx = (size_t)(q0 + row) * a.num_q_heads + h;
        const float lse = a.lse[idx];
        if (lse != -INFINITY) {
          float s = 0.f, dp = 0.f;
          dot2<D>(qp + idx * D, dop + idx * D, ks, vs, s, dp);
          p = fast_exp2(s * a.scale_log2 - lse * kLog2e);
          ds = p * (dp - a.delta[idx]);
        }
      }
      const int n = min(64, r_hi - r0 + 1);
      for (int j = 0; j < n; ++j) {
        const float pj = __shfl(p, j, 64);
        const float dsj = __shfl(ds, j, 64);
        const size_t idx = (size_t)(q0 + r0 + j) * a.num_q_heads + h;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          dv[e] = fmaf(pj, ld(dop + idx * D + lane + 64 * e), dv[e]);
          dk[e] = fmaf(dsj, ld(qp + idx * D + lane + 64 * e), dk[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    a.dk[kr + lane + 64 * e] = dk[e] * a.scale;
    a.dv[kr + lane + 64 * e] = dv[e];
  }
}

// dQ on MFMA (bf16 caches).  A workgroup of 4 waves takes 128 query rows
// of one (sequence, head), 32 per wave; per 64-key tile, staged in LDS:
//   S^T  = K . Q^T   and  dP^T = V . dO^T  (v_mfma_f32_32x32x16_bf16, keys on
//                                            M, the wave's rows on N),
//   P^T  = exp(s S^T - lse),  dS^T = P^T (dP^T - D)  (rounded to bf16),
//   dQ^T += K^T . dS^T  (K^T read transposed from the staged K rows).
constexpr int kBwRows = 128;
constexpr int kBwKeys = 64;

template <int D>
struct BwCfg {
  // Staged rows are read both as 16-byte rows and transposed
  // (ds_read_b64_tr_b16); a pitch of 2D + 32 bytes keeps both patterns free
  // of bank conflicts.
  static constexpr int kKRow = 2 * D + 32;   // staged K (and Q) row bytes
  static constexpr int kVRow = 2 * D + 32;   // staged V (and dO) row bytes
  static constexpr int kCpr = D / 8;         // 16-byte chunks per row
  static constexpr int kNs = D / 16;         // k-steps over the head dim
  static constexpr int kNdb = D / 32;        // 32-dim output blocks
  static constexpr int kLoads = kBwKeys * kCpr / 256;
};

template <int D>
__device__ __forceinline__ void dq_tile(const BackwardArgs &a, int qt, int h, int b, unsigned char *ksm,
                                        unsigned char *vsm) {
  using C = BwCfg<D>;
  const int q0 = bw_q0(a, b);
  const int q_len = bw_qlen(a, b, q0);
  if (qt * kBwRows >= q_len) return;  // uniform
  const int ctx = bw_ctx(a, b, q_len);
  const int off = ctx - q_len;
  const int hk = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, g = lane >> 5, gam = lane >> 4, tp = lane & 15;
  const int row = qt * kBwRows + w * 32 + col;
  const int rowc = min(row, q_len - 1);
  const int pos = off + row;
  const size_t qidx = (size_t)(q0 + rowc) * a.num_q_heads + h;
  const __bf16 *qp = (const __bf16 *)a.q + qidx * D;
  const __bf16 *dop = (const __bf16 *)a.d_out + qidx * D;
  bf16x8 bq[C::kNs], bdo[C::kNs];
#pragma unroll
  for (int s = 0; s < C::kNs; ++s) {
    bq[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s + 8 * g);
    bdo[s] = *reinterpret_cast<const bf16x8 *>(dop + 16 * s + 8 * g);
  }
  const float lse = a.lse[qidx];
  const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;  // no visible key: every p = 0
  // D = dO . O of this lane's row: the lane holds half of its dims (those
  // of bdo), the lane 32 apart the other half.  Written for the dK/dV
  // kernel, which runs after this one.
  const __bf16 *op = (const __bf16 *)a.out + qidx * D;
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < C::kNs; ++s) {
    const bf16x8 ov = *reinterpret_cast<const bf16x8 *>(op + 16 * s + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)bdo[s][e], (float)ov[e], dpart);
  }
  const float dlt = dpart + __shfl_xor(dpart, 32, 64);
  if (g == 0 && row < q_len) a.delta[qidx] = dlt;
  // Visible keys of the tile's rows: [k_lo, k_hi].
  const int p_first = off + qt * kBwRows;
  const int p_last = off + min(qt * kBwRows + kBwRows - 1, q_len - 1);
  const int k_lo = a.window_left >= 0 ? max(0, p_first - a.window_left) : 0;
  const int k_hi = a.causal ? min(p_last, ctx - 1) : ctx - 1;
  // This lane's row sees keys [lo_r, hi_r]; every row of the workgroup
  // (valid or not) sees [max_lo, min_hi].
  const int hi_r = a.causal ? min(pos, ctx - 1) : ctx - 1;
  const int lo_r = a.window_left >= 0 ? pos - a.window_left : 0;
  const int min_hi = a.causal ? min(p_first, ctx - 1) : ctx - 1;
  const int max_lo = a.window_left >= 0 ? off + qt * kBwRows + kBwRows - 1 - a.window_left : 0;
  f32x16 acc[C::kNdb];
#pragma unroll
  for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  const size_t row_elems = (size_t)a.c.num_kv_heads * D;
  const __bf16 *kpool = (const __bf16 *)a.c.k + (size_t)hk * D;
  const __bf16 *vpool = (const __bf16 *)a.c.v + (size_t)hk * D;
  const int lrow = tid / C::kCpr, lch = tid % C::kCpr;
  constexpr int kRowsPerPass = 256 / C::kCpr;
  // K/V of a tile through registers into LDS (rows past the context read
  // the last valid row).
  // The page ids of a tile's rows are looked up two tiles ahead and its K /
  // V rows loaded one tile ahead, so neither round trip to memory waits in
  // front of a tile's products (loaded synchronously, the two dependent
  // round trips took about half of each tile's time).
  u32x4 kreg[C::kLoads], vreg[C::kLoads];
  int pgs[C::kLoads];
  auto lookup = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int key = min(kt * kBwKeys + lrow + i * kRowsPerPass, ctx - 1);
      pgs[i] = bw_page(a, b, key >> a.c.log2_page);
    }
  };
  auto fetch = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int key = min(kt * kBwKeys + lrow + i * kRowsPerPass, ctx - 1);
      const size_t ro = ((size_t)pgs[i] * a.c.page_size + (key & (a.c.page_size - 1))) * row_elems + lch * 8;
      kreg[i] = *reinterpret_cast<const u32x4 *>(kpool + ro);
      vreg[i] = *reinterpret_cast<const u32x4 *>(vpool + ro);
    }
  };
  const int kt_beg = k_lo / kBwKeys;
  const int kt_end = k_hi / kBwKeys;
  lookup(kt_beg);
  fetch(kt_beg);
  lookup(min(kt_beg + 1, kt_end));
  for (int kt = kt_beg; kt <= kt_end; ++kt) {
    const int key0 = kt * kBwKeys;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int r = lrow + i * kRowsPerPass;
      *reinterpret_cast<u32x4 *>(ksm + r * C::kKRow + lch * 16) = kreg[i];
      *reinterpret_cast<u32x4 *>(vsm + r * C::kVRow + lch * 16) = vreg[i];
    }
    __syncthreads();
    // Next tile's rows, then the page ids of the one after (clamped to the
    // last tile: the same loads on every path).
    fetch(min(kt + 1, kt_end));
    lookup(min(kt + 2, kt_end));
    f32x16 sacc[2], dpacc[2];
    {
      // Four chains interleaved (u % 4: S^T of key block 0, dP^T of block 0,
      // S^T of block 1, dP^T of block 1; k-step u / 4), their K / V fragments
      // read kAhead products ahead (a ring of registers), so no MFMA waits
      // for an LDS read issued just before it.  The first product of each
      // chain starts from a zero operand.
      constexpr int kSteps = 4 * C::kNs;
      constexpr int kAhead = 8;
      auto rd = [&](int u) __attribute__((always_inline)) {
        const int kb = (u >> 1) & 1, s = u >> 2;
        const unsigned char *base = (u & 1) ? vsm : ksm;
        return *reinterpret_cast<const bf16x8 *>(base + (kb * 32 + col) * C::kKRow + (16 * s + 8 * g) * 2);
      };
      static_assert(C::kKRow == C::kVRow, "K and V staged with one pitch");
      bf16x8 fa[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) fa[u] = rd(u);
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int kb = (u >> 1) & 1, s = u >> 2;
        const bf16x8 cur = fa[u % kAhead];
        if (u + kAhead < kSteps) fa[u % kAhead] = rd(u + kAhead);
        if (u & 1)
          dpacc[kb] = mfma32(cur, bdo[s], s == 0 ? f32x16{} : dpacc[kb]);
        else
          sacc[kb] = mfma32(cur, bq[s], s == 0 ? f32x16{} : sacc[kb]);
        __builtin_amdgcn_sched_barrier(0);  // keep each read kAhead products ahead
      }
    }
    // dS^T = P^T (dP^T - D), masked; element i of block kb is key
    // key0 + kb*32 + (i/4)*8 + g*4 + i%4 of this lane's row.
    bf16x8 bds[4];
    // Every key of the tile visible to every row of the workgroup: no mask.
    const bool interior = key0 >= max_lo && key0 + kBwKeys - 1 <= min_hi;
    // (The choice is made once per tile: inside the loop the compiler
    // evaluated the mask on every element of every tile.)
    auto probs = [&](auto MASKED) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(sacc[kb][i] * a.scale_log2 - lse2);
          if constexpr (decltype(MASKED)::value) {
            const int key = key0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
            p = (key >= lo_r && key <= hi_r) ? p : 0.f;
          }
          bds[2 * kb + (i >> 3)][i & 7] = (__bf16)(p * (dpacc[kb][i] - dlt));
        }
    };
    if (interior)
      probs(std::false_type{});
    else
      probs(std::true_type{});
    // dQ^T += K^T . dS^T over four 16-key steps (product u: step u / kNdb,
    // output block u % kNdb), K^T fragments read kAhead products ahead.
    {
      constexpr int kSteps = 4 * C::kNdb;
      constexpr int kAhead = 4;
      auto rd = [&](int u) __attribute__((always_inline)) {
        const int t = u / C::kNdb, db = u % C::kNdb;
        const int r0 = (t >> 1) * 32 + (t & 1) * 16 + g * 4;
        const unsigned char *p1 = ksm + (r0 + (tp >> 2)) * C::kKRow + (db * 32 + 16 * (gam & 1) + 4 * (tp & 3)) * 2;
        return cat(lds_read_tr16(p1), lds_read_tr16(p1 + 8 * C::kKRow));
      };
      bf16x8 fa[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) fa[u] = rd(u);
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int t = u / C::kNdb, db = u % C::kNdb;
        const bf16x8 cur = fa[u % kAhead];
        if (u + kAhead < kSteps) fa[u % kAhead] = rd(u + kAhead);
        acc[db] = mfma32(cur, bds[t], acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // the tile is restaged next
  }
  if (row < q_len) {
    float *dq = a.dq + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[db * 32 + (i >> 2) * 8 + g * 4 + (i & 3)] = acc[db][i] * a.scale;
  }
}

// dK / dV on MFMA (bf16 caches).  A workgroup of 4 waves takes 128 keys of
// one (sequence, KV head), 32 per wave, their K and V rows held as MFMA B
// operands; for each query head of the GQA group and each 64-row query tile
// that sees the keys (staged in LDS: Q, dO, lse, D):
//   S  = Q . K^T  and  dP = dO . V^T   (rows on M, the wave's keys on N),
//   P  = exp(s S - lse),  dS = P (dP - D)  (rounded to bf16),
//   dV^T += dO^T . P,   dK^T += Q^T . dS   (Q^T, dO^T read transposed).
constexpr int kBwKeyTile = 128;
constexpr int kBwRowTile = 32;  // query rows per step (one 32-row MFMA block)

template <int D>
__device__ __forceinline__ void dkv_tile(const BackwardArgs &a, int kt, int hk, int b, unsigned char *qsm,
                                         unsigned char *dosm, float *lse_s, float *dl_s) {
  using C = BwCfg<D>;
  constexpr int kPitch = C::kKRow;
  const int q0 = bw_q0(a, b);
  const int q_len = bw_qlen(a, b, q0);
  const int ctx = bw_ctx(a, b, q_len);
  if (kt * kBwKeyTile >= ctx) return;  // uniform
  const int off = ctx - q_len;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, g = lane >> 5, gam = lane >> 4, tp = lane & 15;
  const int key = kt * kBwKeyTile + w * 32 + col;  // this lane's key (B-operand column)
  const int keyc = min(key, ctx - 1);
  const size_t row_elems = (size_t)a.c.num_kv_heads * D;
  const int kpage = bw_page(a, b, keyc >> a.c.log2_page);
  const size_t krow = ((size_t)kpage * a.c.page_size + (keyc & (a.c.page_size - 1))) * row_elems + (size_t)hk * D;
  bf16x8 bk[C::kNs], bv[C::kNs];
#pragma unroll
  for (int s = 0; s < C::kNs; ++s) {
    bk[s] = *reinterpret_cast<const bf16x8 *>((const __bf16 *)a.c.k + krow + 16 * s + 8 * g);
    bv[s] = *reinterpret_cast<const bf16x8 *>((const __bf16 *)a.c.v + krow + 16 * s + 8 * g);
  }
  f32x16 dk[C::kNdb], dv[C::kNdb];
#pragma unroll
  for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;
  // Query rows that can see some key of the tile: positions in
  // [first key, last key + W] (causal), rows = positions - off.
  const int key_first = kt * kBwKeyTile, key_last = min(kt * kBwKeyTile + kBwKeyTile - 1, ctx - 1);
  const int r_lo = a.causal ? max(0, key_first - off) : 0;
  const int r_hi = a.window_left >= 0 ? min(q_len - 1, key_last + a.window_left - off) : q_len - 1;
  const int lrow = tid / C::kCpr, lch = tid % C::kCpr;
  constexpr int kRowsPerPass = 256 / C::kCpr;
  constexpr int kLoads = kBwRowTile * C::kCpr / 256;
  // Steps j = (head gi, row tile) pairs; Q, dO, lse, D of a step in
  // registers (rows past the sequence read its last row), one step ahead.
  const int rt0 = r_lo - (r_lo % kBwRowTile);
  const int n_rt = r_hi >= rt0 ? (r_hi - rt0) / kBwRowTile + 1 : 0;
  const int n_steps = a.group * n_rt;
  u32x4 qreg[kLoads], dreg[kLoads];
  float lreg = 0.f, dlreg = 0.f;
  auto load_step = [&](int j) __attribute__((always_inline)) {
    const int h = hk * a.group + j / n_rt;
    const int rt = rt0 + (j % n_rt) * kBwRowTile;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const size_t idx = (size_t)(q0 + min(rt + lrow + i * kRowsPerPass, q_len - 1)) * a.num_q_heads + h;
      qreg[i] = *reinterpret_cast<const u32x4 *>((const __bf16 *)a.q + idx * D + lch * 8);
      dreg[i] = *reinterpret_cast<const u32x4 *>((const __bf16 *)a.d_out + idx * D + lch * 8);
    }
    const int r = rt + (tid & (kBwRowTile - 1));
    const size_t idx = (size_t)(q0 + min(r, q_len - 1)) * a.num_q_heads + h;
    const float l = a.lse[idx];
    lreg = (r < q_len && l != -INFINITY) ? l * kLog2e : INFINITY;  // INFINITY: p = 0
    dlreg = a.delta[idx];
  };
  if (n_steps > 0) load_step(0);
  for (int j = 0; j < n_steps; ++j) {
    const int rt = rt0 + (j % n_rt) * kBwRowTile;
    {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = lrow + i * kRowsPerPass;
        *reinterpret_cast<u32x4 *>(qsm + r * kPitch + lch * 16) = qreg[i];
        *reinterpret_cast<u32x4 *>(dosm + r * kPitch + lch * 16) = dreg[i];
      }
      if (tid < kBwRowTile) {
        lse_s[tid] = lreg;
        dl_s[tid] = dlreg;
      }
      __syncthreads();
      load_step(min(j + 1, n_steps - 1));  // unconditional: exact wait counts
      constexpr int kMb = kBwRowTile / 32;  // 32-row blocks
      static_assert(kMb == 1, "one 32-row block per step");
      // lse and D of this lane's 16 rows (rows q4*8 + g*4 + 0..3: four
      // vectors each), read before the products so their latency hides
      // behind them.
      f32x4 l4v[4], d4v[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        l4v[q4] = *reinterpret_cast<const f32x4 *>(lse_s + q4 * 8 + g * 4);
        d4v[q4] = *reinterpret_cast<const f32x4 *>(dl_s + q4 * 8 + g * 4);
      }
      f32x16 sacc[kMb], dpacc[kMb];
      {
        // S and dP alternate (u even: Q . K^T, u odd: dO . V^T, k-step u / 2);
        // their Q / dO fragments are read kAhead products ahead (a ring of
        // registers), so each MFMA finds its operand in place instead of
        // waiting for an LDS read issued just before it.  The first product
        // of each starts from a zero operand.
        constexpr int kSteps = 2 * C::kNs;
        constexpr int kAhead = 6;
        auto rd = [&](int u) __attribute__((always_inline)) {
          const int ro = col * kPitch + (16 * (u >> 1) + 8 * g) * 2;
          return *reinterpret_cast<const bf16x8 *>(((u & 1) ? dosm : qsm) + ro);
        };
        bf16x8 fa[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) fa[u] = rd(u);
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
          const int s = u >> 1;
          const bf16x8 cur = fa[u % kAhead];
          if (u + kAhead < kSteps) fa[u % kAhead] = rd(u + kAhead);
          if (u & 1)
            dpacc[0] = mfma32(cur, bv[s], s == 0 ? f32x16{} : dpacc[0]);
          else
            sacc[0] = mfma32(cur, bk[s], s == 0 ? f32x16{} : sacc[0]);
          __builtin_amdgcn_sched_barrier(0);  // keep each read kAhead products ahead
        }
      }
      // Element i of block mb is row rt + mb*32 + (i/4)*8 + g*4 + i%4 against
      // this lane's key; 16-row step t of the products below holds block
      // t/2, elements 8(t%2) .. 8(t%2)+7.
      bf16x8 bp[2 * kMb], bds[2 * kMb];
      // Every (row, key) pair of the step visible: no mask (the usual case
      // away from the diagonal and the window's edge).
      const bool interior = key_first + kBwKeyTile <= ctx && rt + kBwRowTile <= q_len &&
                            (!a.causal || key_first + kBwKeyTile - 1 <= off + rt) &&
                            (a.window_left < 0 || off + rt + kBwRowTile - 1 - key_first <= a.window_left);
      // P and dS; the mask is decided once per step (interior steps skip it).
      auto probs = [&](auto MASKED) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q4 = i >> 2, e = i & 3;
          const int rr = q4 * 8 + g * 4 + e;
          float p = fast_exp2(sacc[0][i] * a.scale_log2 - l4v[q4][e]);
          if constexpr (decltype(MASKED)::value) {
            const int pos = off + rt + rr;
            bool vis = key < ctx && rt + rr < q_len;
            if (a.causal) vis = vis && key <= pos;
            if (a.window_left >= 0) vis = vis && pos - key <= a.window_left;
            p = vis ? p : 0.f;
          }
          bp[i >> 3][i & 7] = (__bf16)p;
          bds[i >> 3][i & 7] = (__bf16)(p * (dpacc[0][i] - d4v[q4][e]));
        }
      };
      if (interior)
        probs(std::false_type{});
      else
        probs(std::true_type{});
      // dV^T += dO^T . P and dK^T += Q^T . dS over two 16-row steps (product
      // u: step u / (2 kNdb), output block (u / 2) % kNdb, dV for even u and
      // dK for odd), the transposed fragments read kAhead products ahead.
      {
        constexpr int kSteps = 4 * C::kNdb;
        constexpr int kAhead = 4;
        auto rd = [&](int u) __attribute__((always_inline)) {
          const int t = u / (2 * C::kNdb), db = (u >> 1) % C::kNdb;
          const int r0 = (t >> 1) * 32 + (t & 1) * 16 + g * 4;
          const int c = (db * 32 + 16 * (gam & 1) + 4 * (tp & 3)) * 2;
          const unsigned char *pr = ((u & 1) ? qsm : dosm) + (r0 + (tp >> 2)) * kPitch + c;
          return cat(lds_read_tr16(pr), lds_read_tr16(pr + 8 * kPitch));
        };
        bf16x8 fa[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) fa[u] = rd(u);
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
          const int t = u / (2 * C::kNdb), db = (u >> 1) % C::kNdb;
          const bf16x8 cur = fa[u % kAhead];
          if (u + kAhead < kSteps) fa[u % kAhead] = rd(u + kAhead);
          if (u & 1)
            mfma32_agpr(dk[db], cur, bds[t]);
          else
            mfma32_agpr(dv[db], cur, bp[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();  // the tiles are restaged next
    }
  }
  // The accumulators were written by MFMAs the compiler does not see
  // (asm): wait out the MFMA-to-VALU read latency before reading them.
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if (key < ctx) {
    float *dkr = a.dk + krow;
    float *dvr = a.dv + krow;
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = db * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        dkr[d] = dk[db][i] * a.scale;
        dvr[d] = dv[db][i];
      }
  }
}

// dQ: a workgroup takes the pair of query tiles (n-1-p, p), heavier first:
// under a causal mask the key-tile counts of the two add up to the same
// total for every p, so all workgroups carry equal work.  (One tile per
// workgroup, all resident at once, left the kernel as long as its heaviest
// tile, about twice the average.)  One workgroup per CU: the prefetched
// tile needs more than 256 registers per lane.
template <int D>
__global__ __launch_bounds__(256) void dq_mfma_kernel(BackwardArgs a) {
  using C = BwCfg<D>;
  __shared__ __align__(16) unsigned char ksm[kBwKeys * C::kKRow];
  __shared__ __align__(16) unsigned char vsm[kBwKeys * C::kVRow];
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = (bw_qlen(a, b, bw_q0(a, b)) + kBwRows - 1) / kBwRows;
  if (p >= (n + 1) / 2) return;  // uniform
  dq_tile<D>(a, n - 1 - p, h, b, ksm, vsm);
  if (n - 1 - p != p) {
    __syncthreads();
    dq_tile<D>(a, p, h, b, ksm, vsm);
  }
}

// dK / dV: one workgroup per CU (its accumulators need more than 256
// registers per lane).  Under a causal mask the work of key tile i shrinks
// with i; a workgroup takes the pair of tiles (p, n-1-p), so all carry the
// same.
template <int D>
__global__ __launch_bounds__(256) void dkv_mfma_kernel(BackwardArgs a) {
  using C = BwCfg<D>;
  __shared__ __align__(16) unsigned char qsm[kBwRowTile * C::kKRow];
  __shared__ __align__(16) unsigned char dosm[kBwRowTile * C::kKRow];
  __shared__ float lse_s[kBwRowTile], dl_s[kBwRowTile];
  const int p = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int n = (bw_ctx(a, b, bw_qlen(a, b, bw_q0(a, b))) + kBwKeyTile - 1) / kBwKeyTile;
  if (p >= (n + 1) / 2) return;  // uniform
  dkv_tile<D>(a, p, hk, b, qsm, dosm, lse_s, dl_s);
  if (n - 1 - p != p) {
    __syncthreads();
    dkv_tile<D>(a, n - 1 - p, hk, b, qsm, dosm, lse_s, dl_s);
  }
}

template <int D, typename T>
hipError_t launch_t(const BackwardArgs &a, hipStream_t s) {
  hipError_t e = hipSuccess;
  if constexpr (sizeof(T) != 2) {  // the bf16 dQ kernel computes D itself
    hipLaunchKernelGGL((delta_kernel<D, T>), dim3(a.total_q), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((dq_mfma_kernel<D>),
                       dim3(((a.max_q_len + kBwRows - 1) / kBwRows + 1) / 2, a.num_q_heads, a.batch), dim3(256), 0, s,
                       a);
  else
    hipLaunchKernelGGL((dq_kernel<D, T>), dim3(a.max_q_len, a.num_q_heads, a.batch), dim3(64), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((dkv_mfma_kernel<D>), dim3(((a.max_ctx + kBwKeyTile - 1) / kBwKeyTile + 1) / 2, a.c.num_kv_heads,
                                                  a.batch),
                       dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dkv_kernel<D, T>), dim3(a.max_ctx, a.c.num_kv_heads, a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

PA_DEFINE_FAULT_READER(take_fault_backward)

hipError_t launch_backward(const BackwardArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.total_q == 0) return hipSuccess;
  const bool bf = a.c.dtype == 1;
  if (a.c.head_dim == 64) return bf ? launch_t<64, __bf16>(a, s) : launch_t<64, float>(a, s);
  return bf ? launch_t<128, __bf16>(a, s) : launch_t<128, float>(a, s);
}

}  // namespace pa
