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
// Work split: one workgroup = (sequence b, KV head hk, split s of
// split_tokens consecutive keys); all G = Hq/Hkv query heads of hk are handled
// together so each K/V byte is read from HBM once.  Each of the 4 waves takes
// every 4th 32-key tile of the split.
//
// Per 32-key tile a wave computes S^T = K . Q^T with v_mfma_f32_16x16x32_bf16
// (keys on the M side, query heads on the N side, zero-padded to 16), the
// online softmax on the S^T registers, then O^T += V^T . P^T with V staged
// through LDS and read back transposed by ds_read_b64_tr_b16 (ds_read_b64_tr_b8
// for int8, converted to exact bf16 integers).  K/V tiles are loaded with
// 16-byte global loads one tile ahead of the one being computed.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kDecWaves = 4;
constexpr int kDecTile = 32;            // keys per wave iteration
constexpr int kMaxSplitPages = 520;     // split_tokens / page_size + 1

int decode_split_tokens(int batch, int num_kv_heads, int max_pages_per_seq, int page_size) {
  // Aim for about 4096 workgroups at the largest possible contexts (about
  // 16 per CU), with splits a power of two between 256 and 8192 keys that
  // is a multiple of the page size.
  const long long upper = (long long)batch * num_kv_heads * max_pages_per_seq * page_size;
  long long want = upper / 4096;
  int s = 256;
  while (s < want && s < 8192) s <<= 1;
  if (s < page_size) s = page_size;
  if (const char *env = getenv("PAGEDATTN_SPLIT_TOKENS")) {
    int v = atoi(env);
    if (v >= 128 && v <= 8192 && (v & (v - 1)) == 0 && v >= page_size) s = v;
  }
  return s;
}

template <int D, bool I8>
struct DecodeCfg {
  static constexpr int kEsz = I8 ? 1 : 2;
  static constexpr int kCpr = D * kEsz / 16;               // 16-byte chunks per cache row
  static constexpr int kVLoads = kDecTile * kCpr / 64;     // V loads per lane per tile
  static constexpr int kKPerBlock = I8 ? D / 64 : D / 32;  // K loads per lane per 16-key block
  static constexpr int kKLoads = 2 * kKPerBlock;
  static constexpr int kVRow = I8 ? D + 16 : 2 * D + 32;   // staged V row bytes (bank spread)
  static constexpr int kNdb = D / 16;                      // 16-dim output blocks
  static constexpr int kNst = D / 32;                      // 32-dim QK k-steps
  static constexpr int kStage = kDecWaves * kDecTile * kVRow;
  static constexpr int kMerge = kDecWaves * 16 * D * 4 + 2 * kDecWaves * 16 * 4;
  static constexpr int kSmem = kStage > kMerge ? kStage : kMerge;
};

template <int D, bool I8>
struct TileRegs {
  uint4 k[DecodeCfg<D, I8>::kKLoads];
  uint4 v[DecodeCfg<D, I8>::kVLoads];
};

// Position (0..31) inside the tile of S^T row i (0..3) of 16-key block kb held
// by lane group g.  bf16: block kb = keys 16kb..16kb+15.  int8: lane group g
// holds the 8 consecutive keys 8g..8g+7 so that one ds_read_b64_tr_b8 gives a
// lane its V^T operand.
template <bool I8>
__device__ __forceinline__ int tile_key(int kb, int g, int i) {
  return I8 ? 8 * g + 4 * kb + i : 16 * kb + 4 * g + i;
}

template <int D, bool I8>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  using C = DecodeCfg<D, I8>;
  __shared__ __align__(16) unsigned char smem[C::kSmem];
  __shared__ int s_pages[kMaxSplitPages];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = a.ctx_lens[b];
  const int S = a.split_tokens;
  const int lo = a.window_left >= 0 ? max(0, ctx - 1 - a.window_left) : 0;
  const int k_begin = max(split * S, lo);
  const int k_end = min((split + 1) * S, ctx);
  if (k_begin >= k_end) return;

  const int P = a.c.page_size;
  const int lp = a.c.log2_page;
  const int hkv = a.c.num_kv_heads;
  const int pg0 = k_begin >> lp;
  const int pg1 = (k_end - 1) >> lp;
  for (int i = threadIdx.x; i <= pg1 - pg0; i += blockDim.x)
    s_pages[i] = a.block_table[(size_t)b * a.max_pages + pg0 + i];
  __syncthreads();

  const size_t row_bytes = (size_t)hkv * D * C::kEsz;
  const char *kbase = (const char *)a.c.k + (size_t)hk * D * C::kEsz;
  const char *vbase = (const char *)a.c.v + (size_t)hk * D * C::kEsz;
  // Keys outside [k_begin, k_end) are clamped to a page of this split, so the
  // address stays inside an assigned page; their data is masked or zeroed.
  auto page_of = [&](int key) {
    const int kc = min(max(key, k_begin), k_end - 1);
    return s_pages[(kc >> lp) - pg0];
  };
  auto row_ptr = [&](const char *base, int key) {
    return base + ((size_t)page_of(key) * P + (key & (P - 1))) * row_bytes;
  };

  // Q^T operand: lane (head column r16, k-group g).
  const int G = a.group;
  const bool head_ok = r16 < G;
  const __bf16 *qrow = (const __bf16 *)a.q + ((size_t)b * a.num_q_heads + hk * G + (head_ok ? r16 : 0)) * D;
  bf16x8 bq[C::kNst];
#pragma unroll
  for (int st = 0; st < C::kNst; ++st) {
    const int dim = I8 ? 64 * (st >> 1) + 16 * g + 8 * (st & 1) : 32 * st + 8 * g;
    uint4 raw = head_ok ? *reinterpret_cast<const uint4 *>(qrow + dim) : make_uint4(0, 0, 0, 0);
    bq[st] = __builtin_bit_cast(bf16x8, raw);
  }

  auto load_tile = [&](int t, TileRegs<D, I8> &R) {
    const int key0 = t * kDecTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = r16;
      const int key = key0 + (I8 ? 8 * (r >> 2) + 4 * kb + (r & 3) : 16 * kb + r);
      const char *rp = row_ptr(kbase, key);
#pragma unroll
      for (int j = 0; j < C::kKPerBlock; ++j) {
        const int dim = I8 ? 64 * j + 16 * g : 32 * j + 8 * g;
        R.k[kb * C::kKPerBlock + j] = *reinterpret_cast<const uint4 *>(rp + dim * C::kEsz);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kVLoads; ++i) {
      const int c = i * 64 + lane;
      const char *rp = row_ptr(vbase, key0 + c / C::kCpr);
      R.v[i] = *reinterpret_cast<const uint4 *>(rp + (c % C::kCpr) * 16);
    }
  };

  float m = -INFINITY;
  float lsum = 0.f;
  f32x4 o[C::kNdb];
#pragma unroll
  for (int db = 0; db < C::kNdb; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t0 = k_begin / kDecTile;
  const int t1 = (k_end + kDecTile - 1) / kDecTile;
  unsigned char *vs = smem + w * kDecTile * C::kVRow;
  TileRegs<D, I8> cur, nxt;
  int t = t0 + w;
  if (t < t1) load_tile(t, cur);
  for (; t < t1; t += kDecWaves) {
    const int key0 = t * kDecTile;
    if (t + kDecWaves < t1) load_tile(t + kDecWaves, nxt);

    // Stage this tile's V rows (zero outside [k_begin, k_end): those slots
    // may hold anything, and 0 * NaN would poison the sum).
#pragma unroll
    for (int i = 0; i < C::kVLoads; ++i) {
      const int c = i * 64 + lane;
      const int row = c / C::kCpr;
      const int key = key0 + row;
      const uint4 val = (key >= k_begin && key < k_end) ? cur.v[i] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(vs + row * C::kVRow + (c % C::kCpr) * 16) = val;
    }

    // S^T = K . Q^T for the two 16-key blocks.
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < C::kNst; ++st) {
        bf16x8 ka;
        if constexpr (I8) {
          const uint4 raw = cur.k[kb * C::kKPerBlock + (st >> 1)];
          ka = (st & 1) ? i8x8_to_bf16x8(raw.z, raw.w) : i8x8_to_bf16x8(raw.x, raw.y);
        } else {
          ka = __builtin_bit_cast(bf16x8, cur.k[kb * C::kKPerBlock + st]);
        }
        sacc[kb] = mfma16(ka, bq[st], sacc[kb]);
      }
    }

    float sl = a.scale_log2;
    float vsc = 1.f;
    if constexpr (I8) {
      const int page = page_of(key0 + 8 * g);
      sl *= a.c.k_scales[(size_t)page * hkv + hk];
      vsc = a.c.v_scales[(size_t)page * hkv + hk];
    }
    const bool edge = key0 < k_begin || key0 + kDecTile > k_end;
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + tile_key<I8>(kb, g, i);
        float v = sacc[kb][i] * sl;
        if (edge && (key < k_begin || key >= k_end)) v = -INFINITY;
        x[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx);  // finite: every tile holds a visible key
    const float corr = fast_exp2(m - m_new);
    float ps = 0.f;
    bf16x8 bp;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(x[kb][i] - m_new);
        ps += p;
        bp[kb * 4 + i] = (__bf16)(p * vsc);
      }
    lsum = lsum * corr + ps;
    m = m_new;

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
      o[db] *= corr;
      o[db] = mfma16(va, bp, o[db]);
    }
    cur = nxt;
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // Merge the 4 waves' (m, l, O) through LDS.
  __syncthreads();
  float *wo = reinterpret_cast<float *>(smem);
  float *wm = wo + kDecWaves * 16 * D;
  float *wl = wm + kDecWaves * 16;
  if (head_ok) {
#pragma unroll
    for (int db = 0; db < C::kNdb; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[(w * 16 + r16) * D + db * 16 + 4 * g + i] = o[db][i];
    if (g == 0) {
      wm[w * 16 + r16] = m;
      wl[w * 16 + r16] = lsum;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int c = e / D;
    const int d = e % D;
    float big_m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) big_m = fmaxf(big_m, wm[ww * 16 + c]);
    float big_l = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float f = fast_exp2(wm[ww * 16 + c] - big_m);
      big_l += wl[ww * 16 + c] * f;
      acc += wo[(ww * 16 + c) * D + d] * f;
    }
    const size_t idx = ((size_t)b * a.num_q_heads + hk * G + c) * a.max_splits + split;
    a.ws_o[idx * D + d] = acc;
    if (d == 0) {
      a.ws_ml[idx * 2] = big_m;
      a.ws_ml[idx * 2 + 1] = big_l;
    }
  }
}

// Merge the splits of one (sequence, query head): M = max m_s,
// L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M) / L.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int ctx = a.ctx_lens[b];
  const int S = a.split_tokens;
  const int lo = a.window_left >= 0 ? max(0, ctx - 1 - a.window_left) : 0;
  const int s_lo = lo / S;
  const int s_hi = (ctx - 1) / S;
  const size_t base = ((size_t)b * a.num_q_heads + h) * a.max_splits;
  float big_m = -INFINITY;
  for (int s = s_lo; s <= s_hi; ++s) big_m = fmaxf(big_m, a.ws_ml[(base + s) * 2]);
  constexpr int kPer = D / 64;
  float acc[kPer] = {};
  float big_l = 0.f;
  for (int s = s_lo; s <= s_hi; ++s) {
    const float f = fast_exp2(a.ws_ml[(base + s) * 2] - big_m);
    big_l += a.ws_ml[(base + s) * 2 + 1] * f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) acc[j] += a.ws_o[(base + s) * D + threadIdx.x + 64 * j] * f;
  }
  const float inv = 1.f / big_l;
  uint16_t *out = (uint16_t *)a.out + ((size_t)b * a.num_q_heads + h) * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) out[threadIdx.x + 64 * j] = f32_to_bf16_bits(acc[j] * inv);
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[(size_t)b * a.num_q_heads + h] = (big_m + __log2f(big_l)) * kLn2;
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
  const int q0 = cu_q != nullptr ? cu_q[b] : b;
  const int q_len = cu_q != nullptr ? cu_q[b + 1] - q0 : 1;
  if (row >= q_len) return;
  const int ctx = ctx_lens[b];
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
    const int page = block_table[(size_t)b * max_pages + (key >> c.log2_page)];
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
  const float inv = 1.f / l;
  float *orow = out + ((size_t)(q0 + row) * num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[lane + 64 * e] = o[e] * inv;
  if (lse != nullptr && lane == 0) lse[(size_t)(q0 + row) * num_q_heads + h] = (m + __log2f(l)) * kLn2;
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

template <int D, bool I8>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  dim3 grid(a.max_splits, a.c.num_kv_heads, a.batch);
  hipLaunchKernelGGL((decode_split_kernel<D, I8>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(a.num_q_heads, a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const bool i8 = a.c.dtype == 2;
  if (a.c.head_dim == 64) return i8 ? launch_decode_t<64, true>(a, s) : launch_decode_t<64, false>(a, s);
  return i8 ? launch_decode_t<128, true>(a, s) : launch_decode_t<128, false>(a, s);
}

}  // namespace pa
