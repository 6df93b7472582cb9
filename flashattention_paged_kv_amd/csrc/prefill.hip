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
// Work split: one workgroup of 4 waves = 128 query rows of one (sequence,
// query head); wave w owns rows 32w..32w+31.  Query tiles are launched last
// tile first, so the longest causal rows start earliest.  For each 64-key
// tile, K and V rows are gathered from their pages into LDS; each wave
// computes S^T = K . Q^T (v_mfma_f32_32x32x16_bf16, keys on M, its 32 query
// rows on N, Q^T held in registers for the whole loop), applies the mask and
// the online softmax to the S^T registers (one query per lane column, so only
// one cross-lane max per tile), and accumulates O^T += V^T . P^T with V^T read
// transposed from LDS by ds_read_b64_tr_b16 and P^T taken straight from the
// S^T registers (rounded to bf16).  exp is computed as exp2 with log2(e)
// folded into the scale.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_rowwise_f32(const PrefillArgs &a, hipStream_t s);

constexpr int kPfRows = 128;
constexpr int kPfKeys = 64;

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int kKRow = 2 * D + 16;  // staged K row bytes (bank spread for b128 reads)
  constexpr int kVRow = 2 * D + 64;  // staged V row bytes (bank spread for transpose reads)
  constexpr int kCpr = D / 8;        // 16-byte chunks per row
  constexpr int kNs = D / 16;        // QK k-steps
  constexpr int kNdb = D / 32;       // O^T 32-dim blocks
  __shared__ __align__(16) unsigned char ks[kPfKeys * kKRow];
  __shared__ __align__(16) unsigned char vs[kPfKeys * kVRow];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int h = blockIdx.x;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = a.cu_q[b];
  const int q_len = a.cu_q[b + 1] - q0;
  if (qt * kPfRows >= q_len) return;
  const int ctx = a.ctx_lens[b];
  const int off = ctx - q_len;
  const int hk = h / a.group;
  const int col = lane & 31;
  const int g = lane >> 5;
  const int qrow = qt * kPfRows + w * 32 + col;
  const int pos = off + qrow;
  const int W = a.window_left;
  const int causal = a.causal;

  // Q^T operand: lane (query column col, k-group g), dims 16s + 8g .. +7.
  const __bf16 *qp = (const __bf16 *)a.q + ((size_t)(q0 + min(qrow, q_len - 1)) * a.num_q_heads + h) * D;
  bf16x8 bq[kNs];
#pragma unroll
  for (int s = 0; s < kNs; ++s) bq[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 16 * s + 8 * g));

  const int p_first = off + qt * kPfRows;
  const int p_last = off + min(qt * kPfRows + kPfRows - 1, q_len - 1);
  const int k_lo = W >= 0 ? max(0, p_first - W) : 0;
  const int k_hi = causal ? min(p_last + 1, ctx) : ctx;  // exclusive

  const int P = a.c.page_size;
  const int lp = a.c.log2_page;
  const size_t row_bytes = (size_t)a.c.num_kv_heads * D * 2;
  const char *kbase = (const char *)a.c.k + (size_t)hk * D * 2;
  const char *vbase = (const char *)a.c.v + (size_t)hk * D * 2;
  const int32_t *bt = a.block_table + (size_t)b * a.max_pages;

  float m = -INFINITY;
  float lsum = 0.f;
  f32x16 o[kNdb];
#pragma unroll
  for (int db = 0; db < kNdb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  const int gam = lane >> 4;
  const int tp = lane & 15;
  for (int key0 = (k_lo / kPfKeys) * kPfKeys; key0 < k_hi; key0 += kPfKeys) {
    __syncthreads();
    for (int c = threadIdx.x; c < kPfKeys * kCpr; c += blockDim.x) {
      const int row = c / kCpr;
      const int ch = c % kCpr;
      const int key = key0 + row;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < ctx) {
        const size_t ro = ((size_t)bt[key >> lp] * P + (key & (P - 1))) * row_bytes + ch * 16;
        kv = *reinterpret_cast<const uint4 *>(kbase + ro);
        vv = *reinterpret_cast<const uint4 *>(vbase + ro);
      }
      *reinterpret_cast<uint4 *>(ks + row * kKRow + ch * 16) = kv;
      *reinterpret_cast<uint4 *>(vs + row * kVRow + ch * 16) = vv;
    }
    __syncthreads();

    // S^T = K . Q^T: two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < kNs; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(ks + (kb * 32 + col) * kKRow + (16 * s + 8 * g) * 2);
        sacc[kb] = mfma32(ka, bq[s], sacc[kb]);
      }
    }

    // Mask (only tiles that cross a boundary) and online softmax.
    const bool edge = (causal && key0 + kPfKeys - 1 > p_first) || (W >= 0 && key0 < p_last - W) ||
                      (key0 + kPfKeys > ctx);
    float x[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        float v = sacc[kb][i] * a.scale_log2;
        if (edge) {
          const bool vis = key < ctx && (!causal || key <= pos) && (W < 0 || pos - key <= W);
          v = vis ? v : -INFINITY;
        }
        x[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // row has seen no key yet
    const float corr = fast_exp2(m - m_use);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[kb][i] = fast_exp2(x[kb][i] - m_use);
        ps += x[kb][i];
      }
    lsum = lsum * corr + ps;
    m = m_new;
#pragma unroll
    for (int db = 0; db < kNdb; ++db) o[db] *= corr;

    // O^T += V^T . P^T over four 16-key steps.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1;
      const int half = t & 1;
      bf16x8 bp;
#pragma unroll
      for (int e = 0; e < 8; ++e) bp[e] = (__bf16)x[kb][8 * half + e];
      const int r0 = kb * 32 + half * 16 + g * 4;
#pragma unroll
      for (int db = 0; db < kNdb; ++db) {
        const unsigned char *p1 = vs + (r0 + (tp >> 2)) * kVRow + (db * 32 + 16 * (gam & 1) + 4 * (tp & 3)) * 2;
        const bf16x8 va = cat(lds_read_tr16(p1), lds_read_tr16(p1 + 8 * kVRow));
        o[db] = mfma32(va, bp, o[db]);
      }
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (qrow < q_len) {
    const float inv = 1.f / ltot;
    uint16_t *orow = (uint16_t *)a.out + ((size_t)(q0 + qrow) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < kNdb; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = f32_to_bf16_bits(o[db][4 * j] * inv) | ((uint32_t)f32_to_bf16_bits(o[db][4 * j + 1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_bits(o[db][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16_bits(o[db][4 * j + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + db * 32 + j * 8 + g * 4) = make_uint2(lo, hi);
      }
    if (a.lse != nullptr && g == 0) a.lse[(size_t)(q0 + qrow) * a.num_q_heads + h] = (m + __log2f(ltot)) * kLn2;
  }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.max_q_len == 0) return hipSuccess;
  if (a.c.dtype == 0) return launch_rowwise_f32(a, s);
  dim3 grid(a.num_q_heads, (a.max_q_len + kPfRows - 1) / kPfRows, a.batch);
  if (a.c.head_dim == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
