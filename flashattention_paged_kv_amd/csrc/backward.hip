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
// Three kernels, all fp32 arithmetic on the vector ALUs:
//   delta_kernel : D = dO . O per (row, head);
//   dq_kernel    : one wave per (query row, head); keys one per lane for the
//                  dot products, then the wave accumulates dQ with lanes over
//                  head dims;
//   dkv_kernel   : one wave per (key position, KV head); query rows (of all
//                  G query heads of the group) one per lane, then dK / dV
//                  accumulated with lanes over head dims and written once, so
//                  no atomics and no zero fill are needed.
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

// Row offset of token `key` of sequence b, KV head hk, in a pool.
__device__ __forceinline__ size_t key_row(const BackwardArgs &a, int b, int key, int hk, int D) {
  const int page = a.block_table[(size_t)b * a.max_pages + (key >> a.c.log2_page)];
  return (((size_t)page * a.c.page_size + (key & (a.c.page_size - 1))) * a.c.num_kv_heads + hk) * D;
}

template <int D, typename T>
__global__ __launch_bounds__(64) void dq_kernel(BackwardArgs a) {
  const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int q0 = a.cu_q[b];
  const int q_len = a.cu_q[b + 1] - q0;
  if (row >= q_len) return;
  const int ctx = a.ctx_lens[b];
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
  const int ctx = a.ctx_lens[b];
  if (key >= ctx) return;
  const int q0 = a.cu_q[b];
  const int q_len = a.cu_q[b + 1] - q0;
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

template <int D, typename T>
hipError_t launch_t(const BackwardArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((delta_kernel<D, T>), dim3(a.total_q), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<D, T>), dim3(a.max_q_len, a.num_q_heads, a.batch), dim3(64), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((dkv_kernel<D, T>), dim3(a.max_ctx, a.c.num_kv_heads, a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.total_q == 0) return hipSuccess;
  const bool bf = a.c.dtype == 1;
  if (a.c.head_dim == 64) return bf ? launch_t<64, __bf16>(a, s) : launch_t<64, float>(a, s);
  return bf ? launch_t<128, __bf16>(a, s) : launch_t<128, float>(a, s);
}

}  // namespace pa
