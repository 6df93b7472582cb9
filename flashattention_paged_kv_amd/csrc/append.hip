// KV-cache append (scatter of new token rows into their page slots) and the
// int8 page quantiser.
//
// Append follows the cache-growth step of "大模型推理优化实战：KV Cache + Flash
// Attention，让 Token 生成快 3 倍" (KV Cache section): new K/V rows are added to
// the cache; the slot comes from the page table of "Flash Attention与Paged KV
// Cache优化大模型计算效率" section 3.2 (token t -> page t / P, slot t % P).
// A token's row of all KV heads is contiguous both in the input and in the
// page ([P, Hkv, D] pages), so the kernel is a row copy with 16-byte lanes.
//
// The quantiser follows section 3.2 of "LLM推理系统优化：KV缓存管理与动态批处理
// 技术" (group quantisation) with 8 bits and one group per (page, KV head).
//
// Appending into an int8 cache keeps that grouping for pages that are only
// partly filled: every (page, KV head) group that receives rows is
// requantised over its valid slots (those of positions before the
// sequence's new end), the old slots entering as code * old scale.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kAppendRowsPerBlock = 4;

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int n0 = checked(a.cu_new[b], 0, 0x7fffffff, kSiteRowOffset, b);
  const int n_new = checked(a.cu_new[b + 1] - n0, 0, min(a.max_new, a.max_pages << a.log2_page), kSiteNewLen, b);
  const int r_begin = blockIdx.x * kAppendRowsPerBlock;
  if (r_begin >= n_new) return;
  const int start = checked(a.start_pos != nullptr ? a.start_pos[b] : a.ctx_lens[b] - n_new, 0,
                            (a.max_pages << a.log2_page) - n_new, kSiteStartPos, b);
  const int chunks = a.row_bytes >> 4;
  const int rows = min(kAppendRowsPerBlock, n_new - r_begin);
  for (int c = threadIdx.x; c < rows * chunks; c += blockDim.x) {
    const int r = r_begin + c / chunks;
    const int ch = c % chunks;
    const int pos = start + r;
    const int page = checked(a.block_table[(size_t)b * a.max_pages + (pos >> a.log2_page)], 0, a.num_pages - 1,
                             kSitePageId, b);
    const size_t dst_row = (size_t)page * a.page_size + (pos & (a.page_size - 1));
    const size_t src_row = (size_t)(n0 + r);
    const uint4 kv = reinterpret_cast<const uint4 *>(a.k_new)[src_row * chunks + ch];
    const uint4 vv = reinterpret_cast<const uint4 *>(a.v_new)[src_row * chunks + ch];
    reinterpret_cast<uint4 *>(a.k_pages)[dst_row * chunks + ch] = kv;
    reinterpret_cast<uint4 *>(a.v_pages)[dst_row * chunks + ch] = vv;
  }
}

PA_DEFINE_FAULT_READER(take_fault_append)

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.max_new == 0) return hipSuccess;
  dim3 grid((a.max_new + kAppendRowsPerBlock - 1) / kAppendRowsPerBlock, a.batch);
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// One workgroup per (page, KV head): the group's P x D bf16 values sit in P
// rows of D contiguous elements, rows num_kv_heads * D apart.
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  const int page = blockIdx.x;
  const int hk = blockIdx.y;
  const int d = a.head_dim;
  const int per_row = d >> 3;  // 8 bf16 per 16-byte chunk
  const int n_chunks = a.page_size * per_row;
  const size_t row_stride = (size_t)a.num_kv_heads * d;
  const size_t base = ((size_t)page * a.page_size * a.num_kv_heads + hk) * d;

  float amax = 0.f;
  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) {
    const int slot = c / per_row, ch = c % per_row;
    const uint4 v = *reinterpret_cast<const uint4 *>(a.src + base + slot * row_stride + ch * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[j] >> 16)));
    }
  }
  __shared__ float red[256];
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  amax = red[0];
  const float scale = (amax == 0.f) ? 1.f : amax / 127.f;  // IEEE division
  if (threadIdx.x == 0) a.scales[(size_t)page * a.num_kv_heads + hk] = scale;

  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) {
    const int slot = c / per_row, ch = c % per_row;
    const size_t off = base + slot * row_stride + ch * 8;
    const uint4 v = *reinterpret_cast<const uint4 *>(a.src + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
      float y = bf16_bits_to_f32(bits) / scale;  // IEEE division
      y = fminf(fmaxf(y, -128.f), 127.f);
      const int code = (int)rintf(y);            // round half to even
      packed[j >> 2] |= ((uint32_t)code & 0xffu) << (8 * (j & 3));
    }
    *reinterpret_cast<uint2 *>(a.codes + off) = make_uint2(packed[0], packed[1]);
  }
}

// One workgroup per (touched logical page j of sequence b, KV head hk), K
// then V.  Pass 1: the largest magnitude over the group's valid slots (old
// slots as code * old scale in float32, new slots from the bf16 rows).
// Pass 2: scale = largest / 127 (1 if 0; IEEE division) and every valid
// slot's code = round-half-even(clamp(value / scale)).  Slots past the
// sequence's new end are not touched.
__global__ __launch_bounds__(256) void append_i8_kernel(AppendI8Args a) {
  const int j = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int r0 = checked(a.cu_new[b], 0, 0x7fffffff, kSiteRowOffset, b);
  const int n = checked(a.cu_new[b + 1] - r0, 0, min(a.max_new, a.max_pages << a.log2_page), kSiteNewLen, b);
  if (n <= 0) return;
  const int P = a.page_size;
  const int s0 = checked(a.start_pos[b], 0, (a.max_pages << a.log2_page) - n, kSiteStartPos, b);
  const int end = s0 + n;
  const int lp = (s0 >> a.log2_page) + j;
  const int p0 = lp * P;
  if (p0 >= end) return;  // uniform
  const int phys = checked(a.block_table[(size_t)b * a.max_pages + lp], 0, a.num_pages - 1, kSitePageId, b);
  const int n_old = max(0, min(s0, p0 + P) - p0);  // old valid slots [0, n_old)
  const int hi = min(end, p0 + P) - p0;            // valid slots after the append: [0, hi)
  const int first_row = r0 + (p0 + n_old - s0);    // input row of slot n_old
  const int D = a.head_dim;
  const int hkv = a.num_kv_heads;
  const size_t slot_stride = (size_t)hkv * D;
  const size_t gbase = ((size_t)phys * P * hkv + hk) * D;
  const size_t sidx = (size_t)phys * hkv + hk;
  __shared__ float red[256];

  for (int which = 0; which < 2; ++which) {
    int8_t *codes = which ? a.v_codes : a.k_codes;
    float *scales = which ? a.v_scales : a.k_scales;
    const uint16_t *src = which ? a.v_new : a.k_new;
    const float s_old = scales[sidx];
    auto value = [&](int e) {
      const int slot = e / D, d = e - slot * D;
      if (slot < n_old) return (float)codes[gbase + slot * slot_stride + d] * s_old;
      return bf16_bits_to_f32(src[((size_t)(first_row + slot - n_old) * hkv + hk) * D + d]);
    };
    float amax = 0.f;
    for (int e = threadIdx.x; e < hi * D; e += blockDim.x) amax = fmaxf(amax, fabsf(value(e)));
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if ((int)threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
      __syncthreads();
    }
    amax = red[0];
    const float scale = (amax == 0.f) ? 1.f : amax / 127.f;  // IEEE division
    for (int e = threadIdx.x; e < hi * D; e += blockDim.x) {
      float y = value(e) / scale;                            // IEEE division
      y = fminf(fmaxf(y, -128.f), 127.f);
      const int slot = e / D, d = e - slot * D;
      codes[gbase + slot * slot_stride + d] = (int8_t)(int)rintf(y);  // round half to even
    }
    __syncthreads();  // every read of the old scale and of red[] is done
    if (threadIdx.x == 0) scales[sidx] = scale;
  }
}

hipError_t launch_append_i8(const AppendI8Args &a, hipStream_t s) {
  if (a.batch == 0 || a.max_new == 0) return hipSuccess;
  // A sequence's new rows span at most max_new / P + 1 logical pages.
  const dim3 grid((a.max_new + a.page_size - 1) / a.page_size + 1, a.num_kv_heads, a.batch);
  hipLaunchKernelGGL(append_i8_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s) {
  if (a.num_pages == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3(a.num_pages, a.num_kv_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
