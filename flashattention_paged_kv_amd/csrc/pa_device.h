// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, MFMA / LDS-transpose wrappers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define PA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN): the hardware
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_mfma_f32_16x16x32_bf16.  Lane l: A row l%16 / B column l%16, k elements
// 8*(l/16) .. 8*(l/16)+7; result column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16.  Lane l: A row l%32 / B column l%32, k elements
// 8*(l/32) .. +7; result column l%32, element i at row
// (i/4)*8 + (l/32)*4 + i%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane t receives element
// t%4 of the 4-element chunks addressed by lanes t/4, t/4+4, t/4+8, t/4+12.
// If lane i of the group addresses row (r0 + i/4), columns c0 + 4*(i%4) ..+3
// of a row-major bf16 matrix, lane t receives rows r0..r0+3 of column c0+t.
// `p` must point into LDS (__shared__ memory).
__device__ __forceinline__ bf16x4 lds_read_tr16(const void *p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane t receives byte t%8
// of the 8-byte chunks addressed by lanes t/8 + 2k, k = 0..7.  If lane i
// addresses row (r0 + i/2), bytes c0 + 8*(i%2) .. +7 of a row-major int8
// matrix, lane t receives rows r0..r0+7 of column c0+t.
__device__ __forceinline__ i32x2 lds_read_tr8(const void *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2 *)(p));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// Cross-row exchanges without LDS (gfx950 v_permlane16/32_swap).  Called with
// the same value for both operands, the two results hold, lane by lane, the
// value of this lane and of lane l ^ 16 (resp. l ^ 32) in some order, so a
// symmetric op of the pair is the pairwise reduction.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes) (gfx9 raw buffer, stride 0):
// loads through it are range-checked by the hardware (out of range -> 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Pack 8 signed int8 (in two dwords) into 8 exact bf16 values.
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x8 r;
  r[0] = (__bf16)(float)(int8_t)(lo & 0xff);
  r[1] = (__bf16)(float)(int8_t)((lo >> 8) & 0xff);
  r[2] = (__bf16)(float)(int8_t)((lo >> 16) & 0xff);
  r[3] = (__bf16)(float)(int8_t)(lo >> 24);
  r[4] = (__bf16)(float)(int8_t)(hi & 0xff);
  r[5] = (__bf16)(float)(int8_t)((hi >> 8) & 0xff);
  r[6] = (__bf16)(float)(int8_t)((hi >> 16) & 0xff);
  r[7] = (__bf16)(float)(int8_t)(hi >> 24);
  return r;
}

// ---- Device checks of device-resident integers (debug builds) -----------
//
// checked(v, lo, hi, site, b): v when lo <= v <= hi.  In a build with
// PA_DEVICE_CHECKS=1 an out-of-range v is recorded in this source file's
// fault record (the first one wins) and lo is returned instead, so that the
// kernel's accesses stay inside the caller's buffers (callers choose ranges
// with lo <= hi, lo itself safe); the host reads the record after the
// launch and reports it.  Release builds return v.
#if PA_DEVICE_CHECKS
static __device__ DeviceFault g_device_fault;

__device__ __noinline__ void record_fault(int site, int v, int lo, int hi, int b) {
  if (atomicCAS(&g_device_fault.flag, 0, -1) == 0) {
    g_device_fault.site = site;
    g_device_fault.value = v;
    g_device_fault.lo = lo;
    g_device_fault.hi = hi;
    g_device_fault.batch = b;
    __threadfence();
    atomicExch(&g_device_fault.flag, 1);
  }
}

#define PA_DEFINE_FAULT_READER(NAME)                                                          \
  hipError_t NAME(DeviceFault *f) {                                                           \
    hipError_t e = hipMemcpyFromSymbol(f, HIP_SYMBOL(g_device_fault), sizeof(DeviceFault));   \
    if (e != hipSuccess || f->flag == 0) return e;                                            \
    const DeviceFault zero = {};                                                              \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_device_fault), &zero, sizeof(DeviceFault));         \
  }
#else
#define PA_DEFINE_FAULT_READER(NAME)
#endif

__device__ __forceinline__ int checked(int v, int lo, int hi, int site, int b) {
#if PA_DEVICE_CHECKS
  if (v < lo || v > hi) {
    record_fault(site, v, lo, hi, b);
    return lo;
  }
#endif
  return v;
}

}  // namespace pa
