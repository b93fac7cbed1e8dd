// 16x16 MFMA helpers for the gfx950 attention kernels (16-bit inputs,
// float32 accumulation), shared by decode and prefill.
//
// Operand layouts (wave64; lane l, t = l % 16, qa = l / 16):
//   v_mfma_f32_16x16x32: A[i][k] lane holds i = t, k = 8qa .. 8qa+7;
//                        B[k][j] lane holds j = t, the same 8 k;
//   v_mfma_f32_16x16x16: A and B the same with k = 4qa .. 4qa+3;
//   C[i][j]: lane holds j = t and i = 4qa + r in register r.
//   ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
//   j % 4 of the 4-element window addressed by lane 4e + j / 4, for e = 0..3
//   (a 4x4 transpose of 16-bit elements per group of lanes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT> struct MfmaOps;
template <> struct MfmaOps<PA_DTYPE_BF16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x4 __attribute__((ext_vector_type(4)));
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) x4 lds_x4;
  static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint2 read_tr(lds_x4* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p));
  }
  static __device__ __forceinline__ void split(const float (&p)[4], uint2& hi, uint2& lo) {
    x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = static_cast<__bf16>(p[i]);
      l[i] = static_cast<__bf16>(p[i] - static_cast<float>(h[i]));
    }
    hi = __builtin_bit_cast(uint2, h);
    lo = __builtin_bit_cast(uint2, l);
  }
};
template <> struct MfmaOps<PA_DTYPE_F16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  typedef __fp16 tr4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) tr4 lds_x4;
  static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint2 read_tr(lds_x4* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
  }
  static __device__ __forceinline__ void split(const float (&p)[4], uint2& hi, uint2& lo) {
    x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = static_cast<_Float16>(p[i]);
      l[i] = static_cast<_Float16>(p[i] - static_cast<float>(h[i]));
    }
    hi = __builtin_bit_cast(uint2, h);
    lo = __builtin_bit_cast(uint2, l);
  }
};

}  // namespace pkv
