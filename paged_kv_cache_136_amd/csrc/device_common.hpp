// Device helpers for the gfx950 kernels: element conversion from 16-byte
// loads and wave64 cross-lane reductions built on DPP / ds_swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Element types: 0 = float32, 1 = float16, 2 = bfloat16 (pa_dtype values).
template <int DT> struct ElemTraits;
template <> struct ElemTraits<PA_DTYPE_F32> { static constexpr int bytes = 4; };
template <> struct ElemTraits<PA_DTYPE_F16> { static constexpr int bytes = 2; };
template <> struct ElemTraits<PA_DTYPE_BF16> { static constexpr int bytes = 2; };

// Unpack one 16-byte chunk (4 dwords) into 16/bytes floats.
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& w, float* f);

template <>
__device__ __forceinline__ void unpack16<PA_DTYPE_F32>(const uint4& w, float* f) {
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}

__device__ __forceinline__ float half_lo(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
}
__device__ __forceinline__ float half_hi(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
}

template <>
__device__ __forceinline__ void unpack16<PA_DTYPE_F16>(const uint4& w, float* f) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = half_lo(d[i]);
    f[2 * i + 1] = half_hi(d[i]);
  }
}

// bfloat16 is the top half of a float32: widening is a shift / mask.
template <>
__device__ __forceinline__ void unpack16<PA_DTYPE_BF16>(const uint4& w, float* f) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(d[i] << 16);
    f[2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
  }
}

// ---- wave64 lane exchange -------------------------------------------------
// perm<OFF>(x) returns x from lane (lane ^ OFF), exactly, so a butterfly over
// OFF = FROM, 2*FROM, ... reduces across aligned groups while keeping each
// lane's position inside its group (needed when lanes of a group hold
// different data, e.g. different head_dim chunks of an output row):
//   OFF 1, 2 : quad_perm DPP [1,0,3,2] / [2,3,0,1]
//   OFF 4    : row_half_mirror then quad_perm [3,2,1,0] (7-i, then 3-j)
//   OFF 8    : row_ror:8 DPP (rotating a 16-lane row by 8 swaps its halves)
//   OFF 16   : ds_swizzle, bit mode, xor mask 0x10 (within 32 lanes)
//   OFF 32   : ds_bpermute, lane ^ 32
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  // Every source lane of these permutations is valid; with bound_ctrl set
  // the old operand is dead and the move can fold into the consuming VALU op.
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

template <int OFF>
__device__ __forceinline__ float perm(float x) {
  if constexpr (OFF == 1) return dpp_f<0xB1>(x);                  // quad_perm [1,0,3,2]
  else if constexpr (OFF == 2) return dpp_f<0x4E>(x);             // quad_perm [2,3,0,1]
  else if constexpr (OFF == 4) return dpp_f<0x1B>(dpp_f<0x141>(x));  // half_mirror, quad [3,2,1,0]
  else if constexpr (OFF == 8) return dpp_f<0x128>(x);            // row_ror:8
  else if constexpr (OFF == 16)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  else
    return __shfl_xor(x, 32);
}

// Sum / max over the TO/FROM lanes {lane ^ k*FROM} (exact xor butterfly):
// with FROM = 1 every lane of an aligned TO-group gets the group total; with
// FROM > 1 lanes at the same position in each FROM-group are combined.
template <int FROM, int TO>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (FROM < TO) {
    x += perm<FROM>(x);
    return group_sum<FROM * 2, TO>(x);
  } else {
    return x;
  }
}

template <int FROM, int TO>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (FROM < TO) {
    x = fmaxf(x, perm<FROM>(x));
    return group_max<FROM * 2, TO>(x);
  } else {
    return x;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// c ? a : b for 16-byte chunks, component by component: a ternary on the
// uint4 struct itself is lowered as a select between two stack copies,
// which puts both in scratch memory.
__device__ __forceinline__ uint4 select4(bool c, const uint4& a, const uint4& b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// ---- 16-byte chunk arithmetic ------------------------------------------
// A lane holds one 16-byte chunk of a K/V row (4 floats or 8 halves) and the
// matching chunk of q in the same raw form.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// <q chunk, k chunk> in float32 (dot2 instructions for 16-bit types).
template <int DT>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k) {
  if constexpr (DT == PA_DTYPE_F32) {
    float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  } else if constexpr (DT == PA_DTYPE_F16) {
    float acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.x), __builtin_bit_cast(half2_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.y), __builtin_bit_cast(half2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.z), __builtin_bit_cast(half2_t, k.z), acc, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w), __builtin_bit_cast(half2_t, k.w), acc, false);
  } else {
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.x), __builtin_bit_cast(bf162_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.y), __builtin_bit_cast(bf162_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.z), __builtin_bit_cast(bf162_t, k.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.w), __builtin_bit_cast(bf162_t, k.w), acc, false);
  }
}

// o[e] += p * v[e] over the chunk, float32 accumulation.
template <int DT>
__device__ __forceinline__ void chunk_axpy(float* o, float p, const uint4& v) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == PA_DTYPE_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = fmaf(p, __uint_as_float(d[i]), o[i]);
  } else if constexpr (DT == PA_DTYPE_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = fmaf(p, half_lo(d[i]), o[2 * i]);
      o[2 * i + 1] = fmaf(p, half_hi(d[i]), o[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = fmaf(p, __uint_as_float(d[i] << 16), o[2 * i]);
      o[2 * i + 1] = fmaf(p, __uint_as_float(d[i] & 0xffff0000u), o[2 * i + 1]);
    }
  }
}

}  // namespace pkv
