// Shared device helpers for the gfx950 kernels of the decoder-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static constexpr int kWave = 64;      // CDNA wavefront width
static constexpr int kKvBlock = 16;   // tokens per paged KV block

// Element <-> fp32.  bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest
// even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 16-byte vector of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Max / sum over the four 16-lane rows of a wave: lanes l, l^16, l^32 and
// l^48 all end with the same value.  gfx950's v_permlane16_swap and
// v_permlane32_swap, given one value for both operands, hand each lane the
// pair {x[l], x[l^16]} (resp. {x[l], x[l^32]}), in VALU without a trip
// through LDS.  Both orders of a pair add to the same fp32 sum.
__device__ __forceinline__ float row_group_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over a group of `W` consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// 16-byte global load that bypasses nothing; kept in one place so the load
// width is visible.
template <typename V>
__device__ __forceinline__ V ld16(const void* p) {
  return *reinterpret_cast<const V*>(p);
}

// 16- and 8-byte global loads with the nontemporal hint, for data a launch
// reads exactly once (decode weights, KV blocks): measured on MI355X, a
// read-only stream of 4 GiB reaches 7.2-7.4 TB/s with the hint against
// 6.0-6.3 TB/s without.  Not for data other workgroups re-read through the
// caches (activations, the prefill GEMM's tiles).
template <typename V>
__device__ __forceinline__ V ld16_nt(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
template <typename V>
__device__ __forceinline__ V ld8_nt(const void* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
}
