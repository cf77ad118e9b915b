// Device-side helpers: storage types and conversions (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

template <int DT>
struct Elem;
template <>
struct Elem<PA_FP32> {
  static constexpr int kBytes = 4;
};
template <>
struct Elem<PA_FP16> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<PA_BF16> {
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fp16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float fp16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Unpack one 16-byte vector into 16/bytes floats.
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == PA_FP32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == PA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = fp16_lo(w[i]);
      f[2 * i + 1] = fp16_hi(w[i]);
    }
  }
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_fp16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// Pack 16/bytes floats into one 16-byte vector of the storage type.
template <int DT>
__device__ __forceinline__ uint4 pack16(const float* f) {
  uint32_t w[4];
  if constexpr (DT == PA_FP32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
  } else if constexpr (DT == PA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32_to_fp16_bits(f[2 * i]) | (f32_to_fp16_bits(f[2 * i + 1]) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t idx, float x) {
  if constexpr (DT == PA_FP32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else if constexpr (DT == PA_BF16) {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(x);
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_fp16_bits(x);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa
