// Shared device helpers of the ISD kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstring>

#include "isd.h"

// 0 if the current HIP device is a gfx950, else ISD_E_DEVICE (isd_runtime.hip).
extern "C" int isd_check_device_internal(void);
extern "C" int isd_device_cus_internal(void);

namespace isd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Vocabulary entries per chunk of the softmax statistics (max, sum of
// exp(l - max)) that the accept step and the LM head exchange.
constexpr int kVocabChunk = 8192;

// Unnormalised softmax weight relative to the max M (as exp2 of a
// log2-scaled argument). Every place that needs P(x) uses these helpers so
// that equal inputs give equal bits.
__device__ __forceinline__ float weight_of(float l, float m_log2) { return fast_exp2(fmaf(l, kLog2e, -m_log2)); }
__device__ __forceinline__ float prob_of(float l, float M, float S) { return weight_of(l, M * kLog2e) / S; }

// Merge two (max, sum exp(l - max)) pairs.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    s = 0.f;
    return;
  }
  s = s * fast_exp2((m - mm) * kLog2e) + s2 * fast_exp2((m2 - mm) * kLog2e);
  m = mm;
}

// Element type traits for the two storage types.
template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int kPerVec = 8;  // elements per 16 bytes
  static __device__ __forceinline__ float to_f32(uint16_t h) { return bf16_bits_to_f32(h); }
};
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
  static __device__ __forceinline__ float to_f32(float f) { return f; }
};

// Unpack a 16-byte vector into kPerVec floats.
__device__ __forceinline__ void unpack16(const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}
__device__ __forceinline__ void unpack16(const u32x4& v, float (&f)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

__device__ __forceinline__ void set_dev_err(int32_t* err, uint32_t bits) {
  if (err) atomicOr(reinterpret_cast<unsigned int*>(err), bits);
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

}  // namespace isd
