// Device-side helpers shared by the H2O kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Storage types: bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;  // elements per 16-byte chunk
  __device__ static inline void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
  __device__ static inline void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
};

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Non-temporal 16-byte load for data read exactly once per launch (K/V slots).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ inline uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = __shfl_xor(v, m, kWave);
    v = o < v ? o : v;
  }
  return v;
}

// Eviction order key: scores are non-negative, so their IEEE bit patterns order
// like the values; the low word breaks ties by position (lower position first).
__device__ inline uint64_t evict_key(float score, int32_t pos) {
  return (static_cast<uint64_t>(__float_as_uint(score)) << 32) | static_cast<uint32_t>(pos);
}

}  // namespace h2o
