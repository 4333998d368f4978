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

// DPP lane moves inside rows of 16 lanes: register-to-register, no LDS traffic.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowRor1 = 0x121;       // row_ror:1
constexpr int kDppRowRor2 = 0x122;       // row_ror:2
constexpr int kDppRowRor4 = 0x124;       // row_ror:4
constexpr int kDppRowRor8 = 0x128;       // row_ror:8
constexpr int kDppRowHalfMirror = 0x141; // reverse each half-row of 8 lanes

template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of the
// group receives the total.  Groups of 16 and 8 use DPP.
template <int G>
__device__ inline float group_sum(float v) {
  if constexpr (G == 16) {
    v += dpp_f<kDppRowRor8>(v);
    v += dpp_f<kDppRowRor4>(v);
    v += dpp_f<kDppRowRor2>(v);
    v += dpp_f<kDppRowRor1>(v);
  } else if constexpr (G == 8) {
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
  } else {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  }
  return v;
}

// Minimum over the wave, returned wave-uniform: DPP within rows of 16, then the
// four row minima through readlane.
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, static_cast<uint32_t>(dpp_i<kDppRowRor8>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<kDppRowRor4>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<kDppRowRor2>(static_cast<int>(v))));
  v = min(v, static_cast<uint32_t>(dpp_i<kDppRowRor1>(static_cast<int>(v))));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return min(min(r0, r1), min(r2, r3));
}

// Eviction order key: scores are non-negative, so their IEEE bit patterns order
// like the values; the low word breaks ties by position (lower position first).
__device__ inline uint64_t evict_key(float score, int32_t pos) {
  return (static_cast<uint64_t>(__float_as_uint(score)) << 32) | static_cast<uint32_t>(pos);
}

// Sparse attention pattern kept in preference to heavy hitters (strided: the
// positions j with (i - j) mod period = 0 for the query at i; fixed: the last
// `width` positions of every block of `period`).  Its entries get the top key
// bit, so they order after every unprotected entry: score bits of non-negative
// floats stay below 2^31 and never reach it.
constexpr int kPatternNone = 0, kPatternStrided = 1, kPatternFixed = 2;
__device__ inline uint64_t pattern_bit(int kind, int period, int width, int32_t j, int32_t i) {
  bool p = false;
  if (kind == kPatternStrided) p = (i - j) % period == 0;
  else if (kind == kPatternFixed) p = j % period >= period - width;
  return p ? (1ull << 63) : 0ull;
}

// Wave-uniform lexicographic minimum of (score bits, position) pairs: the
// minimum score first, then the minimum position among the lanes holding it.
__device__ inline uint64_t wave_min_key(uint64_t key) {
  const uint32_t hi = static_cast<uint32_t>(key >> 32), lo = static_cast<uint32_t>(key);
  const uint32_t mhi = wave_min_u32(hi);
  const uint32_t mlo = wave_min_u32(hi == mhi ? lo : 0xffffffffu);
  return (static_cast<uint64_t>(mhi) << 32) | mlo;
}

}  // namespace h2o
