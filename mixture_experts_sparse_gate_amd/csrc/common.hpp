// Shared device-side definitions for the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element types

// Elements of a 16-byte chunk, and widening to fp32.
template <typename E> struct ElemTraits;
template <> struct ElemTraits<float> {
  static constexpr int kPerChunk = 4;
  __device__ static inline float to_f32(float v) { return v; }
};
template <> struct ElemTraits<bf16> {
  static constexpr int kPerChunk = 8;
  __device__ static inline float to_f32(bf16 v) { return (float)v; }
};

// Element i (0 <= i < kPerChunk) of a 16-byte chunk, widened to fp32.
template <typename E> __device__ inline float chunk_elem(const u32x4& c, int i);
template <> __device__ inline float chunk_elem<float>(const u32x4& c, int i) {
  return __uint_as_float(c[i]);
}
template <> __device__ inline float chunk_elem<bf16>(const u32x4& c, int i) {
  uint32_t w = c[i >> 1];
  return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Packs fp32 values into the output element type.
template <typename E> struct Store;
template <> struct Store<float> {
  // 4 values -> 16 bytes
  __device__ static inline void four(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
};
template <> struct Store<bf16> {
  // 4 values -> 8 bytes
  __device__ static inline void four(bf16* p, float a, float b, float c, float d) {
    u32x2 v;
    v[0] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
    v[1] = f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16);
    *reinterpret_cast<u32x2*>(p) = v;
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// Raw buffer descriptor (gfx9 family: word 3 = 0x00020000) over [base, base + bytes):
// loads outside the range return zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// A buffer offset past the range of every descriptor here (all ranges are
// below 2^31 bytes): a load at it reads zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------- wave helpers

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, kWave);
  hi = __shfl_xor(hi, m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is first mapped to +0.0 so that the two compare equal.
__device__ inline uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe
