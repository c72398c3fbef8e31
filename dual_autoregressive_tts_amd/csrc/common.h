// Device-side helpers shared by the Dual-AR kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 held as raw bits
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DUALAR_WG 256

// Status bits latched in the workspace status word.
enum { ST_BAD_TOKEN = 1, ST_NONFINITE = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element-type traits: a 16-byte vector holds EPV elements.
template <typename T> struct ElemT;
template <> struct ElemT<float> {
  static constexpr int EPV = 4;
  __device__ static __forceinline__ void unpack(const u32x4 v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float load(const void* p, size_t i) { return ((const float*)p)[i]; }
  __device__ static __forceinline__ float round(float x) { return x; }
  __device__ static __forceinline__ void store(void* p, size_t i, float x) { ((float*)p)[i] = x; }
};
template <> struct ElemT<bf16_t> {
  static constexpr int EPV = 8;
  __device__ static __forceinline__ void unpack(const u32x4 v, float* o) {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float load(const void* p, size_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static __forceinline__ float round(float x) { return bf16_bits_to_f32(f32_to_bf16_rne(x)); }
  __device__ static __forceinline__ void store(void* p, size_t i, float x) { ((uint16_t*)p)[i] = f32_to_bf16_rne(x); }
};

__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ u32x4 ld_vec(const void* p) { return *(const u32x4*)p; }

// Butterfly sum over the 64 lanes of a wave (fixed order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }
