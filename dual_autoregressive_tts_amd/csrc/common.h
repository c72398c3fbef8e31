// Device-side helpers shared by the Dual-AR kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 held as raw bits
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DUALAR_WG 256

// Status bits latched in the workspace status word.
enum { ST_BAD_TOKEN = 1, ST_NONFINITE = 2, ST_INDEX = 4 };

// Index checks of the checked build (compiled with -DDUALAR_DEVICE_CHECKS).
// checked_index(i, n, status) is i when 0 <= i < n; otherwise it latches
// ST_INDEX in the status word (when status is set) and returns 0, so the
// access it guards stays inside its buffer and the call reports the failure
// at dualar_sync instead of touching memory it does not own.  In the normal
// build it is i itself and costs nothing.
#ifdef DUALAR_DEVICE_CHECKS
__device__ __forceinline__ long long checked_index_ll(long long i, long long n, int* status) {
  if (i >= 0 && i < n) return i;
  if (status) atomicOr(status, ST_INDEX);
  return 0;
}
#define checked_index(i, n, status) ((decltype(i))checked_index_ll((long long)(i), (long long)(n), (status)))
#else
#define checked_index(i, n, status) (i)
#endif

// Row b's position (pos == NULL: pos_const for every row); a negative one
// marks an inactive row.  The checked build holds the others below max_pos,
// the length of the cache and of the RoPE table.
__device__ __forceinline__ int row_position(const int* pos, int pos_const, int b, int max_pos, int* status) {
  const int v = pos ? pos[b] : pos_const;
  return v < 0 ? v : checked_index(v, max_pos, status);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet): gfx950's
// v_cvt_pk_bf16_f32, branch-free.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// v as three bf16 terms t0 + t1 + t2 (+ a residual below 2^-24 |v|) at
// base[at], base[plane + at], base[2*plane + at]: the activation planes read
// by the matrix-core products.
__device__ __forceinline__ void store_planes(uint16_t* base, size_t plane, size_t at, float v) {
  const uint16_t a0 = f32_to_bf16_rne(v);
  const float r1 = v - bf16_bits_to_f32(a0);
  const uint16_t a1 = f32_to_bf16_rne(r1);
  base[at] = a0;
  base[plane + at] = a1;
  base[2 * plane + at] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
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

// Cross-lane reductions on VALU instructions: DPP row permutations inside a
// row of 16 lanes and the gfx950 permlane16/32 swaps across rows.  Every
// step adds a lane's value to its partner's with the same two operands in
// the same order on both lanes, so results are identical across lanes and
// deterministic.
#define DPP_F(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, true))
__device__ __forceinline__ float xor1_of(float v) { return DPP_F(v, 0xB1); }   // quad_perm [1,0,3,2]
__device__ __forceinline__ float xor2_of(float v) { return DPP_F(v, 0x4E); }   // quad_perm [2,3,0,1]
__device__ __forceinline__ float mir8_of(float v) { return DPP_F(v, 0x141); }  // row_half_mirror
__device__ __forceinline__ float mir16_of(float v) { return DPP_F(v, 0x140); } // row_mirror
__device__ __forceinline__ float xor8_of(float v) { return DPP_F(v, 0x128); }  // row_ror:8
// v(lane) + v(lane ^ 16) and v(lane) + v(lane ^ 32), lower lane's value first
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of `width` lanes (8, 16, 32 or 64); every lane of a
// group ends with the group's sum.  The pairing (x + partner) is arranged so
// that both lanes of a pair add the same operands: after each step all lanes
// of the group-so-far hold one value.
__device__ __forceinline__ float group_sum(float v, int width) {
  v = v + xor1_of(v);
  v = v + xor2_of(v);
  v = v + mir8_of(v);
  if (width >= 16) v = v + mir16_of(v);
  if (width >= 32) v = add_xor16(v);
  if (width >= 64) v = add_xor32(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor1_of(v));
  v = fmaxf(v, xor2_of(v));
  v = fmaxf(v, mir8_of(v));
  v = fmaxf(v, mir16_of(v));
  v = max_xor16(v);
  return max_xor32(v);
}
// Sum over the lanes sharing (lane % width), width 8, 16 or 32: the 64/width
// groups are added together.
__device__ __forceinline__ float across_groups_sum(float v, int width) {
  if (width <= 8) v = v + xor8_of(v);
  if (width <= 16) v = add_xor16(v);
  return add_xor32(v);
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }
