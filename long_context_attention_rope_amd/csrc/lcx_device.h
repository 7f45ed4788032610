// Device-side helpers shared by the gfx950 kernels of liblcx: vector types,
// 16-bit conversions and the bit-exact bf16/f16 packing used by the tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcx {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// bf16 bits -> fp32 (exact)
// Load of data that one pass reads exactly once (global_load ... nt): the
// non-temporal policy streams it past the caches (a plain read kernel: 7.0
// against 6.2 TB/s on this part).
template <class T>
__device__ __forceinline__ T load_once(const T* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // lowers to v_cvt_pk_bf16_f32 on gfx950
  return __builtin_bit_cast(uint32_t, v);
}

// two fp32 -> packed f16x2, round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
  f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Rotate 4 adjacent (even, odd) pairs held as bf16x2 words:
//   (x0, x1) -> (x0 c - x1 s, x0 s + x1 c)
// and repack as f16x2 (OUT_F16) or bf16x2.
template <bool OUT_F16>
__device__ __forceinline__ u32x4 rotate4_bf16(u32x4 x, f32x4 c, f32x4 s) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = bf16lo(x[i]), x1 = bf16hi(x[i]);
    float y0 = x0 * c[i] - x1 * s[i];
    float y1 = x0 * s[i] + x1 * c[i];
    y[i] = OUT_F16 ? pack_f16x2(y0, y1) : pack_bf16x2(y0, y1);
  }
  return y;
}

// bf16x2 words -> f16x2 words (exact for normal-range values)
__device__ __forceinline__ u32x4 bf16_to_f16_4(u32x4 x) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = pack_f16x2(bf16lo(x[i]), bf16hi(x[i]));
  return y;
}

// max / sum with lane l ^ 32 (permlane32_swap: r[0] and r[1] together hold
// the lane's own value and its partner's)
__device__ __forceinline__ float xor32_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace lcx
