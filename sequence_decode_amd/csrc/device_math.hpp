// device_math.hpp -- device helpers with a fixed operation order.
//
// Every floating-point operation that decides output bits goes through one of
// the helpers below, each a single IEEE operation that the compiler may not
// contract into a fused multiply-add (the pragma holds whatever the build
// flags say).  A row is therefore rounded the same way in every template
// instantiation, whatever the batch size.  fp32 division and square root are
// the correctly rounded ones (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

__device__ __forceinline__ float fadd(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}
__device__ __forceinline__ float fsub(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}
__device__ __forceinline__ float fmul(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float fdiv(float a, float b) {
#pragma clang fp contract(off)
  return a / b;
}
__device__ __forceinline__ float ffma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(16)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(16)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
  return (float)h;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <int ctrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl,
                                                               0xF, 0xF, true));
}

// Sum over the 64 lanes of a wave with a fixed tree: partners at lane distance
// 1 and 2 (DPP quad permutations), then the mirrored lane within 8 and within
// 16 (DPP row mirrors), then lanes 16 and 32 apart (v_permlane16/32_swap,
// which return the lower and the upper partner in fixed operand order).  Every
// level adds two equal-shaped subtree sums, so all 64 lanes end with the same
// bits, and the tree depends on nothing but the lane index.
__device__ __forceinline__ float row16_sum_fixed(float v) {
  v = fadd(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = fadd(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = fadd(v, dpp_mov<0x141>(v));  // row_half_mirror: 7 - lane within 8
  v = fadd(v, dpp_mov<0x140>(v));  // row_mirror: 15 - lane within 16
  return v;
}

// Sum of the four 16-lane rows (lanes l, l^16, l^32, l^48): the last two levels.
__device__ __forceinline__ float cross_row_sum_fixed(float v) {
  {
    auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = fadd(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = fadd(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  }
  return v;
}

__device__ __forceinline__ float wave_sum_fixed(float v) { return cross_row_sum_fixed(row16_sum_fixed(v)); }

// Maximum over an aligned group of `width` (32 or 64) lanes, exact and
// order-free, so any pairing gives the same result: the quad and row
// patterns of the sums above (within 16 lanes), then the lanes 16 (and 32)
// apart.  DPP and permlane moves stay in registers; a lane shuffle through
// the LDS crossbar would cost a round trip per level.  Every lane of the group
// must be active.
template <int width>
__device__ __forceinline__ float group_max(float v) {
  static_assert(width == 32 || width == 64, "groups of 32 or 64 lanes");
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  {
    auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  }
  if constexpr (width == 64) {
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  }
  return v;
}

// q8 activation code of x for block scale d (the library-wide convention):
// IEEE fp32 division, round half away from zero, clamp to [-127, 127].
__device__ __forceinline__ int q8_code(float x, float d) {
  if (d == 0.0f) return 0;
  float r = roundf(fdiv(x, d));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ float q8_scale(float amax) { return fdiv(amax, 127.0f); }

}  // namespace sd
