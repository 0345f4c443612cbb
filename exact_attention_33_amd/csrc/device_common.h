// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32 /
// v_log_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Row-local lane permutations (DPP) on 32-bit values.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of 8 or 16 lanes; every lane of a group ends with
// the bitwise-identical sum (each step adds a value and its partner, and
// float addition commutes).
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "group of 8 or 16 lanes");
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (LANES == 16) x += dpp_f32<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ int clamp_kv(const int32_t* kv_len, int b, int M) {
  if (!kv_len) return M;
  const int x = kv_len[b];
  return x < 0 ? 0 : (x > M ? M : x);
}

}  // namespace fa
