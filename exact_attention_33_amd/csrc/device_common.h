// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <cstdint>
#include <type_traits>
#include <utility>

#include <hip/hip_runtime.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// The two halves of a wave combined: every lane receives op(x[i], x[i ^ 32]).
__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int clamp_kv(const int32_t* kv_len, int b, int M) {
  if (!kv_len) return M;
  const int x = kv_len[b];
  return x < 0 ? 0 : (x > M ? M : x);
}

// XCDs of a gfx950 GPU; workgroups are dealt to them round-robin.
constexpr int kNumXcd = 8;
// Word 3 of a raw buffer descriptor on gfx9-family GPUs (untyped 32-bit
// data, no swizzle); out-of-range reads return zeros.
constexpr int kBufferFlags = 0x00020000;

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane j supplies the address of 4 consecutive bf16 of row j / 4 of a 4 x 16
// block, and lane i receives the 4 rows' elements of column i.
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from base + voff into LDS at dst + 16 * lane (one buffer
// load into LDS), against a descriptor of `nbytes` bytes: lanes whose offset
// is out of range read zeros.  The body exists only in the device pass: the
// host pass of a HIP source has no buffer-descriptor type, and clang then
// drops the host stubs of the kernels that use it.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int nbytes, uint32_t voff,
                                                  lds_ptr dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags), dst,
      16, voff, 0, 0, 0);
#endif
}

// 4 bytes per lane from base + voff into LDS at dst + 4 * lane, as above.
// STREAM marks the load non-temporal (data read once, so it should not push
// reused lines out of L2).
template <bool STREAM = false>
__device__ __forceinline__ void buffer_load_lds4(const void* base, int nbytes, uint32_t voff,
                                                 lds_ptr dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags), dst,
      4, voff, 0, 0, STREAM ? 2 : 0);
#endif
}

// 16 bytes per lane to base + voff, against a descriptor of `nbytes` bytes:
// stores of lanes whose offset is out of range are dropped.
__device__ __forceinline__ void buffer_store16(void* base, int nbytes, uint32_t voff, u32x4 v) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b128(v, __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, kBufferFlags),
                                         voff, 0, 0);
#endif
}

// Logical work item of workgroup `wg` when workgroups are dealt round-robin
// to kNumXcd XCDs: XCD x gets a contiguous range of logical items.
__device__ __forceinline__ int64_t xcd_logical(int64_t wg, int64_t G) {
  const int64_t x = wg % kNumXcd, j = wg / kNumXcd;
  const int64_t q = G / kNumXcd, r = G % kNumXcd;
  return x * q + (x < r ? x : r) + j;
}

// f(integral_constant<int, J>) for J = 0 .. N-1, expanded at compile time (the
// pipelined loops are too large for the unroller, and their register arrays
// must only ever see constant indices).
template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace fa
