// Inline-asm MFMAs with fixed register classes, their hazard guards, and the
// LDS stage layout shared by the backward and the key/value-outer forward
// kernels (gfx950).
#pragma once

#include "device_common.h"

namespace fa {
namespace asmk {

constexpr int NW = 4;  // waves per workgroup of the kernels that use Stage

// v_mfma_f32_32x32x16_bf16 with the register file of each operand fixed
// (the compiler's own choice moves accumulators between VGPRs and AGPRs on
// every iteration).  D = A B (+ D); A, B hold 8 bf16 per lane.
//   _vv: D in VGPRs (read by the VALU afterwards), A and B in VGPRs;
//   _va: D in VGPRs, A in VGPRs, B in AGPRs;
//   _aa: D in AGPRs (accumulated over the whole kernel), A and B in VGPRs.
// The asm is invisible to the compiler's hazard tracking, so the rules are
// kept here: each MFMA starts with 2 wait states (a VALU write of a register
// an MFMA reads needs 2, and the compiler may place a copy of an operand
// right before the asm); a VALU (or v_accvgpr_read) access to a result waits
// 16 wait states after the last MFMA that wrote it (mfma_guard, tied to the
// results); registers written by the VALU wait 5 more before an MFMA reads
// them (valu_guard, tied to the operands).
__device__ __forceinline__ void mfma_vv0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vv(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_va0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_va(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_aa(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// The same without the 2 leading wait states, for kernels whose compiled code
// puts no VALU write of an operand within 2 wait states ahead of any MFMA,
// branch targets included (the assembly scan in the tests checks every
// kernel for both cases).
__device__ __forceinline__ void mfma_vv0_nw(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vv_nw(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_aa_nw(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// 16 wait states, ordered after the MFMAs that wrote x and y and before
// every later access to them.
__device__ __forceinline__ void mfma_guard_v(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
// The same for four results at once (one wait covers all of them).
__device__ __forceinline__ void mfma_guard_v4(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void mfma_guard_a(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7" : "+a"(x)); }
__device__ __forceinline__ void valu_guard(bf16x8& x, bf16x8& y) {
  asm volatile("s_nop 4" : "+v"(x), "+v"(y));
}
// The same for four operands at once.
__device__ __forceinline__ void valu_guard4(bf16x8& a, bf16x8& b, bf16x8& c, bf16x8& d) {
  asm volatile("s_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void agpr_guard(f32x16& x) { asm volatile("s_nop 4" : "+a"(x)); }

// vmcnt(0), other counters untouched (gfx9 s_waitcnt encoding).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <class T>
__device__ __forceinline__ const T* lds_at(const void* base, int byte_off) {
  return (const T*)((const char*)base + byte_off);
}

// ---------------------------------------------------------------------------
// Staged tiles.  A stage holds 64 rows of a [rows][D] bf16 tensor, row r at
// byte r * ROWB, its 16-byte chunk c at position c ^ ((r >> 2) & 3).
// ---------------------------------------------------------------------------
template <int D>
struct Stage {
  static constexpr int ROWB = 2 * D + 64;   // LDS bytes per row
  static constexpr int CPR = D / 8;         // data chunks per row
  static constexpr int CH = ROWB / 16;      // 16-byte slots per row
  static constexpr int ROWS = 64;
  static constexpr int BLK = ROWS * CH / 64;  // 1 KB load blocks per stage
  static constexpr int BPW = BLK / NW;        // blocks per wave
  static_assert(BLK % NW == 0, "load blocks split evenly over the waves");
  static constexpr int BYTES = ROWS * ROWB;

  // Global byte offset (relative to the stage's first row) of slot `slot`.
  // Padding slots load the row's chunk 0 (valid data, never read).
  __device__ static uint32_t slot_src(int slot) {
    const int r = slot / CH, pos = slot % CH;
    const int c = pos < CPR ? (pos ^ ((r >> 2) & 3)) : 0;
    return (uint32_t)(r * (2 * D) + 16 * c);
  }
};

}  // namespace asmk
}  // namespace fa
