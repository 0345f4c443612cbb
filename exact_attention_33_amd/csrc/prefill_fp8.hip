// Fused tiled exact-attention forward with fp8 (OCP E4M3) Q, K, V on the
// gfx950 fp8 matrix cores, float32 accumulation, bf16 output.
//
// Method: the online-softmax forward of "Flash Attention: The Hidden Gem"
// (The Algorithm, The Correction Factor) on 8-bit inputs ("Flash Attention:
// The Hidden Gem", FA1, FA2, FA3: FP8 doubles the matrix throughput at some
// cost in precision).  With per-tensor descale factors dq, dk, dv the
// inputs stand for dq*Q8, dk*K8, dv*V8, so
//   S = scale * dq * dk * (Q8 K8^T),  O = dv * softmax(S) V8.
// Both products run on v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8, float32
// accumulate); the weights P are rounded to fp8 before P V8, as FP8 needs.
//
// gfx950 mapping:
//  * workgroup = 8 waves x 32 queries, two waves per SIMD: with 1-byte
//    elements a wave of 32 queries reads no more LDS bytes per MFMA cycle
//    than the bf16 kernel's 64-query waves, and the second wave on each SIMD
//    issues its softmax while the other's MFMAs run (the hardware interleaves
//    the two; no software pipeline);
//  * S^T = K Q^T: K rows from LDS are the A operand (32 bytes of d per lane),
//    Q stays in registers as the B operand; one query per lane, 16 keys per
//    lane per 32-key block, so the row max and row sum are in-lane plus one
//    swap between half-waves;
//  * weights against a lazy reference m with no row max per tile: a lane's
//    sum of at most 2^8 bounds each of its weights by 2^8, which E4M3 holds
//    (largest finite 448).  A larger sum, a row with no reference yet, or
//    (checked only then) a row max more than 8 (log2 units) above m moves m
//    to that max, rescales l and the output accumulator by 2^(m_old - m_new)
//    ("The Correction Factor") and forms the tile's weights again;
//  * O^T += V8^T P8^T: the fp8 weights go straight into the B operand in the
//    order the score layout hands them over (32 keys per lane), and V8^T
//    comes from ds_read_b64_tr_b8 transposing reads of V's [key][d] rows;
//  * LDS tiles of 64 keys, two stages, HBM -> LDS buffer loads (ragged
//    tails read zeros).  K rows: the 16-byte chunks of a row are permuted
//    by XOR with (row / rows-per-256-B) mod chunks-per-row; V rows: the
//    32-byte pairs are permuted by XOR with two (one at D = 64) row bits.
//    Row reads (16 rows x 16 B per 16 lanes) and transposing reads (8 rows x
//    32 B per 32 lanes) are then both free of bank conflicts;
//  * causal: tiles past the last query's diagonal are never loaded, tiles
//    that cross it run in their own loop with every element masked.
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNW8 = kFp8Threads / 64;  // waves per workgroup
constexpr int kQW8 = 32;                // queries per wave

// D = A B (+ D) on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3).  Inline asm
// fixes every operand in VGPRs; the compiler cannot see into the asm, so the
// hazards are kept by hand: a VALU write of an operand needs 2 wait states
// before the MFMA (the compiled kernels place none closer, branch targets
// included, which the assembly scan in the tests checks on every build;
// valu8_guard covers the weights the kernel itself writes), and results are
// read after mfma8_guard (16 wait states, tied to them; the scan checks that
// 19 have passed at every read).
__device__ __forceinline__ void mfma8_0(f32x16& d, const i32x8& a, const i32x8& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8(f32x16& d, const i32x8& a, const i32x8& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_guard(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void mfma8_guard1(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x)); }
__device__ __forceinline__ void valu8_guard(i32x8& x) { asm volatile("s_nop 4" : "+v"(x)); }

__device__ __forceinline__ void wait_vm0_8() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint2 lds_read_tr8(const char* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
  return make_uint2((uint32_t)r[0], (uint32_t)r[1]);
}

// Two floats -> two E4M3 bytes (round to nearest even) in half HI of `old`.
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

template <int D>
struct Fp8Layout {
  static constexpr int C = D / 16;        // 16-byte chunks per row
  static constexpr int R = 256 / D;       // rows per 256-byte bank line
  static constexpr int TILE = 64 * D;     // bytes of one K (or V) tile
  static constexpr int BLK = TILE / 1024; // 1 KB load blocks per tile
  // K: chunk c of row r at position c ^ fK(r)
  __device__ static int fK(int r) { return (r / R) % C; }
  // V: 32-byte pair p of row r at position p ^ gV(r)
  __device__ static int gV(int r) {
    return D == 128 ? (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) : ((r >> 3) & 1);
  }
  // global byte offset (within the tile) of LDS slot `slot`
  __device__ static uint32_t k_src(int slot) {
    const int r = slot / C, pos = slot % C;
    return (uint32_t)(r * D + 16 * (pos ^ fK(r)));
  }
  __device__ static uint32_t v_src(int slot) {
    const int r = slot / C, pos = slot % C;
    return (uint32_t)(r * D + 16 * (2 * ((pos / 2) ^ gV(r)) + pos % 2));
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFp8Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(Problem p, int n_qtiles) {
  using L = Fp8Layout<D>;
  constexpr int BQ = kFp8BlockQ, BK = 64, NW = kNW8, QW = kQW8;
  constexpr int DK8 = D / 64;   // 64-wide k-steps of S
  constexpr int DB = D / 32;    // 32-wide d blocks of O
  static_assert(NW * QW == BQ, "queries per workgroup");
  static_assert((2 * L::BLK) % NW == 0 || 2 * L::BLK < NW, "load blocks per wave");

  __shared__ __attribute__((aligned(1024))) char Kb0[L::TILE];
  __shared__ __attribute__((aligned(1024))) char Kb1[L::TILE];
  __shared__ __attribute__((aligned(1024))) char Vb0[L::TILE];
  __shared__ __attribute__((aligned(1024))) char Vb1[L::TILE];

  // Causal: persistent workgroups walking their XCD's query tiles, heavy
  // and light alternating round by round, as in the bf16 prefill.
  constexpr bool PERSIST = CAUSAL;
  const int64_t n_items = (int64_t)n_qtiles * p.B * p.H;
  const int xcd = blockIdx.x % kNumXcd, u = blockIdx.x / kNumXcd, W = gridDim.x / kNumXcd;
  const int64_t qx = n_items / kNumXcd, rx = n_items % kNumXcd;
  const int64_t x_start = xcd * qx + (xcd < rx ? xcd : rx), x_count = qx + (xcd < rx ? 1 : 0);
  for (int64_t k = 0;; ++k) {
    int64_t logical;
    if constexpr (PERSIST) {
      const int64_t within = k * W + ((k & 1) ? W - 1 - u : u);
      if (within >= x_count) break;
      logical = x_start + within;
      // the previous item's loads into LDS have landed, every wave is done
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    } else {
      if (k > 0) break;
      logical = xcd_logical(blockIdx.x, gridDim.x);
    }
  {
    int qt = (int)(logical % n_qtiles);
    const int64_t bh = logical / n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest query tiles first
    const int b = (int)(bh / p.H);
    const int N = p.N, M = p.M;
    const int tid = threadIdx.x;
    const int lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int ws = __builtin_amdgcn_readfirstlane(tid / 64);
    const int kvl = __builtin_amdgcn_readfirstlane(clamp_kv(p.kv_len, b, M));
    const int off = kvl - N;
    const int q0 = qt * BQ;
    const int qw0 = q0 + ws * QW;
    const int q_last = min(q0 + BQ, N) - 1;
    const int kv_end = CAUSAL ? min(kvl, q_last + off + 1) : kvl;
    const int n_tiles = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;

    const uint8_t* Qg = (const uint8_t*)p.q + (size_t)bh * N * D;
    const uint8_t* Kg = (const uint8_t*)p.k + (size_t)bh * M * D;
    const uint8_t* Vg = (const uint8_t*)p.v + (size_t)bh * M * D;

    // ---- Q in registers: B operand of S^T, 32 bytes of d per lane and k-step ----
    const int row = qw0 + l32;
    const bool row_ok = row < N;
    i32x8 qf[DK8];
  #pragma unroll
    for (int ks = 0; ks < DK8; ++ks) {
      const int4* src = (const int4*)(Qg + (size_t)(row_ok ? row : 0) * D + 64 * ks + 32 * h);
      const int4 a = row_ok ? src[0] : make_int4(0, 0, 0, 0);
      const int4 c = row_ok ? src[1] : make_int4(0, 0, 0, 0);
      qf[ks] = i32x8{a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    }
    const int lim = CAUSAL ? min(row + off, kvl - 1) : kvl - 1;  // last key this query sees

    // ---- tile loads: K blocks then V blocks of tile t ----
    constexpr int NBLK = 2 * L::BLK;                      // K and V blocks per tile
    constexpr int BPW = (NBLK + NW - 1) / NW;             // blocks per wave
    const int nrec = kvl * D;                             // the planner keeps M * D below 2^31
    uint32_t boff[BPW];
  #pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = ws + i * NW;
      const int kb = blk < L::BLK ? blk : blk - L::BLK;
      const int slot = kb * 64 + lane;
      boff[i] = blk < L::BLK ? L::k_src(slot) : L::v_src(slot);
    }
    auto load_tile = [&](int t, char* Kd, char* Vd) __attribute__((always_inline)) {
  #pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int blk = ws + i * NW;  // uniform
        if (blk < NBLK) {
          const uint32_t u = boff[i] + (uint32_t)t * BK * D;
          if (blk < L::BLK) buffer_load_lds16(Kg, nrec, u, (lds_ptr)(Kd + blk * 1024));
          else buffer_load_lds16(Vg, nrec, u, (lds_ptr)(Vd + (blk - L::BLK) * 1024));
        }
      }
    };

    // ---- per-lane LDS read offsets ----
    // K rows (A operand of S^T): row 32 kb2 + l32, 16-byte chunk 4 ks + 2 h + x.
    int kofs[DK8][2];
  #pragma unroll
    for (int ks = 0; ks < DK8; ++ks)
  #pragma unroll
      for (int x = 0; x < 2; ++x) kofs[ks][x] = l32 * D + 16 * ((4 * ks + 2 * h + x) ^ L::fK(l32));
    // V transposing reads (A operand of O^T): read q of d block db; lane j of
    // 16-lane group g addresses key 16 q + 4 h + (u < 4 ? u : u + 4), u = j / 2,
    // bytes 32 db + 16 (g % 2) + 8 (j % 2) of that row.
    const int j16 = lane % 16, u8 = j16 / 2;
    const int vkey = 4 * h + (u8 < 4 ? u8 : u8 + 4);     // + 16 q
    int vofs[DB];
  #pragma unroll
    for (int db = 0; db < DB; ++db)
      vofs[db] = vkey * D + 32 * (db ^ L::gV(vkey)) + 16 * ((lane / 16) % 2) + 8 * (j16 % 2);

    // ---- state: one query per lane ----
    f32x16 oacc[DB];
  #pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = -INFINITY;  // reference max (log2 units of the scaled score)
    float l_run = 0.f;        // this lane's part of the row sum (its half of the keys)
    const float c = fmaxf(p.scale * p.q_descale * p.k_descale * kLog2e, 1e-30f);

    auto tile = [&](int t, const char* Ks, const char* Vs, auto MASK) __attribute__((always_inline)) {
      constexpr bool mask = decltype(MASK)::value;
      // S^T: lane = query row, register r of block kb2 = key 64 t + 32 kb2 + 8 (r / 4) + 4 h + r % 4
      f32x16 s[2];
  #pragma unroll
      for (int ks = 0; ks < DK8; ++ks)
  #pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int4 a0 = *(const int4*)(Ks + 32 * kb2 * D + kofs[ks][0]);
          const int4 a1 = *(const int4*)(Ks + 32 * kb2 * D + kofs[ks][1]);
          const i32x8 ka = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          if (ks == 0) mfma8_0(s[kb2], ka, qf[ks]);
          else mfma8(s[kb2], ka, qf[ks]);
        }
      mfma8_guard(s[0], s[1]);
      if constexpr (mask) {
  #pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t * BK + 32 * kb2 + 8 * (r / 4) + 4 * h + r % 4;
            s[kb2][r] = key > lim ? -INFINITY : s[kb2][r];
          }
      }
      // Weights against the current reference with no row max: a lane's sum
      // of at most 2^8 bounds each of its weights by 2^8 (E4M3 holds them).
      // A larger sum, or a row with no reference yet, takes the rare path:
      // such rows, and rows whose tile max exceeds the reference by more than
      // 8, move it to that max (l and the output accumulator rescaled) and the
      // weights are formed again.
      i32x8 pf;
      float ps = 0.f;
      auto weights = [&](float m_use) __attribute__((always_inline)) {
        ps = 0.f;
  #pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb2 = w / 4, r0 = 4 * (w % 4);
          float e[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = fast_exp2(fmaf(s[kb2][r0 + i], c, -m_use));
            ps += e[i];
          }
          int packed = cvt_fp8x2<false>(e[0], e[1], 0);
          packed = cvt_fp8x2<true>(e[2], e[3], packed);
          pf[w] = packed;
        }
      };
      weights(m_ref == -INFINITY ? 0.f : m_ref);
      if (__builtin_amdgcn_ballot_w64(!(ps <= 256.f) || m_ref == -INFINITY)) {
        float mx = -INFINITY;
  #pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
  #pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb2][r]);
        mx = swap_halves_max(mx) * c;
        // a row whose sum went over moves up to its max (weights <= 1), so
        // the following tiles do not come back here; any row moves when its
        // max is more than 8 above the reference
        const float over = swap_halves_max(!(ps <= 256.f) ? 1.f : 0.f);
        const bool move = (over > 0.f && mx > m_ref) || mx > m_ref + 8.f;
        if (__builtin_amdgcn_ballot_w64(move)) {
          const float m_new = move ? mx : m_ref;
          const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
          l_run *= alpha;
  #pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          m_ref = m_new;
          weights(m_ref == -INFINITY ? 0.f : m_ref);
        }
      }
      l_run += ps;
      valu8_guard(pf);
      // O^T += V8^T P8^T, 64 keys = one k-step per d block
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8 va;
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 x = lds_read_tr8(Vs + 16 * q * D + vofs[db]);
          va[2 * q] = (int)x.x;
          va[2 * q + 1] = (int)x.y;
        }
        mfma8(oacc[db], va, pf);
      }
    };

    auto iteration = [&](int t, const char* Ks, const char* Vs, char* Kn, char* Vn, auto MASK)
                         __attribute__((always_inline)) {
      wait_vm0_8();
      __syncthreads();
      if (t + 1 < n_tiles) load_tile(t + 1, Kn, Vn);
      // causal: a tile that none of this wave's queries sees
      if (!CAUSAL || t * BK <= qw0 + QW - 1 + off) tile(t, Ks, Vs, MASK);
    };

    // Tiles before n_clean (an even number) are seen whole by every query of
    // the workgroup; the rest are masked element by element.
    int n_clean = kvl / BK;
    if (CAUSAL) n_clean = min(n_clean, q0 + off + 1 > 0 ? (q0 + off + 1) / BK : 0);
    n_clean = min(n_clean, n_tiles) / 2 * 2;
    if (n_tiles > 0) load_tile(0, Kb0, Vb0);
    int t = 0;
    for (; t < n_clean; t += 2) {
      iteration(t, Kb0, Vb0, Kb1, Vb1, std::false_type{});
      iteration(t + 1, Kb1, Vb1, Kb0, Vb0, std::false_type{});
    }
    for (; t + 1 < n_tiles; t += 2) {
      iteration(t, Kb0, Vb0, Kb1, Vb1, std::true_type{});
      iteration(t + 1, Kb1, Vb1, Kb0, Vb0, std::true_type{});
    }
    if (t < n_tiles) iteration(t, Kb0, Vb0, Kb1, Vb1, std::true_type{});

    // ---- epilogue: O = dv * acc / l, LSE = ln 2 * (m + log2 l) ----
  #pragma unroll
    for (int db = 0; db < DB; ++db) mfma8_guard1(oacc[db]);
    const float l_tot = swap_halves_sum(l_run);
    if (row_ok) {
      const float inv = l_tot > 0.f ? p.v_descale / l_tot : 0.f;
      __bf16* Orow = (__bf16*)p.o + (size_t)bh * N * D + (size_t)row * D;
  #pragma unroll
      for (int db = 0; db < DB; ++db)
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 ov;
  #pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][4 * g + i] * inv);
          *(bf16x4*)(Orow + 32 * db + 8 * g + 4 * h) = ov;
        }
      if (h == 0) p.lse[(size_t)bh * N + row] = l_tot > 0.f ? kLn2 * (m_ref + fast_log2(l_tot)) : -INFINITY;
    }
  }
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const Problem& p, const Plan& plan, hipStream_t stream) {
  if (plan.grid == 0) return hipSuccess;
  const int n_qtiles = (p.N + kFp8BlockQ - 1) / kFp8BlockQ;
  const dim3 grid((unsigned)plan.grid), block(kFp8Threads);
  if (p.D == 64) {
    if (p.causal) hipLaunchKernelGGL((prefill_fp8_kernel<64, true>), grid, block, 0, stream, p, n_qtiles);
    else hipLaunchKernelGGL((prefill_fp8_kernel<64, false>), grid, block, 0, stream, p, n_qtiles);
  } else {
    if (p.causal) hipLaunchKernelGGL((prefill_fp8_kernel<128, true>), grid, block, 0, stream, p, n_qtiles);
    else hipLaunchKernelGGL((prefill_fp8_kernel<128, false>), grid, block, 0, stream, p, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace fa
