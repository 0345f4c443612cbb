// Backward of the fused exact attention, bf16 inputs, float32 accumulation,
// for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// Method ("Flash Attention: The Hidden Gem", Phase 2: Backward Pass):
//  * the row statistic D_i = rowsum(dO_i * O_i) (The D Shortcut) is computed
//    once, in its own pass over dO and O, before anything else (The
//    Algorithm, step 4);
//  * the weights are recomputed from the saved log-sum-exp, P = exp(S - L),
//    never stored (steps 10-11), and the score gradient is
//    dS = P * (dP - D) with dP = dO V^T (steps 13-14, The Softmax Jacobian);
//  * dV = P^T dO and dK = dS^T Q accumulate on chip over all query tiles and
//    are written once per key tile (steps 5-8, 12, 16, 18: key/value tiles
//    on the outside);
//  * dQ = dS K.  The pages accumulate it with a read-modify-write of dQ in
//    HBM on every inner step (step 15).  Here it has a pass of its own with
//    the query tiles on the outside: it recomputes S and dP (two more tile
//    products out of seven) and then writes each dQ row once, with no
//    read-modify-write traffic, no atomics and a result that does not
//    depend on the order in which workgroups run.
// With S = scale * Q K^T the chain rule puts the scale on both score
// gradients: dQ = scale * dS K and dK = scale * dS^T Q.
//
// gfx950 mapping (both tile passes):
//  * v_mfma_f32_32x32x16_bf16, 4 waves per workgroup, one per SIMD, 512
//    registers per wave;
//  * dK/dV pass: wave w owns 64 keys.  Their K and V fragments stay in
//    registers (B operands of S = Q K^T and dP = dO V^T) and their dK^T and
//    dV^T accumulators too.  Query tiles of 64 stream through LDS (Q, dO,
//    LSE, D) and are processed 32 queries at a time.  S and dP come out
//    with one key per lane and 16 queries per lane, so the weights and score
//    gradients convert to bf16 straight into the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS (the contraction over queries runs in
//    the order in which the accumulator layout hands the queries over);
//    dO^T and Q^T come from transposing LDS reads;
//  * dQ pass: wave w owns 64 queries.  Their Q and dO fragments stay in
//    registers (B operands of S^T = K Q^T and dP^T = V dO^T) with the dQ^T
//    accumulator; key tiles of 64 stream through LDS.  S^T has one query per
//    lane, so LSE and D are two per-lane values, and dS^T converts straight
//    into the B operand of dQ^T += K^T dS^T, with K^T from transposing reads;
//  * each wave reads every staged tile twice (row reads for S and dP,
//    transposing reads for the gradient products): 64 keys (or queries) per
//    wave keep that to 16 bytes of LDS per MFMA cycle;
//  * LDS tiles: rows of 2 D + 64 bytes, and the four 16-byte chunks of each
//    64-byte group of a row are permuted by XOR with bits 2-3 of the row
//    index.  Row reads (16 rows x 16 bytes per 16 lanes) and transposing
//    reads (4 rows x 64 bytes per 32 lanes) are then both free of bank
//    conflicts; no single padding serves both patterns;
//  * tiles move HBM -> LDS with buffer loads into LDS against descriptors
//    that end at the last valid row, so ragged tails read as zeros; two
//    stages, the next one loading while the current one is computed;
//  * causal: tiles that no query of a wave sees are skipped, and only tiles
//    that cross the diagonal are masked element by element;
//  * element masks: the dQ pass walks the forward's list of key tiles per
//    query tile, the dK/dV pass a list of query stages per key tile built
//    the same way (stages and tiles the mask drops are skipped).  Both stage
//    the mask words of a stage in
//    LDS beside the tiles and apply the bits on every stage: dQ as the
//    forward does (lane = query, a word per 32 keys), dK/dV transposed
//    (lane = key: words stored [word][query row], so one 16-byte read gives
//    a lane the words of four consecutive queries).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "fa_internal.h"
#include "mfma_asm.h"

namespace fa {
namespace {

using namespace asmk;
static_assert(NW == kBwdThreads / 64, "waves per workgroup");

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Output staging: 32 rows of a wave's accumulator go out through the wave's
// LDS area (32 rows of 2 D + 16 bytes) as 16-byte pieces of whole rows, not
// as 8 bytes of 32 rows per store.  acc[db] register r holds row l32,
// d = 32 db + 8 (r / 4) + 4 h + r % 4 of the block; the row gets acc * sc,
// or zeros where `ok` is false.  dst is the block's first row (row stride
// D); rows from `rows` on are not written (a buffer descriptor of `rows`
// rows drops their stores).  `rows` and dst are wave-uniform.
template <int D>
__device__ __forceinline__ void store_block_staged(uint8_t* st, const f32x16 (&acc)[D / 32], float sc, bool ok,
                                                   __bf16* dst, int rows) {
  constexpr int OSTR = 2 * D + 16, CPR = D / 8, RPI = 64 / CPR;
  // lane-dependent addresses formed here (not hoisted and kept live)
  int ln = (int)threadIdx.x % 64;
  asm volatile("" : "+v"(ln));
  const int l32 = ln % 32, h = ln / 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(ok ? acc[db][4 * g + e] * sc : 0.f);
      *(bf16x4*)(st + l32 * OSTR + (32 * db + 8 * g + 4 * h) * 2) = v4;
    }
  // the wave's LDS writes before its reads of other lanes' rows
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int bytes = __builtin_amdgcn_readfirstlane(rows < 0 ? 0 : (rows > 32 ? 32 : rows) * D * 2);
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + ln / CPR, c16 = ln % CPR;
    const u32x4 v = *(const u32x4*)(st + r * OSTR + c16 * 16);
    buffer_store16(dst, bytes, (uint32_t)(r * D * 2 + c16 * 16), v);
  }
  // every lane has read the rows before the area is written again
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A wave-uniform pointer kept in scalar registers.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* x) {
  const uint64_t v = (uint64_t)x;
  return (T*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v));
}

// ---------------------------------------------------------------------------
// Pass 1: Lg[i] = LSE_i * log2(e) (+inf where LSE = -inf or i >= N) and
// D_i = rowsum(dO_i * O_i), per (batch, head), Npad rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_rowstat_kernel(BwdProblem p, int nchunk) {
  constexpr int LPR = D / 8;                 // lanes per row, 16 bytes each
  constexpr int RPP = kBwdThreads / LPR;     // rows per pass
  constexpr int ROWS = 64;                   // rows per workgroup
  const int chunk = (int)(blockIdx.x % nchunk);
  const int64_t bh = blockIdx.x / nchunk;
  const int N = p.N;
  const int sub = threadIdx.x % LPR;
  const __bf16* O = (const __bf16*)p.o + (size_t)bh * N * D;
  const __bf16* dO = (const __bf16*)p.dout + (size_t)bh * N * D;
  float* Lg = p.ws + (size_t)bh * 2 * p.Npad;
  float* Dg = Lg + p.Npad;
#pragma unroll
  for (int pass = 0; pass < ROWS / RPP; ++pass) {
    const int row = chunk * ROWS + pass * RPP + (int)threadIdx.x / LPR;
    float acc = 0.f;
    if (row < N) {
      const bf16x8 o = *(const bf16x8*)(O + (size_t)row * D + sub * 8);
      const bf16x8 g = *(const bf16x8*)(dO + (size_t)row * D + sub * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
    acc = group_sum<LPR>(acc);
    if (sub == 0) {
      const float L = row < N ? p.lse[(size_t)bh * N + row] : -INFINITY;
      Lg[row] = L == -INFINITY ? INFINITY : L * kLog2e;
      Dg[row] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 2: dK and dV.  Workgroup = 4 waves x 64 keys; query stages of 64.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool WINDOW, bool BITS>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdProblem p, int n_ktiles) {
  using St = Stage<D>;
  constexpr int ROWB = St::ROWB;
  constexpr int KBW = 2;             // 32-key blocks per wave (the guards below name both)
  constexpr int KW = 32 * KBW;       // keys per wave
  constexpr int DK = D / 16;         // k-steps over d
  constexpr int DB = D / 32;         // 32-wide d blocks
  static_assert(NW * KW == kBwdBlockKV, "keys per workgroup");
  static_assert(St::ROWS == kBwdStageQ, "stage rows");

  __shared__ __attribute__((aligned(1024))) char Qs0[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Qs1[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Gs0[St::BYTES];   // dO
  __shared__ __attribute__((aligned(1024))) char Gs1[St::BYTES];
  __shared__ __attribute__((aligned(1024))) float Ls0[256];        // [0,64) Lg, [64,128) D
  __shared__ __attribute__((aligned(1024))) float Ls1[256];
  // element mask: the stage's words [8 words of the workgroup's keys][64 rows]
  __shared__ __attribute__((aligned(256))) uint32_t Ms0[BITS ? 512 : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Ms1[BITS ? 512 : 1];
  __shared__ int tlist[BITS ? kMaskMaxTiles : 1];   // the key tile's listed query stages
  __shared__ __attribute__((aligned(16))) uint8_t ostage[NW * 32 * (2 * D + 16)];  // output staging

  // Causal without a window or a mask: persistent workgroups walking their
  // XCD's tiles, heavy and light alternating round by round, as in the
  // forward prefill.
  constexpr bool PERSIST = CAUSAL && !WINDOW && !BITS;
  const int64_t n_items = (int64_t)n_ktiles * p.B * p.H;
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
    const int kt = (int)(logical % n_ktiles);   // causal: low key tiles see the most queries
    const int64_t bh = logical / n_ktiles;
    const int b = (int)(bh / p.H);
    const int N = p.N, M = p.M;
    const int tid = threadIdx.x;
    const int lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int ws = __builtin_amdgcn_readfirstlane(tid / 64);
    const int kvl = __builtin_amdgcn_readfirstlane(clamp_kv(p.kv_len, b, M));
    const int off = kvl - N;                    // key j visible to query i iff j <= i + off
    const int k0 = kt * kBwdBlockKV;
    const int jw0 = k0 + ws * KW;               // first key of this wave

    const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * N * D;
    const __bf16* Gg = (const __bf16*)p.dout + (size_t)bh * N * D;
    const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D;
    const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D;
    const float* Wg = p.ws + (size_t)bh * 2 * p.Npad;

    // Local window: key j is seen by queries j - off - wr .. j - off + wl
    // (causal: wr = 0).  LOWQ: a key has a first query; WINDOW: and a last.
    constexpr bool LOWQ = CAUSAL || WINDOW;
    const int wl = WINDOW ? min(p.wl, N + kvl) : 0;
    const int wr = CAUSAL ? 0 : (WINDOW ? min(p.wr, N + kvl) : 0);
    // Query stages this workgroup visits.
    const int n_stage_all = (N + St::ROWS - 1) / St::ROWS;
    int s_lo = 0;
    if (LOWQ) s_lo = min(max(k0 - off - wr, 0) / St::ROWS, n_stage_all);
    int s_end = n_stage_all;
    if (WINDOW) s_end = clampi(floor_div(k0 + kBwdBlockKV - 1 - off + wl, St::ROWS) + 1, s_lo, n_stage_all);
    int n_stages = k0 < kvl ? s_end - s_lo : 0;
    // Element mask: the listed stages in [s_lo, s_lo + n_stages), from list
    // position lo (the list ascends).
    int lo = 0;
    if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int stride = mask_stage_stride(N);
      const int32_t* L = p.stage_lists + ((int64_t)(bm * p.mask_h + hm) * n_ktiles + kt) * stride;
      const int cnt = __builtin_amdgcn_readfirstlane(L[0]);
      for (int i = tid; i < cnt; i += kBwdThreads) tlist[i] = L[1 + i];
      __syncthreads();
      int below_lo = 0, below_hi = 0;
      for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int e = i0 + lane < cnt ? (tlist[i0 + lane] & 0x7FFFFFFF) : 0x7FFFFFFF;
        below_lo += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < s_lo));
        below_hi += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < s_lo + n_stages));
      }
      lo = __builtin_amdgcn_readfirstlane(below_lo);
      n_stages = __builtin_amdgcn_readfirstlane(below_hi) - lo;
    }
    // List entry of the t-th visited stage (bit 31 set where the mask does
    // not keep the whole tile), and its query stage.
    auto entry_of = [&](int t) -> int {
      if constexpr (BITS) return __builtin_amdgcn_readfirstlane(tlist[lo + t]);
      else return s_lo + t;
    };
    auto stage_of = [&](int t) -> int { return entry_of(t) & 0x7FFFFFFF; };

    // ---- K and V fragments of the wave's keys (B operands), zero past kv_len ----
    bf16x8 kf[KBW][DK], vf[KBW][DK];
  #pragma unroll
    for (int kb2 = 0; kb2 < KBW; ++kb2) {
      const int key = jw0 + 32 * kb2 + l32;
      const bool ok = key < kvl;
  #pragma unroll
      for (int kb = 0; kb < DK; ++kb) {
        const size_t e = (size_t)(ok ? key : 0) * D + kb * 16 + h * 8;
        kf[kb2][kb] = ok ? *(const bf16x8*)(Kg + e) : bf16x8{};
        vf[kb2][kb] = ok ? *(const bf16x8*)(Vg + e) : bf16x8{};
      }
    }

    // ---- stage loads: rows [64 s, 64 s + 64) of Q, dO, Lg, D ----
    uint32_t soff[St::BPW];
  #pragma unroll
    for (int i = 0; i < St::BPW; ++i) soff[i] = St::slot_src((ws + i * NW) * 64 + lane);
    const int nrec_q = N * 2 * D;  // the planner keeps this below 2^31
    // Lane l of wave 0's extra block: Lg (l < 16) or D (16 <= l < 32) chunk.
    const uint32_t loff = (uint32_t)((lane < 16 ? lane : (lane < 32 ? p.Npad / 4 + lane - 16 : 0)) * 16);
    // Element mask: wave ws loads words 2 ws and 2 ws + 1 of the workgroup's
    // 256 keys for the stage's 64 rows (lane = row) from the stage's block,
    // where the pre-pass stored them [word][row] (rows past N copy row N - 1):
    // 256 contiguous bytes per wave and word.  A stage the mask keeps whole
    // reads the key tile's all-ones block (block 0; stage s has block s + 1),
    // every lane the same word, so the wave touches one line.
    const uint32_t* Mg = nullptr;
    int mbytes = 0;
    if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int n_st = mask_stage_stride(N) - 1;
      Mg = p.stage_blocks + ((size_t)(bm * p.mask_h + hm) * n_ktiles + kt) * (n_st + 1) * (kMaskBlockBytes / 4);
      mbytes = (n_st + 1) * kMaskBlockBytes;
    }
    auto load_stage = [&](int e, char* Qd, char* Gd, float* Ld, uint32_t* Md) __attribute__((always_inline)) {
      const int s = e & 0x7FFFFFFF;
      const uint32_t rb = (uint32_t)s * St::ROWS * 2 * D;
  #pragma unroll
      for (int i = 0; i < St::BPW; ++i) {
        int wofs = (ws + i * NW) * 1024;
        asm volatile("" : "+s"(wofs));
        buffer_load_lds16(Qg, nrec_q, soff[i] + rb, (lds_ptr)(Qd + wofs));
        buffer_load_lds16(Gg, nrec_q, soff[i] + rb, (lds_ptr)(Gd + wofs));
      }
      if (ws == 0)
        buffer_load_lds16(Wg + s * St::ROWS, (int)((2 * p.Npad - s * St::ROWS) * 4), loff, (lds_ptr)Ld);
      if constexpr (BITS) {
  #pragma unroll
        for (int w = 0; w < 2; ++w) {
          int mofs = (2 * ws + w) * 64;
          asm volatile("" : "+s"(mofs));
          const uint32_t at = ((uint32_t)(s + 1) * (uint32_t)kMaskBlockBytes + (uint32_t)(mofs + lane) * 4u) &
                              (uint32_t)(e >> 31);  // whole: every lane reads word 0 of the all-ones block
          buffer_load_lds4<true>(Mg, mbytes, at, (lds_ptr)(Md + mofs));
        }
      }
    };

    // ---- per-lane LDS read bases ----
    // Row reads (A operand of S and dP): row 32 u + l32, chunk 2 kb + h.
    const int G = (l32 >> 2) & 3;
    const int rbase0 = l32 * ROWB + 16 * ((0 + h) ^ G);   // kb even; + 32 u ROWB + 64 (kb / 2)
    const int rbase1 = l32 * ROWB + 16 * ((2 + h) ^ G);   // kb odd
    // Transposing reads (A operand of dV^T, dK^T): lane j of 16-lane group g
    // reads row 32 u + 16 s' + 8 hi + 4 h + j / 4, columns 32 db + 16 (g % 2) +
    // 4 (j % 4) .. + 4.
    const int j16 = lane % 16, g2 = (lane / 16) % 2;
    const int tbase0 = (4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (0 + h)) + 8 * (j16 % 2);
    const int tbase1 = (8 + 4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (2 + h)) + 8 * (j16 % 2);

    f32x16 dkacc[KBW][DB], dvacc[KBW][DB];
  #pragma unroll
    for (int kb2 = 0; kb2 < KBW; ++kb2)
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        dkacc[kb2][db] = f32x16{};
        dvacc[kb2][db] = f32x16{};
        agpr_guard(dkacc[kb2][db]);
        agpr_guard(dvacc[kb2][db]);
      }
    const float c = fmaxf(p.scale * kLog2e, 1e-30f);
    // Query i sees the lane's key j iff j - off - wr <= i (causal, window) and
    // i <= j - off + wl (window); register r of a step holds query
    // qs0 + 8 (r / 4) + 4 h + r % 4, masked iff qs0 + 8 (r / 4) + r % 4 < thr
    // or > thr_hi.
    int thr[KBW], thr_hi[KBW];
  #pragma unroll
    for (int kb2 = 0; kb2 < KBW; ++kb2) {
      thr[kb2] = jw0 + 32 * kb2 + l32 - off - wr - 4 * h;
      thr_hi[kb2] = jw0 + 32 * kb2 + l32 - off + wl - 4 * h;
    }

    // One 32-query step of stage s from buffers (Qs, Gs, Ls, Ms).
    auto qstep = [&](int s, int u, const char* Qs, const char* Gs, const float* Ls, const uint32_t* Ms,
                     auto MASK) __attribute__((always_inline)) {
      constexpr bool mask = decltype(MASK)::value;
      const int qs0 = s * St::ROWS + 32 * u;
      f32x16 sacc[KBW], pacc[KBW];
      // Operands are read one fragment ahead of their MFMAs, in a ring of
      // three: a read overwrites a register two fragments after the asm MFMAs
      // last read it.  Scheduling barriers keep the reads where they are (the
      // scheduler would otherwise sink them next to their use and expose the
      // LDS latency before every fragment).
      bf16x8 qa[3], ga[3];
      auto read_qg = [&](int kb) __attribute__((always_inline)) {
        const int o = 32 * u * ROWB + 64 * (kb / 2) + ((kb & 1) ? rbase1 : rbase0);
        qa[kb % 3] = *lds_at<bf16x8>(Qs, o);
        ga[kb % 3] = *lds_at<bf16x8>(Gs, o);
      };
      read_qg(0);
      static_for<DK>([&](auto kc) {
        constexpr int kb = decltype(kc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kb + 1 < DK) read_qg(kb + 1);
  #pragma unroll
        for (int kb2 = 0; kb2 < KBW; ++kb2) {
          if constexpr (kb == 0) {
            mfma_vv0_nw(sacc[kb2], qa[kb % 3], kf[kb2][kb]);
            mfma_vv0_nw(pacc[kb2], ga[kb % 3], vf[kb2][kb]);
          } else {
            mfma_vv_nw(sacc[kb2], qa[kb % 3], kf[kb2][kb]);
            mfma_vv_nw(pacc[kb2], ga[kb % 3], vf[kb2][kb]);
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      mfma_guard_v4(sacc[0], pacc[0], sacc[1], pacc[1]);
      // P = 2^(S c - Lg), dS = P (dP - D).  Lane: key jw0 + 32 kb2 + l32,
      // register r: query qs0 + 8 (r / 4) + 4 h + r % 4.
      bf16x8 pf[KBW][2], sf[KBW][2];
  #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 L4 = *(const float4*)(Ls + 32 * u + 8 * g + 4 * h);
        const float4 D4 = *(const float4*)(Ls + 64 + 32 * u + 8 * g + 4 * h);
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
        const float Dv[4] = {D4.x, D4.y, D4.z, D4.w};
        // mask words of the four queries 32 u + 8 g + 4 h + e, for each of the
        // wave's 32-key blocks: bit l32 is the lane's key; the eight bits the
        // lane needs are gathered into one register, bit 4 kb2 + e
        [[maybe_unused]] uint32_t mvis = 0u;
        if constexpr (BITS) {
  #pragma unroll
          for (int kb2 = 0; kb2 < KBW; ++kb2) {
            const uint4 w4 = *(const uint4*)(Ms + (2 * ws + kb2) * 64 + 32 * u + 8 * g + 4 * h);
            const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  #pragma unroll
            for (int e = 0; e < 4; ++e) mvis |= ((w[e] >> l32) & 1u) << (4 * kb2 + e);
          }
        }
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
  #pragma unroll
          for (int kb2 = 0; kb2 < KBW; ++kb2) {
            float pv = fast_exp2(fmaf(sacc[kb2][r], c, -Lv[e]));
            if constexpr (mask) {
              const int qi = qs0 + 8 * g + e;
              bool hide = false;
              if constexpr (LOWQ) hide = qi < thr[kb2];
              if constexpr (WINDOW) hide = hide | (qi > thr_hi[kb2]);
              if constexpr (BITS) hide = hide | (((mvis >> (4 * kb2 + e)) & 1u) == 0u);
              pv = hide ? 0.f : pv;
            }
            const float dsv = pv * (pacc[kb2][r] - Dv[e]);
            pf[kb2][r / 8][r % 8] = (__bf16)pv;
            sf[kb2][r / 8][r % 8] = (__bf16)dsv;
          }
        }
      }
      asm volatile("s_nop 4" : "+v"(pf[0][0]), "+v"(sf[0][0]), "+v"(pf[0][1]), "+v"(sf[0][1]),
                   "+v"(pf[1][0]), "+v"(sf[1][0]), "+v"(pf[1][1]), "+v"(sf[1][1]));  // valu_guard, all eight
      // dV^T += dO^T P, dK^T += Q^T dS over the step's 32 queries; fragment
      // i = (sp, db), operands read one fragment ahead in a ring of three.
      bf16x8 gt[3], qt[3];
      auto read_t = [&](int i) __attribute__((always_inline)) {
        const int o = (32 * u + 16 * (i / DB)) * ROWB + 64 * (i % DB);
        const s16x4 glo = lds_read_tr16((const __bf16*)(Gs + o + tbase0));
        const s16x4 ghi = lds_read_tr16((const __bf16*)(Gs + o + tbase1));
        const s16x4 qlo = lds_read_tr16((const __bf16*)(Qs + o + tbase0));
        const s16x4 qhi = lds_read_tr16((const __bf16*)(Qs + o + tbase1));
        gt[i % 3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7));
        qt[i % 3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      read_t(0);
      static_for<2 * DB>([&](auto ic) {
        constexpr int i = decltype(ic)::value, sp = i / DB, db = i % DB;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i + 1 < 2 * DB) read_t(i + 1);
  #pragma unroll
        for (int kb2 = 0; kb2 < KBW; ++kb2) {
          mfma_aa_nw(dvacc[kb2][db], gt[i % 3], pf[kb2][sp]);
          mfma_aa_nw(dkacc[kb2][db], qt[i % 3], sf[kb2][sp]);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    // Every branch below is uniform over the workgroup and no step is skipped
    // inside a loop: control flow that joins with the accumulators live makes
    // the register allocator shuffle them between AGPRs.
    auto iteration = [&](int t, const char* Qs, const char* Gs, const float* Ls, const uint32_t* Ms,
                         char* Qn, char* Gn, float* Ln, uint32_t* Mn, auto MASK) __attribute__((always_inline)) {
      wait_vm0();
      __syncthreads();
      const int s_cur = stage_of(t);
      if (t + 1 < n_stages) load_stage(entry_of(t + 1), Qn, Gn, Ln, Mn);
      qstep(s_cur, 0, Qs, Gs, Ls, Ms, MASK);
      qstep(s_cur, 1, Qs, Gs, Ls, Ms, MASK);
    };

    if (n_stages > 0) load_stage(entry_of(0), Qs0, Gs0, Ls0, Ms0);
    if constexpr (BITS) {
      // element mask: every listed stage applies its bits (and the causal
      // and window rules)
      int t = 0;
      for (; t + 1 < n_stages; t += 2) {
        iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::true_type{});
        iteration(t + 1, Qs1, Gs1, Ls1, Ms1, Qs0, Gs0, Ls0, Ms0, std::true_type{});
      }
      if (t < n_stages) iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::true_type{});
    } else if constexpr (!WINDOW) {
      // Causal: the first n_mask stages hold queries that do not see every key
      // of the workgroup and are masked element by element (an even number, so
      // that the unmasked loop starts on buffer 0, or all stages).
      int n_mask = 0;
      if (CAUSAL) {
        const int rows = k0 + kBwdBlockKV - 1 - off - s_lo * St::ROWS;  // masked rows from stage s_lo on
        n_mask = rows > 0 ? min((rows + 2 * St::ROWS - 1) / (2 * St::ROWS) * 2, n_stages) : 0;
      }
      int t = 0;
      for (; t + 1 < n_mask; t += 2) {
        iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::true_type{});
        iteration(t + 1, Qs1, Gs1, Ls1, Ms1, Qs0, Gs0, Ls0, Ms0, std::true_type{});
      }
      if (t < n_mask) {  // n_mask == n_stages, odd: the last stage
        iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::true_type{});
        ++t;
      }
      for (; t + 1 < n_stages; t += 2) {
        iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::false_type{});
        iteration(t + 1, Qs1, Gs1, Ls1, Ms1, Qs0, Gs0, Ls0, Ms0, std::false_type{});
      }
      if (t < n_stages) iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, std::false_type{});
    } else {
      // Window: stages before nA hold queries before some key's first viewer,
      // stages from nC on queries past some key's last viewer; both masked,
      // the stages between are seen whole.  Stage t uses buffer t % 2.
      const int nA = clampi(floor_div(k0 + kBwdBlockKV - 1 - off - wr + St::ROWS - 1, St::ROWS) - s_lo,
                            0, n_stages);
      const int nC = clampi(floor_div(k0 - off + wl - (St::ROWS - 1), St::ROWS) + 1 - s_lo, nA, n_stages);
      auto segment = [&](int t, int t_end, auto MASK) __attribute__((always_inline)) {
        if ((t & 1) && t < t_end) {
          iteration(t, Qs1, Gs1, Ls1, Ms1, Qs0, Gs0, Ls0, Ms0, MASK);
          ++t;
        }
        for (; t + 1 < t_end; t += 2) {
          iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, MASK);
          iteration(t + 1, Qs1, Gs1, Ls1, Ms1, Qs0, Gs0, Ls0, Ms0, MASK);
        }
        if (t < t_end) iteration(t, Qs0, Gs0, Ls0, Ms0, Qs1, Gs1, Ls1, Ms1, MASK);
      };
      segment(0, nA, std::true_type{});
      segment(nA, nC, std::false_type{});
      segment(nC, n_stages, std::true_type{});
    }

  #pragma unroll
    for (int kb2 = 0; kb2 < KBW; ++kb2)
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        mfma_guard_a(dkacc[kb2][db]);
        mfma_guard_a(dvacc[kb2][db]);
      }
    // ---- write dK = scale * dK^T^T and dV (zero for keys at or past kv_len) ----
    // Accumulator (kb2, db), register r: d = 32 db + 8 (r / 4) + 4 h + r % 4,
    // key jw0 + 32 kb2 + l32.
    const float sc = p.scale;
    uint8_t* st = ostage + (tid / 64) * 32 * (2 * D + 16);
  #pragma unroll
    for (int kb2 = 0; kb2 < KBW; ++kb2) {
      const int k_blk = __builtin_amdgcn_readfirstlane(jw0 + 32 * kb2);
      const bool ok = k_blk + l32 < kvl;
      const size_t at = ((size_t)bh * M + k_blk) * D;
      store_block_staged<D>(st, dkacc[kb2], sc, ok, uniform_ptr((__bf16*)p.dk + at), M - k_blk);
      store_block_staged<D>(st, dvacc[kb2], 1.f, ok, uniform_ptr((__bf16*)p.dv + at), M - k_blk);
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Pass 3: dQ.  Workgroup = 4 waves x 64 queries; key stages of 64.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool WINDOW, bool BITS>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdProblem p, int n_qtiles) {
  using St = Stage<D>;
  constexpr int ROWB = St::ROWB;
  constexpr int QW = 64;             // queries per wave
  constexpr int NQB = QW / 32;       // 32-query blocks per wave (two; the guards name both)
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  static_assert(NW * QW == kBwdBlockQ, "queries per workgroup");
  static_assert(St::ROWS == kBwdStageK, "stage rows");

  __shared__ __attribute__((aligned(1024))) char Ks0[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Ks1[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs0[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs1[St::BYTES];
  // element mask: the workgroup's list of key tiles (stages), and per stage
  // each wave's mask words [word][64 rows]
  __shared__ int tlist[BITS ? kMaskMaxTiles : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Mq0[BITS ? NW * 128 : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Mq1[BITS ? NW * 128 : 1];
  __shared__ __attribute__((aligned(16))) uint8_t ostage[NW * 32 * (2 * D + 16)];  // output staging

  // Causal without a window or a mask: persistent workgroups walking their
  // XCD's tiles, heavy and light alternating round by round, as in the
  // forward prefill.
  constexpr bool PERSIST = CAUSAL && !WINDOW && !BITS;
  // A stage as one pipeline (stage_piped) rather than two ksteps: for plain
  // causal attention, the one form whose registers hold the scores and dP of
  // both blocks at D = 128 without spills.  Measured (B = 2, H = 32,
  // N = 8192, causal, one box, interleaved, bit-identical): the whole
  // backward 3.556 -> 3.470 ms at D = 128 and 2.140 -> 2.083 ms at D = 64.
  // With only the second overlap (dS of block 1 under the dQ MFMAs of block
  // 0), which is all that fits beside a mask or a window, the pass ran 1-2%
  // slower than two ksteps, so those keep kstep.
  constexpr bool PIPE = CAUSAL && !WINDOW && !BITS;
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
    if (CAUSAL) qt = n_qtiles - 1 - qt;   // heaviest query tiles first
    const int b = (int)(bh / p.H);
    const int N = p.N, M = p.M;
    const int tid = threadIdx.x;
    const int lane = tid % 64, h = lane / 32, l32 = lane % 32;
    const int ws = __builtin_amdgcn_readfirstlane(tid / 64);
    const int kvl = __builtin_amdgcn_readfirstlane(clamp_kv(p.kv_len, b, M));
    const int off = kvl - N;
    const int q0 = qt * kBwdBlockQ;
    const int qw0 = q0 + ws * QW;
    const int q_last = min(q0 + kBwdBlockQ, N) - 1;
    // Local window: query i sees keys i + off - wl .. i + off + wr (causal: wr = 0).
    constexpr bool UPPER = CAUSAL || WINDOW;
    const int wl = WINDOW ? min(p.wl, N + kvl) : 0;
    const int wr = CAUSAL ? 0 : (WINDOW ? min(p.wr, N + kvl) : 0);
    const int kv_end = UPPER ? min(kvl, q_last + off + wr + 1) : kvl;
    // first key stage (window: the first query's first key)
    const int t0 = WINDOW ? max(0, q0 + off - wl) / St::ROWS : 0;
    int n_stages = kv_end > t0 * St::ROWS ? (kv_end + St::ROWS - 1) / St::ROWS - t0 : 0;
    // Element mask: the listed stages in [t0, t0 + n_stages), from list
    // position lo (the list ascends; see the forward).
    int lo = 0;
    if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int stride = mask_list_stride(M);
      const int32_t* L = p.lists + ((int64_t)(bm * p.mask_h + hm) * n_qtiles + qt) * stride;
      const int cnt = __builtin_amdgcn_readfirstlane(L[0]);
      for (int i = tid; i < cnt; i += kBwdThreads) tlist[i] = L[1 + i];
      __syncthreads();
      int below_lo = 0, below_hi = 0;
      for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int e = i0 + lane < cnt ? (tlist[i0 + lane] & 0x7FFFFFFF) : 0x7FFFFFFF;
        below_lo += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < t0));
        below_hi += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < t0 + n_stages));
      }
      lo = __builtin_amdgcn_readfirstlane(below_lo);
      n_stages = __builtin_amdgcn_readfirstlane(below_hi) - lo;
    }
    // List entry of the t-th visited stage (bit 31 set where the mask does
    // not keep the whole tile), and its key stage.
    auto entry_of = [&](int t) -> int {
      if constexpr (BITS) return __builtin_amdgcn_readfirstlane(tlist[lo + t]);
      else return t0 + t;
    };
    auto stage_of = [&](int t) -> int { return entry_of(t) & 0x7FFFFFFF; };

    const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * N * D;
    const __bf16* Gg = (const __bf16*)p.dout + (size_t)bh * N * D;
    const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D;
    const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D;
    const float* Wg = p.ws + (size_t)bh * 2 * p.Npad;

    // ---- Q and dO fragments of the wave's queries (B operands) ----
    // Rows past N hold zeros; their Lg is +inf, so their weights are 0.
    bf16x8 qf[NQB][DK], gf[NQB][DK];
    float Lq[NQB], Dq[NQB];
    int lim[NQB];                  // last key the lane's query sees
    int lim_lo[NQB];               // first key (window)
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = qw0 + 32 * qb + l32;
      const bool ok = row < N;
  #pragma unroll
      for (int kb = 0; kb < DK; ++kb) {
        const size_t e = (size_t)(ok ? row : 0) * D + kb * 16 + h * 8;
        qf[qb][kb] = ok ? *(const bf16x8*)(Qg + e) : bf16x8{};
        gf[qb][kb] = ok ? *(const bf16x8*)(Gg + e) : bf16x8{};
      }
      Lq[qb] = Wg[row];            // row < Npad
      Dq[qb] = Wg[p.Npad + row];
      lim[qb] = UPPER ? min(row + off + wr, kvl - 1) : kvl - 1;
      lim_lo[qb] = row + off - wl;
    }

    uint32_t soff[St::BPW];
  #pragma unroll
    for (int i = 0; i < St::BPW; ++i) soff[i] = St::slot_src((ws + i * NW) * 64 + lane);
    const int nrec_k = kvl * 2 * D;  // the planner keeps M * D * 2 below 2^31
    // Element mask: words 2 s and 2 s + 1 of the wave's 64 query rows (lane =
    // row) from the (query tile, key stage) block, stored by the pre-pass as
    // the forward's (rows past N copy row N - 1): 256 contiguous bytes per
    // wave and word.  A stage the mask keeps whole reads the query tile's
    // all-ones block (block 0; stage s has block s + 1), every lane the same
    // word, so the wave touches one line.
    const uint32_t* Mg = nullptr;
    int mbytes = 0;
    if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int n_kt = mask_list_stride(M) - 1;
      Mg = p.blocks + ((size_t)(bm * p.mask_h + hm) * n_qtiles + qt) * (n_kt + 1) * (kMaskBlockBytes / 4);
      mbytes = (n_kt + 1) * kMaskBlockBytes;
    }
    auto load_stage = [&](int e, char* Kd, char* Vd, uint32_t* Md) __attribute__((always_inline)) {
      const int s = e & 0x7FFFFFFF;
      if constexpr (BITS) {
  #pragma unroll
        for (int w = 0; w < 2; ++w) {
          int mofs = ws * 128 + w * 64;
          asm volatile("" : "+s"(mofs));
          const uint32_t at = ((uint32_t)(s + 1) * (uint32_t)kMaskBlockBytes + (uint32_t)(mofs + lane) * 4u) &
                              (uint32_t)(e >> 31);  // whole: every lane reads word 0 of the all-ones block
          buffer_load_lds4<true>(Mg, mbytes, at, (lds_ptr)(Md + mofs));
        }
      }
      const uint32_t rb = (uint32_t)s * St::ROWS * 2 * D;
  #pragma unroll
      for (int i = 0; i < St::BPW; ++i) {
        int wofs = (ws + i * NW) * 1024;
        asm volatile("" : "+s"(wofs));
        buffer_load_lds16(Kg, nrec_k, soff[i] + rb, (lds_ptr)(Kd + wofs));
        buffer_load_lds16(Vg, nrec_k, soff[i] + rb, (lds_ptr)(Vd + wofs));
      }
    };

    const int G = (l32 >> 2) & 3;
    const int rbase0 = l32 * ROWB + 16 * ((0 + h) ^ G);
    const int rbase1 = l32 * ROWB + 16 * ((2 + h) ^ G);
    const int j16 = lane % 16, g2 = (lane / 16) % 2;
    const int tbase0 = (4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (0 + h)) + 8 * (j16 % 2);
    const int tbase1 = (8 + 4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (2 + h)) + 8 * (j16 % 2);

    f32x16 dqacc[NQB][DB];
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        dqacc[qb][db] = f32x16{};
        agpr_guard(dqacc[qb][db]);
      }
    const float c = fmaxf(p.scale * kLog2e, 1e-30f);

    // 32 keys (block kb2) of stage s.
    auto kstep = [&](int s, int kb2, const char* Ks, const char* Vs, const uint32_t* Ms, auto MASK)
                     __attribute__((always_inline)) {
      constexpr bool mask = decltype(MASK)::value;
      const int kk0 = s * St::ROWS + 32 * kb2;
      f32x16 sacc[NQB], pacc[NQB];
      // Operands one fragment ahead, in a ring of three (as in the dK/dV pass).
      bf16x8 ka[3], va[3];
      auto read_kv = [&](int kb) __attribute__((always_inline)) {
        const int o = 32 * kb2 * ROWB + 64 * (kb / 2) + ((kb & 1) ? rbase1 : rbase0);
        ka[kb % 3] = *lds_at<bf16x8>(Ks, o);
        va[kb % 3] = *lds_at<bf16x8>(Vs, o);
      };
      read_kv(0);
      static_for<DK>([&](auto kc) {
        constexpr int kb = decltype(kc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kb + 1 < DK) read_kv(kb + 1);
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          if constexpr (kb == 0) {
            mfma_vv0_nw(sacc[qb], ka[kb % 3], qf[qb][kb]);
            mfma_vv0_nw(pacc[qb], va[kb % 3], gf[qb][kb]);
          } else {
            mfma_vv_nw(sacc[qb], ka[kb % 3], qf[qb][kb]);
            mfma_vv_nw(pacc[qb], va[kb % 3], gf[qb][kb]);
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      mfma_guard_v4(sacc[0], pacc[0], sacc[1], pacc[1]);
      // Lane: query qw0 + 32 qb + l32; register r: key kk0 + 8 (r / 4) + 4 h + r % 4.
      bf16x8 sf[NQB][2];
      // mask: key kk0 + 8 (r / 4) + 4 h + r % 4 is bit 8 (r / 4) + r % 4 of the
      // row's word shifted down by 4 h (bit set: hidden)
      [[maybe_unused]] uint32_t hid[NQB];
      if constexpr (BITS) {
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) hid[qb] = ~Ms[ws * 128 + kb2 * 64 + 32 * qb + l32] >> (4 * h);
      }
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(sacc[qb][r], c, -Lq[qb]));
          if constexpr (mask) {
            const int key = kk0 + 8 * (r / 4) + 4 * h + r % 4;
            bool hide = key > lim[qb];
            if constexpr (WINDOW) hide = hide | (key < lim_lo[qb]);
            if constexpr (BITS) hide = hide | (((hid[qb] >> (8 * (r / 4) + r % 4)) & 1u) != 0u);
            pv = hide ? 0.f : pv;
          }
          sf[qb][r / 8][r % 8] = (__bf16)(pv * (pacc[qb][r] - Dq[qb]));
        }
      valu_guard4(sf[0][0], sf[0][1], sf[1][0], sf[1][1]);
      // dQ^T += K^T dS^T over the 32 keys; fragment i = (sp, db), operands
      // one fragment ahead in a ring of three.
      bf16x8 kt[3];
      auto read_t = [&](int i) __attribute__((always_inline)) {
        const int o = (32 * kb2 + 16 * (i / DB)) * ROWB + 64 * (i % DB);
        const s16x4 klo = lds_read_tr16((const __bf16*)(Ks + o + tbase0));
        const s16x4 khi = lds_read_tr16((const __bf16*)(Ks + o + tbase1));
        kt[i % 3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(klo, khi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      read_t(0);
      static_for<2 * DB>([&](auto ic) {
        constexpr int i = decltype(ic)::value, sp = i / DB, db = i % DB;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i + 1 < 2 * DB) read_t(i + 1);
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) mfma_aa_nw(dqacc[qb][db], kt[i % 3], sf[qb][sp]);
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    // A whole stage (64 keys, two 32-key blocks) as a software pipeline, so
    // that the VALU work of one block runs under the MFMAs of the other:
    //   1: S and dP of block 0;
    //   2: S and dP of block 1, with dS of block 0 (one pair of scores every
    //      second MFMA);
    //   3: dQ^T += K^T dS^T of block 0, with dS of block 1 (a pair per MFMA);
    //   4: the same product for block 1.
    // The arithmetic of every score and every product is kstep's, in the same
    // order per accumulator, so the result is bitwise the same.  dO sits in
    // AGPRs as the B operand of dP (Q stays in VGPRs), which leaves room in
    // the VGPRs for the scores and dP of both blocks.
    auto stage_piped = [&](int s, const char* Ks, const char* Vs, const uint32_t* Ms, auto MASK)
                           __attribute__((always_inline)) {
      constexpr bool mask = decltype(MASK)::value;
      f32x16 sa[2][NQB], pa[2][NQB];  // scores and dP of blocks 0 and 1
      bf16x8 sd[2][NQB][2];           // dS of blocks 0 and 1 (16 keys per vector)
      [[maybe_unused]] uint32_t hid[2][NQB];
      bf16x8 ka[3], va[3], kt[3];
      // fragment kb of block kb2 into ring slot `slot`
      auto read_kv = [&](int kb2, int kb, int slot) __attribute__((always_inline)) {
        const int o = 32 * kb2 * ROWB + 64 * (kb / 2) + ((kb & 1) ? rbase1 : rbase0);
        ka[slot] = *lds_at<bf16x8>(Ks, o);
        va[slot] = *lds_at<bf16x8>(Vs, o);
      };
      // MFMA m of the S and dP products of block kb2: fragment kb = m / 4, then
      // S of query block 0, dP of 0, S of 1, dP of 1 (kstep's order).  Ring
      // slots continue from block 0 into block 1 (fragment DK kb2 + kb), so a
      // slot is rewritten only after the MFMAs of the fragments between.
      auto sdp_step = [&](auto kbc, auto mc) __attribute__((always_inline)) {
        constexpr int kb2 = decltype(kbc)::value, m = decltype(mc)::value;
        constexpr int kb = m / 4, qb = (m / 2) % 2, w = m % 2, f = DK * kb2 + kb;
        if constexpr (m % 4 == 0 && kb + 1 < DK) read_kv(kb2, kb + 1, (f + 1) % 3);
        if constexpr (w == 0) {
          if constexpr (kb == 0) mfma_vv0_nw(sa[kb2][qb], ka[f % 3], qf[qb][kb]);
          else mfma_vv_nw(sa[kb2][qb], ka[f % 3], qf[qb][kb]);
        } else {
          // dO's fragments are copied into AGPRs right before some of these: keep the wait
          if constexpr (kb == 0) mfma_va0(pa[kb2][qb], va[f % 3], gf[qb][kb]);
          else mfma_va(pa[kb2][qb], va[f % 3], gf[qb][kb]);
        }
      };
      // dS of scores 2 j and 2 j + 1 of query block qb of block kb2 (unit
      // u = 8 qb + j), as kstep computes each.
      auto ds_unit = [&](auto kbc, auto uc) __attribute__((always_inline)) {
        constexpr int kb2 = decltype(kbc)::value, u = decltype(uc)::value, qb = u / 8;
        const int kk0 = s * St::ROWS + 32 * kb2;
  #pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * (u % 8) + e;
          float pv = fast_exp2(fmaf(sa[kb2][qb][r], c, -Lq[qb]));
          if constexpr (mask) {
            const int key = kk0 + 8 * (r / 4) + 4 * h + r % 4;
            bool hide = key > lim[qb];
            if constexpr (WINDOW) hide = hide | (key < lim_lo[qb]);
            if constexpr (BITS) hide = hide | (((hid[kb2][qb] >> (8 * (r / 4) + r % 4)) & 1u) != 0u);
            pv = hide ? 0.f : pv;
          }
          sd[kb2][qb][r / 8][r % 8] = (__bf16)(pv * (pa[kb2][qb][r] - Dq[qb]));
        }
        // keep the pair's pack here (IR passes would sink it past the
        // scheduling barrier that follows)
        asm volatile("" ::"v"(sd[kb2][qb][(2 * (u % 8)) / 8]));
      };
      // K^T fragment i of block kb2 (as kstep's read_t) into ring slot `slot`
      auto read_t = [&](int kb2, int i, int slot) __attribute__((always_inline)) {
        const int o = (32 * kb2 + 16 * (i / DB)) * ROWB + 64 * (i % DB);
        const s16x4 klo = lds_read_tr16((const __bf16*)(Ks + o + tbase0));
        const s16x4 khi = lds_read_tr16((const __bf16*)(Ks + o + tbase1));
        kt[slot] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(klo, khi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // MFMA j of dQ^T += K^T dS^T for block kb2: fragment i = j / 2 =
      // (sp, db), query block j % 2 (kstep's order).
      auto dq_step = [&](auto kbc, auto jc) __attribute__((always_inline)) {
        constexpr int kb2 = decltype(kbc)::value, j = decltype(jc)::value;
        constexpr int i = j / 2, qb = j % 2, sp = i / DB, db = i % DB, f = 2 * DB * kb2 + i;
        if constexpr (qb == 0 && i + 1 < 2 * DB) read_t(kb2, i + 1, (f + 1) % 3);
        mfma_aa_nw(dqacc[qb][db], kt[f % 3], sd[kb2][qb][sp]);
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      if constexpr (BITS) {
  #pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb) hid[kb2][qb] = ~Ms[ws * 128 + kb2 * 64 + 32 * qb + l32] >> (4 * h);
      }
      // 1
      read_kv(0, 0, 0);
      static_for<4 * DK>([&](auto mc) {
        __builtin_amdgcn_sched_barrier(0);
        sdp_step(I0{}, mc);
      });
      __builtin_amdgcn_sched_barrier(0);
      mfma_guard_v4(sa[0][0], pa[0][0], sa[0][1], pa[0][1]);
      // 2
      read_kv(1, 0, DK % 3);
      static_for<4 * DK>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        __builtin_amdgcn_sched_barrier(0);
        sdp_step(I1{}, mc);
        constexpr int u0 = m * 16 / (4 * DK), u1 = (m + 1) * 16 / (4 * DK);
        static_for<u1 - u0>([&](auto uc) { ds_unit(I0{}, std::integral_constant<int, u0 + decltype(uc)::value>{}); });
      });
      __builtin_amdgcn_sched_barrier(0);
      mfma_guard_v4(sa[1][0], pa[1][0], sa[1][1], pa[1][1]);
      valu_guard4(sd[0][0][0], sd[0][0][1], sd[0][1][0], sd[0][1][1]);
      // 3
      read_t(0, 0, 0);
      static_for<4 * DB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        dq_step(I0{}, jc);
        constexpr int u0 = j * 16 / (4 * DB), u1 = (j + 1) * 16 / (4 * DB);
        static_for<u1 - u0>([&](auto uc) { ds_unit(I1{}, std::integral_constant<int, u0 + decltype(uc)::value>{}); });
      });
      __builtin_amdgcn_sched_barrier(0);
      valu_guard4(sd[1][0][0], sd[1][0][1], sd[1][1][0], sd[1][1][1]);
      // 4
      read_t(1, 0, (2 * DB) % 3);
      static_for<4 * DB>([&](auto jc) {
        __builtin_amdgcn_sched_barrier(0);
        dq_step(I1{}, jc);
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(16 % (4 * DB) == 0 && (4 * DK) % 16 == 0, "dS units (16 pairs per block) spread evenly");

    // As in the dK/dV pass: uniform branches only, no step skipped in a loop.
    auto iteration = [&](int t, const char* Ks, const char* Vs, const uint32_t* Ms, char* Kn, char* Vn,
                         uint32_t* Mn, auto MASK) __attribute__((always_inline)) {
      wait_vm0();
      __syncthreads();
      const int s_cur = stage_of(t);
      if (t + 1 < n_stages) load_stage(entry_of(t + 1), Kn, Vn, Mn);
      if constexpr (PIPE) {
        stage_piped(s_cur, Ks, Vs, Ms, MASK);
      } else {
        kstep(s_cur, 0, Ks, Vs, Ms, MASK);
        kstep(s_cur, 1, Ks, Vs, Ms, MASK);
      }
    };

    // Stages before n_clean (an even number) are seen whole by every query of
    // the workgroup: no key past kv_len and, causal, none past the first
    // query's last key.  The rest are masked element by element.
    if (n_stages > 0) load_stage(entry_of(0), Ks0, Vs0, Mq0);
    if constexpr (BITS) {
      // element mask: every listed stage applies its bits (and the causal,
      // window and kv_len rules)
      int t = 0;
      for (; t + 1 < n_stages; t += 2) {
        iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, std::true_type{});
        iteration(t + 1, Ks1, Vs1, Mq1, Ks0, Vs0, Mq0, std::true_type{});
      }
      if (t < n_stages) iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, std::true_type{});
    } else if constexpr (!WINDOW) {
      int n_clean = kvl / St::ROWS;
      if (CAUSAL) n_clean = min(n_clean, q0 + off + 1 > 0 ? (q0 + off + 1) / St::ROWS : 0);
      n_clean = min(n_clean, n_stages) / 2 * 2;
      int t = 0;
      for (; t < n_clean; t += 2) {
        iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, std::false_type{});
        iteration(t + 1, Ks1, Vs1, Mq1, Ks0, Vs0, Mq0, std::false_type{});
      }
      for (; t + 1 < n_stages; t += 2) {
        iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, std::true_type{});
        iteration(t + 1, Ks1, Vs1, Mq1, Ks0, Vs0, Mq0, std::true_type{});
      }
      if (t < n_stages) iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, std::true_type{});
    } else {
      // Window: stages before nA hold keys before the last query's first key,
      // stages from nC on keys past the first query's last key (or kv_len);
      // both masked, the stages between are seen whole.  Stage t uses buffer
      // t % 2.
      const int nA = clampi(floor_div(q_last + off - wl + St::ROWS - 1, St::ROWS) - t0, 0, n_stages);
      const int last_all = min(UPPER ? q0 + off + wr : kvl - 1, kvl - 1);  // last key every query sees
      const int nC = clampi(floor_div(last_all - (St::ROWS - 1), St::ROWS) + 1 - t0, nA, n_stages);
      auto segment = [&](int t, int t_end, auto MASK) __attribute__((always_inline)) {
        if ((t & 1) && t < t_end) {
          iteration(t, Ks1, Vs1, Mq1, Ks0, Vs0, Mq0, MASK);
          ++t;
        }
        for (; t + 1 < t_end; t += 2) {
          iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, MASK);
          iteration(t + 1, Ks1, Vs1, Mq1, Ks0, Vs0, Mq0, MASK);
        }
        if (t < t_end) iteration(t, Ks0, Vs0, Mq0, Ks1, Vs1, Mq1, MASK);
      };
      segment(0, nA, std::true_type{});
      segment(nA, nC, std::false_type{});
      segment(nC, n_stages, std::true_type{});
    }

  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
      for (int db = 0; db < DB; ++db) mfma_guard_a(dqacc[qb][db]);
    // ---- write dQ = scale * (dQ^T)^T ----
    // Accumulator (qb, db), register r: d = 32 db + 8 (r / 4) + 4 h + r % 4,
    // query qw0 + 32 qb + l32.
    const float sc = p.scale;
    uint8_t* st = ostage + (tid / 64) * 32 * (2 * D + 16);
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int q_blk = __builtin_amdgcn_readfirstlane(qw0 + 32 * qb);
      store_block_staged<D>(st, dqacc[qb], sc, true, uniform_ptr((__bf16*)p.dq + ((size_t)bh * N + q_blk) * D),
                            N - q_blk);
    }
  }
  }
}

// Workgroups of a pass: one per item, or, persistent, at most one per CU (a
// multiple of the 8 XCDs).
int64_t persist_grid(int64_t items, bool persistent) {
  return persistent ? std::min<int64_t>((items + 7) / 8 * 8, kPrefillPersistGrid) : items;
}

template <int D, bool BITS>
void launch_bwd_passes(const BwdProblem& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  const dim3 block(kBwdThreads);
  if (p.M > 0) {
    const int n_kt = (p.M + kBwdBlockKV - 1) / kBwdBlockKV;
    const dim3 grid((unsigned)persist_grid(bh * n_kt, p.causal && !p.window && !BITS));
    if (p.window) {
      if (p.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true, BITS>), grid, block, 0, stream, p, n_kt);
      else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true, BITS>), grid, block, 0, stream, p, n_kt);
    } else {
      if (p.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false, BITS>), grid, block, 0, stream, p, n_kt);
      else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false, BITS>), grid, block, 0, stream, p, n_kt);
    }
  }
  if (p.N > 0) {
    const int n_qt = (p.N + kBwdBlockQ - 1) / kBwdBlockQ;
    const dim3 grid((unsigned)persist_grid(bh * n_qt, p.causal && !p.window && !BITS));
    if (p.window) {
      if (p.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, true, BITS>), grid, block, 0, stream, p, n_qt);
      else hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, BITS>), grid, block, 0, stream, p, n_qt);
    } else {
      if (p.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, BITS>), grid, block, 0, stream, p, n_qt);
      else hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, BITS>), grid, block, 0, stream, p, n_qt);
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdProblem& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  const dim3 block(kBwdThreads);
  if (p.N > 0) {
    const int nchunk = p.Npad / 64;
    hipLaunchKernelGGL(bwd_rowstat_kernel<D>, dim3((unsigned)(bh * nchunk)), block, 0, stream, p, nchunk);
  }
  if (p.mask) {
    // the dQ pass's tile lists (the forward's) and the dK/dV pass's stage
    // lists, then both passes with bits
    const fa_shape s{p.B, p.H, p.N, p.M, p.D};
    launch_mask_prep(p.mask, p.N, p.M, p.mask_w, p.mask_b, p.mask_h, p.ws,
                     mask_workspace(p.N, p.M, p.mask_b, p.mask_h, bwd_mask_lists_offset(s), true), true,
                     stream);
    launch_bwd_passes<D, true>(p, stream);
  } else {
    launch_bwd_passes<D, false>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdProblem& p, hipStream_t stream) {
  if ((int64_t)p.B * p.H == 0) return hipSuccess;
  return p.D == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace fa
