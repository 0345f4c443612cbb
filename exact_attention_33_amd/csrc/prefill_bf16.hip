// Fused tiled exact-attention forward, bf16 inputs, float32 accumulation,
// for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// Method ("Flash Attention: The Hidden Gem", The Algorithm and The Correction
// Factor; "FlashAttention: attention was never compute-bound", The one
// formula): each workgroup owns a tile of queries and keeps, per query row, a
// running max m, a running sum l and an unnormalised output accumulator.  K
// and V tiles stream through LDS; for each tile the score tile S = Q K^T is
// formed on chip, the tile's weights e^(S - m) are added (l += rowsum,
// O += P V), and whenever m has to move, l and the accumulator are rescaled
// by e^(m_old - m_new).  The output is divided by l once, after the last tile
// ("Understanding FlashAttention", From loops to tiling: keep the numerator
// and divide at the end), and L = m + log(l) is written beside it.  The score
// and weight tiles never leave registers.
//
// gfx950 mapping:
//  * workgroup = 8 waves = 256 queries; wave w owns queries [32w, 32w + 32).
//    Waves w and w + 4 share a SIMD.  They run the per-tile work in two
//    phases -- an MFMA phase (S(t+1) = K(t+1) Q^T and O += P(t) V(t)) and a
//    VALU phase (mask, row max and exponentials of tile t+1) -- offset by one
//    phase: while waves 0-3 are in their MFMA phase, waves 4-7 are in their
//    VALU phase and vice versa, with a workgroup barrier between phases.
//    MFMA and VALU instructions of two waves on one SIMD overlap almost
//    perfectly (measured on MI355X), so each SIMD keeps its matrix pipe busy
//    while the other wave does the softmax arithmetic;
//  * the score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: Q is the B operand and stays in registers for
//    the whole sweep, K comes from LDS.  Lane (h, c) of a wave (h = lane / 32,
//    c = lane % 32) then holds 16 scores of query c per 32-key block, at keys
//    8*(r/4) + 4*h + r%4, so row max and row sum are in-lane plus one
//    exchange between the two half-waves;
//  * scores are kept in base 2: t = s * scale * log2(e), weights 2^(t - m) on
//    v_exp_f32; the scale is applied in float32 to the float32 score;
//  * the reference max m moves only when a row's max exceeds it by more than
//    2^8 (or on the first visible key): the pages subtract the max only to
//    keep the exponentials finite, and any reference at or above
//    (row max - 8) keeps every weight <= 256.  The rescale of l and the
//    accumulator then almost never runs; the result is the same function;
//  * the output is accumulated transposed, O^T += V^T P^T, with the same MFMA:
//    the weights convert to bf16 straight into the B operand (no LDS round
//    trip) and V^T comes from V's natural [key][d] layout in LDS through two
//    ds_read_b64_tr_b16 transposing reads per MFMA.  The row sum adds the
//    float32 weights before rounding (a sum of bf16-rounded weights would
//    carry their 2^-9 relative error into LSE for rows with few keys);
//  * K and V move HBM -> LDS directly (global_load_lds_dwordx4: each lane's
//    16 bytes land at M0 + 16 * lane, so one wave instruction fills a 1 KB
//    block and the per-lane global address picks what goes where), with no
//    staging registers.  Two K and two V buffers, each its own LDS array so
//    the compiler can see that reading one never waits on a load into another;
//  * pipeline: K(t+2) and V(t+1) are loaded while tiles t and t+1 are in use;
//    a load has two phases (one tile) to land before the barrier that
//    waits for it;
//  * LDS layouts are padded so that every operand read is one per-lane base
//    register plus a compile-time offset (no per-step address arithmetic, no
//    address registers held across the loop) and conflict-free on the 64
//    banks: K and Q rows carry 16 bytes of padding, so the 16 rows that a
//    16-lane group reads with ds_read_b128 start 4 banks apart; V rows carry
//    64 bytes, so the 4 rows x 64 bytes that 32 lanes read with
//    ds_read_b64_tr_b16 start 16 banks apart.  Loads into LDS are 1 KB
//    blocks of 64 lanes x 16 bytes; the slots that fall on padding receive
//    a copy of valid data that is never read;
//  * Q stays in LDS (each wave's 32 rows) and is read as the B operand in the
//    MFMA phase, which leaves the registers for operand prefetch: each MFMA's
//    operands are fetched a few MFMAs ahead;
//  * causal: tiles past the workgroup's last visible key are never visited,
//    waves skip tiles they cannot see, and only tiles that cross the diagonal
//    or the kv_len boundary are masked element by element;
//  * workgroup order: gfx950 deals workgroups round-robin to its 8 XCDs, each
//    with its own L2.  Consecutive logical work items (the query tiles of one
//    (batch, head), heaviest first when causal) are mapped to one XCD so that
//    the workgroups sharing a head's K/V run together on one L2.
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kNumXcd = 8;
constexpr float kLazyRescale = 8.0f;  // log2 of the largest weight allowed

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// Logical work item of workgroup `wg` when workgroups are dealt round-robin
// to kNumXcd XCDs: XCD x gets a contiguous range of logical items.
__device__ __forceinline__ int64_t xcd_logical(int64_t wg, int64_t G) {
  const int64_t x = wg % kNumXcd, j = wg / kNumXcd;
  const int64_t q = G / kNumXcd, r = G % kNumXcd;
  return x * q + (x < r ? x : r) + j;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16_kernel(Problem p, int n_qtiles) {
  constexpr int BQ = kPrefillBlockQ, BK = kPrefillBlockK;
  constexpr int NW = kPrefillThreads / 64;   // waves per workgroup
  constexpr int CPR = D / 8;                 // 16-byte chunks of data per row
  constexpr int KROW = D + 8;                // K/Q row stride in LDS (elements)
  constexpr int VROW = D + 32;               // V row stride in LDS (elements)
  constexpr int KCH = KROW / 8, VCH = VROW / 8;        // 16-byte slots per row
  constexpr int KBLK = (BK * KCH + 63) / 64;           // 1 KB blocks per K tile
  constexpr int VBLK = (BK * VCH + 63) / 64;           // 1 KB blocks per V tile
  constexpr int QBLK = (32 * KCH + 63) / 64;           // 1 KB blocks per wave's Q rows
  static_assert(NW == 8 && BQ == 32 * NW, "8 waves of 32 queries");
  __shared__ __attribute__((aligned(1024))) __bf16 Kb0[KBLK * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Kb1[KBLK * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb0[VBLK * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb1[VBLK * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Qs_all[NW * QBLK * 512];

  const int64_t logical = xcd_logical(blockIdx.x, gridDim.x);
  int qt = (int)(logical % n_qtiles);
  const int64_t bh = logical / n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest query tiles first
  const int b = (int)(bh / p.H);
  const int N = p.N, M = p.M;
  const int tid = threadIdx.x;
  const int w = tid / 64, lane = tid % 64, hl = lane / 32, ql = lane % 32;
  const bool group_a = w < NW / 2;  // waves 0-3 lead, waves 4-7 follow one phase behind
  const int kvl = clamp_kv(p.kv_len, b, M);
  const int q0 = qt * BQ;
  const int qw0 = q0 + 32 * w;  // first query of this wave
  const int qrow = qw0 + ql;    // this lane's query
  const int off = kvl - N;      // key j visible to query i iff j < kvl and (!causal or j <= i + off)
  const int q_last = min(q0 + BQ, N) - 1;
  const int kv_end = CAUSAL ? min(kvl, q_last + off + 1) : kvl;
  const int n_tiles = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;

  const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * N * D;
  const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D;
  const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D;

  // Slot s of a padded tile holds row s / CH, chunk s % CH; slots on the
  // padding (chunk >= CPR) load chunk 0 of that row (valid data, never read).
  auto load_padded = [&](const __bf16* src, int row0, int row_max, __bf16* dst, int nblk, int ch,
                         int first_blk, int blk_step) {
    for (int blk = first_blk; blk < nblk; blk += blk_step) {
      const int slot = blk * 64 + lane;
      const int r = slot / ch, c = slot % ch;
      const int row = min(row0 + r, row_max);
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)row * D + (c < CPR ? c * 8 : 0)),
                                       (lds_ptr)(dst + blk * 512), 16, 0, 0);
    }
  };
  // K and V tiles: this wave loads blocks w, w + NW, ... of each.  The
  // per-lane byte offsets of those blocks' slots within a tile (< 64 KB) are
  // fixed, so they are computed once and kept two to a register; a tile load
  // is then a shift or mask and an add per block, with the tile base in
  // scalar registers.  Rows past kv_len (last tile only) repeat the last
  // valid row (finite data whose weights are exactly 0).
  constexpr int KPW = (KBLK + NW - 1) / NW, VPW = (VBLK + NW - 1) / NW;
  constexpr int ROWB = D * 2, LOG_ROWB = D == 128 ? 8 : 7;  // bytes per global row
  static_assert(ROWB == 1 << LOG_ROWB && BK * ROWB <= 65536, "row bytes");
  const int ws = __builtin_amdgcn_readfirstlane(w);
  auto slot_off = [&](int blk, int ch) -> uint32_t {
    const int slot = blk * 64 + lane, r = slot / ch, cc = slot % ch;
    return (uint32_t)(r * ROWB + (cc < CPR ? cc * 16 : 0));
  };
  uint32_t koff[(KPW + 1) / 2], voff[(VPW + 1) / 2];
#pragma unroll
  for (int i = 0; i < KPW; i += 2)
    koff[i / 2] = slot_off(ws + i * NW, KCH) | (i + 1 < KPW ? slot_off(ws + (i + 1) * NW, KCH) << 16 : 0u);
#pragma unroll
  for (int i = 0; i < VPW; i += 2)
    voff[i / 2] = slot_off(ws + i * NW, VCH) | (i + 1 < VPW ? slot_off(ws + (i + 1) * NW, VCH) << 16 : 0u);
  auto load_tile = [&](const __bf16* src, int t, __bf16* dst, const uint32_t* offs, int nblk,
                       auto npw_c) {
    constexpr int npw = decltype(npw_c)::value;
    const char* base = (const char*)(src + (size_t)t * BK * D);
    const int rmax = kvl - 1 - t * BK;  // last valid row of this tile (>= 0)
    // Opaque copies: the unpacked offsets must not be hoisted out of the
    // main loop, where they would hold twice the registers.
    uint32_t pk[(npw + 1) / 2];
#pragma unroll
    for (int i = 0; i < (npw + 1) / 2; ++i) {
      pk[i] = offs[i];
      asm volatile("" : "+v"(pk[i]));
    }
    offs = pk;
    if (rmax >= BK - 1) {
#pragma unroll
      for (int i = 0; i < npw; ++i)
        if (ws + i * NW < nblk) {
          const uint32_t o = i % 2 ? offs[i / 2] >> 16 : offs[i / 2] & 0xFFFFu;
          __builtin_amdgcn_global_load_lds((const void*)(base + o),
                                           (lds_ptr)(dst + (ws + i * NW) * 512), 16, 0, 0);
        }
    } else {
#pragma unroll
      for (int i = 0; i < npw; ++i)
        if (ws + i * NW < nblk) {
          const uint32_t u = i % 2 ? offs[i / 2] >> 16 : offs[i / 2] & 0xFFFFu;
          const uint32_t o = (uint32_t)min((int)(u >> LOG_ROWB), rmax) << LOG_ROWB | (u & (ROWB - 1));
          __builtin_amdgcn_global_load_lds((const void*)(base + o),
                                           (lds_ptr)(dst + (ws + i * NW) * 512), 16, 0, 0);
        }
    }
  };
  auto load_k = [&](int t, __bf16* dst) { load_tile(Kg, t, dst, koff, KBLK, std::integral_constant<int, KPW>{}); };
  auto load_v = [&](int t, __bf16* dst) { load_tile(Vg, t, dst, voff, VBLK, std::integral_constant<int, VPW>{}); };

  // This wave's 32 query rows (rows past N: any finite data, never written out).
  __bf16* Qs = Qs_all + w * QBLK * 512;
  load_padded(Qg, qw0, N - 1, Qs, QBLK, KCH, 0, 1);

  // Per-lane base offsets (elements) of the three operand reads.
  const int kbase = ql * KROW + hl * 8;   // + (32 nb) KROW + 16 kb
  const int vbase = (4 * hl + (lane % 16) / 4) * VROW + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
                                          // + (32 nb + 16 t2) VROW + 32 db, + 8 VROW for the upper 4 keys

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  f32x16 sacc0[BK / 32], sacc1[BK / 32];
  bf16x8 pf[BK / 16];       // weights of the tile whose PV is next
  float m_run = -INFINITY;  // reference max of t = s * scale * log2(e)
  float l_run = 0.f;        // this lane's part of the running sum
  // A scale of 0 would turn a masked -inf score into NaN (-inf * 0); a floor
  // of 1e-30 changes the weights of finite scores by less than 1e-20.
  const float c = fmaxf(p.scale * kLog2e, 1e-30f);

  // a wave none of whose queries sees a key of tile t skips its math
  auto active = [&](int t) { return t < n_tiles && (!CAUSAL || t * BK <= qw0 + 31 + off); };

  // ---- operand fetches ----
  auto fetch_k = [&](const __bf16* Ks, int kb, int nb) -> bf16x8 {
    return *(const bf16x8*)(Ks + kbase + nb * 32 * KROW + kb * 16);
  };
  auto fetch_q = [&](int kb) -> bf16x8 { return *(const bf16x8*)(Qs + kbase + kb * 16); };
  // V^T operand of PV MFMA i = (nb, t2, db).  B operand slot 8*hl + e of
  // 16-key block (nb, t2) is key 32 nb + 16 t2 + 8 (e / 4) + 4 hl + e % 4;
  // the A operand for the same slots comes from two transposing reads of 4
  // consecutive keys each: within a 16-lane group, lane j reads row
  // kbase + j / 4 at column dsrc + 4 (j % 4), and lane i receives the 4 keys
  // at column dsrc + i.
  auto fetch_v = [&](const __bf16* Vs, int i) -> bf16x8 {
    const int nb = i / (2 * (D / 32)), t2 = (i / (D / 32)) % 2, db = i % (D / 32);
    const __bf16* a = Vs + vbase + (nb * 32 + t2 * 16) * VROW + db * 32;
    const s16x4 lo = lds_read_tr16(a);
    const s16x4 hi = lds_read_tr16(a + 8 * VROW);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- S^T = K Q^T for 64 keys x 32 queries (prologue only) ----
  auto compute_s = [&](const __bf16* Ks, f32x16* sacc) {
#pragma unroll
    for (int nb = 0; nb < BK / 32; ++nb) sacc[nb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      const bf16x8 qv = fetch_q(kb);
#pragma unroll
      for (int nb = 0; nb < BK / 32; ++nb)
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fetch_k(Ks, kb, nb), qv, sacc[nb], 0, 0, 0);
    }
  };

  // ---- softmax of tile t: mask, running max, weights 2^(t - m) as the
  //      bf16 B operand of the PV product, row sums ----
  auto softmax = [&](int t, f32x16* sacc) {
    const int k0 = t * BK;
    const bool need_mask = (k0 + BK > kvl) || (CAUSAL && k0 + BK - 1 > qw0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? min(kvl - 1, qrow + off) : kvl - 1;  // last visible key
#pragma unroll
      for (int nb = 0; nb < BK / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + nb * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
          if (key > lim) sacc[nb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < BK / 32; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxc = mx * c;  // -inf stays -inf (c > 0)
    if (__any(mxc > m_run + kLazyRescale)) {
      const float m_new = fmaxf(m_run, mxc);
      // e^(m_old - m_new); nothing accumulated yet when m_old = -inf
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;  // no visible key yet: all weights 0
    float psum = 0.f;
#pragma unroll
    for (int nb = 0; nb < BK / 32; ++nb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = (2 * t2 + e / 4) * 4 + (e % 4);
          const float pv = fast_exp2(fmaf(sacc[nb][r], c, -m_use));
          psum += pv;
          pf[nb * 2 + t2][e] = (__bf16)pv;
        }
    l_run += psum;
  };

  // MFMA phase of tile t: S(t+1) from Knext into snext (when with_s), then
  // O += P(t) V(t), as one sequence of MFMAs whose LDS operands are fetched
  // ahead (KPD steps of S, VPD MFMAs of PV).  Scheduling barriers pin this
  // order: left alone, the compiler fetches each operand just before its
  // MFMA and every MFMA then waits out a full LDS round trip.
  constexpr int NPV = (BK / 16) * (D / 32);  // MFMAs of O += P V
  constexpr int KPD = 2, VPD = 4;
  auto mfma_phase = [&](bool with_s, const __bf16* Ks, const __bf16* Vs, f32x16* snext) {
    bf16x8 vfr[VPD];
    if (with_s) {
      bf16x8 kfr[KPD][BK / 32], qfr[KPD];
#pragma unroll
      for (int kb = 0; kb < KPD; ++kb) {
        qfr[kb] = fetch_q(kb);
#pragma unroll
        for (int nb = 0; nb < BK / 32; ++nb) kfr[kb][nb] = fetch_k(Ks, kb, nb);
      }
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        __builtin_amdgcn_sched_barrier(0);
        const int slot = kb % KPD;
        const bf16x8 qcur = qfr[slot];
        bf16x8 kcur[BK / 32];
#pragma unroll
        for (int nb = 0; nb < BK / 32; ++nb) kcur[nb] = kfr[slot][nb];
        const int nx = kb + KPD;  // next fetch: S operands, then the first PV operands
        if (nx < D / 16) {
          qfr[slot] = fetch_q(nx);
#pragma unroll
          for (int nb = 0; nb < BK / 32; ++nb) kfr[slot][nb] = fetch_k(Ks, nx, nb);
        } else if (nx - D / 16 < VPD) {
          vfr[nx - D / 16] = fetch_v(Vs, nx - D / 16);
        }
#pragma unroll
        for (int nb = 0; nb < BK / 32; ++nb)
          snext[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[nb], qcur, kb == 0 ? f32x16{} : snext[nb], 0, 0, 0);
      }
#pragma unroll
      for (int i = KPD; i < VPD; ++i) vfr[i] = fetch_v(Vs, i);
    } else {
#pragma unroll
      for (int i = 0; i < VPD; ++i) vfr[i] = fetch_v(Vs, i);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 vcur = vfr[i % VPD];
      if (i + VPD < NPV) vfr[i % VPD] = fetch_v(Vs, i + VPD);
      const int nb = i / (2 * (D / 32)), t2 = (i / (D / 32)) % 2, db = i % (D / 32);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pf[nb * 2 + t2], oacc[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_mfma = [&](int t, const __bf16* Knext, const __bf16* Vcur, f32x16* snext) {
    if (active(t + 1)) {
      mfma_phase(true, Knext, Vcur, snext);  // active(t+1) implies active(t)
    } else {
      // snext is not read again; defining it on this path too ends the live
      // range of the value it held (otherwise both accumulators stay live)
#pragma unroll
      for (int nb = 0; nb < BK / 32; ++nb) snext[nb] = f32x16{};
      if (active(t)) mfma_phase(false, Knext, Vcur, snext);
    }
  };
  // VALU phase of tile t: softmax of tile t+1 (its weights feed the next PV).
  auto phase_valu = [&](int t, f32x16* snext) {
    if (active(t + 1)) softmax(t + 1, snext);
  };
  // Barrier that only aligns the phases of the two wave groups: nothing is
  // written to LDS that a read on its far side depends on, so it carries no
  // memory fence (a fence would also wait for the in-flight tile loads).
  auto align = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: Q, tiles 0 (K, V) and 1 (K) in LDS; S(0) and its softmax in
  // every wave (the following group then idles through its first VALU phase).
  if (n_tiles > 0) {
    load_k(0, Kb0);
    load_v(0, Vb0);
    if (n_tiles > 1) load_k(1, Kb1);
  }
  __syncthreads();
  if (active(0)) {
    compute_s(Kb0, sacc0);
    softmax(0, sacc0);
  }
  __syncthreads();  // every wave is done with K(0) before slot 0 loads K(2) over it

  // Phase slots: the leading group runs M(t) in slot 2t and V(t) in slot
  // 2t + 1; the following group runs V(t - 1) in slot 2t and M(t) in slot
  // 2t + 1.  Slot 2t also issues the loads of K(t+2) and V(t+1); the full
  // barrier after slot 2t + 1 waits for them.  Each group has its own loop
  // (same barriers, same count), so each keeps only one score accumulator
  // live at a time; both loops are unrolled by two tiles so that every LDS
  // buffer and accumulator is fixed at compile time.
  auto loads = [&](int t, __bf16* Kdst, __bf16* Vdst) {
    if (t + 2 < n_tiles) load_k(t + 2, Kdst);
    if (t + 1 < n_tiles) load_v(t + 1, Vdst);
  };
  if (group_a) {
    for (int t = 0; t < n_tiles; t += 2) {
      loads(t, Kb0, Vb1);
      phase_mfma(t, Kb1, Vb0, sacc1);
      align();
      phase_valu(t, sacc1);
      __syncthreads();
      if (t + 1 >= n_tiles) break;
      loads(t + 1, Kb1, Vb0);
      phase_mfma(t + 1, Kb0, Vb1, sacc0);
      align();
      phase_valu(t + 1, sacc0);
      __syncthreads();
    }
  } else {
    for (int t = 0; t < n_tiles; t += 2) {
      loads(t, Kb0, Vb1);
      if (t > 0) phase_valu(t - 1, sacc0);
      align();
      phase_mfma(t, Kb1, Vb0, sacc1);
      __syncthreads();
      if (t + 1 >= n_tiles) break;
      loads(t + 1, Kb1, Vb0);
      phase_valu(t, sacc1);
      align();
      phase_mfma(t + 1, Kb0, Vb1, sacc0);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* Orow = (__bf16*)p.o + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][4 * j + i] * inv);
        *(bf16x4*)(Orow + db * 32 + 8 * j + 4 * hl) = ov;
      }
    if (hl == 0)
      p.lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const Problem& p, const Plan& plan, hipStream_t stream) {
  if (plan.grid == 0) return hipSuccess;
  const int n_qtiles = (p.N + kPrefillBlockQ - 1) / kPrefillBlockQ;
  const dim3 grid((unsigned)plan.grid), block(kPrefillThreads);
  if (p.D == 64) {
    if (p.causal) hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), grid, block, 0, stream, p, n_qtiles);
    else hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), grid, block, 0, stream, p, n_qtiles);
  } else {
    if (p.causal) hipLaunchKernelGGL((prefill_bf16_kernel<128, true>), grid, block, 0, stream, p, n_qtiles);
    else hipLaunchKernelGGL((prefill_bf16_kernel<128, false>), grid, block, 0, stream, p, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace fa
