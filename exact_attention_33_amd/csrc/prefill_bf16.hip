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
//  * workgroup = 4 waves = 128 queries; wave w owns queries [32w, 32w + 32);
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
//  * software pipeline inside each wave: iteration t issues the loads of
//    K(t+2) and V(t+1), computes the softmax of tile t while the MFMAs of
//    S(t+1) = K(t+1) Q^T run, then O += P(t) V(t); one barrier per tile;
//  * LDS bank conflicts: rows are unpadded and their 16-byte chunks are
//    XOR-swizzled by row: for K so that the 16 rows a 16-lane group reads
//    with ds_read_b128 hit 16 different bank groups, for V so that the
//    4 rows x 64 bytes that 32 lanes read with ds_read_b64_tr_b16 cover all
//    64 banks once.  Rows past kv_len in the last tile are filled from the
//    last valid row (finite data; their weights are exactly 0);
//  * causal: tiles past the workgroup's last visible key are never visited,
//    waves skip tiles they cannot see, and only tiles that cross the diagonal
//    or the kv_len boundary are masked element by element;
//  * workgroup order: gfx950 deals workgroups round-robin to its 8 XCDs, each
//    with its own L2.  Consecutive logical work items (the query tiles of one
//    (batch, head), heaviest first when causal) are mapped to one XCD so that
//    the workgroups sharing a head's K/V run together on one L2.
#include <cmath>

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
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_bf16_kernel(Problem p, int n_qtiles) {
  constexpr int BQ = kPrefillBlockQ, BK = kPrefillBlockK;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BK * D;               // elements of one K or V tile
  constexpr int NLD = TILE * 2 / 1024 / 4;   // 1 KB load instructions per wave per tile
  static_assert(NLD >= 1 && TILE * 2 == NLD * 4 * 1024, "tile must split into 1 KB blocks");
  __shared__ __attribute__((aligned(1024))) __bf16 Kb0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 Kb1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb1[TILE];
  // Chunk swizzles (see the header): K keeps 16 consecutive rows on distinct
  // bank groups, V keeps rows r..r+3 (r % 4 == 0) x 4 aligned chunks distinct.
  auto kswz = [](int row) { return CPR == 16 ? (row & 15) : ((row >> 1) & 7); };
  auto vswz = [](int row) { return CPR == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); };

  const int64_t logical = xcd_logical(blockIdx.x, gridDim.x);
  int qt = (int)(logical % n_qtiles);
  const int64_t bh = logical / n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest query tiles first
  const int b = (int)(bh / p.H);
  const int N = p.N, M = p.M;
  const int tid = threadIdx.x;
  const int w = tid / 64, lane = tid % 64, hl = lane / 32, ql = lane % 32;
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

  // Q as the B operand of S^T = K Q^T: lane (hl, ql) holds Q[qrow][16 kb + 8 hl .. + 8).
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    if (qrow < N)
      qf[kb] = *(const bf16x8*)(Qg + (size_t)qrow * D + kb * 16 + hl * 8);
    else
      qf[kb] = bf16x8{};
  }

  // Per-lane source rows/columns of this wave's 1 KB load blocks: LDS chunk
  // slot = (block * 64 + lane) holds row slot / CPR, swizzled chunk slot % CPR.
  int lrow[NLD], kcol[NLD], vcol[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int slot = (w * NLD + i) * 64 + lane;
    lrow[i] = slot / CPR;
    kcol[i] = ((slot % CPR) ^ kswz(lrow[i])) * 8;
    vcol[i] = ((slot % CPR) ^ vswz(lrow[i])) * 8;
  }
  auto load_tile = [&](const __bf16* src, int t, const int* col, __bf16* dst) {
    const int k0 = t * BK;
    __bf16* d = dst + w * NLD * 512;
    if (k0 + BK <= kvl) {
      const __bf16* base = src + (size_t)k0 * D;  // uniform
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(base + lrow[i] * D + col[i]),
                                         (lds_ptr)(d + i * 512), 16, 0, 0);
    } else {  // last tile: rows past kv_len repeat the last valid row
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = min(k0 + lrow[i], kvl - 1);
        __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)row * D + col[i]),
                                         (lds_ptr)(d + i * 512), 16, 0, 0);
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  f32x16 sacc0[BK / 32], sacc1[BK / 32];
  float m_run = -INFINITY;  // reference max of t = s * scale * log2(e)
  float l_run = 0.f;        // this lane's part of the running sum
  // A scale of 0 would turn a masked -inf score into NaN (-inf * 0); a floor
  // of 1e-30 changes the weights of finite scores by less than 1e-20.
  const float c = fmaxf(p.scale * kLog2e, 1e-30f);

  // a wave none of whose queries sees a key of tile t skips its math
  auto active = [&](int t) { return !CAUSAL || t * BK <= qw0 + 31 + off; };

  // ---- S^T = K Q^T for 64 keys x 32 queries ----
  auto compute_s = [&](const __bf16* Ks, f32x16* sacc) {
#pragma unroll
    for (int nb = 0; nb < BK / 32; ++nb) sacc[nb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
#pragma unroll
      for (int nb = 0; nb < BK / 32; ++nb) {
        const int row = nb * 32 + ql;
        const int ch = (2 * kb + hl) ^ kswz(row);
        const bf16x8 kf = *(const bf16x8*)(Ks + row * D + ch * 8);
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], sacc[nb], 0, 0, 0);
      }
    }
  };

  // ---- softmax, part A: mask, running max, move the reference if needed ----
  auto softmax_max = [&](int t, f32x16* sacc) {
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
  };

  // ---- softmax, part B: weights 2^(t - m) as the bf16 B operand, row sums ----
  auto softmax_exp = [&](const f32x16* sacc, bf16x8* pf) {
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

  // ---- O^T += V^T P^T ----
  // B operand slot 8*hl + e of 16-key block (nb, t2) is key
  // 32 nb + 16 t2 + 8 (e / 4) + 4 hl + e % 4.  The A operand (V^T) for the
  // same slots comes from two transposing reads of 4 consecutive keys each:
  // within a 16-lane group, lane j reads row kbase + j / 4 at column
  // dsrc + 4 (j % 4), and lane i receives the 4 keys at column dsrc + i.
  // Rows krow and krow + 8 share one swizzle pattern.
  auto pv = [&](const __bf16* Vs, const bf16x8* pf) {
#pragma unroll
    for (int nb = 0; nb < BK / 32; ++nb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int krow = nb * 32 + t2 * 16 + 4 * hl + (lane % 16) / 4;
        const int sw = vswz(krow);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int dsrc = db * 32 + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
          const int col = (((dsrc >> 3) ^ sw) << 3) + (dsrc & 7);
          const s16x4 lo = lds_read_tr16(Vs + krow * D + col);
          const s16x4 hi = lds_read_tr16(Vs + (krow + 8) * D + col);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb * 2 + t2], oacc[db], 0, 0, 0);
        }
      }
  };

  // One pipeline step for tile t with buffers fixed at compile time:
  // reads K(t+1) from Knext and V(t) from Vcur; loads K(t+2) into Kload and
  // V(t+1) into Vload; S(t) is in scur, S(t+1) goes to snext.  The MFMAs of
  // S(t+1) do not depend on the softmax of tile t, so the two overlap.
  auto step = [&](int t, const __bf16* Knext, const __bf16* Vcur, __bf16* Kload, __bf16* Vload,
                  f32x16* scur, f32x16* snext) {
    if (t + 2 < n_tiles) load_tile(Kg, t + 2, kcol, Kload);
    if (t + 1 < n_tiles) load_tile(Vg, t + 1, vcol, Vload);
    if (active(t)) {
      bf16x8 pf[BK / 16];
      softmax_max(t, scur);
      softmax_exp(scur, pf);
      if (t + 1 < n_tiles && active(t + 1)) compute_s(Knext, snext);
      pv(Vcur, pf);
    }
    __syncthreads();  // loads of this step have landed; buffers read here are free
  };

  if (n_tiles > 0) {
    load_tile(Kg, 0, kcol, Kb0);
    load_tile(Vg, 0, vcol, Vb0);
    if (n_tiles > 1) load_tile(Kg, 1, kcol, Kb1);
  }
  __syncthreads();
  if (n_tiles > 0 && active(0)) compute_s(Kb0, sacc0);
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, Kb1, Vb0, Kb0, Vb1, sacc0, sacc1);
    if (t + 1 < n_tiles) step(t + 1, Kb0, Vb1, Kb1, Vb0, sacc1, sacc0);
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
