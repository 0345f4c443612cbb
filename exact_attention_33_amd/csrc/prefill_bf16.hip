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
//  * K and V move HBM -> registers -> LDS with 16-byte loads into a double
//    buffer: tile t+1 is written while tile t is read, tile t+2 is in flight
//    from HBM, and one barrier per tile separates them;
//  * LDS bank conflicts: K rows are padded by 16 bytes, so the 16 rows a
//    16-lane group reads with ds_read_b128 start 4 banks apart; V rows are
//    not padded but their 16-byte chunks are XOR-swizzled by row, so the 4
//    rows x 64 bytes that 32 lanes read with ds_read_b64_tr_b16 cover all 64
//    banks once;
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_bf16_kernel(Problem p, int n_qtiles) {
  constexpr int BQ = kPrefillBlockQ, BK = kPrefillBlockK;
  constexpr int LROW = D + kPrefillPad;           // K row length in LDS (bf16 elements)
  constexpr int KTILE = BK * LROW;                // one K tile in LDS
  constexpr int VTILE = BK * D;                   // one V tile in LDS (swizzled, unpadded)
  constexpr int BUF = KTILE + VTILE;
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int CH = BK * CPR / kPrefillThreads;  // chunks per thread per tile
  static_assert(BK * CPR % kPrefillThreads == 0, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];  // K0 V0 K1 V1
  // V chunk swizzle: rows r..r+3 (r % 4 == 0) x any 4 aligned chunks land on
  // 16 distinct 16-byte bank groups (D = 128: 16 chunks per row; D = 64: 8).
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

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // reference max of t = s * scale * log2(e)
  float l_run = 0.f;        // this lane's part of the running sum
  // A scale of 0 would turn a masked -inf score into NaN (-inf * 0); a floor
  // of 1e-30 changes the weights of finite scores by less than 1e-20.
  const float c = fmaxf(p.scale * kLog2e, 1e-30f);

  uint4 kreg[CH], vreg[CH];
  auto gload = [&](int t) {
    const int k0 = t * BK;
    if (k0 + BK <= kvl) {  // whole tile inside the sequence
#pragma unroll
      for (int r = 0; r < CH; ++r) {
        const int ch = r * kPrefillThreads + tid;
        const int key = ch / CPR, dc = ch % CPR;
        kreg[r] = *(const uint4*)(Kg + (size_t)(k0 + key) * D + dc * 8);
        vreg[r] = *(const uint4*)(Vg + (size_t)(k0 + key) * D + dc * 8);
      }
    } else {
#pragma unroll
      for (int r = 0; r < CH; ++r) {
        const int ch = r * kPrefillThreads + tid;
        const int key = ch / CPR, dc = ch % CPR;
        if (k0 + key < kvl) {
          kreg[r] = *(const uint4*)(Kg + (size_t)(k0 + key) * D + dc * 8);
          vreg[r] = *(const uint4*)(Vg + (size_t)(k0 + key) * D + dc * 8);
        } else {  // past the keys of this sequence: zeros, never read from HBM
          kreg[r] = make_uint4(0, 0, 0, 0);
          vreg[r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    __bf16* Ks = lds + buf * BUF;
    __bf16* Vs = Ks + KTILE;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int ch = r * kPrefillThreads + tid;
      const int key = ch / CPR, dc = ch % CPR;
      *(uint4*)(Ks + key * LROW + dc * 8) = kreg[r];
      *(uint4*)(Vs + key * D + ((dc ^ vswz(key)) * 8)) = vreg[r];
    }
  };

  if (n_tiles > 0) {
    gload(0);
    lstore(0);
    if (n_tiles > 1) gload(1);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BK;
    const __bf16* Ks = lds + (t & 1) * BUF;
    const __bf16* Vs = Ks + KTILE;
    // a wave none of whose queries sees a key of this tile skips the math
    const bool active = !CAUSAL || k0 <= qw0 + 31 + off;
    if (active) {
      // ---- S^T = K Q^T for 64 keys x 32 queries ----
      f32x16 sacc[BK / 32];
#pragma unroll
      for (int nb = 0; nb < BK / 32; ++nb) sacc[nb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
#pragma unroll
        for (int nb = 0; nb < BK / 32; ++nb) {
          const bf16x8 kf = *(const bf16x8*)(Ks + (nb * 32 + ql) * LROW + kb * 16 + hl * 8);
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], sacc[nb], 0, 0, 0);
        }
      }

      // ---- mask (only on tiles that cross the kv_len end or the diagonal) ----
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

      // ---- row max; move the reference only when needed ----
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

      // ---- weights 2^(t - m), bf16 B operand of the PV product, row sums ----
      bf16x8 pf[BK / 16];
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

      // ---- O^T += V^T P^T ----
      // B operand slot 8*hl + e of 16-key block (nb, t2) is key
      // 32 nb + 16 t2 + 8 (e / 4) + 4 hl + e % 4.  The A operand (V^T) for the
      // same slots comes from two transposing reads of 4 consecutive keys each:
      // within a 16-lane group, lane j reads row kbase + j / 4 at column
      // dsrc + 4 (j % 4), and lane i receives the 4 keys at column dsrc + i.
      // Rows krow and krow + 8 share one swizzle pattern.
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
    }

    // ---- stage the next tile; start loading the one after ----
    if (t + 1 < n_tiles) {
      lstore((t + 1) & 1);  // that buffer's last readers passed the previous barrier
      if (t + 2 < n_tiles) gload(t + 2);
    }
    __syncthreads();
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
