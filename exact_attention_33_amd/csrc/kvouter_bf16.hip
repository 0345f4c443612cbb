// Key/value-outer forward ("FA1 loop order"), bf16 inputs, float32
// accumulation, for gfx950.  An ablation path: it computes the same O and
// LSE as the prefill kernel with the opposite loop nest.
//
// Method ("Flash Attention: The Hidden Gem", FA1, FA2, FA3: the first
// version looped over key blocks outside and query blocks inside;
// "Understanding FlashAttention", From loops to tiling: with key/value tiles
// in the outer loop, the query and output tiles are read and written again
// for every key/value tile): a workgroup stages one 64-key K/V tile in LDS
// and then sweeps its query tiles.  For each query tile it reads the queries,
// their running max m, running sum l and unnormalised output accumulator
// from HBM, applies the tile (online softmax with the correction
// e^(m_old - m_new), "Flash Attention: The Hidden Gem", The Correction
// Factor), and writes m, l and the accumulator back.  After the last key
// tile it divides by l and writes O and LSE.  The accumulator is float32 in
// a caller-provided workspace: B H N (D + 2) floats.
//
// A workgroup owns `tiles_per_group` consecutive 256-query tiles of one
// (batch, head): 1 gives the grid of the prefill kernel (the loop order is
// the only difference); the whole sequence gives the first version's
// parallelism over batch and heads only.
//
// gfx950 mapping: 4 waves, 64 queries each per query tile; S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the same operand layouts
// as the backward's dQ pass (K rows and transposing V reads from the
// XOR-swizzled LDS stage); the output accumulator of a wave is read,
// rescaled and written 32 columns at a time.
#include <cmath>

#include "device_common.h"
#include "fa_internal.h"
#include "mfma_asm.h"

namespace fa {
namespace {

using namespace asmk;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void kvouter_kernel(Problem p, int n_qtiles, int tiles_per_group, float* ws) {
  using St = Stage<D>;
  constexpr int ROWB = St::ROWB;
  constexpr int BQ = 256, QW = 64, NQB = 2, DK = D / 16, DB = D / 32, BK = St::ROWS;

  __shared__ __attribute__((aligned(1024))) char Ks[St::BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs[St::BYTES];

  const int n_groups = (n_qtiles + tiles_per_group - 1) / tiles_per_group;
  const int64_t logical = xcd_logical(blockIdx.x, gridDim.x);
  const int grp = (int)(logical % n_groups);
  const int64_t bh = logical / n_groups;
  const int b = (int)(bh / p.H);
  const int N = p.N, M = p.M;
  const int tid = threadIdx.x;
  const int lane = tid % 64, h = lane / 32, l32 = lane % 32;
  const int ws_ = __builtin_amdgcn_readfirstlane(tid / 64);
  const int kvl = __builtin_amdgcn_readfirstlane(clamp_kv(p.kv_len, b, M));
  const int off = kvl - N;
  const int qt_lo = grp * tiles_per_group, qt_hi = min(qt_lo + tiles_per_group, n_qtiles);
  const int q_last = min(qt_hi * BQ, N) - 1;
  const int kv_end = CAUSAL ? min(kvl, q_last + off + 1) : kvl;
  const int n_kt = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;

  const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * N * D;
  const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D;
  const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D;
  const int64_t BH = (int64_t)p.B * p.H;
  float* Ow = ws + (size_t)bh * N * D;                 // accumulator [N][D]
  float* Mw = ws + (size_t)BH * N * D + (size_t)bh * N;  // running max (base 2)
  float* Lw = Mw + (size_t)BH * N;                       // running sum

  uint32_t soff[St::BPW];
#pragma unroll
  for (int i = 0; i < St::BPW; ++i) soff[i] = St::slot_src((ws_ + i * NW) * 64 + lane);
  const int nrec = kvl * 2 * D;  // the planner keeps M * D * 2 below 2^31

  const int G = (l32 >> 2) & 3;
  const int rbase0 = l32 * ROWB + 16 * ((0 + h) ^ G);
  const int rbase1 = l32 * ROWB + 16 * ((2 + h) ^ G);
  const int j16 = lane % 16, g2 = (lane / 16) % 2;
  const int tbase0 = (4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (0 + h)) + 8 * (j16 % 2);
  const int tbase1 = (8 + 4 * h + j16 / 4) * ROWB + 16 * ((2 * g2 + (j16 % 4) / 2) ^ (2 + h)) + 8 * (j16 % 2);
  const float c = fmaxf(p.scale * kLog2e, 1e-30f);

  // One key tile j (in LDS) applied to the 64 queries of this wave from qw0.
  auto step = [&](int j, int qw0, bool first) __attribute__((always_inline)) {
    bf16x8 qf[NQB][DK];
    float m_old[NQB], l_old[NQB];
    int lim[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = qw0 + 32 * qb + l32;
      const bool ok = row < N;
#pragma unroll
      for (int kb = 0; kb < DK; ++kb)
        qf[qb][kb] = ok ? *(const bf16x8*)(Qg + (size_t)row * D + kb * 16 + h * 8) : bf16x8{};
      m_old[qb] = (first || !ok) ? -INFINITY : Mw[row];
      l_old[qb] = (first || !ok) ? 0.f : Lw[row];
      lim[qb] = CAUSAL ? min(row + off, kvl - 1) : kvl - 1;
    }
    // S^T = K Q^T: lane = query qw0 + 32 qb + l32, register r of key block
    // kb2 = key 64 j + 32 kb2 + 8 (r / 4) + 4 h + r % 4
    f32x16 s[2][NQB];
#pragma unroll
    for (int kb = 0; kb < DK; ++kb) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 ka = *lds_at<bf16x8>(Ks, 32 * kb2 * ROWB + 64 * (kb / 2) + ((kb & 1) ? rbase1 : rbase0));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          if (kb == 0) mfma_vv0(s[kb2][qb], ka, qf[qb][kb]);
          else mfma_vv(s[kb2][qb], ka, qf[qb][kb]);
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mfma_guard_v(s[0][qb], s[1][qb]);
    // online softmax of the tile
    bf16x8 pf[NQB][2][2];
    float alpha[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BK + 32 * kb2 + 8 * (r / 4) + 4 * h + r % 4;
          if (key > lim[qb]) s[kb2][qb][r] = -INFINITY;
          mx = fmaxf(mx, s[kb2][qb][r]);
        }
      mx = swap_halves_max(mx);
      const float m_new = fmaxf(m_old[qb], mx * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[qb] = m_old[qb] == -INFINITY ? 0.f : fast_exp2(m_old[qb] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(fmaf(s[kb2][qb][r], c, -m_use));
          ps += pv;
          pf[qb][kb2][r / 8][r % 8] = (__bf16)pv;
        }
      ps = swap_halves_sum(ps);
      const float l_new = alpha[qb] * l_old[qb] + ps;
      const int row = qw0 + 32 * qb + l32;
      if (h == 0 && row < N) {
        Mw[row] = m_new;
        Lw[row] = l_new;
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      valu_guard(pf[qb][0][0], pf[qb][0][1]);
      valu_guard(pf[qb][1][0], pf[qb][1][1]);
    }
    // O^T += V^T P^T, 32 columns of the accumulator at a time: read from
    // HBM, rescale by alpha, accumulate, write back.  Register r of
    // accumulator (qb, db): column 32 db + 8 (r / 4) + 4 h + r % 4.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16 o[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw0 + 32 * qb + l32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
          if (!first && row < N) x = *(const float4*)(Ow + (size_t)row * D + 32 * db + 8 * g + 4 * h);
          o[qb][4 * g + 0] = x.x * alpha[qb];
          o[qb][4 * g + 1] = x.y * alpha[qb];
          o[qb][4 * g + 2] = x.z * alpha[qb];
          o[qb][4 * g + 3] = x.w * alpha[qb];
        }
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const int o_ = (32 * kb2 + 16 * sp) * ROWB + 64 * db;
          const s16x4 lo = lds_read_tr16((const __bf16*)(Vs + o_ + tbase0));
          const s16x4 hi = lds_read_tr16((const __bf16*)(Vs + o_ + tbase1));
          const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) mfma_vv(o[qb], vt, pf[qb][kb2][sp]);
        }
      mfma_guard_v(o[0], o[1]);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw0 + 32 * qb + l32;
        if (row < N) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(Ow + (size_t)row * D + 32 * db + 8 * g + 4 * h) =
                make_float4(o[qb][4 * g], o[qb][4 * g + 1], o[qb][4 * g + 2], o[qb][4 * g + 3]);
        }
      }
    }
  };

  for (int j = 0; j < n_kt; ++j) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < St::BPW; ++i) {
      int wofs = (ws_ + i * NW) * 1024;
      asm volatile("" : "+s"(wofs));
      const uint32_t u = soff[i] + (uint32_t)j * BK * 2 * D;
      buffer_load_lds16(Kg, nrec, u, (lds_ptr)(Ks + wofs));
      buffer_load_lds16(Vg, nrec, u, (lds_ptr)(Vs + wofs));
    }
    wait_vm0();
    __syncthreads();
    for (int qt = qt_lo; qt < qt_hi; ++qt) {
      const int qw0 = qt * BQ + ws_ * QW;
      if (qw0 >= N) continue;
      // causal: a later key tile that none of the wave's queries sees
      if (CAUSAL && j > 0 && j * BK > qw0 + QW - 1 + off) continue;
      step(j, qw0, j == 0);
    }
  }

  // ---- O = accumulator / l, LSE = ln 2 (m + log2 l) ----
  for (int qt = qt_lo; qt < qt_hi; ++qt) {
    const int qw0 = qt * BQ + ws_ * QW;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = qw0 + 32 * qb + l32;
      if (row >= N) continue;
      const float l = n_kt > 0 ? Lw[row] : 0.f;
      const float m = n_kt > 0 ? Mw[row] : -INFINITY;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      __bf16* Orow = (__bf16*)p.o + (size_t)bh * N * D + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n_kt > 0) x = *(const float4*)(Ow + (size_t)row * D + 32 * db + 8 * g + 4 * h);
          bf16x4 ov = {(__bf16)(x.x * inv), (__bf16)(x.y * inv), (__bf16)(x.z * inv), (__bf16)(x.w * inv)};
          *(bf16x4*)(Orow + 32 * db + 8 * g + 4 * h) = ov;
        }
      if (h == 0) p.lse[(size_t)bh * N + row] = l > 0.f ? kLn2 * (m + fast_log2(l)) : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_kvouter_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream) {
  if (plan.grid == 0) return hipSuccess;
  const int n_qtiles = (p.N + 255) / 256;
  const dim3 grid((unsigned)plan.grid), block(256);
  float* ws = (float*)workspace;
  const int tpg = plan.block_q / 256;
  if (p.D == 64) {
    if (p.causal) hipLaunchKernelGGL((kvouter_kernel<64, true>), grid, block, 0, stream, p, n_qtiles, tpg, ws);
    else hipLaunchKernelGGL((kvouter_kernel<64, false>), grid, block, 0, stream, p, n_qtiles, tpg, ws);
  } else {
    if (p.causal) hipLaunchKernelGGL((kvouter_kernel<128, true>), grid, block, 0, stream, p, n_qtiles, tpg, ws);
    else hipLaunchKernelGGL((kvouter_kernel<128, false>), grid, block, 0, stream, p, n_qtiles, tpg, ws);
  }
  return hipGetLastError();
}

}  // namespace fa
