// Float32 path: float32 Q/K/V/O, float64 arithmetic inside.
//
// The tiled forward of "Flash Attention: The Hidden Gem", The Algorithm: a
// tile of 16 queries stays on chip with its running max m, running sum l and
// unnormalised output; K and V tiles of 32 keys stream through LDS; each tile
// updates m, rescales l and the output by e^(m_old - m_new) (The Correction
// Factor) and adds the tile's weights; the output is divided by l once at the
// end and L = m + log(l) is written beside it.
//
// An element mask (bit j % 32 of word j / 32 of the query's mask row) hides
// keys on top of kv_len, causal and the window; its bits are read per score.
//
// This path exists for exactness, not speed: scores, exponentials and sums are
// float64 so that O and LSE round to float32 only once (an fp32 score at
// |S| ~ 90 already carries an ulp of 7.6e-6).
#include <cmath>

#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(Problem p, int n_qtiles) {
  constexpr int BQ = kF32BlockQ, BK = kF32BlockK, E = D / 16;
  __shared__ float Ks[BK * D];
  __shared__ float Vs[BK * D];

  const int64_t wg = blockIdx.x;
  const int qt = (int)(wg % n_qtiles);
  const int64_t bh = wg / n_qtiles;
  const int b = (int)(bh / p.H);
  const int N = p.N, M = p.M;
  const int r = threadIdx.x / 16, sub = threadIdx.x % 16;
  const int i = qt * BQ + r;
  const int kvl = clamp_kv(p.kv_len, b, M);
  const int off = kvl - N;  // causal: key j visible to query i iff j <= i + off
  // Local window: query i sees keys i + off - wl .. i + off + wr only; causal
  // caps wr at 0.
  const bool upper = p.causal || p.window;
  const int wl = p.window ? min(p.wl, N + kvl) : 0;
  const int wr = p.causal ? 0 : (p.window ? min(p.wr, N + kvl) : 0);
  const int i_last = min(qt * BQ + BQ, N) - 1;
  const int kv_end = upper ? min(kvl, i_last + off + wr + 1) : kvl;
  const int kv_start = p.window ? max(0, qt * BQ + off - wl) / BK * BK : 0;

  // this query's row of the element mask (none: nullptr)
  const uint32_t* mrow = nullptr;
  if (p.mask && i < N) {
    const int64_t mb = p.mask_b > 1 ? b : 0, mh = p.mask_h > 1 ? bh % p.H : 0;
    mrow = p.mask + ((size_t)(mb * p.mask_h + mh) * N + i) * p.mask_w;
  }

  const float* Q = (const float*)p.q + (size_t)bh * N * D;
  const float* K = (const float*)p.k + (size_t)bh * M * D;
  const float* V = (const float*)p.v + (size_t)bh * M * D;

  double q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = i < N ? (double)Q[(size_t)i * D + sub + 16 * e] : 0.0;
    acc[e] = 0.0;
  }
  double m = -INFINITY, l = 0.0;
  const double sc = (double)p.scale;

  for (int j0 = kv_start; j0 < kv_end; j0 += BK) {
    __syncthreads();
    for (int c = threadIdx.x; c < BK * D / 4; c += kF32Threads) {
      const int key = c / (D / 4), dc = c % (D / 4);
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (j0 + key < kvl) {
        kk = *(const float4*)(K + (size_t)(j0 + key) * D + 4 * dc);
        vv = *(const float4*)(V + (size_t)(j0 + key) * D + 4 * dc);
      }
      *(float4*)(Ks + key * D + 4 * dc) = kk;
      *(float4*)(Vs + key * D + 4 * dc) = vv;
    }
    __syncthreads();

    double s[BK];
    double mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fma(q[e], (double)Ks[jj * D + sub + 16 * e], part);
      part += __shfl_xor(part, 8, 16);
      part += __shfl_xor(part, 4, 16);
      part += __shfl_xor(part, 2, 16);
      part += __shfl_xor(part, 1, 16);
      const int key = j0 + jj;
      const bool vis = key < kvl && (!upper || key <= i + off + wr) &&
                       (!p.window || key >= i + off - wl) &&
                       (!p.mask || (mrow && ((mrow[key >> 5] >> (key & 31)) & 1u)));
      s[jj] = vis ? part * sc : -INFINITY;
      mx = fmax(mx, s[jj]);
    }
    const double m_new = fmax(m, mx);
    // e^(m_old - m_new); a row with nothing seen so far has nothing to rescale.
    const double corr = (m == -INFINITY) ? 0.0 : exp(m - m_new);
    double psum = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= corr;
#pragma unroll
    for (int jj = 0; jj < BK; ++jj) {
      const double pj = (s[jj] == -INFINITY) ? 0.0 : exp(s[jj] - m_new);
      psum += pj;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fma(pj, (double)Vs[jj * D + sub + 16 * e], acc[e]);
    }
    l = l * corr + psum;
    m = m_new;
  }

  if (i < N) {
    float* O = (float*)p.o + (size_t)bh * N * D + (size_t)i * D;
    const double inv = l > 0.0 ? 1.0 / l : 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) O[sub + 16 * e] = (float)(acc[e] * inv);
    if (sub == 0) p.lse[(size_t)bh * N + i] = l > 0.0 ? (float)(m + log(l)) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const Plan& plan, hipStream_t stream) {
  if (plan.grid == 0) return hipSuccess;
  const int n_qtiles = (p.N + kF32BlockQ - 1) / kF32BlockQ;
  if (p.D == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)plan.grid), dim3(kF32Threads), 0,
                       stream, p, n_qtiles);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)plan.grid), dim3(kF32Threads), 0,
                       stream, p, n_qtiles);
  return hipGetLastError();
}

}  // namespace fa
