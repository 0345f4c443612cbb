// Split-KV decode: one query per (batch, head) against a long KV cache
// ("Understanding FlashAttention", Attention: when decoding one token N = 1
// while M holds the history in the KV cache).  With one query there is no
// dense contraction to speak of -- every key and value is read once and used
// once -- so the work is a bandwidth-bound stream of the cache and runs on
// the vector ALUs, not on MFMA.
//
// Kernel 1 (partial): the keys of each sequence are cut into splits of
// `split_keys` keys.  A workgroup streams one split with the online softmax of
// "FlashAttention: attention was never compute-bound", The one formula (running
// max m, running sum l, unnormalised output rescaled by e^(m_old - m_new)),
// and writes the split's normalised output O_s and log-sum-exp L_s (base 2).
// Splits that start at or past kv_len[b] write nothing.
//
// Kernel 2 (merge): per (batch, head), L = M* + log2 sum_s 2^(L_s - M*) with
// M* = max_s L_s and O = sum_s 2^(L_s - L) O_s.  The pages do not print this
// step; it is the rescale identity e^(a - c) = e^(a - b) e^(b - c) ("On the
// maths anxiety") applied to two partial states as in "Flash Attention: The
// Hidden Gem", The Algorithm, step 5.  The merge order is fixed, so results
// are deterministic run to run.
//
// Memory access: D/8 lanes share one key (16 bytes each, one key row = 256 B
// at D = 128), so each wave-wide load moves 4 whole consecutive rows (1 KB);
// every lane keeps 8 keys' K and V rows in flight per step.  The cache is read
// once, so the loads are non-temporal (measured: +5% HBM throughput over
// ordinary loads on MI355X).
#include <cmath>

#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kUnroll = 8;  // keys per lane group in flight per step

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load that bypasses cache retention (streamed once).
__device__ __forceinline__ uint4 load_stream(const __bf16* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void unpack8(const uint4 u, float f[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
  }
}

template <int D>
__global__ __launch_bounds__(kSplitThreads) void splitkv_partial_kernel(
    Problem p, int splits, int split_keys, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int LPK = D / 8;                 // lanes per key
  constexpr int G = kSplitThreads / LPK;     // key groups per workgroup
  __shared__ float sm[G], sl[G];
  __shared__ float so[G * D];

  const int64_t wg = blockIdx.x;
  const int s = (int)(wg % splits);
  const int64_t bh = wg / splits;
  const int b = (int)(bh / p.H);
  const int M = p.M;
  const int kvl = clamp_kv(p.kv_len, b, M);
  const int k_begin = s * split_keys;
  if (k_begin >= kvl) return;  // empty split: the merge never reads it
  const int k_end = min(k_begin + split_keys, kvl);

  const int tid = threadIdx.x, g = tid / LPK, sub = tid % LPK;
  const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * D;  // N == 1
  const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D;
  const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D;

  // This lane's 8 query values, pre-multiplied by scale * log2(e) in float32:
  // dot products then come out directly as base-2 exponents.
  float qc[8];
  {
    float qf[8];
    unpack8(*(const uint4*)(Qg + sub * 8), qf);
    const float c = p.scale * kLog2e;
#pragma unroll
    for (int e = 0; e < 8; ++e) qc[e] = qf[e] * c;
  }

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int kb = k_begin + g; kb < k_end; kb += G * kUnroll) {
    uint4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = kb + u * G;
      if (key < k_end) {
        kr[u] = load_stream(Kg + (size_t)key * D + sub * 8);
        vr[u] = load_stream(Vg + (size_t)key * D + sub * 8);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float t[kUnroll];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qc[e], kf[e], part);
      part = group_sum<LPK>(part);
      t[u] = (kb + u * G < k_end) ? part : -INFINITY;
      mx = fmaxf(mx, t[u]);
    }
    // kb < k_end, so t[0] is finite and so is m_new.
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);  // 0 on the first step (m = -inf)
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pu = fast_exp2(t[u] - m_new);  // 0 for keys past the split
      float vf[8];
      unpack8(vr[u], vf);
      l += pu;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(pu, vf[e], o[e]);
    }
    m = m_new;
  }

  // Combine the G lane groups of this workgroup (each saw a strided subset).
  if (sub == 0) {
    sm[g] = m;
    sl[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) so[g * D + sub * 8 + e] = o[e];
  __syncthreads();
  if (tid < D) {
    float mstar = -INFINITY;
    for (int i = 0; i < G; ++i) mstar = fmaxf(mstar, sm[i]);
    float L = 0.f, acc = 0.f;
    for (int i = 0; i < G; ++i) {
      const float w = fast_exp2(sm[i] - mstar);  // groups that saw no key: 2^-inf = 0
      L += sl[i] * w;
      acc += so[i * D + tid] * w;
    }
    const size_t part = (size_t)bh * splits + s;
    ws_o[part * D + tid] = acc / L;
    if (tid == 0) ws_lse[part] = mstar + fast_log2(L);
  }
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void splitkv_merge_kernel(
    Problem p, int splits, int split_keys, const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse) {
  // Threads form (row group, 4-column slice): DQ = D/4 threads cover one
  // partial output row with float4 loads, RG = 256/DQ rows are read at once.
  constexpr int DQ = D / 4, RG = kMergeThreads / DQ;
  __shared__ float red[kMergeThreads];
  __shared__ float4 acc_s[RG][DQ];
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / p.H);
  const int kvl = clamp_kv(p.kv_len, b, p.M);
  const int ns = (kvl + split_keys - 1) / split_keys;  // splits that hold keys
  const int tid = threadIdx.x;
  __bf16* O = (__bf16*)p.o + (size_t)bh * D;
  if (ns == 0) {  // no visible key: O = 0, LSE = -inf
    for (int d = tid; d < D; d += kMergeThreads) O[d] = (__bf16)0.f;
    if (tid == 0) p.lse[bh] = -INFINITY;
    return;
  }
  const float* L = ws_lse + (size_t)bh * splits;
  // M* = max_s L_s
  float mx = -INFINITY;
  for (int i = tid; i < ns; i += kMergeThreads) mx = fmaxf(mx, L[i]);
  red[tid] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float mstar = red[0];
  __syncthreads();
  // sum_s 2^(L_s - M*)
  float tot = 0.f;
  for (int i = tid; i < ns; i += kMergeThreads) tot += fast_exp2(L[i] - mstar);
  red[tid] = tot;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float inv = 1.f / red[0];
  // O = sum_s 2^(L_s - M*) O_s / sum_s 2^(L_s - M*), rows of O_s read whole
  const int rg = tid / DQ, dq = tid % DQ;
  const float4* Os = (const float4*)(ws_o + (size_t)bh * splits * D);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int i = rg; i < ns; i += RG) {
    const float w = fast_exp2(L[i] - mstar);
    const float4 x = Os[(size_t)i * DQ + dq];
    acc.x = fmaf(w, x.x, acc.x);
    acc.y = fmaf(w, x.y, acc.y);
    acc.z = fmaf(w, x.z, acc.z);
    acc.w = fmaf(w, x.w, acc.w);
  }
  acc_s[rg][dq] = acc;
  __syncthreads();
  if (tid < DQ) {
    float4 t = acc_s[0][tid];
    for (int r = 1; r < RG; ++r) {
      const float4 u = acc_s[r][tid];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    bf16x4 ov = {(__bf16)(t.x * inv), (__bf16)(t.y * inv), (__bf16)(t.z * inv), (__bf16)(t.w * inv)};
    *(bf16x4*)(O + 4 * tid) = ov;
  }
  if (tid == 0) p.lse[bh] = (mstar + fast_log2(red[0])) * kLn2;
}

}  // namespace

hipError_t launch_splitkv_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh == 0) return hipSuccess;
  float* ws_o = (float*)workspace;
  float* ws_lse = workspace ? (float*)((char*)workspace + plan.ws_lse_offset) : nullptr;
  if (plan.grid > 0) {
    if (p.D == 64)
      hipLaunchKernelGGL(splitkv_partial_kernel<64>, dim3((unsigned)plan.grid), dim3(kSplitThreads),
                         0, stream, p, plan.splits, plan.block_k, ws_o, ws_lse);
    else
      hipLaunchKernelGGL(splitkv_partial_kernel<128>, dim3((unsigned)plan.grid), dim3(kSplitThreads),
                         0, stream, p, plan.splits, plan.block_k, ws_o, ws_lse);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.D == 64)
    hipLaunchKernelGGL(splitkv_merge_kernel<64>, dim3((unsigned)bh), dim3(kMergeThreads), 0, stream,
                       p, plan.splits, plan.block_k, ws_o, ws_lse);
  else
    hipLaunchKernelGGL(splitkv_merge_kernel<128>, dim3((unsigned)bh), dim3(kMergeThreads), 0, stream,
                       p, plan.splits, plan.block_k, ws_o, ws_lse);
  return hipGetLastError();
}

}  // namespace fa
