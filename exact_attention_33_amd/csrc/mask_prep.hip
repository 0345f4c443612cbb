// Element-mask pre-pass ("Understanding FlashAttention", Attention: a mask is
// an elementwise constant, so which tiles hold a kept key is known before any
// score is computed).  Two launches:
//   1. mask_blocks_kernel classifies every (256-query tile, 64-key tile) pair
//      for the prefill and the dQ pass and, for the backward, every (256-key
//      tile, 64-query stage) pair for the dK/dV pass, and copies the words of
//      the pairs the mask keeps in part into 2 KB blocks laid out the way a
//      wave loads them (one coalesced load per wave instead of one cache line
//      per row); pairs kept whole share one all-ones block per row of blocks;
//   2. mask_lists_kernel compacts the classes into the ascending tile lists
//      the kernels walk (bit 31 set on tiles the mask keeps in part only).
#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kPrepRows = kPrefillBlockQ;     // rows per workgroup: one 256-query tile
constexpr int kPrepWords = 32;                // words per row: 1024 keys
constexpr int kPrepPitch = kPrepWords + 1;    // LDS row pitch (words), conflict-free columns
constexpr int kPrepTiles = kPrepWords / 2;    // 64-key tiles per workgroup
constexpr int kPrepKTiles = kPrepWords / 8;   // 256-key tiles per workgroup
constexpr int kPrepStages = kPrepRows / kBwdStageQ;  // 64-query stages per workgroup
static_assert(kPrefillBlockK == 64 && kBwdBlockKV == 256 && kBwdStageQ == 64 && kBwdBlockQ == kPrepRows,
              "tile sizes the block layouts assume");

__device__ __forceinline__ uint32_t keys_below(int M, int word) {  // bits of keys < M in a word
  const int n = min(max(M - word * 32, 0), 32);
  return n == 32 ? ~0u : (1u << n) - 1u;
}

// One workgroup per (mask batch, mask head, query tile qt, group gi of 32
// words).  Rows past N copy row N - 1 into the blocks (the kernels read that
// row for their padding lanes) but are not classified; words past the row
// read as zeros (keys >= M, which the kernels mask by kv_len anyway).
__global__ __launch_bounds__(256) void mask_blocks_kernel(const uint32_t* __restrict__ mask, int N,
                                                          int M, int W, int n_qt,
                                                          uint8_t* __restrict__ cls,
                                                          uint32_t* __restrict__ blocks,
                                                          uint8_t* __restrict__ stage_cls,
                                                          uint32_t* __restrict__ stage_blocks) {
  __shared__ uint32_t rows[kPrepRows * kPrepPitch];
  __shared__ uint32_t red_o[4][kPrepStages][kPrepWords], red_a[4][kPrepStages][kPrepWords];
  __shared__ int c_tile[kPrepTiles], c_stage[kPrepKTiles * kPrepStages];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int qt = blockIdx.x % n_qt, gi = blockIdx.y;
  const int64_t mbh = blockIdx.x / n_qt;
  const int r0 = qt * kPrepRows;
  const int n_kt = mask_list_stride(M) - 1;
  const int n_kt256 = (M + kBwdBlockKV - 1) / kBwdBlockKV;
  const int n_st = mask_stage_stride(N) - 1;

  // ---- stage the 256 rows x 32 words; OR / AND per (stage, word) ----
  const int wd = tid % kPrepWords, gw = gi * kPrepWords + wd;
  const uint32_t* src = mask + (size_t)mbh * N * W + gw;
  uint32_t o[kPrepStages], a[kPrepStages];
#pragma unroll
  for (int v = 0; v < kPrepStages; ++v) { o[v] = 0u; a[v] = ~0u; }
#pragma unroll
  for (int v = 0; v < kPrepStages; ++v)
#pragma unroll
    for (int i = 0; i < kBwdStageQ / 8; ++i) {  // row 64 v + 8 i + tid / 32
      const int rr = v * kBwdStageQ + i * 8 + tid / kPrepWords;
      const int gr = min(r0 + rr, N - 1);
      const uint32_t x = gw < W ? src[(size_t)gr * W] : 0u;
      rows[rr * kPrepPitch + wd] = x;
      if (r0 + rr < N) {
        o[v] |= x;
        a[v] &= x;
      }
    }
#pragma unroll
  for (int v = 0; v < kPrepStages; ++v) {  // lanes l and l + 32 hold one word
    o[v] |= __shfl_xor(o[v], 32);
    a[v] &= __shfl_xor(a[v], 32);
    if (lane < 32) {
      red_o[wv][v][wd] = o[v];
      red_a[wv][v][wd] = a[v];
    }
  }
  __syncthreads();

  // ---- classes: 0 no key kept, 1 every key < M of every real row, 2 some ----
  auto classify = [](uint32_t any_bits, uint32_t all_bits) { return any_bits ? (all_bits == ~0u ? 1 : 2) : 0; };
  if (tid < kPrepTiles) {  // 64-key tile i of the query tile
    const int i = tid, kt = gi * kPrepTiles + i;
    uint32_t any_bits = 0u, all_bits = ~0u;
    for (int w = 0; w < 2; ++w) {
      const uint32_t valid = keys_below(M, gi * kPrepWords + 2 * i + w);
      for (int s = 0; s < 4; ++s)
        for (int v = 0; v < kPrepStages; ++v) {
          any_bits |= red_o[s][v][2 * i + w] & valid;
          all_bits &= red_a[s][v][2 * i + w] | ~valid;
        }
    }
    const int c = classify(any_bits, all_bits);
    c_tile[i] = c;
    if (kt < n_kt) cls[((size_t)mbh * n_qt + qt) * n_kt + kt] = (uint8_t)c;
  } else if (stage_cls && tid >= 64 && tid < 64 + kPrepKTiles * kPrepStages) {
    // (256-key tile u, 64-query stage v) of the dK/dV pass
    const int j = tid - 64, u = j / kPrepStages, v = j % kPrepStages;
    const int kt = gi * kPrepKTiles + u, st = qt * kPrepStages + v;
    uint32_t any_bits = 0u, all_bits = ~0u;
    for (int w = 0; w < 8; ++w) {
      const uint32_t valid = keys_below(M, gi * kPrepWords + 8 * u + w);
      for (int s = 0; s < 4; ++s) {
        any_bits |= red_o[s][v][8 * u + w] & valid;
        all_bits &= red_a[s][v][8 * u + w] | ~valid;
      }
    }
    const int c = classify(any_bits, all_bits);
    c_stage[j] = c;
    if (kt < n_kt256 && st < n_st) stage_cls[((size_t)mbh * n_kt256 + kt) * n_st + st] = (uint8_t)c;
  }
  __syncthreads();

  // ---- blocks: tile t of a row of blocks is block t + 1; block 0 all ones ----
  constexpr int BW = kMaskBlockBytes / 4;  // words per block
  uint32_t* frow = blocks + ((size_t)mbh * n_qt + qt) * (n_kt + 1) * BW;
  if (gi == 0) {
    frow[tid] = ~0u;
    frow[tid + 256] = ~0u;
  }
  // Forward block of tile i, word e = 128 ws + 64 w + l: row 64 ws + l, word 2 i + w.
  for (int i = 0; i < kPrepTiles; ++i) {
    const int kt = gi * kPrepTiles + i;
    if (kt >= n_kt || c_tile[i] != 2) continue;
    uint32_t* dst = frow + (size_t)(kt + 1) * BW;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h, row = (e / 128) * 64 + e % 64, w = (e / 64) % 2;
      dst[e] = rows[row * kPrepPitch + 2 * i + w];
    }
  }
  if (!stage_cls) return;
  // dK/dV block of (u, v), word e = 64 w + l: row 64 v + l, word 8 u + w.
  for (int u = 0; u < kPrepKTiles; ++u) {
    const int kt = gi * kPrepKTiles + u;
    if (kt >= n_kt256) break;
    uint32_t* srow = stage_blocks + ((size_t)mbh * n_kt256 + kt) * (n_st + 1) * BW;
    if (qt == 0) {
      srow[tid] = ~0u;
      srow[tid + 256] = ~0u;
    }
    for (int v = 0; v < kPrepStages; ++v) {
      const int st = qt * kPrepStages + v;
      if (st >= n_st || c_stage[u * kPrepStages + v] != 2) continue;
      uint32_t* dst = srow + (size_t)(st + 1) * BW;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = tid + 256 * h, row = v * 64 + e % 64, w = e / 64;
        dst[e] = rows[row * kPrepPitch + 8 * u + w];
      }
    }
  }
}

// One workgroup per list: lists [0, n_fwd) take `n` classes each from cls,
// the rest (stage lists) `n_s` classes each from stage_cls.  Entries ascend;
// bit 31 marks class 2; entry 0 of a list holds its length.
// walk_n_qt > 0 (causal forward on the pipelined walk, N >= 256, M >= N,
// no kv_len): each forward list (query tile qt = list % walk_n_qt) is cut at
// the causal limit, the first tile past the tile's last query's last key,
// and a list left with fewer than 4 tiles is filled up to 4 with tiles the
// mask does not touch, flagged as kept in part and given an all-zero block
// (every key masked: weights of exactly 0).  A list of such a query tile
// then holds exactly the tiles the prefill visits.
__global__ __launch_bounds__(256) void mask_lists_kernel(const uint8_t* __restrict__ cls, int n,
                                                         int32_t* __restrict__ lists, int64_t n_fwd,
                                                         const uint8_t* __restrict__ stage_cls, int n_s,
                                                         int32_t* __restrict__ stage_lists, int walk_n_qt,
                                                         int N, int M, uint32_t* __restrict__ blocks) {
  __shared__ int wave_n[4];
  __shared__ int pad_tiles[4], n_pad;
  const int64_t g = blockIdx.x;
  const bool fwd = g < n_fwd;
  const int len = fwd ? n : n_s;
  const uint8_t* C = fwd ? cls + g * n : stage_cls + (g - n_fwd) * n_s;
  int32_t* L = fwd ? lists + g * (n + 1) : stage_lists + (g - n_fwd) * (n_s + 1);
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  int base = 0;
  for (int c0 = 0; c0 < len; c0 += 256) {
    const int idx = c0 + tid;
    const int k = idx < len ? C[idx] : 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(k != 0);
    if (lane == 0) wave_n[wv] = __builtin_popcountll(bal);
    __syncthreads();
    int pos = base + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    for (int w = 0; w < wv; ++w) pos += wave_n[w];
    if (k != 0) L[1 + pos] = k == 2 ? (int32_t)((uint32_t)idx | 0x80000000u) : idx;
    base += wave_n[0] + wave_n[1] + wave_n[2] + wave_n[3];
    __syncthreads();
  }
  if (!fwd || walk_n_qt == 0) {
    if (tid == 0) L[0] = base;
    return;
  }
  __syncthreads();  // the entries are written
  const int qt = (int)(g % walk_n_qt);
  const int kv_end = min(M, min(qt * kPrefillBlockQ + kPrefillBlockQ, N) + (M - N));
  const int t_end = (kv_end + kPrefillBlockK - 1) / kPrefillBlockK;
  // entries below t_end (the list ascends)
  int keep = 0;
  for (int c0 = 0; c0 < base; c0 += 256) {
    const int idx = c0 + tid;
    const bool below = idx < base && (L[1 + idx] & 0x7FFFFFFF) < t_end;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(below);
    if (lane == 0) wave_n[wv] = __builtin_popcountll(bal);
    __syncthreads();
    keep += wave_n[0] + wave_n[1] + wave_n[2] + wave_n[3];
    __syncthreads();
  }
  if (tid == 0) {
    int np = 0;
    if (keep < 4) {
      // merge the kept entries with the first untouched tiles, in order
      int out[4], nk = 0, pos = 0;
      for (int t = 0; t < t_end && nk < 4; ++t) {
        if (C[t] != 0) {
          out[nk++] = L[1 + pos++];
        } else if (np < 4 - keep) {
          out[nk++] = (int32_t)((uint32_t)t | 0x80000000u);
          pad_tiles[np++] = t;
        }
      }
      for (int i = 0; i < nk; ++i) L[1 + i] = out[i];
      keep = nk;
    }
    n_pad = np;
    L[0] = keep;
  }
  __syncthreads();
  // zero the blocks of the filler tiles (tile t: block t + 1 of the row)
  constexpr int BW = kMaskBlockBytes / 4;
  uint32_t* frow = blocks + g * (int64_t)(n + 1) * BW;
  for (int i = 0; i < n_pad; ++i) {
    frow[(int64_t)(pad_tiles[i] + 1) * BW + tid] = 0u;
    frow[(int64_t)(pad_tiles[i] + 1) * BW + tid + 256] = 0u;
  }
}

// Order of the causal prefill's pipelined walk.  The walk deals each XCD a
// contiguous range of work items (as the prefill's persistent grid does) and
// takes them round by round, W workgroups a round, alternating direction; in
// mask order, round k takes the k-th W items of the range sorted by tile
// count, most first (ties by item), so that a workgroup's items are as heavy
// as any other's: a snake over the sorted range.  One workgroup per XCD;
// at most kOrderMax items per range.
constexpr int kOrderMax = 4096;
__global__ __launch_bounds__(1024) void mask_order_kernel(const int32_t* __restrict__ lists, int stride,
                                                          int64_t n_items, int n_qt, int H, int mask_b,
                                                          int mask_h, int32_t* __restrict__ order) {
  __shared__ uint64_t key[kOrderMax];
  const int x = blockIdx.x, tid = threadIdx.x;
  const int64_t qx = n_items / kNumXcd, rx = n_items % kNumXcd;
  const int64_t x_start = x * qx + (x < rx ? x : rx);
  const int x_count = (int)(qx + (x < rx ? 1 : 0));
  int P = 1;
  while (P < x_count) P *= 2;
  for (int j = tid; j < P; j += 1024) {
    uint64_t kj = ~0ull;  // past the range: sorts last
    if (j < x_count) {
      const int64_t it = x_start + j, bh = it / n_qt;
      const int qt = n_qt - 1 - (int)(it % n_qt);
      const int bm = mask_b > 1 ? (int)(bh / H) : 0, hm = mask_h > 1 ? (int)(bh % H) : 0;
      const uint32_t n = (uint32_t)lists[((int64_t)(bm * mask_h + hm) * n_qt + qt) * stride];
      kj = ((uint64_t)(~n) << 32) | (uint32_t)j;  // most tiles first, then by item
    }
    key[j] = kj;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= P; size *= 2)
    for (int stride2 = size / 2; stride2 > 0; stride2 /= 2) {
      for (int j = tid; j < P; j += 1024) {
        const int partner = j ^ stride2;
        if (partner > j) {
          const bool up = (j & size) == 0;
          const uint64_t a = key[j], b = key[partner];
          if ((a > b) == up) {
            key[j] = b;
            key[partner] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int j = tid; j < x_count; j += 1024) order[x_start + j] = (int32_t)(uint32_t)(key[j] & 0xFFFFFFFFu);
}

}  // namespace

void launch_mask_prep(const uint32_t* mask, int N, int M, int mask_w, int mask_b, int mask_h,
                      void* ws, const MaskWorkspace& w, bool stages, hipStream_t stream, bool walk, int B,
                      int H) {
  char* base = (char*)ws;
  const int64_t mbh = (int64_t)mask_b * mask_h;
  const int n_qt = (N + kPrefillBlockQ - 1) / kPrefillBlockQ;
  const int n_kt256 = (M + kBwdBlockKV - 1) / kBwdBlockKV;
  if (mbh == 0) return;
  const int n_grp = (mask_w + kPrepWords - 1) / kPrepWords;
  if (n_qt > 0 && n_grp > 0)
    hipLaunchKernelGGL(mask_blocks_kernel, dim3((unsigned)(mbh * n_qt), (unsigned)n_grp), dim3(256), 0,
                       stream, mask, N, M, mask_w, n_qt, (uint8_t*)(base + w.cls),
                       (uint32_t*)(base + w.blocks), stages ? (uint8_t*)(base + w.stage_cls) : nullptr,
                       stages ? (uint32_t*)(base + w.stage_blocks) : nullptr);
  // every list is written, also empty ones (N or M of 0)
  const int64_t n_fwd = mbh * n_qt, n_bwd = stages ? mbh * n_kt256 : 0;
  if (n_fwd + n_bwd > 0)
    hipLaunchKernelGGL(mask_lists_kernel, dim3((unsigned)(n_fwd + n_bwd)), dim3(256), 0, stream,
                     (const uint8_t*)(base + w.cls), mask_list_stride(M) - 1, (int32_t*)(base + w.lists),
                     n_fwd, (const uint8_t*)(base + w.stage_cls), mask_stage_stride(N) - 1,
                     (int32_t*)(base + w.stage_lists), walk ? n_qt : 0, N, M, (uint32_t*)(base + w.blocks));
  if (walk && n_qt > 0 && (int64_t)B * H > 0)
    hipLaunchKernelGGL(mask_order_kernel, dim3(kNumXcd), dim3(1024), 0, stream, (const int32_t*)(base + w.lists),
                       mask_list_stride(M), (int64_t)B * H * n_qt, n_qt, H, mask_b, mask_h,
                       (int32_t*)(base + w.order));
}

}  // namespace fa
