// Tiling and launch planner: a pure host function of the shape and options.
//
// The tile sizes follow the counting argument of "FlashAttention: attention
// was never compute-bound", How big should a tile be?: K and V are re-read
// once per query tile, so the query tile is the largest that keeps its
// working set on chip.  On gfx950 the prefill's working set lives in
// registers (Q, the score and weight tiles, the output accumulator: one wave
// of 64 queries per SIMD with all 512 registers) and LDS (a ring of K and V
// tiles of 64 keys, about 120 KB at D = 128), so a workgroup holds 256
// queries and one workgroup runs per compute unit.  Batch, heads and query
// tiles are independent ("Understanding FlashAttention", Attention: batch
// and heads only repeat the problem), so the grid spans all three; causal
// attention without a window or mask gets a persistent grid of one
// workgroup per compute unit that walks the query tiles of its XCD.
#include <algorithm>
#include <climits>
#include <cstdint>

#include "fa_internal.h"

namespace fa {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Keys per split for split-KV decode: large enough to stream long runs of
// contiguous K/V rows (512 keys = 256 KB of K and V at D = 128), small enough
// that the grid covers the GPU many times over (measured on MI355X: 512 beats
// 256, 1024 and 2048 on the B=32, H=32, kv_len up to 32768 decode).
int32_t auto_split_keys(const fa_shape& s) {
  int32_t sk = 512;
  while (sk > 128 && (int64_t)s.B * s.H * ceil_div(s.M, sk) < 4096) sk /= 2;
  return sk;
}

}  // namespace

fa_status make_plan(const fa_shape& s, fa_dtype dt, int causal,
                    const fa_options* opt, Plan* plan, const char** why) {
  *plan = Plan{};
  if (s.B < 0 || s.H < 0 || s.N < 0 || s.M < 0 || s.D < 0) {
    *why = "B, H, N, M and D must be non-negative";
    return FA_ERR_SHAPE;
  }
  if (dt != FA_F32 && dt != FA_BF16 && dt != FA_FP8) {
    *why = "dtype must be FA_F32, FA_BF16 or FA_FP8";
    return FA_ERR_UNSUPPORTED;
  }
  if (s.D != 64 && s.D != 128) {
    *why = "head dimension D must be 64 or 128";
    return FA_ERR_UNSUPPORTED;
  }
  const int32_t req = opt ? opt->path : FA_PATH_AUTO;
  if (req < FA_PATH_AUTO || req > FA_PATH_FP8) {
    *why = "options.path is not a fa_path value";
    return FA_ERR_ARG;
  }
  if (opt && (opt->split_keys < 0 || opt->split_keys % 64 != 0)) {
    *why = "options.split_keys must be 0 or a positive multiple of 64";
    return FA_ERR_ARG;
  }
  const bool window = opt && opt->window;
  if (opt && (opt->window != 0 && opt->window != 1)) {
    *why = "options.window must be 0 or 1";
    return FA_ERR_ARG;
  }
  if (opt && opt->kvouter_query_tiles < 0) {
    *why = "options.kvouter_query_tiles must be >= 0";
    return FA_ERR_ARG;
  }
  if (window && (opt->window_left < 0 || opt->window_right < 0)) {
    *why = "options.window_left and window_right must be >= 0";
    return FA_ERR_ARG;
  }
  const bool mask = opt && opt->mask;
  const int32_t mask_b = mask && opt->mask_batches ? opt->mask_batches : 1;
  const int32_t mask_h = mask && opt->mask_heads ? opt->mask_heads : 1;
  if (mask && ((mask_b != 1 && mask_b != s.B) || (mask_h != 1 && mask_h != s.H))) {
    *why = "options.mask_batches must be 1 or B and options.mask_heads 1 or H";
    return FA_ERR_ARG;
  }
  // Element counts must fit comfortably in 64-bit byte offsets.
  const int64_t bh = (int64_t)s.B * s.H;
  if (bh > INT32_MAX || (bh > 0 && ((int64_t)s.N * s.D > INT64_MAX / 8 / bh ||
                                    (int64_t)s.M * s.D > INT64_MAX / 8 / bh))) {
    *why = "tensor sizes overflow 64-bit offsets";
    return FA_ERR_SHAPE;
  }

  if (opt && !(opt->q_descale >= 0.f && opt->k_descale >= 0.f && opt->v_descale >= 0.f &&
               opt->q_descale < 3.4e38f && opt->k_descale < 3.4e38f && opt->v_descale < 3.4e38f)) {
    *why = "options.q_descale, k_descale and v_descale must be finite and >= 0";
    return FA_ERR_ARG;
  }
  fa_path path;
  if (dt == FA_FP8) {
    if (req != FA_PATH_AUTO && req != FA_PATH_FP8) {
      *why = "FA_FP8 inputs run only on FA_PATH_FP8";
      return FA_ERR_UNSUPPORTED;
    }
    if (window || mask) {
      *why = "FA_PATH_FP8 takes no window and no element mask";
      return FA_ERR_UNSUPPORTED;
    }
    path = FA_PATH_FP8;
  } else if (req == FA_PATH_FP8) {
    *why = "FA_PATH_FP8 needs FA_FP8 inputs";
    return FA_ERR_UNSUPPORTED;
  } else if (dt == FA_F32) {
    if (req != FA_PATH_AUTO && req != FA_PATH_F32) {
      *why = "float32 inputs run only on FA_PATH_F32";
      return FA_ERR_UNSUPPORTED;
    }
    path = FA_PATH_F32;
  } else {
    if (req == FA_PATH_F32) {
      *why = "FA_PATH_F32 needs float32 inputs";
      return FA_ERR_UNSUPPORTED;
    }
    if (req == FA_PATH_SPLITKV && s.N != 1) {
      *why = "FA_PATH_SPLITKV needs N == 1 (one query per sequence)";
      return FA_ERR_UNSUPPORTED;
    }
    if (req == FA_PATH_KVOUTER && (window || mask)) {
      *why = "FA_PATH_KVOUTER takes no window and no element mask";
      return FA_ERR_UNSUPPORTED;
    }
    if (req == FA_PATH_SPLITKV && (window || mask)) {
      *why = "FA_PATH_SPLITKV has no window and no element mask; such a query runs on "
             "FA_PATH_PREFILL";
      return FA_ERR_UNSUPPORTED;
    }
    // A window bounds a query's keys, so one query is cheap on the prefill
    // kernel, and the prefill kernel is the one that reads element masks; the
    // split-KV path streams whole caches.
    path = req == FA_PATH_AUTO
               ? (s.N == 1 && !window && !mask ? FA_PATH_SPLITKV : FA_PATH_PREFILL)
               : (fa_path)req;
  }

  plan->path = path;
  switch (path) {
    case FA_PATH_PREFILL:
      // The prefill kernel addresses one (batch, head) of K or V with 32-bit
      // byte offsets.
      if ((int64_t)s.M * s.D * 2 > INT32_MAX) {
        *why = "FA_PATH_PREFILL needs M * D * 2 < 2^31 (K/V bytes per batch and head)";
        return FA_ERR_UNSUPPORTED;
      }
      plan->block_q = kPrefillBlockQ;
      plan->block_k = kPrefillBlockK;
      plan->threads = kPrefillThreads;
      plan->lds_bytes = prefill_lds_bytes(s.D);
      plan->grid = ceil_div(s.N, kPrefillBlockQ) * bh;
      if (opt && opt->split_keys > 0) {
        // key splits: one workgroup per (query tile, chunk of split_keys
        // keys), each writing float32 partial results, then one merge launch
        if (window || mask) {
          *why = "key splits (options.split_keys) on FA_PATH_PREFILL take no window and no element mask";
          return FA_ERR_UNSUPPORTED;
        }
        plan->split_tiles = opt->split_keys / kPrefillBlockK;
        plan->splits = (int32_t)std::max<int64_t>(1, ceil_div(s.M, opt->split_keys));
        plan->grid *= plan->splits;
        if (plan->grid > INT32_MAX) {
          *why = "too many key splits: B * H * ceil(N / 256) * ceil(M / split_keys) must stay below 2^31";
          return FA_ERR_UNSUPPORTED;
        }
        const size_t rows = (size_t)bh * (size_t)s.N * (size_t)plan->splits;
        plan->ws_lse_offset = align_up(rows * (size_t)s.D * sizeof(float), 256);
        plan->ws_bytes = rows ? align_up(plan->ws_lse_offset + rows * sizeof(float), 256) : 0;
        break;
      }
      // causal without a window or a mask: persistent workgroups, one per CU
      // (a multiple of the 8 XCDs), each walking several query tiles
      if (causal && !window && !mask)
        plan->grid = std::min<int64_t>((plan->grid + 7) / 8 * 8, kPrefillPersistGrid);
      if (mask) {
        // the kernel holds one query tile's list of key tiles in LDS, and
        // addresses one (mask batch, mask head) of the mask with 32-bit byte
        // offsets
        plan->mask_tiles = mask_list_stride(s.M);
        if (plan->mask_tiles > kMaskMaxTiles) {
          *why = "an element mask on FA_PATH_PREFILL needs M <= 262080";
          return FA_ERR_UNSUPPORTED;
        }
        if ((int64_t)s.N * mask_words(s.M) * 4 > INT32_MAX) {
          *why = "an element mask on FA_PATH_PREFILL needs N * ceil(M / 32) * 4 < 2^31";
          return FA_ERR_UNSUPPORTED;
        }
        // the pre-pass's tile lists, tile classes and blocks of mask words,
        // and the order of the work items for the pipelined causal walk
        plan->ws_bytes = mask_workspace(s.N, s.M, mask_b, mask_h, 0, false, causal ? bh * ceil_div(s.N, kPrefillBlockQ) : 0).end;
      }
      break;
    case FA_PATH_F32:
      plan->block_q = kF32BlockQ;
      plan->block_k = kF32BlockK;
      plan->threads = kF32Threads;
      plan->lds_bytes = f32_lds_bytes(s.D);
      plan->grid = ceil_div(s.N, kF32BlockQ) * bh;
      break;
    case FA_PATH_SPLITKV: {
      const int32_t sk = (opt && opt->split_keys) ? opt->split_keys : auto_split_keys(s);
      plan->block_q = 1;
      plan->block_k = sk;
      plan->threads = kSplitThreads;
      plan->splits = (int32_t)ceil_div(s.M, sk);
      plan->lds_bytes = 0;
      plan->grid = (int64_t)plan->splits * bh;
      const size_t parts = (size_t)bh * (size_t)plan->splits;
      plan->ws_lse_offset = align_up(parts * (size_t)s.D * sizeof(float), 256);
      plan->ws_bytes = parts ? align_up(plan->ws_lse_offset + parts * sizeof(float), 256) : 0;
      break;
    }
    case FA_PATH_FP8:
      // one (batch, head) of K or V is addressed with 32-bit byte offsets
      if ((int64_t)s.M * s.D > INT32_MAX) {
        *why = "FA_PATH_FP8 needs M * D < 2^31 (K/V bytes per batch and head)";
        return FA_ERR_UNSUPPORTED;
      }
      plan->block_q = kFp8BlockQ;
      plan->block_k = 64;
      plan->threads = kFp8Threads;
      plan->lds_bytes = 4 * 64 * s.D;
      plan->grid = ceil_div(s.N, kFp8BlockQ) * bh;
      if (causal)  // persistent, as the causal bf16 prefill
        plan->grid = std::min<int64_t>((plan->grid + 7) / 8 * 8, kPrefillPersistGrid);
      break;
    case FA_PATH_KVOUTER: {
      if ((int64_t)s.M * s.D * 2 > INT32_MAX) {
        *why = "FA_PATH_KVOUTER needs M * D * 2 < 2^31 (K/V bytes per batch and head)";
        return FA_ERR_UNSUPPORTED;
      }
      const int64_t n_qt = ceil_div(s.N, 256);
      const int64_t tpg = std::max<int64_t>(1, std::min<int64_t>(
          n_qt, (opt && opt->kvouter_query_tiles) ? opt->kvouter_query_tiles : 1));
      plan->block_q = (int32_t)(256 * tpg);
      plan->block_k = 64;
      plan->threads = 256;
      plan->lds_bytes = 2 * 64 * (2 * s.D + 64);
      plan->grid = n_qt ? ceil_div(n_qt, tpg) * bh : 0;
      // float32 accumulator [B,H,N,D], then m and l [B,H,N] each
      plan->ws_bytes = align_up((size_t)bh * (size_t)s.N * ((size_t)s.D + 2) * sizeof(float), 256);
      break;
    }
    default:
      *why = "internal: no path";
      return FA_ERR_UNSUPPORTED;
  }
  if (plan->grid > INT32_MAX) {
    *why = "grid exceeds 2^31 - 1 workgroups";
    return FA_ERR_SHAPE;
  }
  return FA_OK;
}

}  // namespace fa
