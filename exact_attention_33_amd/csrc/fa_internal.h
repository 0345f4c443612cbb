// Internal interface between the C-ABI shim, the planner and the kernels.
// Not installed; the public interface is include/fa_mi355x.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fa_mi355x.h"

namespace fa {

// Problem description handed to every launcher.  Pointers are device
// pointers; tensors are contiguous [B,H,N|M,D] with D fastest.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_len;  // [B] or nullptr (= M for all)
  void* o;
  float* lse;
  int32_t B, H, N, M, D;
  float scale;
  int causal;
  // Local window (options.window): key j visible to query i only if
  // i + off - wl <= j <= i + off + wr, off = kv_len - N.  window == 0: none.
  int window;
  int32_t wl, wr;
  // FA_FP8: the inputs stand for q_descale * Q8, k_descale * K8, v_descale * V8.
  float q_descale, k_descale, v_descale;
  // Element mask (options.mask): words [mask_b][mask_h][N][mask_w], bit j % 32
  // of word j / 32 set = key j visible; nullptr: none.
  const uint32_t* mask;
  int32_t mask_b, mask_h, mask_w;
};

// Planner output (host-only; see plan.cpp).
struct Plan {
  fa_path path;
  int32_t block_q;
  int32_t block_k;
  int32_t threads;
  int32_t lds_bytes;
  int32_t splits;       // split-KV only
  int64_t grid;
  size_t ws_bytes;
  size_t ws_lse_offset;  // split-KV: byte offset of the partial LSE array
  int32_t mask_tiles;    // prefill with a mask: int32 entries per tile list
  int32_t split_tiles;   // prefill with key splits: 64-key tiles per chunk (0: none)
};

// Returns FA_OK and fills `plan`, or an error status with `why` set.
fa_status make_plan(const fa_shape& s, fa_dtype dt, int causal,
                    const fa_options* opt, Plan* plan, const char** why);

// Kernel launchers: enqueue on `stream`, return the launch status.
hipError_t launch_prefill_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream);
hipError_t launch_fwd_f32(const Problem& p, const Plan& plan, hipStream_t stream);
hipError_t launch_splitkv_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream);
hipError_t launch_kvouter_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream);
hipError_t launch_prefill_fp8(const Problem& p, const Plan& plan, hipStream_t stream);

// Tile constants shared by the planner and the kernels.
constexpr int kPrefillBlockQ = 256;   // 4 waves x 64 queries
constexpr int kPrefillBlockK = 64;    // keys per K/V tile
constexpr int kPrefillThreads = 256;
// Persistent causal prefill: at most one workgroup per CU of an MI355X.
constexpr int kPrefillPersistGrid = 256;

// Element mask on the prefill path: the workspace holds, per (mask batch,
// mask head, 256-query tile), a list of kMaskListStride(M) int32: the count,
// then the key tiles (64 keys) in which some query of the tile sees a masked-in
// key, ascending, bit 31 set on tiles the mask does not keep whole.  The
// kernel copies a list into LDS, so a list holds at most kMaskMaxTiles - 1
// tiles.
constexpr int kMaskMaxTiles = 4096;
// The causal prefill's pipelined walk with a mask holds the lists of all of a
// workgroup's work items in LDS (at most kMaskMaxTiles - 5 entries), for at
// most kWalkMaxItems items.
constexpr int kWalkMaxItems = 64;
__host__ __device__ inline int32_t mask_list_stride(int M) { return (M + kPrefillBlockK - 1) / kPrefillBlockK + 1; }
__host__ __device__ inline int32_t mask_words(int M) { return (M + 31) / 32; }
// Mask words of one (query tile, key tile) pair, copied by the pre-pass into
// a contiguous block so that each wave reads its rows' words with one
// coalesced load: 256 rows x 2 words, stored [wave][word][row of the wave]
// (2 KB).  The dK/dV pass's blocks hold one (256-key tile, 64-query stage)
// pair: 64 rows x 8 words, stored [word][row] (2 KB).  Only pairs the mask
// keeps in part have a block (tile t: block t + 1 of its row of blocks);
// block 0 of each row is all ones and stands for the pairs kept whole.
constexpr int kMaskBlockBytes = 2048;

constexpr int kF32BlockQ = 16;        // 16 query rows x 16 lanes
constexpr int kF32BlockK = 32;
constexpr int kF32Threads = 256;

constexpr int kFp8BlockQ = 256;       // 8 waves x 32 queries
constexpr int kFp8Threads = 512;

constexpr int kSplitThreads = 256;
constexpr int kMergeThreads = 256;

inline int prefill_lds_bytes(int D) {
  // Three K and three V tiles, padded, in 1 KB blocks, rounded up to a whole
  // number of blocks per wave.
  const int waves = kPrefillThreads / 64;
  const int kblk = (kPrefillBlockK * (D + 8) / 8 + 63) / 64;
  const int vblk = (kPrefillBlockK * (D + 32) / 8 + 63) / 64;
  return 1024 * 3 * ((kblk + waves - 1) / waves * waves + (vblk + waves - 1) / waves * waves);
}
inline int f32_lds_bytes(int D) { return 2 * kF32BlockK * D * 4; }

// ---- backward ----

// Problem description handed to the backward launchers.  q, k, v, o, dout,
// dq, dk, dv are contiguous [B,H,N|M,D] device tensors; lse [B,H,N] float32.
// The workspace holds, per (batch, head), Npad float32 values of
// LSE * log2(e) (+inf for a row with no visible key and for the padding
// rows) followed by Npad values of the row statistic D = rowsum(dO * O).
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const int32_t* kv_len;
  void* dq;
  void* dk;
  void* dv;
  float* ws;
  int32_t B, H, N, M, D, Npad;
  float scale;
  int causal;
  int window;            // as in Problem
  int32_t wl, wr;
  // Element mask, as in Problem (nullptr: none); with a mask the workspace
  // continues, at byte offset bwd_mask_lists_offset, with the pre-pass
  // output (mask_workspace with stages).
  const uint32_t* mask;
  int32_t mask_b, mask_h, mask_w;
  int32_t* lists;        // dQ pass: per 256-query tile, the key stages (64 keys)
  int32_t* stage_lists;  // dK/dV pass: per 256-key tile, the query stages (64 queries)
  const uint32_t* blocks;        // dQ pass: words of each listed (query tile, key stage)
  const uint32_t* stage_blocks;  // dK/dV pass: words of each listed (key tile, query stage)
};

constexpr int kBwdThreads = 256;
constexpr int kBwdRowPad = 256;        // Npad = N rounded up to this
constexpr int kBwdStageQ = 64;         // dK/dV kernel: queries per LDS stage
constexpr int kBwdBlockKV = 256;       // dK/dV kernel: keys per workgroup (4 waves x 64)
constexpr int kBwdBlockQ = 256;        // dQ kernel: queries per workgroup (4 waves x 64)
constexpr int kBwdStageK = 64;         // dQ kernel: keys per LDS stage

inline int64_t bwd_npad(int N) { return ((int64_t)N + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad; }
inline size_t bwd_stats_bytes(const fa_shape& s) {
  return (size_t)s.B * (size_t)s.H * (size_t)bwd_npad(s.N) * 2 * sizeof(float);
}
inline size_t bwd_mask_lists_offset(const fa_shape& s) { return (bwd_stats_bytes(s) + 255) / 256 * 256; }
// dK/dV pass with a mask: per (mask batch, mask head, 256-key tile), the
// count and then the ascending 64-query stages in which some query keeps
// one of the tile's keys.
__host__ __device__ inline int32_t mask_stage_stride(int N) { return (N + kBwdStageQ - 1) / kBwdStageQ + 1; }

// Byte offsets of the element-mask pre-pass output in a workspace, from
// `base`: the forward's tile lists (per mask batch, mask head and 256-query
// tile: mask_list_stride(M) int32), with stages the dK/dV pass's stage lists
// (per 256-key tile: mask_stage_stride(N) int32); then one class byte per
// (query tile, 64-key tile) (0: no key kept, 1: all, 2: some) and per query
// tile a row of 1 + ceil(M / 64) blocks; with stages, one class byte per
// (256-key tile, 64-query stage) and per key tile a row of 1 + ceil(N / 64)
// blocks; without stages, `items` int32 (the order in which the causal
// prefill's pipelined walk takes the work items).  Every region starts on 256
// bytes.
struct MaskWorkspace {
  size_t lists, stage_lists, cls, blocks, stage_cls, stage_blocks, order, end;
};
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }
inline MaskWorkspace mask_workspace(int N, int M, int mask_b, int mask_h, size_t base, bool stages,
                                    int64_t items = 0) {
  const size_t mbh = (size_t)mask_b * (size_t)mask_h;
  const size_t n_qt = (size_t)((N + kPrefillBlockQ - 1) / kPrefillBlockQ);
  const size_t n_kt = (size_t)(mask_list_stride(M) - 1);
  const size_t n_kt256 = (size_t)((M + kBwdBlockKV - 1) / kBwdBlockKV);
  const size_t n_st = (size_t)(mask_stage_stride(N) - 1);
  MaskWorkspace w{};
  w.lists = base;
  w.stage_lists = align256(w.lists + mbh * n_qt * (n_kt + 1) * sizeof(int32_t));
  w.cls = stages ? align256(w.stage_lists + mbh * n_kt256 * (n_st + 1) * sizeof(int32_t)) : w.stage_lists;
  w.blocks = align256(w.cls + mbh * n_qt * n_kt);
  w.stage_cls = align256(w.blocks + mbh * n_qt * (n_kt + 1) * kMaskBlockBytes);
  w.stage_blocks = stages ? align256(w.stage_cls + mbh * n_kt256 * n_st) : w.stage_cls;
  w.order = w.stage_cls;
  w.end = stages ? w.stage_blocks + mbh * n_kt256 * (n_st + 1) * kMaskBlockBytes
                 : (items > 0 ? align256(w.stage_cls) + (size_t)items * sizeof(int32_t) : w.stage_cls);
  if (!stages && items > 0) w.order = align256(w.stage_cls);
  return w;
}
// mask_b, mask_h: 0 without a mask
inline size_t bwd_workspace_bytes(const fa_shape& s, int mask_b = 0, int mask_h = 0) {
  if (!mask_b) return bwd_stats_bytes(s);
  return mask_workspace(s.N, s.M, mask_b, mask_h, bwd_mask_lists_offset(s), true).end;
}
// Row stride in LDS of a staged [rows][D] bf16 tile: 64 bytes of padding.
inline int bwd_lds_row_bytes(int D) { return 2 * D + 64; }
inline int bwd_dkdv_lds_bytes(int D) { return 2 * (2 * kBwdStageQ * bwd_lds_row_bytes(D) + 1024); }
inline int bwd_dq_lds_bytes(int D) { return 2 * (2 * kBwdStageK * bwd_lds_row_bytes(D)); }

hipError_t launch_bwd_bf16(const BwdProblem& p, hipStream_t stream);

// Element-mask pre-pass: classifies the mask's tiles, lists them, and copies
// the words of the tiles the mask keeps in part into blocks (layout above),
// into the workspace regions `w` names relative to `ws`; with stages also
// the dK/dV pass's stage lists and blocks.  walk (B, H given): the forward
// lists are cut at the causal limit (no kv_len, M >= N >= 256) and filled up
// to 4 tiles with fully masked ones, and the work items of each XCD's range
// are ordered by tile count, most first, into w.order, for the causal
// prefill's pipelined walk.
void launch_mask_prep(const uint32_t* mask, int N, int M, int mask_w, int mask_b, int mask_h,
                      void* ws, const MaskWorkspace& w, bool stages, hipStream_t stream, bool walk = false,
                      int B = 0, int H = 0);

// Records a failure for fa_last_error() on the calling thread (printf-style
// detail) and returns `st`; shared by every C entry point.
fa_status report_error(fa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace fa
