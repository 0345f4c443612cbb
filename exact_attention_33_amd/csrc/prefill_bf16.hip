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
//  * workgroup = 4 waves = 256 queries, one wave per SIMD; wave w owns the 64
//    queries [64w, 64w + 64) as two 32-query blocks.  With one wave per SIMD
//    a wave has 512 registers: Q (64 rows), the output accumulator, two score
//    tiles and two weight tiles all stay in registers.  Each wave reads whole
//    K and V tiles from LDS, so 64 queries per wave halve the LDS traffic per
//    FLOP against 32 (LDS bandwidth, about 150-185 B/clk per CU measured on
//    MI355X, bounds a 32-query design);
//  * software pipeline inside the wave: iteration t issues the MFMAs of
//    S(t+2) = K(t+2) Q^T and O += P(t) V(t) and, between them, the softmax of
//    tile t+1 (mask, exponentials, row sum) on the VALU.  The three
//    have no data dependence, and one wave keeps its matrix pipe nearly full
//    while it issues about four VALU instructions per MFMA (measured: 64
//    MFMAs with that VALU mix and their LDS operand reads take about 2,600
//    cycles against 2,048 for the MFMAs alone).  Scheduling barriers fix the
//    interleave: step j of an iteration holds one MFMA, the LDS reads of the
//    operands two fragments ahead, and a slice of the softmax or a tile
//    load (the loads go with the S MFMAs of key block 1, which carry no
//    softmax work);
//  * the score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: Q is the B operand, K comes from LDS.  Lane
//    (h, c) of a wave (h = lane / 32, c = lane % 32) then holds, per 32-query
//    block, 16 scores of query c per 32-key block, at keys 8*(r/4) + 4*h + r%4,
//    so a row's sum (and, on the rare path, its max) is in-lane plus one swap
//    between the half-waves (v_permlane32_swap);
//  * scores are kept in base 2: t = s * scale * log2(e), weights 2^(t - m) on
//    v_exp_f32; the scale is applied in float32 to the float32 score;
//  * no row max on the common path: the pages subtract the max only to keep
//    the exponentials finite, and any reference m that keeps every weight at
//    most 2^20 gives the same l, O and L.  A weight above that shows in the
//    lane's sum of the tile's weights; that, or a row's first visible key,
//    sends the wave to a rare path that moves m up to the row max of the key
//    block and rescales l and the output accumulator (after the iteration's
//    P V products, which still use the old reference);
//  * the output is accumulated transposed, O^T += V^T P^T, with the same MFMA:
//    the weights convert to bf16 straight into the B operand (no LDS round
//    trip) and V^T comes from V's natural [key][d] layout in LDS through two
//    ds_read_b64_tr_b16 transposing reads per fragment.  The row sum adds the
//    float32 weights before rounding (a sum of bf16-rounded weights would
//    carry their 2^-9 relative error into LSE for rows with few keys);
//  * K and V move HBM -> LDS directly (buffer loads into LDS, 16 bytes per
//    lane: each lane's bytes land at M0 + 16 * lane, so one wave instruction
//    fills a 1 KB block and the per-lane offset picks what goes where), with
//    no staging registers.  Three K and three V buffers, each its own LDS array
//    so the compiler can see that reading one never waits on a load into
//    another.  Iteration t loads K(t+4) and V(t+2), spread over its phase A,
//    and iteration t + 1 ends by waiting for them: every load has a whole
//    iteration more than its issue to land;
//  * LDS layouts are padded so that every operand read is one per-lane base
//    register plus a compile-time offset and conflict-free on the 64 banks:
//    K rows carry 16 bytes of padding, so the 16 rows that a 16-lane group
//    reads with ds_read_b128 start 4 banks apart; V rows carry 64 bytes, so
//    the 4 rows x 64 bytes that 32 lanes read with ds_read_b64_tr_b16 start
//    16 banks apart.  The slots of a 1 KB load block that fall on padding
//    receive a copy of valid data that is never read;
//  * causal: tiles past the workgroup's last visible key are never visited,
//    a wave skips the work of tiles none of its queries sees, and only tiles
//    that cross the diagonal or the kv_len boundary are masked element by
//    element;
//  * workgroup order: gfx950 deals workgroups round-robin to its 8 XCDs, each
//    with its own L2.  Consecutive logical work items (the query tiles of one
//    (batch, head), heaviest first when causal) are mapped to one XCD so that
//    the workgroups sharing a head's K/V run together on one L2;
//  * causal with no window, mask or kv_len: one persistent workgroup per CU
//    walks several work items, and its software pipeline runs straight from
//    one item into the next (the tiles of one query block are independent of
//    every other block's, "Understanding FlashAttention", From loops to
//    tiling): the iterations on an item's last tiles already load, score and
//    weigh the next item's first tiles, Q of the next item is reloaded once
//    the last S MFMAs on the current Q have issued, and the output of an item
//    is written out between two iterations.  Against draining the pipeline
//    at every item (a prologue per item, two iterations on tiles past its
//    end) this measured +1.2% at N = 8192, +2.2% at 4096 and +4.6% at 2048
//    (D = 128), with bit-identical results;
//  * element masks ("Understanding FlashAttention", Attention: mask() is any
//    elementwise constant, causal being one kind): a pre-pass reduces the
//    mask over each 256-query x 64-key tile and lists, per query tile, the
//    key tiles in which some query keeps a key, flagging those it does not
//    keep whole.  The workgroup copies its list to LDS and visits only the
//    listed tiles (the general form of the causal tile skip).  The pre-pass
//    also copies each flagged tile's words into a contiguous 2 KB block, so
//    each wave's words for a tile (64 rows x 2 words) travel HBM -> LDS as
//    two coalesced 256-byte loads with the tile loads, three tiles ahead,
//    and the bits are applied only on flagged tiles.
#include <algorithm>
#include <cmath>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "fa_internal.h"

namespace fa {
namespace {




// S^T += K Q^T fragment products with the accumulator in VGPRs.  The score
// tile is read by the softmax right after it is formed; the compiler places
// every MFMA accumulator of this kernel in AGPRs, and reading AGPRs back
// between MFMAs costs about twice a VALU operation per value (measured).
// The output accumulator stays in AGPRs (it is read only at the end).  These
// asm MFMAs are invisible to the compiler's hazard tracking, so their users
// keep the rules themselves: back-to-back accumulation into the same VGPRs
// (same opcode, exact overlap) needs no wait; a VALU read of a result waits
// 16 wait states after the last MFMA that wrote it (mfma_guard; an 8-pass
// MFMA needs 11); an operand register is overwritten no sooner than two
// fragments (four MFMAs) after its last use.
// The B operand (Q) is taken from AGPRs: Q is read only here, and keeping its
// 64 registers out of the VGPRs leaves room for the score tile.
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// The same with two wait states ahead, inside the asm: outside the pipelined
// loop the compiler may write an operand (a copy into a free register) right
// before the MFMA, and a VALU write needs 2 wait states before an MFMA reads
// it as SrcA or SrcB.
__device__ __forceinline__ void mfma_s_first_safe(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s_acc_safe(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// max of three floats as one v_max3_f32 (fmaxf would first quiet each
// operand with an extra instruction; the scores are never signalling NaNs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

__device__ __forceinline__ void mfma_guard() { asm volatile("s_nop 7\n\ts_nop 7"); }


// Key splits of the prefill: each query tile's keys in chunks of
// split_tiles tiles, one workgroup per (query tile, chunk), each writing its
// chunk's normalised output and log-sum-exp (float32) for the merge.
struct SplitArgs {
  float* part_o;    // [splits][B H][N][D]
  float* part_lse;  // [splits][B H][N]
  int split_tiles;  // 64-key tiles per chunk
  int splits;
};

// The kernel body, shared by the prefill kernel and its key-split form.
template <int D, bool CAUSAL, bool WINDOW, bool BITS, bool SPLIT, bool CONT = false>
__device__ __forceinline__ void prefill_body(const Problem& p, int n_qtiles, const int32_t* __restrict__ tile_lists,
                                             int list_stride, const uint32_t* __restrict__ mask_blocks,
                                             const SplitArgs& sp, const int32_t* __restrict__ walk_order = nullptr) {
  static_assert(!SPLIT || (!WINDOW && !BITS), "key splits take no window and no mask");
  static_assert(!CONT || (!SPLIT && (!BITS || (CAUSAL && !WINDOW))),
                "one pipeline over the walk: no key splits; a mask only with causal attention");
  constexpr int BQ = kPrefillBlockQ, BK = kPrefillBlockK;
  constexpr int NW = kPrefillThreads / 64;   // waves per workgroup
  constexpr int QW = BQ / NW;                // queries per wave
  constexpr int NQB = QW / 32;               // 32-query blocks per wave
  constexpr int NKB = BK / 32;               // 32-key blocks per tile
  constexpr int NP = BK / 16;                // 16-key weight fragments per query block
  constexpr int DK = D / 16;                 // k-steps of S
  constexpr int DB = D / 32;                 // 32-wide d-blocks of O
  constexpr int NF = NKB * DK;               // K fragments per tile (= V fragments)
  static_assert(NF == NP * DB, "K and V fragment counts match");
  constexpr int CPR = D / 8;                 // 16-byte chunks of data per row
  constexpr int KROW = D + 8;                // K row stride in LDS (elements)
  constexpr int VROW = D + 32;               // V row stride in LDS (elements)
  constexpr int KCH = KROW / 8, VCH = VROW / 8;        // 16-byte slots per row
  constexpr int KBLK = (BK * KCH + 63) / 64;           // 1 KB blocks per K tile
  constexpr int VBLK = (BK * VCH + 63) / 64;           // 1 KB blocks per V tile
  constexpr int KPW = (KBLK + NW - 1) / NW, VPW = (VBLK + NW - 1) / NW;  // blocks per wave
  static_assert(NW == 4 && QW == 64, "4 waves of 64 queries");
  // Every wave loads the same number of blocks; the blocks past a tile's last
  // (KBLK .. NW * KPW) receive bytes that are never read.
  __shared__ __attribute__((aligned(1024))) __bf16 Kb0[NW * KPW * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Kb1[NW * KPW * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Kb2[NW * KPW * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb0[NW * VPW * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb1[NW * VPW * 512];
  __shared__ __attribute__((aligned(1024))) __bf16 Vb2[NW * VPW * 512];
  // Element mask: the workgroup's list of key tiles, and a ring of three
  // tiles' mask words, per wave [word][64 rows].
  __shared__ int tlist[BITS ? kMaskMaxTiles : 1];
  // CONT with a mask: tlist holds the workgroup's whole tile stream (its
  // items' lists one after another), walk_n the tiles of each item
  __shared__ int walk_n[CONT && BITS ? kWalkMaxItems : 1];
  __shared__ int walk_item[CONT && BITS ? kWalkMaxItems : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Mb0[BITS ? NW * 128 : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Mb1[BITS ? NW * 128 : 1];
  __shared__ __attribute__((aligned(256))) uint32_t Mb2[BITS ? NW * 128 : 1];
  // Output staging: a wave writes the normalised output of 32 of its rows
  // here and reads it back as 16-byte pieces of whole rows, so that each
  // store to O covers whole rows instead of 16 bytes of 32 rows (measured:
  // the scattered stores held an item's write-out to about 8,000 cycles).
  // With a mask at D = 128 the LDS has no room for it.
  constexpr bool OSTAGE = !SPLIT && !(BITS && D == 128);
  constexpr int OSTR = 2 * D + 16;  // staging row stride in bytes
  __shared__ __attribute__((aligned(16))) uint8_t ostage[OSTAGE ? NW * 32 * OSTR : 16];

  // Causal without a window or a mask: persistent workgroups, one per CU
  // (the planner's grid), each walking the work items of its XCD.  Round k
  // takes item k W + u (even k) or k W + W - 1 - u (odd k), W workgroups
  // per XCD and u this workgroup's place among them: the items of one
  // (batch, head) run together on one XCD as before, and since a causal
  // head's query tiles come heaviest first, a workgroup's heavy and light
  // tiles alternate (measured on MI355X: -3% at N = 8192, -14% at N = 4096
  // against one workgroup per item, results identical; with uneven work
  // per item -- windows, masks -- the dispatcher's own balancing wins).
  constexpr bool PERSIST = CAUSAL && !WINDOW && !BITS && !SPLIT;
  const int64_t n_items = (int64_t)n_qtiles * p.B * p.H * (SPLIT ? sp.splits : 1);
  const int xcd = blockIdx.x % kNumXcd, u = blockIdx.x / kNumXcd, W = gridDim.x / kNumXcd;
  const int64_t qx = n_items / kNumXcd, rx = n_items % kNumXcd;
  const int64_t x_start = xcd * qx + (xcd < rx ? xcd : rx), x_count = qx + (xcd < rx ? 1 : 0);
  // CONT: the same walk, as one software pipeline: the body below starts with
  // the workgroup's first item and runs into each next item without draining
  // (no kv_len, so every (batch, head) has M keys; the launcher checks that
  // every item visits at least 4 key tiles).
  for (int64_t k = 0;; ++k) {
    int64_t logical;
    if constexpr (CONT) {
      if (k > 0 || u >= x_count) break;
      // with a mask, the pre-pass's order (the range sorted by tile count)
      logical = x_start + (BITS ? walk_order[x_start + u] : u);
    } else if constexpr (PERSIST) {
      const int64_t within = k * W + ((k & 1) ? W - 1 - u : u);
      if (within >= x_count) break;
      logical = x_start + within;
      // the previous item's loads into LDS (some past its last tile) have
      // landed, and every wave is done reading
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    } else {
      if (k > 0) break;
      logical = xcd_logical(blockIdx.x, gridDim.x);
    }
  {
    const int split = SPLIT ? (int)(logical % sp.splits) : 0;  // key chunk
    const int64_t item = SPLIT ? logical / sp.splits : logical;
    int qt = (int)(item % n_qtiles);
    int64_t bh = item / n_qtiles;  // (CONT: of the current item, as qw0, Qg, Kg, Vg, n_tiles)
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // heaviest query tiles first
    const int b = (int)(bh / p.H);
    const int N = p.N, M = p.M;
    const int tid = threadIdx.x;
    const int lane = tid % 64, hl = lane / 32, ql = lane % 32;
    const int ws = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index (uniform)
    // uniform in fact; readfirstlane lets the compiler keep it (and every tile
    // descriptor built from it) in scalar registers
    const int kvl = __builtin_amdgcn_readfirstlane(clamp_kv(p.kv_len, b, M));
    const int q0 = qt * BQ;
    int qw0 = q0 + QW * ws;  // first query of this wave
    const int off = kvl - N;       // key j visible to query i iff j < kvl and (!causal or j <= i + off)
    // Local window: query i sees keys i + off - wl .. i + off + wr only; causal
    // caps wr at 0.  (Clamped so that no bound overflows.)
    constexpr bool UPPER = CAUSAL || WINDOW;   // rows have a last key before kvl - 1
    const int wl = WINDOW ? min(p.wl, N + kvl) : 0;
    const int wr = CAUSAL ? 0 : (WINDOW ? min(p.wr, N + kvl) : 0);
    const int q_last = min(q0 + BQ, N) - 1;
    // Keys past kend are not this workgroup's: kv_len, or the end of its key
    // chunk (the causal alignment off stays that of kv_len).
    const int kend = SPLIT ? min(kvl, (split + 1) * sp.split_tiles * BK) : kvl;
    const int kv_end = UPPER ? min(kend, q_last + off + wr + 1) : kend;
    // Window: tiles before the first query's first key are never visited.
    // Without a mask the K/V descriptors start at that tile, t0, and the loop
    // counts tiles from there; with a mask the loop walks the listed tiles in
    // [tw, t_end) and tiles are addressed from 0.
    const int tw = WINDOW ? max(0, q0 + off - wl) / BK : (SPLIT ? split * sp.split_tiles : 0);
    const int t_end = kv_end > tw * BK ? (kv_end + BK - 1) / BK : tw;
    int t0 = BITS ? 0 : tw;  // (CONT: of the current item)
    int n_tiles = t_end - tw;
    int lo = 0;  // with a mask: list position of the first tile visited
    if constexpr (CONT && BITS) {
      // The workgroup's items in walk order and their tiles, one stream: the
      // pre-pass cut each list at the causal limit and filled it up to 4
      // tiles, so a list holds exactly the item's visited tiles.  Past the
      // last item, 5 entries one past kv_len (zeros, all masked).
      __shared__ int walk_off[kWalkMaxItems + 1];
      __shared__ int walk_list[kWalkMaxItems];
      int n_wk = 0;
      while (n_wk < kWalkMaxItems) {
        const int64_t within = (int64_t)n_wk * W + ((n_wk & 1) ? W - 1 - u : u);
        if (within >= x_count) break;
        ++n_wk;
      }
      if (tid < n_wk) {
        const int64_t within = (int64_t)tid * W + ((tid & 1) ? W - 1 - u : u);
        const int64_t it = x_start + walk_order[x_start + within];
        walk_item[tid] = (int)it;
        const int qt_i = n_qtiles - 1 - (int)(it % n_qtiles);
        const int64_t bh_i = it / n_qtiles;
        const int bm = p.mask_b > 1 ? (int)(bh_i / p.H) : 0, hm = p.mask_h > 1 ? (int)(bh_i % p.H) : 0;
        const int li = (int)(((int64_t)(bm * p.mask_h + hm) * n_qtiles + qt_i) * list_stride);
        walk_list[tid] = li;
        walk_n[tid] = tile_lists[li];
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < n_wk; ++i) {
          walk_off[i] = acc;
          acc += walk_n[i];
        }
        walk_off[n_wk] = acc;
      }
      __syncthreads();
      const int total = walk_off[n_wk];
      for (int j = tid; j < total + 5; j += kPrefillThreads) {
        int e = (kvl + BK - 1) / BK;
        if (j < total) {
          int i = 0;
          while (walk_off[i + 1] <= j) ++i;
          e = tile_lists[walk_list[i] + 1 + (j - walk_off[i])];
        }
        tlist[j] = e;
      }
      __syncthreads();
      n_tiles = __builtin_amdgcn_readfirstlane(walk_n[0]);
    } else if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int32_t* L = tile_lists + ((int64_t)(bm * p.mask_h + hm) * n_qtiles + qt) * list_stride;
      const int cnt = __builtin_amdgcn_readfirstlane(L[0]);
      for (int i = tid; i < cnt; i += kPrefillThreads) tlist[i] = L[1 + i];
      __syncthreads();
      // the list ascends: count the entries below tw and below t_end
      int below_lo = 0, below_hi = 0;
      for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int e = i0 + lane < cnt ? (tlist[i0 + lane] & 0x7FFFFFFF) : 0x7FFFFFFF;
        below_lo += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < tw));
        below_hi += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e < t_end));
      }
      lo = __builtin_amdgcn_readfirstlane(below_lo);
      n_tiles = __builtin_amdgcn_readfirstlane(below_hi) - lo;
      __syncthreads();  // every wave has read the list
      // after the last visited tile: one past kv_len, whose loads read zeros
      // and whose keys are all masked (lo + n_tiles <= cnt < kMaskMaxTiles)
      if (tid == 0) tlist[lo + n_tiles] = (kvl + BK - 1) / BK;
      __syncthreads();
    }
    // Entry of the t-th visited tile: its index (relative to t0), with bit 31
    // set when the mask does not keep it whole.  Without a mask, t itself.
    int gb = 0;  // CONT with a mask: stream position of the current item's first tile
    auto tile_entry = [&](int t) -> int {
      if constexpr (CONT && BITS) return __builtin_amdgcn_readfirstlane(tlist[gb + t]);
      else if constexpr (BITS) return __builtin_amdgcn_readfirstlane(tlist[lo + min(t, n_tiles)]);
      else return t;
    };
    auto tile_index = [&](int e) -> int { return BITS ? (e & 0x7FFFFFFF) : e; };

    const __bf16* Qg = (const __bf16*)p.q + (size_t)bh * N * D;
    const __bf16* Kg = (const __bf16*)p.k + (size_t)bh * M * D + (size_t)t0 * BK * D;
    const __bf16* Vg = (const __bf16*)p.v + (size_t)bh * M * D + (size_t)t0 * BK * D;
    // CONT: the item after the current one in the walk (has_nx false past the
    // last), round kw being the current one's.  Every item has at least 4
    // tiles (the launcher checks).
    // CONT: byte offset of an item's row of blocks among all rows
    auto mask_row = [&](int64_t bhx, int qtx) -> int {
      const int bm = p.mask_b > 1 ? (int)(bhx / p.H) : 0, hm = p.mask_h > 1 ? (int)(bhx % p.H) : 0;
      return (int)(((int64_t)(bm * p.mask_h + hm) * n_qtiles + qtx) * list_stride * kMaskBlockBytes);
    };
    int64_t kw = 0, bh_n = 0;
    bool has_nx = false;
    int qw0_n = 0, n_n = 0, t0_n = 0, mrow_n = 0;
    const __bf16 *Qg_n = nullptr, *Kg_n = nullptr, *Vg_n = nullptr;
    // Round k of a causal walk pairs heavy and light query tiles (above);
    // with a window the items are nearly equal but for a head's first query
    // tiles, and round k takes item k W + (u + k S) mod W (S = W / 8), so
    // that each workgroup's rounds step through the query tiles and meet the
    // short ones as often as any other workgroup.
    auto walk_next = [&]() {
      const int64_t kn = kw + 1;
      const int64_t within = kn * W + (CAUSAL && !WINDOW ? ((kn & 1) ? W - 1 - u : u)
                                                         : (u + kn * max(1, W / 8)) % W);
      has_nx = within < x_count;
      const int64_t it = BITS ? (has_nx ? (int64_t)walk_item[kw + 1] : x_start) : x_start + (has_nx ? within : 0);
      int qt_n = (int)(it % n_qtiles);
      if (CAUSAL) qt_n = n_qtiles - 1 - qt_n;
      bh_n = it / n_qtiles;
      // the item's tiles, as for the current item above (kv_len = M)
      const int q0_n = qt_n * BQ, ql_n = min(q0_n + BQ, N) - 1;
      const int kv_end_n = UPPER ? min(kend, ql_n + off + wr + 1) : kend;
      t0_n = WINDOW ? max(0, q0_n + off - wl) / BK : 0;
      n_n = (kv_end_n > t0_n * BK ? (kv_end_n + BK - 1) / BK : t0_n) - t0_n;
      qw0_n = q0_n + QW * ws;
      if constexpr (BITS) {
        // the pre-pass's list of the item holds exactly its tiles
        n_n = has_nx ? __builtin_amdgcn_readfirstlane(walk_n[kw + 1]) : 0;
        mrow_n = mask_row(bh_n, qt_n);
      }
      Qg_n = (const __bf16*)p.q + (size_t)bh_n * N * D;
      Kg_n = (const __bf16*)p.k + (size_t)bh_n * M * D + (size_t)t0_n * BK * D;
      Vg_n = (const __bf16*)p.v + (size_t)bh_n * M * D + (size_t)t0_n * BK * D;
    };
    if constexpr (CONT) walk_next();

    // ---- tile loads ----
    // Slot s of a padded tile holds row s / CH, chunk s % CH; slots on the
    // padding (chunk >= CPR) load chunk 0 of that row (valid data, never read).
    // Wave ws loads blocks ws, ws + NW, ... of each tile.  The per-lane byte
    // offsets of a wave's slots within a tile (< 64 KB) are fixed, so they are
    // computed once and kept two to a register.  Loads are buffer loads into
    // LDS against one descriptor per (batch, head) that ends at kv_len: rows
    // past it (last tile) and whole tiles past it read as zeros -- finite data
    // whose weights are 0 -- with no clamping arithmetic, and the descriptors
    // stay in 8 scalar registers for the whole kernel.  (Buffer rather than
    // global loads also keep the compiler's LDS wait counting exact: it treats
    // a global load into LDS like a flat access and then waits for every LDS
    // read.)
    constexpr int NMI = BITS ? 2 : 0;  // mask load items (one per word of a row's tile)
    constexpr int NITEM = KPW + VPW + NMI;  // load items per wave per iteration
    constexpr int ROWB = D * 2;       // bytes per global row
    static_assert((NW * KPW * 64 / KCH + 1) * ROWB <= 65536 && (NW * VPW * 64 / VCH + 1) * ROWB <= 65536,
                  "slot offsets fit 16 bits");
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
    // Lane's slot offset (half `hi` of a packed pair) plus a wave-uniform byte
    // offset, as one instruction next to the load that uses it (the volatile
    // asm also keeps the compiler from unpacking every offset once, outside
    // the loop, into registers of their own).
    auto slot_plus = [&](uint32_t packed, int hi, int add) -> uint32_t {
      uint32_t v;
      if (hi)
        asm volatile("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
                     : "=v"(v) : "v"(packed), "s"(add));
      else
        asm volatile("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
                     : "=v"(v) : "v"(packed), "s"(add));
      return v;
    };
    // Byte offset of the wave's first block in an LDS tile buffer, passed
    // through an empty asm once per iteration (relaunder_wofs), so that each
    // load forms its LDS address (M0) with one add next to it instead of the
    // compiler keeping all of them (three buffers x NITEM blocks) in scalar
    // registers across the loop.
    int wofs_it = ws * 1024;
    auto relaunder_wofs = [&]() {
      wofs_it = ws * 1024;
      asm volatile("" : "+s"(wofs_it));
    };
    // K and V bytes this (batch, head) may read; the planner keeps M * D * 2
    // below 2^31, so every offset below fits 32 bits.
    const int nrec = (SPLIT ? max(kend - t0 * BK, 0) : kend - t0 * BK) * ROWB;
    // Block i of this wave: its slots of tile t of src into dst.  The wave's
    // block offset goes through an empty asm so that the compiler forms each
    // LDS address next to its load instead of keeping all of them (three
    // buffers x NITEM blocks) in scalar registers.
    auto load_block = [&](const __bf16* src, int t, __bf16* dst, uint32_t packed, int i) {
      const uint32_t u = slot_plus(packed, i % 2, t * (BK * ROWB));
      buffer_load_lds16(src, nrec, u, (lds_ptr)((char*)dst + wofs_it + i * NW * 1024));
    };
    auto load_k_item = [&](int i, int t, __bf16* dst, const __bf16* src) { load_block(src, t, dst, koff[i / 2], i); };
    auto load_v_item = [&](int i, int t, __bf16* dst, const __bf16* src) { load_block(src, t, dst, voff[i / 2], i); };
    // Mask word w of key tile t for the wave's 64 query rows (lane = row):
    // from the tile's block of the query tile's blocks (the pre-pass copied
    // rows past N from row N - 1), 256 contiguous bytes per wave and word,
    // one 4-byte buffer load per lane into LDS.
    const uint32_t* Mg = nullptr;
    int mbytes = 0;
    uint32_t mlane = 0;
    int mrow_c = 0;
    if constexpr (BITS) {
      const int bm = p.mask_b > 1 ? b : 0, hm = p.mask_h > 1 ? (int)(bh % p.H) : 0;
      const int n_kt = list_stride - 1;  // tile t has block t + 1
      Mg = mask_blocks + ((size_t)(bm * p.mask_h + hm) * n_qtiles + qt) * (n_kt + 1) * (kMaskBlockBytes / 4);
      mbytes = (n_kt + 1) * kMaskBlockBytes;
      mlane = (uint32_t)(ws * 512 + lane * 4);
      if constexpr (CONT) mrow_c = mask_row(bh, qt);
    }
    // A tile the mask keeps whole (entry e >= 0) has no block and never reads
    // its words: its load still goes out (the end-of-iteration wait counts
    // every load) but from offset 0 (the all-ones block).  CONT: one
    // descriptor over every row of blocks (below 2^31 bytes), mrow the byte
    // offset of the tile's item's row.
    const int nrec_m = CONT && BITS ? p.mask_b * p.mask_h * n_qtiles * list_stride * kMaskBlockBytes : 0;
    auto load_mask_item = [&](int w, int e, uint32_t* dst, int mrow) {
      if constexpr (BITS) {
        int wofs = ws * 128 + w * 64;
        asm volatile("" : "+s"(wofs));
        const uint32_t part = (uint32_t)(e >> 31);  // all ones for a partial tile
        const uint32_t at =
            ((uint32_t)(tile_index(e) + 1) * (uint32_t)kMaskBlockBytes + mlane + (uint32_t)w * 256u) & part;
        if constexpr (CONT) buffer_load_lds4<true>(mask_blocks, nrec_m, at + (uint32_t)mrow, (lds_ptr)(dst + wofs));
        else buffer_load_lds4<true>(Mg, mbytes, at, (lds_ptr)(dst + wofs));
      }
    };
    auto load_k = [&](int t, __bf16* dst) {
  #pragma unroll
      for (int i = 0; i < KPW; ++i) load_k_item(i, t, dst, Kg);
    };
    auto load_v = [&](int t, __bf16* dst) {
  #pragma unroll
      for (int i = 0; i < VPW; ++i) load_v_item(i, t, dst, Vg);
    };
    auto load_mask = [&](int e, uint32_t* dst) {
  #pragma unroll
      for (int w = 0; w < NMI; ++w) load_mask_item(w, e, dst, mrow_c);
    };
    // Load item j of iteration t: K(t+4) blocks into Kdst, then V(t+2) blocks
    // into Vdst, then (mask) the mask words of tile t+3 into Mdst; eK, eV, eM
    // are those tiles' entries (tiles past the last read as zeros), Ksrc and
    // Vsrc the (batch, head) they belong to.
    // CONT: one descriptor per tensor (all heads, below 2^31 bytes), so that
    // tiles of the current and the next item differ only in the offset.
    const int nrec_all = CONT ? p.B * p.H * M * ROWB : 0;
    auto load_item = [&](int j, int eK, int eV, int eM, __bf16* Kdst, __bf16* Vdst, uint32_t* Mdst,
                         const __bf16* Ksrc, const __bf16* Vsrc, int mrow) {
      if constexpr (CONT) {
        if (j >= KPW + VPW) {
          load_mask_item(j - KPW - VPW, eM, Mdst, mrow);
          return;
        }
        const uint32_t packed = j < KPW ? koff[j / 2] : voff[(j - KPW) / 2];
        const int i = j < KPW ? j : j - KPW;
        const uint32_t u = slot_plus(packed, i % 2, j < KPW ? eK : eV);
        buffer_load_lds16(j < KPW ? (const void*)p.k : (const void*)p.v, nrec_all, u,
                          (lds_ptr)((char*)(j < KPW ? Kdst : Vdst) + wofs_it + i * NW * 1024));
        return;
      }
      if (j < KPW) load_k_item(j, tile_index(eK), Kdst, Ksrc);
      else if (j < KPW + VPW) load_v_item(j - KPW, tile_index(eV), Vdst, Vsrc);
      else if (j < NITEM) load_mask_item(j - KPW - VPW, eM, Mdst, 0);
    };

    // ---- Q in registers: B operand of S^T = K Q^T ----
    // Fragment (qb, kb): lane (h, c) holds Q[qw0 + 32 qb + c][16 kb + 8 h .. + 8].
    // Rows past N hold a copy of row N - 1 (finite, never written out).
    bf16x8 qf[NQB][DK];
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = min(qw0 + 32 * qb + ql, N - 1);
      if constexpr (CONT) {
        // straight into the AGPRs that the pipeline reloads for each next
        // item (waited for before the first S MFMAs)
  #pragma unroll
        for (int kb = 0; kb < DK; ++kb)
          asm volatile("global_load_dwordx4 %0, %1, off offset:%2"
                       : "=a"(qf[qb][kb]) : "v"(Qg + (size_t)row * D + hl * 8), "n"(kb * 32) : "memory");
      } else {
  #pragma unroll
        for (int kb = 0; kb < DK; ++kb) qf[qb][kb] = *(const bf16x8*)(Qg + (size_t)row * D + kb * 16 + hl * 8);
      }
    }

    // Per-lane base offsets (elements) of the operand reads.
    const int kbase = ql * KROW + hl * 8;   // + (32 nb) KROW + 16 kb
    const int vbase = (4 * hl + (lane % 16) / 4) * VROW + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
                                            // + (32 nb + 16 t2) VROW + 32 db, + 8 VROW for the upper 4 keys

    // K fragment i (kb-major): rows 32 nb .. + 32, columns 16 kb .. + 16.
    auto fetch_k = [&](const __bf16* Ks, int i) -> bf16x8 {
      const int kb = i / NKB, nb = i % NKB;
      return *(const bf16x8*)(Ks + kbase + nb * 32 * KROW + kb * 16);
    };
    // V^T fragment i = (nb, t2, db), db fastest.  B operand slot 8*hl + e of
    // 16-key block (nb, t2) is key 32 nb + 16 t2 + 8 (e / 4) + 4 hl + e % 4 (the
    // order in which the score layout hands the weights over); the A operand
    // for the same slots comes from two transposing reads of 4 consecutive keys
    // each: within a 16-lane group, lane j reads row kbase + j / 4 at column
    // dsrc + 4 (j % 4), and lane i receives the 4 keys at column dsrc + i.
    auto fetch_v = [&](const __bf16* Vs, int i) -> bf16x8 {
      const int nb = i / (2 * DB), t2 = (i / DB) % 2, db = i % DB;
      const __bf16* a = Vs + vbase + (nb * 32 + t2 * 16) * VROW + db * 32;
      const s16x4 lo = lds_read_tr16(a);
      const s16x4 hi = lds_read_tr16(a + 8 * VROW);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 oacc[DB][NQB];
  #pragma unroll
    for (int db = 0; db < DB; ++db)
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) oacc[db][qb] = f32x16{};
    f32x16 sacc[NKB][NQB];  // score tile: S(t+1), then S(t+2), during iteration t
    bf16x8 pacc[NQB][NP];   // weight tile: P(t), then P(t+1), during iteration t
    float m_run[NQB], l_run[NQB];  // reference max (base 2), this lane's part of the sum
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
    }
    // A scale of 0 would turn a masked -inf score into NaN (-inf * 0); a floor
    // of 1e-30 changes the weights of finite scores by less than 1e-20.
    const float c = fmaxf(p.scale * kLog2e, 1e-30f);

    // Tiles that cross the diagonal or the kv_len boundary -- and tiles past
    // the workgroup's last one, whose LDS holds stale data -- are masked
    // element by element; every other tile is fully visible to the wave.
    // qwx, t0x: the wave's first query and the first tile of the tile's
    // work item.
    auto need_mask = [&](int e, int qwx, int t0x) {
      const int k0 = (tile_index(e) + t0x) * BK;
      return (BITS && e < 0) | (k0 + BK > kend) | (UPPER && k0 + BK - 1 > qwx + off + wr) |
             (WINDOW && k0 < qwx + QW - 1 + off - wl);
    };

    // ---- softmax of one tile, in small units that the pipeline spreads out ----
    // The weights of a tile are formed against the current reference m with no
    // row max at all: the pages subtract the max only to keep the exponentials
    // finite, and any reference that keeps every weight at most 2^20 (sums of
    // a million keys stay far inside float32) gives the same l, O and L.  A
    // weight above that shows in the lane's sum of the tile's weights, so two
    // cheap checks replace the max:
    //   EM units (key block 0): weight, sum and bf16 weight of 2 scores;
    //   check 1 (after the EM units and the P V products of the previous tile,
    //     block-0 scores intact): a lane's block-0 sum above 2^20, or a row
    //     with no reference yet (m = -inf) that sees a key of block 0, moves
    //     the reference up to block 0's row max (rare): l and the output
    //     accumulator are rescaled and key block 0 is computed again;
    //   EX units (key block 1): as EM;
    //   check 2 (after the EX units, block-1 scores intact): the same for the
    //     whole tile's sum and block 1 (rarer still): l, the output
    //     accumulator and block 0's weights and sum are rescaled and key block
    //     1 is computed again.
    // Once a row has a reference, its l is at least 1 (the key that set it
    // weighs exactly 1), so weights that underflow are negligible.  Each score
    // is read from the accumulator once and consumed at once.
    constexpr int NU_EM = NQB * 8, NU_EX = NQB * 8;
    constexpr float kSumLimit = 1048576.0f;  // 2^20
    float m_use[NQB], ps0[NQB][2], ps1[NQB][2];  // reference in use; block 0 and block 1 sums
    bool vis[NKB][NQB];  // the row sees a key of key block nb
    auto sm_begin = [&]() {
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        ps0[qb][0] = ps0[qb][1] = ps1[qb][0] = ps1[qb][1] = 0.f;
        m_use[qb] = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      }
    };
    // weights of 2 scores (pair `pair` of 16-key half t2 of key block nb);
    // `first`: the pair starts the lane's sums of the block (they were 0, and
    // 0 + w is w for the weights, which are never -0); not used with a mask,
    // where the changed code makes the allocator spill more at D = 128
    auto exp_pair = [&](f32x16 (&s)[NKB][NQB], int nb, int qb, int t2, int pair, bool first = false) {
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 2 * pair + h, r = (2 * t2 + e / 4) * 4 + (e % 4);
        const float pv = fast_exp2(fmaf(s[nb][qb][r], c, -m_use[qb]));
        if (first) (nb == 0 ? ps0 : ps1)[qb][h] = pv;
        else (nb == 0 ? ps0 : ps1)[qb][h] += pv;
        pacc[qb][nb * 2 + t2][e] = (__bf16)pv;
      }
    };
    // EM unit u: t2-major, so that the units of the first 16-key half come
    // first (the P V products release that half of the weight tile first)
    auto unit_em = [&](f32x16 (&s)[NKB][NQB], auto uc) {
      constexpr int u = decltype(uc)::value, t2 = u / 8, qb = (u / 4) % 2, pair = u % 4;
      exp_pair(s, 0, qb, t2, pair, !BITS && t2 == 0 && pair == 0);
    };
    auto unit_ex = [&](f32x16 (&s)[NKB][NQB], auto uc) {
      constexpr int u = decltype(uc)::value, qb = u / 8, t2 = (u / 4) % 2, pair = u % 4;
      exp_pair(s, 1, qb, t2, pair, !BITS && t2 == 0 && pair == 0);
    };
    // Move row qb's reference to mx (its new row max, base 2): returns the
    // factor e^(m_old - m_new) for everything accumulated so far.
    // Only the rows that ask for it move (trig); the others keep their
    // reference (factor 1).  A row that moves from -inf has accumulated
    // nothing (factor 0 on zeros), so the output accumulator is rescaled only
    // when some row with a reference moves it up (rescale_acc).  Both half-waves
    // hold every row and must take the same decision: trig is combined over
    // the pair first.
    auto row_any = [&](bool x) -> bool {
      const uint32_t v = x ? 1u : 0u;
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (r[0] | r[1]) != 0u;
    };
    auto move_ref = [&](int qb, float mx, bool trig, bool& moved_up) -> float {
      const float m_new = trig ? fmaxf(m_run[qb], mx) : m_run[qb];
      const float a = m_run[qb] == -INFINITY ? 0.f : fast_exp2(m_run[qb] - m_new);  // nothing accumulated yet
      moved_up = (m_run[qb] != -INFINITY) & (m_new > m_run[qb]);
      l_run[qb] *= a;
      m_run[qb] = m_new;
      m_use[qb] = m_new == -INFINITY ? 0.f : m_new;
      return a;
    };
    auto rescale_acc = [&](const float (&a)[NQB]) {
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
        for (int db = 0; db < DB; ++db) {
          // read inside the branch, in place: no copy of the accumulator
          // outside it
          asm volatile("" : "+a"(oacc[db][qb]));
          oacc[db][qb] *= a[qb];
        }
    };
    // qwait (CONT): Q was just reloaded for the S MFMAs that follow; the rare
    // path is taken to wait for the loads there (its recomputation of a block
    // whose rows keep their reference reproduces the same weights and sum).
    auto sm_check1 = [&](f32x16 (&s)[NKB][NQB], bool qwait) __attribute__((always_inline)) {
      if constexpr (CONT && !BITS) {
        if (qwait) {
          // the reloaded Q is read by the S MFMAs that follow: wait for its
          // loads, and tie the wait to the Q registers so that no MFMA moves
          // above it
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
            for (int kb = 0; kb < DK; ++kb) asm volatile("" : "+a"(qf[qb][kb]));
        }
      }
      bool over = CONT && BITS && qwait;
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        over |= (ps0[qb][0] + ps0[qb][1] > kSumLimit) | ((m_run[qb] == -INFINITY) & vis[0][qb]);
      if (__builtin_amdgcn_ballot_w64(over) != 0) {  // wave-uniform, rare
        if constexpr (CONT && BITS) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        float a[NQB];
        bool up = false;
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const bool trig = row_any(ps0[qb][0] + ps0[qb][1] > kSumLimit) |
                            ((m_run[qb] == -INFINITY) & vis[0][qb]);
          float mx = -INFINITY;
  #pragma unroll
          for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[0][qb][r], s[0][qb][r + 1]);
          bool moved_up;
          a[qb] = move_ref(qb, swap_halves_max(mx) * c, trig, moved_up);  // -inf stays -inf (c > 0)
          up |= moved_up;
          ps0[qb][0] = ps0[qb][1] = 0.f;
        }
        if (__builtin_amdgcn_ballot_w64(up) != 0) rescale_acc(a);
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
  #pragma unroll
            for (int pair = 0; pair < 4; ++pair) exp_pair(s, 0, qb, t2, pair);
      }
    };
    // fresh: the tile is its work item's first; the output accumulator still
    // holds the previous item's output (CONT), and this item's is zero, so it
    // is not rescaled.
    auto sm_check2 = [&](f32x16 (&s)[NKB][NQB], bool fresh) __attribute__((always_inline)) {
      bool over = false;
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        over |= (ps0[qb][0] + ps0[qb][1] + ps1[qb][0] + ps1[qb][1] > kSumLimit) |
                ((m_run[qb] == -INFINITY) & vis[1][qb]);
      if (__builtin_amdgcn_ballot_w64(over) != 0) {  // wave-uniform, rarer still
        float a[NQB];
        bool up = false;
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const bool trig = row_any(ps0[qb][0] + ps0[qb][1] + ps1[qb][0] + ps1[qb][1] > kSumLimit) |
                            ((m_run[qb] == -INFINITY) & vis[1][qb]);
          float mx = -INFINITY;
  #pragma unroll
          for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[1][qb][r], s[1][qb][r + 1]);
          bool moved_up;
          a[qb] = move_ref(qb, swap_halves_max(mx) * c, trig, moved_up);
          up |= moved_up;
          ps0[qb][0] *= a[qb];
          ps0[qb][1] *= a[qb];
  #pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
  #pragma unroll
            for (int e = 0; e < 8; ++e) pacc[qb][t2][e] = (__bf16)((float)pacc[qb][t2][e] * a[qb]);
          ps1[qb][0] = ps1[qb][1] = 0.f;
        }
        if (!fresh && __builtin_amdgcn_ballot_w64(up) != 0) rescale_acc(a);
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
  #pragma unroll
            for (int pair = 0; pair < 4; ++pair) exp_pair(s, 1, qb, t2, pair);
      }
    };
    auto sm_end = [&]() {
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) l_run[qb] += (ps0[qb][0] + ps0[qb][1]) + (ps1[qb][0] + ps1[qb][1]);
    };
    // Results computed so far must exist here: an empty statement that reads
    // them keeps the compiler from sinking their arithmetic past the branch
    // that follows (which would pull it out of the interleaved block).
    auto pin_weights = [&](int nb) {
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        asm volatile("" ::"v"(pacc[qb][nb * 2]), "v"(pacc[qb][nb * 2 + 1]));
        asm volatile("" ::"v"(ps0[qb][0]), "v"(ps0[qb][1]), "v"(ps1[qb][0]), "v"(ps1[qb][1]));
      }
    };
    // Scores of keys past a row's last visible key become -inf.  The select is
    // a sign mask and a bit insert, not a compare: a compare per score writes a
    // scalar register pair, and the compiler would keep dozens of them live.
    // With a mask, Ms holds the tile's mask words and key 8 (r / 4) + 4 hl + r % 4
    // of key block nb is bit 8 (r / 4) + r % 4 of this lane's word shifted down
    // by 4 hl.
    auto apply_mask = [&](int e, int qwx, int t0x, f32x16 (&s)[NKB][NQB], const uint32_t* Ms) {
      const int k0 = (tile_index(e) + t0x) * BK;
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qrow = qwx + 32 * qb + ql;
        const int lim = UPPER ? min(kend - 1, qrow + off + wr) : kend - 1;  // last visible key
        const int lo = qrow + off - wl;                                   // first (window)
        uint32_t hid[NKB];  // masked-out keys of the row's two key blocks (bit set)
  #pragma unroll
        for (int nb = 0; nb < NKB; ++nb) {
          vis[nb][qb] = lim >= k0 + 32 * nb && (!WINDOW || lo <= k0 + 32 * nb + 31);
          if constexpr (BITS) {
            // a tile the mask keeps whole has no words in LDS: all ones
            const uint32_t w = Ms[ws * 128 + nb * 64 + 32 * qb + ql] | ~(uint32_t)(e >> 31);
            vis[nb][qb] = vis[nb][qb] && w != 0u;  // a hint: a false "sees" only costs time
            hid[nb] = ~w >> (4 * hl);
          }
        }
        const int base = lim - (k0 + 4 * hl);  // >= 0 iff key k0 + 4 hl is visible
        const int base_lo = k0 + 4 * hl - lo;  // >= 0 iff key k0 + 4 hl is past the window start
  #pragma unroll
        for (int nb = 0; nb < NKB; ++nb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int idx = nb * 32 + 8 * (r / 4) + (r % 4);
            uint32_t hide = (uint32_t)((base - idx) >> 31);
            if constexpr (WINDOW) hide |= (uint32_t)((base_lo + idx) >> 31);
            if constexpr (BITS) hide |= (uint32_t)__builtin_amdgcn_sbfe((int)hid[nb], 8 * (r / 4) + r % 4, 1);
            const uint32_t v = __float_as_uint(s[nb][qb][r]);
            s[nb][qb][r] = __uint_as_float((hide & 0xFF800000u) | (~hide & v));
          }
      }
    };
    // Whole softmax of the tile with entry e (prologue only).
    auto softmax_all = [&](int e, f32x16 (&s)[NKB][NQB], const uint32_t* Ms) {
      mfma_guard();  // compute_s just wrote the scores
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) vis[0][qb] = vis[1][qb] = true;
      if (need_mask(e, qw0, t0)) apply_mask(e, qw0, t0, s, Ms);
      sm_begin();
      static_for<NU_EM>([&](auto uc) { unit_em(s, uc); });
      sm_check1(s, false);
      static_for<NU_EX>([&](auto uc) { unit_ex(s, uc); });
      sm_check2(s, false);
      sm_end();
    };
    // S^T = K Q^T for one tile, not interleaved (prologue only).
    auto compute_s = [&](const __bf16* Ks, f32x16 (&s)[NKB][NQB]) {
  #pragma unroll
      for (int i = 0; i < NF; ++i) {
        const bf16x8 kf = fetch_k(Ks, i);
        const int kb = i / NKB, nb = i % NKB;
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          if (kb == 0) mfma_s_first_safe(s[nb][qb], kf, qf[qb][kb]);
          else mfma_s_acc_safe(s[nb][qb], kf, qf[qb][kb]);
        }
      }
    };

    // ---- one pipelined iteration ----
    // Work of iteration t: O += P(t) V(t), the softmax of S(t+1) into P(t+1),
    // S(t+2) = K(t+2) Q^T.  One score and one weight tile suffice because the
    // steps run in three phases, one MFMA per step:
    //   A: the P V MFMAs (fragment j / 2, query block j % 2), with the EM
    //      units; then check 1;
    //   B: the S MFMAs of key block 0 -- whose scores have been consumed --
    //      with the EX units; then check 2;
    //   C: the S MFMAs of key block 1, with the tile loads.
    // Operands are read PF fragments ahead; tile load item k goes at step
    // 3k + 1 (measured: spreading them over all steps gains nothing).
    constexpr int PF = 2;
    constexpr int NSA = 2 * NF, NSB = NQB * DK;  // steps of phases A and B (C = B)
    // Ksrc, Vsrc: the (batch, head) of the tiles loaded (CONT: eK and eV are
    // the byte offsets of the tiles in the whole K and V, Ksrc and Vsrc
    // unused); fresh: S(t+1) is its work item's first tile; qwait: Q was just
    // reloaded for S(t+2) (CONT), and its loads are waited for before phase B.
    auto iteration = [&](int eK, int eV, int eM, const __bf16* Ks, const __bf16* Vs, __bf16* Kdst,
                         __bf16* Vdst, uint32_t* Mdst, const __bf16* Ksrc, const __bf16* Vsrc, bool fresh,
                         bool qwait, int mrow) {
      relaunder_wofs();
      sm_begin();
      // K operands: a ring of PF + 2, so that a read overwrites a register two
      // fragments after the asm MFMAs last used it
      constexpr int KR = PF + 2;
      bf16x8 vr[PF + 1], kr[KR];
  #pragma unroll
      for (int i = 0; i < PF; ++i) vr[i] = fetch_v(Vs, i);
      // phase A
      static_for<NSA>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        constexpr int i = j / 2, qb = j % 2;
        constexpr int nb = i / (2 * DB), t2 = (i / DB) % 2, db = i % DB;
        oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % (PF + 1)], pacc[qb][nb * 2 + t2],
                                                              oacc[db][qb], 0, 0, 0);
        if constexpr (qb == 0 && i + PF < NF) vr[(i + PF) % (PF + 1)] = fetch_v(Vs, i + PF);
        // EM units over the last three quarters of the steps: an EM unit of
        // 16-key half t2 overwrites weight fragment t2 of P(t), which the P V
        // MFMAs of fragment t2 (steps 2 DB t2 .. + 2 DB) read first
        constexpr int Q1 = NSA / 4;
        if constexpr (j >= Q1) {
          constexpr int W = NSA - Q1;
          constexpr int u0 = ((j - Q1) * NU_EM + W - 1) / W, u1 = ((j - Q1 + 1) * NU_EM + W - 1) / W;
          static_for<u1 - u0>([&](auto uc) {
            constexpr int u = u0 + decltype(uc)::value;
            static_assert(j >= 2 * DB * (u / (NU_EM / 2) + 1), "EM unit after the P V MFMAs of its fragment");
            unit_em(sacc, std::integral_constant<int, u>{});
          });
        }
        // the first K operands of phase B, during the last steps of phase A
        if constexpr (j >= NSA - PF) kr[j - (NSA - PF)] = fetch_k(Ks, (j - (NSA - PF)) * NKB);
      });
      __builtin_amdgcn_sched_barrier(0);
      pin_weights(0);
      sm_check1(sacc, qwait);
      // phases B and C: S fragments (kb, nb) in order nb-major, kb, query block
      static_for<2 * NSB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j == NSB) {
          // check 2, before phase C overwrites key block 1's scores
          pin_weights(1);
          sm_check2(sacc, fresh);
          __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int f = j / NQB, qb = j % NQB;     // f-th S fragment of this iteration
        constexpr int nb = f / DK, kb = f % DK;
        if constexpr (kb == 0) mfma_s_first(sacc[nb][qb], kr[f % KR], qf[qb][kb]);
        else mfma_s_acc(sacc[nb][qb], kr[f % KR], qf[qb][kb]);
        if constexpr (qb == 0 && f + PF < NF) {
          constexpr int f2 = f + PF;
          kr[f2 % KR] = fetch_k(Ks, (f2 % DK) * NKB + f2 / DK);
        }
        // tile loads in phase C, which carries no VALU work: item i at step
        // NSB + i NSB / NITEM
        if constexpr (j >= NSB) {
          static_for<NITEM>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (NSB + i * NSB / NITEM == j) load_item(i, eK, eV, eM, Kdst, Vdst, Mdst, Ksrc, Vsrc, mrow);
          });
        }
        if constexpr (j < NSB) {
          constexpr int u0 = (j * NU_EX + NSB - 1) / NSB, u1 = ((j + 1) * NU_EX + NSB - 1) / NSB;
          static_for<u1 - u0>([&](auto uc) { unit_ex(sacc, std::integral_constant<int, u0 + decltype(uc)::value>{}); });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      pin_weights(1);
      sm_end();
    };
    // Iteration t: K(t+2) in Ks, V(t) in Vs; loads K(t+4) into Kdst and V(t+2)
    // into Vdst.  Every wave runs the whole pipeline every iteration: a tile
    // that none of a wave's queries sees is fully masked and adds weights of
    // exactly 0 (at most two iterations per workgroup and the diagonal tiles of
    // the later waves; one code path keeps the interleave and the register
    // assignment fixed).
    // With a mask, Ms holds the words of tile t+1 and Mdst receives those of
    // tile t+3.
    auto step_tile = [&](int t, const __bf16* Ks, const __bf16* Vs, __bf16* Kdst, __bf16* Vdst,
                         const uint32_t* Ms, uint32_t* Mdst) {
      const int e1 = tile_entry(t + 1), e2 = tile_entry(t + 2), e3 = tile_entry(t + 3),
                e4 = tile_entry(t + 4);
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) vis[0][qb] = vis[1][qb] = true;
      // The last iteration's final MFMAs wrote the scores: the mask reads them
      // at once and waits first; unmasked, the first read is 8 MFMAs into
      // phase A.
      if (need_mask(e1, qw0, t0)) {
        mfma_guard();
        apply_mask(e1, qw0, t0, sacc, Ms);
      }
      iteration(e4, e2, e3, Ks, Vs, Kdst, Vdst, Mdst, Kg, Vg, false, false, 0);
      // This wave's loads of the previous iteration (K(t+3), V(t+1)) are done
      // (loads complete in order: only this iteration's NITEM may be pending),
      // and so are its LDS reads; the barrier then makes every wave's loads
      // visible and frees the buffers read in this iteration for the next
      // iteration's loads.
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NITEM) : "memory");
    };

    // Prologue: K(0) .. K(2), V(0), V(1) in LDS; S(0) and its softmax, S(1);
    // K(3) loaded over K(0) once every wave has read K(0).
    const int e0 = tile_entry(0);
    if (n_tiles > 0) {
      const int e1 = tile_entry(1), e2 = tile_entry(2);
      load_k(tile_index(e0), Kb0);
      load_k(tile_index(e1), Kb1);
      load_k(tile_index(e2), Kb2);
      load_v(tile_index(e0), Vb0);
      load_v(tile_index(e1), Vb1);
      load_mask(e0, Mb0);
      load_mask(e1, Mb1);
      load_mask(e2, Mb2);
    }
    if constexpr (CONT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // Q
    __syncthreads();
    compute_s(Kb0, sacc);
    __syncthreads();  // every wave is done with K(0) before K(3) goes over it
    if (n_tiles > 0) load_k(tile_index(tile_entry(3)), Kb0);
    softmax_all(e0, sacc, Mb0);
    compute_s(Kb1, sacc);
    // K(1) is read by every wave before iteration 0 loads K(4) over it; K(3)
    // may still be in flight (iteration 0 waits for it)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l), for the item of
    // qw0 and bh ----
    auto write_out = [&](const float (&mr)[NQB], const float (&lr)[NQB]) __attribute__((always_inline)) {
  #pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qrow = qw0 + 32 * qb + ql;
      const float l_tot = swap_halves_sum(lr[qb]);
      if constexpr (CONT) {
        // read inside the item-boundary branch, in place
  #pragma unroll
        for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(oacc[db][qb]));
      }
      if (SPLIT && qrow < N) {
        // the chunk's normalised output and log-sum-exp, in float32
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const size_t prow = ((size_t)split * p.B * p.H + bh) * N + qrow;
        float* Orow = sp.part_o + prow * D;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            float4 ov;
            ov.x = oacc[db][qb][4 * j] * inv;
            ov.y = oacc[db][qb][4 * j + 1] * inv;
            ov.z = oacc[db][qb][4 * j + 2] * inv;
            ov.w = oacc[db][qb][4 * j + 3] * inv;
            *(float4*)(Orow + db * 32 + 8 * j + 4 * hl) = ov;
          }
        if (hl == 0) sp.part_lse[prow] = l_tot > 0.f ? (mr[qb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      } else if constexpr (OSTAGE) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // lane-dependent addresses are formed here, not hoisted to the
        // kernel's start and kept live (or spilled) across the whole walk
        int ln = lane;
        asm volatile("" : "+v"(ln));
        uint8_t* st = ostage + ws * 32 * OSTR;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x4 ov;
  #pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][qb][4 * j + i] * inv);
            *(bf16x4*)(st + (ln % 32) * OSTR + (db * 32 + 8 * j + 4 * (ln / 32)) * 2) = ov;
          }
        // the wave's LDS writes before its reads of other lanes' rows
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the block's rows of O, as one buffer: stores to rows past N drop
        // (block offset and size are wave-uniform: scalar registers)
        const int q_blk = __builtin_amdgcn_readfirstlane(qw0 + 32 * qb);
        const int64_t blk = ((int64_t)bh * N + q_blk) * D;
        __bf16* Oblk = (__bf16*)p.o + (((int64_t)__builtin_amdgcn_readfirstlane((int)(blk >> 32)) << 32) |
                                       (uint32_t)__builtin_amdgcn_readfirstlane((int)blk));
        const int blk_bytes = __builtin_amdgcn_readfirstlane(max(0, min(32, N - q_blk)) * D * 2);
        constexpr int RPI = 64 / CPR;  // rows per read: 16-byte piece lane % CPR of row lane / CPR
  #pragma unroll
        for (int r0 = 0; r0 < 32; r0 += RPI) {
          const int r = r0 + ln / CPR, c16 = ln % CPR;
          const u32x4 v = *(const u32x4*)(st + r * OSTR + c16 * 16);
          buffer_store16(Oblk, blk_bytes, (uint32_t)(r * D * 2 + c16 * 16), v);
        }
        // every lane has read the rows before the next block overwrites them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (hl == 0 && qrow < N)
          p.lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (mr[qb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      } else if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        __bf16* Orow = (__bf16*)p.o + (size_t)bh * N * D + (size_t)qrow * D;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x4 ov;
  #pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][qb][4 * j + i] * inv);
            *(bf16x4*)(Orow + db * 32 + 8 * j + 4 * hl) = ov;
          }
        if (hl == 0)
          p.lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (mr[qb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      }
    }
    };

    if constexpr (CONT) {
      // One pipeline over the walk: the iterations of an item's last tiles
      // already load, score and weigh the next item's first tiles.  Item
      // boundary work goes after an iteration's barrier:
      //   after tile n-3: Q of the next item into the Q registers (the last
      //     S MFMAs on this item's Q are done; the next iteration's S MFMAs,
      //     on the next item's first tile, wait for the loads after phase A);
      //   after tile n-2: this item's m and l are final (its last tile's
      //     weights are in); the running ones restart for the next item,
      //     whose first tile the next iteration weighs;
      //   after tile n-1: the output accumulator holds this item's whole
      //     output; it is written out and cleared, and the next item becomes
      //     the current one.
      // The pipeline drains only after the workgroup's last item.
      auto load_q_next = [&]() {
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int row = min(qw0_n + 32 * qb + ql, N - 1);
          const __bf16* a = Qg_n + (size_t)row * D + hl * 8;
  #pragma unroll
          for (int kb = 0; kb < DK; ++kb)
            asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "+a"(qf[qb][kb]) : "v"(a), "n"(kb * 32) : "memory");
        }
      };
      int t = 0;  // tile of the current item
      // first row of the next item's first tile; byte offsets of the last K
      // and V tiles loaded (K(3) and V(1) in the prologue)
      int row_c = (int)bh * M, row_nx = (int)bh_n * M + t0_n * BK;
      int kofs = ((int)bh * M + (t0 + 3) * BK) * ROWB, vofs = ((int)bh * M + (t0 + 1) * BK) * ROWB;
      float m_fin[NQB], l_fin[NQB];
  #pragma unroll
      for (int qb = 0; qb < NQB; ++qb) m_fin[qb] = l_fin[qb] = 0.f;
      // Per item, without a mask: the iterations t at which the loads jump to
      // the next item's first tile (K at t = n - 4, V at t = n - 2; -1 without
      // a next item), and, causal without a window, mth: the weighed tile
      // t + 1 needs masking iff t + 1 >= mth.  A causal wave's tiles that
      // cross the diagonal or end past kv_len are a suffix of its item: tile
      // e is masked iff (e + 1) BK > min(kend, qw0 + off + wr + 1), i.e.
      // e >= that bound / BK.  The next item's first tile (t + 1 = n) always
      // counts as masked: masking a tile that needs none gives the same
      // scores, and it saves the per-iteration test of which item the
      // weighed tile belongs to.
      // With a window the tiles masked at the band's lower edge are a prefix:
      // tile e is masked there iff (e + t0) BK < qw0 + QW - 1 + off - wl, i.e.
      // e < mlo.
      int kjump = -1, vjump = -1, jump_to = 0, mth = 0, mlo = 0;
      auto item_marks = [&]() {
        kjump = has_nx ? n_tiles - 4 : -1;
        vjump = has_nx ? n_tiles - 2 : -1;
        jump_to = row_nx * ROWB;
        mth = min(min(kend, qw0 + off + wr + 1) / BK - t0, n_tiles);
        if constexpr (WINDOW) {
          const int lo_key = qw0 + QW - 1 + off - wl;  // the wave's last query's first key
          // ceil(lo_key / BK), rounding toward minus infinity for negatives
          const int lo_tiles = lo_key > 0 ? (lo_key + BK - 1) / BK : -((-lo_key) / BK);
          mlo = lo_tiles - t0;
        }
      };
      if constexpr (!BITS) item_marks();
      auto cont_step = [&](const __bf16* Ks, const __bf16* Vs, __bf16* Kdst, __bf16* Vdst, const uint32_t* Ms,
                           uint32_t* Mdst) __attribute__((always_inline)) -> bool {
        const int n = n_tiles;
        // tiles t+1 (weighed), t+2 (V loaded), t+3 (mask words loaded), t+4
        // (K loaded): the next item's once past this one's last
        const bool sm_nx = has_nx && t + 1 >= n;
        const int qw_sm = sm_nx ? qw0_n : qw0, t0_sm = sm_nx ? t0_n : t0;
        int e1, e3 = 0, mrow = 0;
        // the masking test is t + 1 >= mth (or t + 1 < mlo with a window)
        constexpr bool MTH = !BITS && (CAUSAL || WINDOW);
        if constexpr (BITS) {
          // the stream runs on into the next item's entries
          e1 = tile_entry(t + 1);
          e3 = tile_entry(t + 3);
          const int e2 = tile_entry(t + 2), e4 = tile_entry(t + 4);
          kofs = ((has_nx && t + 4 >= n ? row_nx : row_c) + tile_index(e4) * BK) * ROWB;
          vofs = ((has_nx && t + 2 >= n ? row_nx : row_c) + tile_index(e2) * BK) * ROWB;
          mrow = has_nx && t + 3 >= n ? mrow_n : mrow_c;
        } else {
          e1 = sm_nx ? t + 1 - n : t + 1;
          // first bytes of K(t+4) and V(t+2) in the whole tensors: a tile on
          // from the last, or the next item's first tile
          kofs = t == kjump ? jump_to : kofs + BK * ROWB;
          vofs = t == vjump ? jump_to : vofs + BK * ROWB;
        }
        // the scores' guard only where the mask reads them at once (as
        // step_tile), but for the masked walk, whose D = 128 form spills more
        // registers with the guard inside the branch
        if constexpr (BITS) mfma_guard();
  #pragma unroll
        for (int qb = 0; qb < NQB; ++qb) vis[0][qb] = vis[1][qb] = true;
        bool nm;
        if constexpr (MTH) nm = (t + 1 >= mth) | (WINDOW && t + 1 < mlo);
        else nm = need_mask(e1, qw_sm, t0_sm);
        if (nm) {
          if constexpr (!BITS) mfma_guard();
          apply_mask(e1, qw_sm, t0_sm, sacc, Ms);
        }
        iteration(kofs, vofs, e3, Ks, Vs, Kdst, Vdst, Mdst, nullptr, nullptr, t == n - 1, has_nx && t == n - 2,
                  mrow);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NITEM) : "memory");
        if (__builtin_expect(t < n - 3, 1)) {
          ++t;
          return false;
        }
        if (t == n - 3) {
          if (has_nx) load_q_next();
          ++t;
          return false;
        }
        if (t == n - 2) {
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            m_fin[qb] = m_run[qb];
            l_fin[qb] = l_run[qb];
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.f;
          }
          ++t;
          return false;
        }
        write_out(m_fin, l_fin);
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb) oacc[db][qb] = f32x16{};
        if (!has_nx) return true;
        ++kw;
        gb += n;
        bh = bh_n;
        qw0 = qw0_n;
        t0 = t0_n;
        mrow_c = mrow_n;
        n_tiles = n_n;
        Qg = Qg_n;
        Kg = Kg_n;
        Vg = Vg_n;
        walk_next();
        row_c = (int)bh * M;
        row_nx = (int)bh_n * M + t0_n * BK;
        if constexpr (!BITS) item_marks();
        t = 0;
        return false;
      };
      for (;;) {
        if (cont_step(Kb2, Vb0, Kb1, Vb2, Mb1, Mb0)) break;
        if (cont_step(Kb0, Vb1, Kb2, Vb0, Mb2, Mb1)) break;
        if (cont_step(Kb1, Vb2, Kb0, Vb1, Mb0, Mb2)) break;
      }
    } else {
      for (int t = 0; t < n_tiles; t += 3) {
        step_tile(t, Kb2, Vb0, Kb1, Vb2, Mb1, Mb0);
        if (t + 1 >= n_tiles) break;
        step_tile(t + 1, Kb0, Vb1, Kb2, Vb0, Mb2, Mb1);
        if (t + 2 >= n_tiles) break;
        step_tile(t + 2, Kb1, Vb2, Kb0, Vb1, Mb0, Mb2);
      }
      write_out(m_run, l_run);
    }
  }
  }
}

template <int D, bool CAUSAL, bool WINDOW, bool BITS>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_bf16_kernel(Problem p, int n_qtiles, const int32_t* __restrict__ tile_lists,
                         int list_stride, const uint32_t* __restrict__ mask_blocks) {
  prefill_body<D, CAUSAL, WINDOW, BITS, false>(p, n_qtiles, tile_lists, list_stride, mask_blocks, SplitArgs{});
}

// Causal or windowed, no mask, key splits or kv_len, M >= N >= 256,
// several items per workgroup: a persistent walk as one pipeline.
template <int D, bool CAUSAL, bool WINDOW, bool BITS>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_cont_kernel(Problem p, int n_qtiles, const int32_t* __restrict__ tile_lists, int list_stride,
                         const uint32_t* __restrict__ mask_blocks, const int32_t* __restrict__ walk_order) {
  prefill_body<D, CAUSAL, WINDOW, BITS, false, true>(p, n_qtiles, tile_lists, list_stride, mask_blocks,
                                                      SplitArgs{}, walk_order);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_split_kernel(Problem p, int n_qtiles, SplitArgs sp) {
  prefill_body<D, CAUSAL, false, false, true>(p, n_qtiles, nullptr, 0, nullptr, sp);
}

// Merge of the key chunks of each row ("Understanding FlashAttention", the
// correction factor: partial results over disjoint key sets combine through
// their log-sum-exps): L = log sum_s e^(L_s), O = sum_s e^(L_s - L) O_s, in
// chunk order.  D / 8 threads per row, 8 elements each; a row no chunk sees
// a key of gets O = 0 and L = -inf.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(Problem p, SplitArgs sp) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;  // threads per row, rows per block
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (r >= rows) return;
  const int S = sp.splits;
  // Groups of four chunks: all of a group's loads go out before any is used
  // (one memory latency per group), then the group folds into a running
  // max, sum and output, rescaled when the max moves (the same identity).
  constexpr int G = 4;
  float mx = -INFINITY, sum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += G) {
    float ls[G];
    float4 a[G], b[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int s = min(s0 + g, S - 1);  // in bounds; chunks past S are left out below
      ls[g] = sp.part_lse[(size_t)s * rows + r];
      const float4* src = (const float4*)(sp.part_o + ((size_t)s * rows + r) * D + 8 * c);
      a[g] = src[0];
      b[g] = src[1];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // a chunk with no key for this row (LSE -inf) takes no part, nor do
      // its outputs (selected away, not multiplied by 0)
      const bool use = s0 + g < S && ls[g] != -INFINITY;
      const float lg = use ? ls[g] : mx;
      const float m_new = fmaxf(mx, lg);
      const float f = mx == -INFINITY ? 0.f : fast_exp2((mx - m_new) * kLog2e);
      const float w = use ? fast_exp2((lg - m_new) * kLog2e) : 0.f;
      const float4 z = {0.f, 0.f, 0.f, 0.f};
      const float4 av = use ? a[g] : z, bv = use ? b[g] : z;
      sum = sum * f + w;
      acc[0] = acc[0] * f + w * av.x; acc[1] = acc[1] * f + w * av.y;
      acc[2] = acc[2] * f + w * av.z; acc[3] = acc[3] * f + w * av.w;
      acc[4] = acc[4] * f + w * bv.x; acc[5] = acc[5] * f + w * bv.y;
      acc[6] = acc[6] * f + w * bv.z; acc[7] = acc[7] * f + w * bv.w;
      mx = m_new;
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  bf16x8 ov;
#pragma unroll
  for (int i = 0; i < 8; ++i) ov[i] = (__bf16)(acc[i] * inv);
  *(bf16x8*)((__bf16*)p.o + r * D + 8 * c) = ov;
  if (c == 0) p.lse[r] = sum > 0.f ? mx + fast_log2(sum) * kLn2 : -INFINITY;
}

template <int D, bool BITS>
void launch_prefill_dm(const Problem& p, dim3 grid, hipStream_t stream, int n_qtiles,
                       const int32_t* lists, int stride, const uint32_t* blocks) {
  const dim3 block(kPrefillThreads);
  if (p.window) {
    if (p.causal)
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true, BITS>), grid, block, 0, stream, p, n_qtiles, lists, stride, blocks);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, BITS>), grid, block, 0, stream, p, n_qtiles, lists, stride, blocks);
  } else {
    if (p.causal)
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, BITS>), grid, block, 0, stream, p, n_qtiles, lists, stride, blocks);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, BITS>), grid, block, 0, stream, p, n_qtiles, lists, stride, blocks);
  }
}

// Fewest key tiles any work item visits, by the kernel's own arithmetic for
// kv_len = M (no mask): the pipelined walk needs at least 4 (it loads K four
// tiles ahead).
int min_item_tiles(const Problem& p, int n_qtiles) {
  const int N = p.N, M = p.M, off = M - N, BQ = kPrefillBlockQ, BK = kPrefillBlockK;
  const int wl = p.window ? std::min<int64_t>(p.wl, (int64_t)N + M) : 0;
  const int wr = p.causal ? 0 : (p.window ? std::min<int64_t>(p.wr, (int64_t)N + M) : 0);
  int fewest = INT32_MAX;
  for (int qt = 0; qt < n_qtiles; ++qt) {
    const int q0 = qt * BQ, q_last = std::min(q0 + BQ, N) - 1;
    const int kv_end = (p.causal || p.window) ? std::min(M, q_last + off + wr + 1) : M;
    const int tw = p.window ? std::max(0, q0 + off - wl) / BK : 0;
    const int t_end = kv_end > tw * BK ? (kv_end + BK - 1) / BK : tw;
    fewest = std::min(fewest, t_end - tw);
  }
  return fewest;
}

void launch_prefill_cont(const Problem& p, dim3 grid, hipStream_t stream, int n_qtiles, const int32_t* lists,
                         int stride, const uint32_t* blocks, const int32_t* order) {
  const dim3 block(kPrefillThreads);
  // causal with a mask, windowed, or plain causal (the caller checks)
  if (p.mask) {
    if (p.D == 64)
      hipLaunchKernelGGL((prefill_cont_kernel<64, true, false, true>), grid, block, 0, stream, p, n_qtiles, lists,
                         stride, blocks, order);
    else
      hipLaunchKernelGGL((prefill_cont_kernel<128, true, false, true>), grid, block, 0, stream, p, n_qtiles, lists,
                         stride, blocks, order);
  } else if (p.D == 64) {
    if (!p.window)
      hipLaunchKernelGGL((prefill_cont_kernel<64, true, false, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
    else if (p.causal)
      hipLaunchKernelGGL((prefill_cont_kernel<64, true, true, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
    else
      hipLaunchKernelGGL((prefill_cont_kernel<64, false, true, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
  } else {
    if (!p.window)
      hipLaunchKernelGGL((prefill_cont_kernel<128, true, false, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
    else if (p.causal)
      hipLaunchKernelGGL((prefill_cont_kernel<128, true, true, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
    else
      hipLaunchKernelGGL((prefill_cont_kernel<128, false, true, false>), grid, block, 0, stream, p, n_qtiles, nullptr,
                         0, nullptr, nullptr);
  }
}

template <int D>
void launch_prefill_d(const Problem& p, dim3 grid, hipStream_t stream, int n_qtiles,
                      const int32_t* lists, int stride, const uint32_t* blocks) {
  if (p.mask) launch_prefill_dm<D, true>(p, grid, stream, n_qtiles, lists, stride, blocks);
  else launch_prefill_dm<D, false>(p, grid, stream, n_qtiles, lists, stride, blocks);
}

}  // namespace

hipError_t launch_prefill_bf16(const Problem& p, const Plan& plan, void* workspace,
                               hipStream_t stream) {
  if (plan.grid == 0) return hipSuccess;
  const int n_qtiles = (p.N + kPrefillBlockQ - 1) / kPrefillBlockQ;
  const dim3 grid((unsigned)plan.grid);
  if (plan.split_tiles > 0) {
    // key chunks, then their merge
    const SplitArgs sp{(float*)workspace, (float*)((char*)workspace + plan.ws_lse_offset), plan.split_tiles,
                       plan.splits};
    const dim3 block(kPrefillThreads);
    if (p.D == 64) {
      if (p.causal) hipLaunchKernelGGL((prefill_split_kernel<64, true>), grid, block, 0, stream, p, n_qtiles, sp);
      else hipLaunchKernelGGL((prefill_split_kernel<64, false>), grid, block, 0, stream, p, n_qtiles, sp);
    } else {
      if (p.causal) hipLaunchKernelGGL((prefill_split_kernel<128, true>), grid, block, 0, stream, p, n_qtiles, sp);
      else hipLaunchKernelGGL((prefill_split_kernel<128, false>), grid, block, 0, stream, p, n_qtiles, sp);
    }
    const int64_t rows = (int64_t)p.B * p.H * p.N;
    const int rpb = 256 / (p.D / 8);
    const dim3 mgrid((unsigned)((rows + rpb - 1) / rpb));
    if (p.D == 64) hipLaunchKernelGGL(prefill_merge_kernel<64>, mgrid, dim3(256), 0, stream, p, sp);
    else hipLaunchKernelGGL(prefill_merge_kernel<128>, mgrid, dim3(256), 0, stream, p, sp);
    return hipGetLastError();
  }
  const int64_t n_items = (int64_t)p.B * p.H * n_qtiles;
  // The pipelined walk: no kv_len, M >= N >= 256, one buffer descriptor over
  // all of K (and of V), and more items than the 256 persistent workgroups.
  const bool walk = !p.kv_len && p.N >= kPrefillBlockQ && p.M >= p.N &&
                    (int64_t)p.B * p.H * p.M * p.D * 2 <= INT32_MAX && n_items > kPrefillPersistGrid;
  if (walk && !p.mask && (p.window || p.causal) && min_item_tiles(p, n_qtiles) >= 4) {
    // every work item has at least 4 key tiles, and each workgroup walks more
    // than one: one pipeline per persistent workgroup (one per CU; with one
    // item each, the item-by-item kernel measured 3-4% faster).  Not for
    // plain non-causal attention, whose long uniform items gain little and
    // whose D = 128 form the compiler cannot allocate without spills.  Plain
    // causal attention at D = 64, whose iterations are half as long, gains
    // 1-3% (N = 8192 down to 2048) since the walk tests a per-item mask
    // threshold instead of working out its bookkeeping every iteration
    // (-0.5% before).
    launch_prefill_cont(p, dim3(kPrefillPersistGrid), stream, n_qtiles, nullptr, 0, nullptr, nullptr);
    return hipGetLastError();
  }
  const int32_t* lists = nullptr;
  const uint32_t* blocks = nullptr;
  if (p.mask) {
    // the tile lists, one per (mask batch, mask head, query tile), and the
    // words of the tiles the mask keeps in part
    const MaskWorkspace w = mask_workspace(p.N, p.M, p.mask_b, p.mask_h, 0, false, p.causal ? n_items : 0);
    // Causal masks take the pipelined walk when the workgroup's lists fit
    // in LDS (the pre-pass then cuts each list at the causal limit and fills
    // short ones up to 4 tiles) and one descriptor covers every row of blocks.
    const int64_t per_wg = ((n_items + kNumXcd - 1) / kNumXcd + kPrefillPersistGrid / kNumXcd - 1) /
                           (kPrefillPersistGrid / kNumXcd);
    const int64_t n_kt = (p.M + kPrefillBlockK - 1) / kPrefillBlockK;
    const bool walk_mask = walk && p.causal && !p.window && per_wg <= kWalkMaxItems &&
                           (n_items + kNumXcd - 1) / kNumXcd <= 4096 &&
                           per_wg * std::max<int64_t>(n_kt, 4) + 5 <= kMaskMaxTiles &&
                           (int64_t)p.mask_b * p.mask_h * n_qtiles * plan.mask_tiles * kMaskBlockBytes <= INT32_MAX;
    launch_mask_prep(p.mask, p.N, p.M, p.mask_w, p.mask_b, p.mask_h, workspace, w, false, stream, walk_mask, p.B,
                     p.H);
    lists = (const int32_t*)((char*)workspace + w.lists);
    blocks = (const uint32_t*)((char*)workspace + w.blocks);
    if (walk_mask) {
      launch_prefill_cont(p, dim3(kPrefillPersistGrid), stream, n_qtiles, lists, plan.mask_tiles, blocks,
                          (const int32_t*)((char*)workspace + w.order));
      return hipGetLastError();
    }
  }
  if (p.D == 64) launch_prefill_d<64>(p, grid, stream, n_qtiles, lists, plan.mask_tiles, blocks);
  else launch_prefill_d<128>(p, grid, stream, n_qtiles, lists, plan.mask_tiles, blocks);
  return hipGetLastError();
}

}  // namespace fa
