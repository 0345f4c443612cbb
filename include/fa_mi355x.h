/*
 * fa_mi355x.h -- C ABI of the fused exact attention for MI355X (gfx950):
 * the forward and its backward.
 *
 * The operation (per batch b and head h, all arithmetic described in real
 * numbers; the library's rounding is documented per path below):
 *
 *   S[i][j]   = scale * sum_d Q[b][h][i][d] * K[b][h][j][d]
 *   visible   : j < kv_len[b]  and  (not causal  or  j <= i + kv_len[b] - N)
 *               and, when fa_options asks for them, inside the local window
 *               and kept by the element mask
 *   O[b][h][i]  = sum_{visible j} softmax_j(S[i][.]) * V[b][h][j]
 *   LSE[b][h][i] = ln sum_{visible j} exp(S[i][j])
 *
 * Sources: "Flash Attention: The Hidden Gem" -- Background (the attention
 * formula softmax(Q K^T / sqrt(d_k)) V), The Algorithm (the forward returns O
 * and the log-sum-exp L = m + log(l) kept for the backward pass);
 * "Understanding FlashAttention" -- Attention (Q [N,D], K [M,D], V [M,D],
 * N = 1 when decoding against a KV cache of M keys, an elementwise mask that
 * does not depend on the scores, batch and heads as independent repeats, D
 * fixed at compile time, scaling by 1/sqrt(D)).
 *
 * Readings where the pages are silent: the causal mask is aligned to the
 * bottom-right corner (the last query sees the last visible key; with
 * N == kv_len it is the usual j <= i, with N == 1 the query sees its whole
 * history); kv_len masks keys only; a query with no visible key gets O = 0
 * and LSE = -inf; LSE is a natural logarithm and always float32.
 *
 * Memory and ownership.  Every pointer argument except `stream` is a device
 * pointer on the current HIP device.  The caller allocates and frees every
 * buffer, including the workspace; the library allocates nothing, never
 * synchronises and never copies to the host, and it holds no device state
 * except the static scratch of fa_fwd_noalloc (below).  Calls are
 * enqueued on `stream` (NULL = the default stream) and return at once; the
 * outputs are ready when the stream reaches that point.  Functions are
 * reentrant and never throw across the ABI.
 *
 * Layout.  Q [B,H,N,D], K and V [B,H,M,D] and O [B,H,N,D] are contiguous,
 * row-major, D fastest, all of element type `dtype` (O is bf16 for FA_FP8);
 * LSE [B,H,N] is float32;
 * kv_len [B] is int32 (NULL means M for every batch).  Device-side kv_len
 * values cannot be checked without a synchronisation: values outside [0, M]
 * are clamped to that range by the kernels.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 8

/* FA_FP8: OCP E4M3 (finite max 448, no infinities) Q, K, V with per-tensor
 * descale factors (fa_options); O is then bf16 and LSE float32. */
typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_FP8 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,       /* a dimension is negative or the sizes overflow       */
  FA_ERR_UNSUPPORTED = 3, /* D not in {64, 128}, unknown dtype, path not usable  */
  FA_ERR_ALIGN = 4,       /* Q/K/V/O not 16-byte aligned, LSE/kv_len not 4-byte  */
  FA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required             */
  FA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch         */
  FA_ERR_ARG = 7          /* scale not finite or negative, bad option value      */
} fa_status;

typedef struct { int32_t B, H, N, M, D; } fa_shape;

typedef enum {
  FA_PATH_AUTO = 0,     /* planner's choice                                      */
  FA_PATH_PREFILL = 1,  /* fused tiled kernel, bf16 MFMA (bf16 only; K/V bytes
                           per batch and head, M * D * 2, below 2^31); with a
                           window or an element mask it also serves N = 1        */
  FA_PATH_SPLITKV = 2,  /* split-KV partial kernel + log-sum-exp merge (bf16, N=1,
                           no window, no element mask)                            */
  FA_PATH_F32 = 3,      /* float32 inputs/outputs, float64 internal arithmetic;
                           takes a window and an element mask                    */
  FA_PATH_KVOUTER = 4,  /* ablation, never chosen by the planner: the same result
                           with key/value tiles in the outer loop and the output
                           accumulator, m and l read and written back in a
                           float32 workspace for every key tile (bf16, no window,
                           no element mask)                                       */
  FA_PATH_FP8 = 5       /* fused tiled kernel on the fp8 matrix cores: FA_FP8
                           inputs only, any N, no window, no element mask; the
                           weights are rounded to E4M3 before the P V product      */
} fa_path;

/* Optional controls; pass NULL for the planner's defaults.  A zero-filled
 * struct means the defaults too. */
typedef struct {
  int32_t path;        /* fa_path                                                */
  int32_t split_keys;  /* a multiple of 64.  FA_PATH_SPLITKV: keys per split
                          (0 = auto).  FA_PATH_PREFILL (N > 1 under
                          FA_PATH_AUTO): 0 = none; otherwise each query tile's
                          keys go in chunks of split_keys to separate
                          workgroups, whose float32 partial results are merged
                          by their log-sum-exps ("Understanding
                          FlashAttention", the correction factor) in one more
                          launch: more workgroups for a small B * H * N (up to
                          256 CUs), at the cost of workspace
                          (fa_fwd_workspace_bytes: (D + 1) * 4 bytes per
                          (chunk, batch, head, query row)); no window, no
                          element mask                                         */
  int32_t window;      /* 0: no window.  1: local (banded) attention: key j is
                          visible to query i only if
                            i + off - window_left <= j <= i + off + window_right
                          with off = kv_len[b] - N (the causal alignment), in
                          addition to j < kv_len[b] and the causal rule (which
                          caps window_right at 0).  window_left = W - 1,
                          window_right = 0 with causal gives each query the W
                          most recent keys: "a 128-wide local window" is
                          window_left = 127.                                    */
  int32_t window_left;   /* >= 0, used when window == 1                         */
  int32_t window_right;  /* >= 0, used when window == 1                         */
  int32_t kvouter_query_tiles;  /* FA_PATH_KVOUTER: 256-query tiles per workgroup
                                   (0 = 1); a value >= ceil(N / 256) gives one
                                   workgroup per (batch, head)                  */
  float q_descale;     /* FA_FP8: Q stands for q_descale * Q8 (0 means 1)       */
  float k_descale;     /* FA_FP8: K stands for k_descale * K8 (0 means 1)       */
  float v_descale;     /* FA_FP8: V stands for v_descale * V8 (0 means 1)       */
  /* Element mask ("Understanding FlashAttention", Attention: mask() covers
   * causal masking and other kinds, each an elementwise constant that does
   * not depend on the scores).  NULL: none.  Otherwise a device array of
   * uint32 words [mask_batches][mask_heads][N][W], W = ceil(M / 32), rows of
   * W words contiguous: key j is visible to query i of batch b, head h only
   * if bit (j % 32) of word [b'][h'][i][j / 32] is 1 (b' = b, or 0 when
   * mask_batches == 1; h' likewise), in addition to kv_len, the causal rule
   * and the window.  Bits of keys >= M are ignored.  4-byte aligned; the
   * caller keeps it alive until the call's work on the stream is done.
   * Paths: FA_PATH_PREFILL (which then needs workspace: a pre-pass lists,
   * per query tile of 256, the 64-key tiles in which some query keeps a
   * key and copies the words of the tiles the mask keeps in part into 2 KB
   * blocks, about N * M / 8 bytes (the size of the mask) per (mask batch,
   * mask head), and, when causal, 4 bytes per 256-query work item for the
   * order in which persistent workgroups take them: fa_fwd_workspace_bytes;
   * M up to 262080 and N * W * 4 below 2^31) and FA_PATH_F32, which reads
   * the words directly.                                                    */
  const uint32_t* mask;
  int32_t mask_batches;  /* 1 or B (0 means 1)                               */
  int32_t mask_heads;    /* 1 or H (0 means 1)                               */
} fa_options;

/* What the planner decided for a shape (host-only, no device call). */
typedef struct {
  int32_t path;            /* fa_path actually used                              */
  int32_t block_q;         /* queries per workgroup                              */
  int32_t block_k;         /* keys per K/V tile (prefill) or per split (split-KV) */
  int32_t threads;         /* threads per workgroup                              */
  int32_t lds_bytes;       /* static LDS per workgroup                           */
  int32_t splits;          /* split-KV: number of key splits per (b, h)          */
  int64_t grid;            /* workgroups of the main kernel                      */
  size_t workspace_bytes;  /* bytes the caller must pass as workspace            */
} fa_plan;

/*
 * fa_plan_query -- run the planner only.  Pure host function: it reads no
 * device state and launches nothing.  Returns the same status fa_fwd_ex
 * would return for the shape-level checks (FA_ERR_SHAPE, FA_ERR_UNSUPPORTED,
 * FA_ERR_ARG); `out` (non-NULL) receives the plan on FA_OK.
 */
fa_status fa_plan_query(fa_shape s, fa_dtype dtype, int causal,
                        const fa_options* opt, fa_plan* out);

/*
 * fa_fwd_workspace_bytes -- bytes of device workspace fa_fwd needs for this
 * shape (0 unless the split-KV path, the key/value-outer path or an element
 * mask on the prefill path is chosen).  Returns 0 for a shape the
 * planner rejects.  The value depends on the shape and options only.
 */
size_t fa_fwd_workspace_bytes(fa_shape s, fa_dtype dtype, int causal,
                              const fa_options* opt);

/*
 * fa_fwd -- the exact-attention forward: O and LSE as defined at the top of
 * this file.  `scale` is applied in float32 to the float32 score (bf16 path)
 * or in float64 (float32 path); pass 1/sqrt(D) for the usual scaling.
 * Checks run before any launch; on a non-OK status nothing is enqueued and
 * fa_last_error() describes the failure.  A problem with no work
 * (B*H*N == 0) returns FA_OK without launching.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v,
                 const int32_t* kv_len, void* o, float* lse,
                 fa_shape s, fa_dtype dtype, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream);

/* fa_fwd_ex -- fa_fwd with explicit options (NULL = defaults). */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v,
                    const int32_t* kv_len, void* o, float* lse,
                    fa_shape s, fa_dtype dtype, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream,
                    const fa_options* opt);

/*
 * fa_fwd_noalloc -- fa_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same computation, arguments, checks and errors as fa_fwd
 * with no options, without the workspace arguments: the workspace fa_fwd
 * would take (the split-KV path's partial results) comes from a static
 * device array of FA_NOALLOC_SCRATCH_BYTES inside the library.  Each GPU
 * the library runs on holds its own copy from the library's load until the
 * process ends; on the first call on a device its address is resolved
 * (hipGetSymbolAddress, with that device current) and kept.  The call makes
 * no hipMalloc, hipFree or other allocating call.
 * Limit: a shape whose fa_fwd_workspace_bytes(s, dtype, causal, NULL)
 * exceeds FA_NOALLOC_SCRATCH_BYTES is rejected with FA_ERR_WORKSPACE before
 * anything is enqueued (the split-KV decode of B * H * ceil(M / 512) splits
 * at D = 128 needs about 516 bytes per split; 48 MiB hold 97,000 splits,
 * e.g. B = 32, H = 32, M = 48,000).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: the kernels write every
 * partial result they later read).  Calls that overlap on one GPU -- on two
 * streams, or from two threads without ordering -- race on the array: the
 * caller must order them.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
fa_status fa_fwd_noalloc(const void* q, const void* k, const void* v,
                         const int32_t* kv_len, void* o, float* lse,
                         fa_shape s, fa_dtype dtype, float scale, int causal, void* stream);

/*
 * ---- Backward ----
 *
 * The gradients of the forward above for an upstream gradient dO = dL/dO
 * (per batch b and head h; P is the softmax of the visible scores):
 *
 *   dV[j]  = sum_i P[i][j] * dO[i]                        (j < kv_len[b])
 *   dP[i][j] = dO[i] . V[j]
 *   D[i]   = sum_j dP[i][j] * P[i][j]  = dO[i] . O[i]
 *   dS[i][j] = P[i][j] * (dP[i][j] - D[i])
 *   dQ[i]  = scale * sum_j dS[i][j] * K[j]
 *   dK[j]  = scale * sum_i dS[i][j] * Q[i]                (j < kv_len[b])
 *
 * and dK[j] = dV[j] = 0 for keys at or past kv_len[b]; a query with no
 * visible key gets dQ = 0.  Sources: "Flash Attention: The Hidden Gem" --
 * Phase 2: Backward Pass (Chain Rule Through a Matrix Multiply: dV = P^T dO,
 * dP = dO V^T; The Softmax Jacobian: dS = P (dP - D); The D Shortcut:
 * D = rowsum(dO * O); The Algorithm: P recomputed as exp(S - L) from the
 * saved log-sum-exp, dQ = dS K, dK = dS^T Q).  The pages write S = Q K^T;
 * with the forward's S = scale * Q K^T the chain rule puts the scale on dQ
 * and dK as above.
 *
 * Inputs are those of the forward plus its outputs: O [B,H,N,D] and LSE
 * [B,H,N] exactly as fa_fwd wrote them for the same q, k, v, kv_len, scale
 * and causal (the backward recomputes P from LSE and takes D from O), and
 * dout [B,H,N,D].  Outputs dq [B,H,N,D], dk and dv [B,H,M,D].  All tensors
 * contiguous, D fastest, element type `dtype` except LSE (float32); the same
 * alignment rules as fa_fwd (16 bytes for tensors, 4 for lse and kv_len,
 * 256 for the workspace).  Every output element is written; no output may
 * alias an input.  Accumulation is float32; P and dS are rounded to bf16
 * before the products that use them; outputs are rounded once (RNE).
 * The result is bitwise reproducible: no atomics, fixed summation order.
 *
 * Memory, streams and errors as for fa_fwd: caller-owned device buffers,
 * enqueued on `stream`, checks before any launch, FA_ERR_* on failure with
 * fa_last_error() describing it.  Supported: dtype FA_BF16, D in {64, 128},
 * N * D * 2 and M * D * 2 below 2^31.  A problem with B * H == 0, or with
 * N == M == 0, returns FA_OK without launching.
 */

/* fa_bwd_workspace_bytes -- device workspace fa_bwd needs: 8 bytes per
 * (batch, head, query row) with the rows rounded up to a multiple of 256
 * (0 for an unsupported dtype). */
size_t fa_bwd_workspace_bytes(fa_shape s, fa_dtype dtype, int causal);

/* fa_bwd_workspace_bytes_ex -- the same for fa_bwd_ex with options `opt`
 * (NULL = none): with an element mask the workspace also holds the dQ
 * pass's lists and blocks of mask words, as the forward's prefill path
 * does, and the same for the dK/dV pass (per 256-key tile, the 64-query
 * stages): about twice the forward's (0 for an unsupported dtype or mask
 * shape). */
size_t fa_bwd_workspace_bytes_ex(fa_shape s, fa_dtype dtype, int causal, const fa_options* opt);

/* fa_bwd -- dq, dk, dv as defined above. */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, const int32_t* kv_len, void* dq, void* dk, void* dv,
                 fa_shape s, fa_dtype dtype, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream);

/* fa_bwd_ex -- fa_bwd for a forward run with options `opt` (NULL = none):
 * a window must be the one the forward used (the gradients above then run
 * over the keys visible under it), and so must an element mask (the same
 * words, mask_batches and mask_heads; the gradients of the entries it hides
 * are 0; workspace from fa_bwd_workspace_bytes_ex; M up to 262080 and
 * N * ceil(M / 32) * 4 below 2^31).  `path`, `split_keys`, the fp8 descales
 * and `kvouter_query_tiles` are ignored. */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, const int32_t* kv_len, void* dq,
                    void* dk, void* dv, fa_shape s, fa_dtype dtype, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream,
                    const fa_options* opt);

/* Static name of a status code. */
const char* fa_status_str(fa_status st);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* fa_last_error(void);

/* FA_ABI_VERSION of the built library. */
int32_t fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
