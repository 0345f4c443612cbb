// C-ABI shim: argument checks, planning and dispatch to the kernels.
// The declarations and their contracts are in include/fa_mi355x.h.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

fa_status vfail(fa_status st, const char* fmt, va_list ap) {
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  return st;
}

fa_status fail(fa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

fa_status fa::report_error(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_str(fa_status st) {
  switch (st) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_ARG: return "FA_ERR_ARG";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

fa_status fa_plan_query(fa_shape s, fa_dtype dtype, int causal,
                        const fa_options* opt, fa_plan* out) {
  if (!out) return fail(FA_ERR_NULL, "fa_plan_query: out is NULL");
  fa::Plan plan;
  const char* why = "";
  fa_status st = fa::make_plan(s, dtype, causal, opt, &plan, &why);
  if (st != FA_OK) return fail(st, "fa_plan_query: %s", why);
  out->path = plan.path;
  out->block_q = plan.block_q;
  out->block_k = plan.block_k;
  out->threads = plan.threads;
  out->lds_bytes = plan.lds_bytes;
  out->splits = plan.splits;
  out->grid = plan.grid;
  out->workspace_bytes = plan.ws_bytes;
  g_last_error[0] = 0;
  return FA_OK;
}

size_t fa_fwd_workspace_bytes(fa_shape s, fa_dtype dtype, int causal,
                              const fa_options* opt) {
  fa::Plan plan;
  const char* why = "";
  if (fa::make_plan(s, dtype, causal, opt, &plan, &why) != FA_OK) return 0;
  return plan.ws_bytes;
}

fa_status fa_fwd_ex(const void* q, const void* k, const void* v,
                    const int32_t* kv_len, void* o, float* lse,
                    fa_shape s, fa_dtype dtype, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream,
                    const fa_options* opt) {
  fa::Plan plan;
  const char* why = "";
  fa_status st = fa::make_plan(s, dtype, causal, opt, &plan, &why);
  if (st != FA_OK) return fail(st, "fa_fwd: %s", why);
  if (!std::isfinite(scale) || scale < 0.0f)
    return fail(FA_ERR_ARG, "fa_fwd: scale must be finite and >= 0 (got %g)", (double)scale);

  const int64_t bh = (int64_t)s.B * s.H;
  const bool no_rows = bh == 0 || s.N == 0;
  if (no_rows) {  // nothing to compute and nothing to write
    g_last_error[0] = 0;
    return FA_OK;
  }
  const bool has_kv = s.M > 0;
  if (!q || !o || !lse) return fail(FA_ERR_NULL, "fa_fwd: q, o and lse must be non-NULL");
  if (has_kv && (!k || !v)) return fail(FA_ERR_NULL, "fa_fwd: k and v must be non-NULL when M > 0");
  if (!aligned(q, 16) || !aligned(o, 16) || (has_kv && (!aligned(k, 16) || !aligned(v, 16))))
    return fail(FA_ERR_ALIGN, "fa_fwd: q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4) || (kv_len && !aligned(kv_len, 4)))
    return fail(FA_ERR_ALIGN, "fa_fwd: lse and kv_len must be 4-byte aligned");
  if (plan.ws_bytes) {
    if (!workspace)
      return fail(FA_ERR_WORKSPACE, "fa_fwd: this shape needs %zu workspace bytes, got NULL",
                  plan.ws_bytes);
    if (workspace_bytes < plan.ws_bytes)
      return fail(FA_ERR_WORKSPACE, "fa_fwd: this shape needs %zu workspace bytes, got %zu",
                  plan.ws_bytes, workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(FA_ERR_ALIGN, "fa_fwd: workspace must be 256-byte aligned");
  }

  const bool win = opt && opt->window;
  auto descale = [](float x) { return x == 0.f ? 1.f : x; };
  const uint32_t* mask = opt ? opt->mask : nullptr;
  if (mask && !aligned(mask, 4)) return fail(FA_ERR_ALIGN, "fa_fwd: options.mask must be 4-byte aligned");
  fa::Problem p{q, k, v, kv_len, o, lse, s.B, s.H, s.N, s.M, s.D, scale, causal ? 1 : 0,
                win ? 1 : 0, win ? opt->window_left : 0, win ? opt->window_right : 0,
                opt ? descale(opt->q_descale) : 1.f, opt ? descale(opt->k_descale) : 1.f,
                opt ? descale(opt->v_descale) : 1.f, mask,
                mask && opt->mask_batches ? opt->mask_batches : 1,
                mask && opt->mask_heads ? opt->mask_heads : 1, fa::mask_words(s.M)};
  hipStream_t hs = (hipStream_t)stream;
  hipError_t err = hipSuccess;
  switch (plan.path) {
    case FA_PATH_PREFILL: err = fa::launch_prefill_bf16(p, plan, workspace, hs); break;
    case FA_PATH_F32: err = fa::launch_fwd_f32(p, plan, hs); break;
    case FA_PATH_SPLITKV: err = fa::launch_splitkv_bf16(p, plan, workspace, hs); break;
    case FA_PATH_KVOUTER: err = fa::launch_kvouter_bf16(p, plan, workspace, hs); break;
    case FA_PATH_FP8: err = fa::launch_prefill_fp8(p, plan, hs); break;
    default: return fail(FA_ERR_UNSUPPORTED, "fa_fwd: internal: no path");
  }
  if (err != hipSuccess)
    return fail(FA_ERR_HIP, "fa_fwd: launch failed: %s", hipGetErrorString(err));
  g_last_error[0] = 0;
  return FA_OK;
}

fa_status fa_fwd(const void* q, const void* k, const void* v,
                 const int32_t* kv_len, void* o, float* lse,
                 fa_shape s, fa_dtype dtype, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return fa_fwd_ex(q, k, v, kv_len, o, lse, s, dtype, scale, causal, workspace,
                   workspace_bytes, stream, nullptr);
}

size_t fa_bwd_workspace_bytes(fa_shape s, fa_dtype dtype, int causal) {
  return fa_bwd_workspace_bytes_ex(s, dtype, causal, nullptr);
}

size_t fa_bwd_workspace_bytes_ex(fa_shape s, fa_dtype dtype, int causal, const fa_options* opt) {
  (void)causal;
  if (dtype != FA_BF16 || s.B < 0 || s.H < 0 || s.N < 0 || s.M < 0) return 0;
  if (!opt || !opt->mask) return fa::bwd_workspace_bytes(s);
  const int32_t mb = opt->mask_batches ? opt->mask_batches : 1;
  const int32_t mh = opt->mask_heads ? opt->mask_heads : 1;
  if ((mb != 1 && mb != s.B) || (mh != 1 && mh != s.H)) return 0;
  return fa::bwd_workspace_bytes(s, mb, mh);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, const int32_t* kv_len, void* dq, void* dk, void* dv,
                 fa_shape s, fa_dtype dtype, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, kv_len, dq, dk, dv, s, dtype, scale, causal, workspace,
                   workspace_bytes, stream, nullptr);
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, const int32_t* kv_len, void* dq,
                    void* dk, void* dv, fa_shape s, fa_dtype dtype, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream,
                    const fa_options* opt) {
  if (opt && opt->window != 0 && opt->window != 1)
    return fail(FA_ERR_ARG, "fa_bwd: options.window must be 0 or 1");
  const uint32_t* mask = opt ? opt->mask : nullptr;
  const int32_t mask_b = mask && opt->mask_batches ? opt->mask_batches : 1;
  const int32_t mask_h = mask && opt->mask_heads ? opt->mask_heads : 1;
  if (mask && ((mask_b != 1 && mask_b != s.B) || (mask_h != 1 && mask_h != s.H)))
    return fail(FA_ERR_ARG, "fa_bwd: options.mask_batches must be 1 or B and options.mask_heads 1 or H");
  const bool win = opt && opt->window;
  if (win && (opt->window_left < 0 || opt->window_right < 0))
    return fail(FA_ERR_ARG, "fa_bwd: options.window_left and window_right must be >= 0");
  if (s.B < 0 || s.H < 0 || s.N < 0 || s.M < 0 || s.D < 0)
    return fail(FA_ERR_SHAPE, "fa_bwd: B, H, N, M and D must be non-negative");
  if (dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: only FA_BF16 inputs are supported");
  if (s.D != 64 && s.D != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: head dimension D must be 64 or 128");
  if (!std::isfinite(scale) || scale < 0.0f)
    return fail(FA_ERR_ARG, "fa_bwd: scale must be finite and >= 0 (got %g)", (double)scale);
  const int64_t bh = (int64_t)s.B * s.H;
  // The tile passes address one (batch, head) of Q, dO, K or V with 32-bit
  // byte offsets, and their grids must fit 32 bits.
  if ((int64_t)s.N * s.D * 2 > INT32_MAX || (int64_t)s.M * s.D * 2 > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: needs N * D * 2 and M * D * 2 below 2^31");
  // With a mask the dQ pass holds a list of key tiles in LDS, and both passes
  // address one (mask batch, mask head) of the mask with 32-bit byte offsets.
  if (mask && (fa::mask_list_stride(s.M) > fa::kMaskMaxTiles ||
               fa::mask_stage_stride(s.N) > fa::kMaskMaxTiles ||
               (int64_t)s.N * fa::mask_words(s.M) * 4 > INT32_MAX))
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: an element mask needs N and M <= 262080 and "
                                    "N * ceil(M / 32) * 4 < 2^31");
  if (bh > INT32_MAX ||
      bh * ((fa::bwd_npad(s.N) + 63) / 64) > INT32_MAX ||
      bh * (((int64_t)s.M + fa::kBwdBlockKV - 1) / fa::kBwdBlockKV) > INT32_MAX)
    return fail(FA_ERR_SHAPE, "fa_bwd: grid exceeds 2^31 - 1 workgroups");
  if (bh == 0 || (s.N == 0 && s.M == 0)) {
    g_last_error[0] = 0;
    return FA_OK;
  }
  const bool has_q = s.N > 0, has_kv = s.M > 0;
  if (has_q && (!q || !o || !lse || !dout || !dq))
    return fail(FA_ERR_NULL, "fa_bwd: q, o, lse, dout and dq must be non-NULL when N > 0");
  if (has_kv && (!k || !v || !dk || !dv))
    return fail(FA_ERR_NULL, "fa_bwd: k, v, dk and dv must be non-NULL when M > 0");
  const void* a16[] = {q, o, dout, dq, k, v, dk, dv};
  for (const void* ptr : a16)
    if (ptr && !aligned(ptr, 16))
      return fail(FA_ERR_ALIGN, "fa_bwd: q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if ((lse && !aligned(lse, 4)) || (kv_len && !aligned(kv_len, 4)) || (mask && !aligned(mask, 4)))
    return fail(FA_ERR_ALIGN, "fa_bwd: lse, kv_len and options.mask must be 4-byte aligned");
  const size_t need = mask ? fa::bwd_workspace_bytes(s, mask_b, mask_h) : fa::bwd_workspace_bytes(s);
  if (need) {
    if (!workspace)
      return fail(FA_ERR_WORKSPACE, "fa_bwd: this shape needs %zu workspace bytes, got NULL", need);
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "fa_bwd: this shape needs %zu workspace bytes, got %zu", need,
                  workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(FA_ERR_ALIGN, "fa_bwd: workspace must be 256-byte aligned");
  }
  // with a mask: the pre-pass output after the row statistics
  const fa::MaskWorkspace mw = fa::mask_workspace(s.N, s.M, mask_b, mask_h, fa::bwd_mask_lists_offset(s), true);
  char* const wsb = (char*)workspace;
  fa::BwdProblem p{q, k, v, o, dout, lse, kv_len, dq, dk, dv, (float*)workspace,
                   s.B, s.H, s.N, s.M, s.D, (int32_t)fa::bwd_npad(s.N), scale, causal ? 1 : 0,
                   win ? 1 : 0, win ? opt->window_left : 0, win ? opt->window_right : 0,
                   mask, mask_b, mask_h, fa::mask_words(s.M),
                   mask ? (int32_t*)(wsb + mw.lists) : nullptr,
                   mask ? (int32_t*)(wsb + mw.stage_lists) : nullptr,
                   mask ? (const uint32_t*)(wsb + mw.blocks) : nullptr,
                   mask ? (const uint32_t*)(wsb + mw.stage_blocks) : nullptr};
  const hipError_t err = fa::launch_bwd_bf16(p, (hipStream_t)stream);
  if (err != hipSuccess)
    return fail(FA_ERR_HIP, "fa_bwd: launch failed: %s", hipGetErrorString(err));
  g_last_error[0] = 0;
  return FA_OK;
}

}  // extern "C"
