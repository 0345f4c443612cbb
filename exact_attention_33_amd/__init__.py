"""exact_attention_33_amd: fused exact attention for MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/fa_mi355x.h``.  It only
marshals arguments: torch allocates the outputs and the workspace and supplies
the stream; every step of the computation runs in the HIP kernels of
``lib/libfa_mi355x.so``.  There is no fallback: if the library is missing the
first call raises.

    o, lse = exact_attention_33_amd.fwd(q, k, v, scale=None, causal=False, kv_len=None)
    dq, dk, dv = exact_attention_33_amd.bwd(q, k, v, o, lse, do, scale=None, causal=False,
                                            kv_len=None)

q [B,H,N,D], k/v [B,H,M,D] contiguous CUDA tensors (bf16 or float32, D in
{64, 128}); kv_len an int32 tensor [B] on the same device (or None).  Returns
O [B,H,N,D] (input dtype) and LSE [B,H,N] (float32, natural log).  ``bwd``
takes the forward's inputs and outputs and the upstream gradient dO (bf16)
and returns dQ, dK, dV (bf16).  ``fwd`` also takes a local window and an
element mask (``pack_mask`` turns a boolean [Bm, Hm, N, M] into the packed
words the library reads).
"""
import ctypes
import math
import os

__all__ = ["fwd", "fwd_noalloc", "bwd", "bwd_workspace_bytes", "plan", "workspace_bytes", "pack_mask", "lib",
           "library_path", "FaError",
           "PATH_AUTO", "PATH_PREFILL", "PATH_SPLITKV", "PATH_F32", "PATH_KVOUTER", "PATH_FP8",
           "FP8",
           "F32", "BF16", "EXPORTS", "NOALLOC_SCRATCH_BYTES"]

F32, BF16, FP8 = 0, 1, 2
PATH_AUTO, PATH_PREFILL, PATH_SPLITKV, PATH_F32, PATH_KVOUTER, PATH_FP8 = 0, 1, 2, 3, 4, 5
PATH_NAMES = {PATH_PREFILL: "prefill", PATH_SPLITKV: "splitkv", PATH_F32: "f32",
              PATH_KVOUTER: "kvouter", PATH_FP8: "fp8"}

# Every symbol include/fa_mi355x.h declares.
EXPORTS = ["fa_plan_query", "fa_fwd_workspace_bytes", "fa_fwd", "fa_fwd_ex", "fa_fwd_noalloc",
           "fa_bwd_workspace_bytes", "fa_bwd_workspace_bytes_ex", "fa_bwd", "fa_bwd_ex",
           "fa_status_str", "fa_last_error", "fa_abi_version"]

# Bytes of the library's static scratch behind fa_fwd_noalloc
# (FA_NOALLOC_SCRATCH_BYTES in include/fa_mi355x.h).
NOALLOC_SCRATCH_BYTES = 48 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "lib", "libfa_mi355x.so")


class FaError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("M", ctypes.c_int32), ("D", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_keys", ctypes.c_int32),
                ("window", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("kvouter_query_tiles", ctypes.c_int32),
                ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float),
                ("v_descale", ctypes.c_float), ("mask", ctypes.c_void_p),
                ("mask_batches", ctypes.c_int32), ("mask_heads", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m exact_attention_33_amd.build` (hipcc, gfx950)")
    # torch first: the library then binds to the HIP runtime torch already
    # loaded.  Loaded the other way round, the process holds two runtimes
    # and the library's launches find no device.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the binding needs torch anyway
        pass
    L = ctypes.CDLL(library_path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    L.fa_plan_query.argtypes = [Shape, i32, i32, ctypes.POINTER(Options), ctypes.POINTER(PlanInfo)]
    L.fa_plan_query.restype = i32
    L.fa_fwd_workspace_bytes.argtypes = [Shape, i32, i32, ctypes.POINTER(Options)]
    L.fa_fwd_workspace_bytes.restype = ctypes.c_size_t
    fwd_args = [vp, vp, vp, vp, vp, vp, Shape, i32, f32, i32, vp, ctypes.c_size_t, vp]
    L.fa_fwd.argtypes = fwd_args
    L.fa_fwd.restype = i32
    L.fa_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(Options)]
    L.fa_fwd_ex.restype = i32
    L.fa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, Shape, i32, f32, i32, vp]
    L.fa_fwd_noalloc.restype = i32
    L.fa_bwd_workspace_bytes.argtypes = [Shape, i32, i32]
    L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd_workspace_bytes_ex.argtypes = [Shape, i32, i32, ctypes.POINTER(Options)]
    L.fa_bwd_workspace_bytes_ex.restype = ctypes.c_size_t
    L.fa_bwd.argtypes = [vp] * 10 + [Shape, i32, f32, i32, vp, ctypes.c_size_t, vp]
    L.fa_bwd.restype = i32
    L.fa_bwd_ex.argtypes = L.fa_bwd.argtypes + [ctypes.POINTER(Options)]
    L.fa_bwd_ex.restype = i32
    L.fa_status_str.argtypes = [i32]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_abi_version.argtypes = []
    L.fa_abi_version.restype = i32
    _lib = L
    return L


def _check(st):
    if st != 0:
        L = lib()
        raise FaError(st, L.fa_status_str(st).decode(), L.fa_last_error().decode())


def _options(path, split_keys, window=None, kvouter_query_tiles=0, descale=None, mask=None):
    """fa_options for the call, or None for the defaults.  ``window`` is None
    or (left, right): key j visible to query i only if
    i + off - left <= j <= i + off + right (off = kv_len - N).  ``descale``
    is None or (dq, dk, dv) for fp8 inputs.  ``mask`` is None or
    (device pointer, mask batches, mask heads) of packed mask words."""
    if (path in (None, PATH_AUTO) and not split_keys and window is None
            and not kvouter_query_tiles and descale is None and mask is None):
        return None
    wl, wr = (int(window[0]), int(window[1])) if window is not None else (0, 0)
    dq, dk, dv = (float(x) for x in descale) if descale is not None else (0.0, 0.0, 0.0)
    mp, mb, mh = mask if mask is not None else (None, 0, 0)
    return Options(PATH_AUTO if path is None else int(path), int(split_keys or 0),
                   1 if window is not None else 0, wl, wr, int(kvouter_query_tiles or 0),
                   dq, dk, dv, mp, int(mb), int(mh))


def _opt_ptr(o):
    return ctypes.byref(o) if o is not None else None


def plan(B, H, N, M, D, dtype=BF16, causal=False, path=None, split_keys=0, window=None,
         kvouter_query_tiles=0, mask_shape=None):
    """The planner's decision for a shape, as a dict (host only).
    ``mask_shape=(Bm, Hm)`` plans for an element mask of that many batches
    and heads (no pointer is needed to plan)."""
    info = PlanInfo()
    o = _options(path, split_keys, window, kvouter_query_tiles,
                 mask=None if mask_shape is None else (1, mask_shape[0], mask_shape[1]))
    _check(lib().fa_plan_query(Shape(B, H, N, M, D), int(dtype), int(bool(causal)),
                               _opt_ptr(o), ctypes.byref(info)))
    d = {f: getattr(info, f) for f, _ in PlanInfo._fields_}
    d["path_name"] = PATH_NAMES.get(d["path"], "?")
    return d


def workspace_bytes(B, H, N, M, D, dtype=BF16, causal=False, path=None, split_keys=0,
                    window=None, kvouter_query_tiles=0, mask_shape=None):
    """Device workspace fwd needs; ``mask_shape=(Bm, Hm)`` for an element mask."""
    o = _options(path, split_keys, window, kvouter_query_tiles,
                 mask=None if mask_shape is None else (1, mask_shape[0], mask_shape[1]))
    return int(lib().fa_fwd_workspace_bytes(Shape(B, H, N, M, D), int(dtype),
                                            int(bool(causal)), _opt_ptr(o)))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float8_e4m3fn:
        return FP8
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16, torch.float32 or "
                    "torch.float8_e4m3fn")


def pack_mask(allowed):
    """Pack a boolean mask [Bm, Hm, N, M] (True = key visible) into the
    library's words: int32 [Bm, Hm, N, ceil(M / 32)], bit j % 32 of word
    j / 32 for key j.  Runs where ``allowed`` lives (torch ops only)."""
    import torch
    if allowed.dim() != 4:
        raise ValueError("mask must be [Bm, Hm, N, M]")
    Bm, Hm, N, M = allowed.shape
    W = (M + 31) // 32
    bits = torch.zeros((Bm, Hm, N, W * 32), dtype=torch.int64, device=allowed.device)
    bits[..., :M] = allowed.to(torch.int64)
    weights = torch.bitwise_left_shift(
        torch.ones(32, dtype=torch.int64, device=allowed.device),
        torch.arange(32, dtype=torch.int64, device=allowed.device))
    words = (bits.view(Bm, Hm, N, W, 32) * weights).sum(dim=-1)      # < 2^32
    words = torch.where(words >= 2 ** 31, words - 2 ** 32, words)     # as int32 bits
    return words.to(torch.int32).contiguous()


def _torch_stream(stream, dev):
    """The stream to run on as a torch stream object: the current stream when
    None, a torch stream as given, or a raw hipStream_t (int) wrapped."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


def _kv_len_arg(kv_len, B, dev):
    """kv_len as a contiguous int32 device tensor of B entries (or None)."""
    import torch
    if kv_len is None:
        return None
    if not isinstance(kv_len, torch.Tensor):
        kv_len = torch.as_tensor(kv_len, dtype=torch.int32)
    kv_len = kv_len.to(device=dev, dtype=torch.int32).contiguous()
    if kv_len.numel() != B:
        raise ValueError("kv_len must have B entries")
    return kv_len


def fwd(q, k, v, scale=None, causal=False, kv_len=None, *, out=None, lse=None,
        workspace=None, path=None, split_keys=0, window=None, kvouter_query_tiles=0,
        descale=None, mask=None, stream=None):
    """Exact attention forward through the C ABI; returns (O, LSE).

    ``window=(left, right)`` restricts query i to keys
    i + off - left .. i + off + right (off = kv_len - N; causal caps right
    at 0): ``causal=True, window=(127, 0)`` is a 128-wide local window.
    float8_e4m3fn inputs (FP8) give a bf16 O; ``descale=(dq, dk, dv)`` says
    that they stand for dq*Q, dk*K, dv*V.  ``mask`` is an element mask as
    packed words, int32 [Bm, Hm, N, ceil(M / 32)] on the device
    (``pack_mask``), Bm in {1, B}, Hm in {1, H}."""
    import torch
    L = lib()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N|M, D]")
    B, H, N, D = q.shape
    M = k.shape[2]
    if tuple(k.shape) != (B, H, M, D) or tuple(v.shape) != (B, H, M, D):
        raise ValueError("k and v must be [B, H, M, D] matching q [B, H, N, D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dt = _dtype_code(q)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _torch_stream(stream, dev)
    # Every temporary (the device copy of kv_len, the workspace) and the
    # outputs are made on the stream the kernels run on, so that the caching
    # allocator never hands their memory to other work while they are in use.
    with torch.cuda.stream(stream):
        kv_len = _kv_len_arg(kv_len, B, dev)
        if out is None:
            out = torch.empty((B, H, N, D), dtype=torch.bfloat16 if dt == FP8 else q.dtype,
                              device=dev)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        opts = _options(path, split_keys, window, kvouter_query_tiles, descale,
                        _mask_arg(mask, B, H, N, M, dev))
        shape = Shape(B, H, N, M, D)
        ws_need = int(L.fa_fwd_workspace_bytes(shape, dt, int(bool(causal)), _opt_ptr(opts)))
        if ws_need and workspace is None:
            workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(),
                kv_len.data_ptr() if kv_len is not None else None,
                out.data_ptr(), lse.data_ptr(), shape, dt, float(scale),
                int(bool(causal)), ws_ptr, ws_len, stream.cuda_stream or None)
        # the plain entry point when no option is set, the extended one otherwise
        st = L.fa_fwd(*args) if opts is None else L.fa_fwd_ex(*args, _opt_ptr(opts))
    _check(st)
    return out, lse


def fwd_noalloc(q, k, v, scale=None, causal=False, kv_len=None, *, out, lse, stream=None):
    """The forward through fa_fwd_noalloc: no workspace, the library's static
    scratch instead.  For callers that cannot allocate, so the outputs must
    be given and ``kv_len`` must be None or an int32 device tensor of B
    entries (nothing is allocated or copied here)."""
    import torch
    L = lib()
    B, H, N, D = q.shape
    M = k.shape[2]
    if tuple(k.shape) != (B, H, M, D) or tuple(v.shape) != (B, H, M, D):
        raise ValueError("k and v must be [B, H, M, D] matching q [B, H, N, D]")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if kv_len is not None and (not isinstance(kv_len, torch.Tensor) or not kv_len.is_cuda
                               or kv_len.dtype != torch.int32 or kv_len.numel() != B
                               or not kv_len.is_contiguous()):
        raise ValueError("kv_len must be None or a contiguous int32 device tensor of B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _torch_stream(stream, q.device)
    st = L.fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          kv_len.data_ptr() if kv_len is not None else None, out.data_ptr(),
                          lse.data_ptr(), Shape(B, H, N, M, D), _dtype_code(q), float(scale),
                          int(bool(causal)), stream.cuda_stream or None)
    _check(st)
    return out, lse


def bwd_workspace_bytes(B, H, N, M, D, dtype=BF16, causal=False, mask_shape=None):
    """Device workspace bwd needs; ``mask_shape=(Bm, Hm)`` for an element mask."""
    o = None if mask_shape is None else _options(None, 0, mask=(1, mask_shape[0], mask_shape[1]))
    return int(lib().fa_bwd_workspace_bytes_ex(Shape(B, H, N, M, D), int(dtype), int(bool(causal)),
                                               _opt_ptr(o)))


def _mask_arg(mask, B, H, N, M, dev):
    """(pointer, Bm, Hm) of packed mask words after checking their shape."""
    import torch
    if mask is None:
        return None
    if mask.dim() != 4 or mask.dtype != torch.int32 or not mask.is_contiguous():
        raise ValueError("mask must be contiguous int32 [Bm, Hm, N, ceil(M / 32)]")
    if not mask.is_cuda or mask.device != dev:
        raise ValueError("mask must be on the device of q")
    Bm, Hm, Nm, Wm = mask.shape
    if Nm != N or Wm != (M + 31) // 32 or Bm not in (1, B) or Hm not in (1, H):
        raise ValueError("mask must be [1 or B, 1 or H, N, ceil(M / 32)]")
    return (mask.data_ptr(), Bm, Hm)


def bwd(q, k, v, o, lse, do, scale=None, causal=False, kv_len=None, *, dq=None, dk=None,
        dv=None, workspace=None, window=None, mask=None, stream=None):
    """Gradients of the forward through the C ABI; returns (dQ, dK, dV).

    ``o`` and ``lse`` must be what ``fwd`` returned for the same q, k, v,
    scale, causal, kv_len, window and mask; ``do`` is the upstream gradient,
    shaped like o.
    """
    import torch
    L = lib()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, N, D = q.shape
    M = k.shape[2]
    if tuple(k.shape) != (B, H, M, D) or tuple(v.shape) != (B, H, M, D):
        raise ValueError("k and v must be [B, H, M, D] matching q [B, H, N, D]")
    if tuple(o.shape) != (B, H, N, D) or tuple(do.shape) != (B, H, N, D):
        raise ValueError("o and do must be shaped like q")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == do.dtype):
        raise TypeError("q, k, v, o and do must share one dtype")
    dt = _dtype_code(q)
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = _torch_stream(stream, dev)
    with torch.cuda.stream(stream):  # temporaries and outputs on the kernels' stream
        kv_len = _kv_len_arg(kv_len, B, dev)
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        shape = Shape(B, H, N, M, D)
        opts = _options(None, 0, window, mask=_mask_arg(mask, B, H, N, M, dev))
        need = int(L.fa_bwd_workspace_bytes_ex(shape, dt, int(bool(causal)), _opt_ptr(opts)))
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = L.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         do.data_ptr(), kv_len.data_ptr() if kv_len is not None else None,
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), shape, dt, float(scale),
                         int(bool(causal)), ws_ptr, ws_len, stream.cuda_stream or None,
                         _opt_ptr(opts))
    _check(st)
    return dq, dk, dv
