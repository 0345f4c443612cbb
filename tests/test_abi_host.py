"""The C-ABI library on the host: it loads, exports what the header declares,
plans shapes, and rejects bad arguments before any launch (no GPU needed).

Every fa_fwd call here fails a host-side check, so nothing is ever launched:
the fake pointers below are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import exact_attention_33_amd as fa
from exact_attention_33_amd import Options, Shape
from tests.mask_layout import mask_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path),
                                reason="library not built (python -m exact_attention_33_amd.build)")

# Fake but 256-byte aligned device addresses; only used where a check fails first.
P = 0x10000


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = fa.lib()
    declared = header_functions()
    assert sorted(fa.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.fa_abi_version() == 8


def test_status_strings():
    L = fa.lib()
    names = [L.fa_status_str(i).decode() for i in range(8)]
    assert names == ["FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED",
                     "FA_ERR_ALIGN", "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_ARG"]
    assert L.fa_status_str(99).decode() == "FA_ERR_UNKNOWN"


def test_planner_paths():
    p = fa.plan(2, 32, 8192, 8192, 128, fa.BF16, True)
    assert p["path_name"] == "prefill" and p["block_k"] == 64
    assert p["block_q"] == p["threads"] and p["block_q"] % 64 == 0  # 64 queries per wave
    assert p["grid"] == 256 and p["workspace_bytes"] == 0         # persistent: one per CU
    assert fa.plan(2, 32, 8192, 8192, 128, fa.BF16, False)["grid"] == 32 * 64
    assert fa.plan(2, 32, 8192, 8192, 128, fa.BF16, True, window=(127, 0))["grid"] == 32 * 64
    assert fa.plan(1, 3, 300, 300, 128, fa.BF16, True)["grid"] == 8   # 6 items, rounded up
    assert p["lds_bytes"] <= 160 * 1024                      # fits one compute unit's LDS
    p = fa.plan(1, 1, 128, 128, 64, fa.F32, False)
    assert p["path_name"] == "f32" and p["grid"] == 8
    p = fa.plan(32, 32, 1, 32768, 128, fa.BF16, False)
    assert p["path_name"] == "splitkv"
    assert p["splits"] * p["block_k"] >= 32768
    assert p["workspace_bytes"] >= 32 * 32 * p["splits"] * (128 + 1) * 4
    # forcing paths
    assert fa.plan(1, 2, 1, 500, 64, fa.BF16, True, path=fa.PATH_PREFILL)["path_name"] == "prefill"
    # the largest K/V that prefill addresses: M * D * 2 = 2^31 - 256 bytes
    assert fa.plan(1, 1, 16, (1 << 23) - 1, 128, fa.BF16, False)["path_name"] == "prefill"
    p = fa.plan(1, 2, 1, 500, 64, fa.BF16, False, path=fa.PATH_SPLITKV, split_keys=64)
    assert p["splits"] == 8 and p["block_k"] == 64
    # empty problems plan fine and need nothing
    assert fa.plan(0, 4, 16, 16, 64)["grid"] == 0
    assert fa.workspace_bytes(1, 1, 1, 0, 64) == 0


@pytest.mark.parametrize("args,status", [
    ((1, 1, 16, 16, 96, fa.BF16, False), "FA_ERR_UNSUPPORTED"),
    ((1, 1, 16, 16, 64, 7, False), "FA_ERR_UNSUPPORTED"),
    ((-1, 1, 16, 16, 64, fa.BF16, False), "FA_ERR_SHAPE"),
    ((1, 1, 16, -16, 64, fa.BF16, False), "FA_ERR_SHAPE"),
    # prefill addresses one (batch, head) of K/V with 32-bit byte offsets
    ((1, 1, 16, 1 << 23, 128, fa.BF16, False), "FA_ERR_UNSUPPORTED"),
])
def test_planner_rejects(args, status):
    with pytest.raises(fa.FaError) as ei:
        fa.plan(*args)
    assert ei.value.name == status


@pytest.mark.parametrize("kw,status", [
    (dict(path=fa.PATH_PREFILL), "FA_ERR_UNSUPPORTED"),   # f32 data on the bf16 path
    (dict(path=9), "FA_ERR_ARG"),
])
def test_planner_rejects_options_f32(kw, status):
    with pytest.raises(fa.FaError) as ei:
        fa.plan(1, 1, 16, 16, 64, fa.F32, False, **kw)
    assert ei.value.name == status


def test_planner_rejects_options_bf16():
    with pytest.raises(fa.FaError) as ei:
        fa.plan(1, 1, 4, 16, 64, fa.BF16, False, path=fa.PATH_SPLITKV)
    assert ei.value.name == "FA_ERR_UNSUPPORTED"
    with pytest.raises(fa.FaError) as ei:
        fa.plan(1, 1, 1, 16, 64, fa.BF16, False, split_keys=100)
    assert ei.value.name == "FA_ERR_ARG"
    with pytest.raises(fa.FaError) as ei:
        fa.plan(1, 1, 1, 16, 64, fa.BF16, False, path=fa.PATH_F32)
    assert ei.value.name == "FA_ERR_UNSUPPORTED"


def call(q=P, k=P, v=P, kvl=None, o=P, lse=P, shape=(1, 2, 16, 16, 64), dt=fa.BF16,
         scale=0.125, causal=0, ws=None, ws_len=0, opt=None):
    L = fa.lib()
    st = L.fa_fwd_ex(q, k, v, kvl, o, lse, Shape(*shape), dt, scale, causal, ws, ws_len,
                     None, ctypes.byref(opt) if opt else None)
    return L.fa_status_str(st).decode(), L.fa_last_error().decode()


def test_fwd_rejects_before_launch():
    assert call(q=None)[0] == "FA_ERR_NULL"
    assert call(o=None)[0] == "FA_ERR_NULL"
    assert call(lse=None)[0] == "FA_ERR_NULL"
    assert call(k=None)[0] == "FA_ERR_NULL"
    assert call(q=P + 8)[0] == "FA_ERR_ALIGN"
    assert call(v=P + 4)[0] == "FA_ERR_ALIGN"
    assert call(lse=P + 2)[0] == "FA_ERR_ALIGN"
    assert call(kvl=P + 1)[0] == "FA_ERR_ALIGN"
    assert call(scale=float("nan"))[0] == "FA_ERR_ARG"
    assert call(scale=float("inf"))[0] == "FA_ERR_ARG"
    assert call(scale=-1.0)[0] == "FA_ERR_ARG"
    assert call(shape=(1, 2, 16, 16, 80))[0] == "FA_ERR_UNSUPPORTED"
    assert call(shape=(1, 2, -3, 16, 64))[0] == "FA_ERR_SHAPE"
    st, msg = call(shape=(1, 2, 1, 4096, 64))   # split-KV needs a workspace
    assert st == "FA_ERR_WORKSPACE" and "workspace" in msg
    need = fa.workspace_bytes(1, 2, 1, 4096, 64)
    assert call(shape=(1, 2, 1, 4096, 64), ws=P, ws_len=need - 1)[0] == "FA_ERR_WORKSPACE"
    assert call(shape=(1, 2, 1, 4096, 64), ws=P + 16, ws_len=need)[0] == "FA_ERR_ALIGN"


def test_fwd_empty_problem_is_a_no_op():
    # B*H*N == 0: nothing to compute, so OK without touching any pointer.
    assert call(q=None, k=None, v=None, o=None, lse=None, shape=(0, 2, 16, 16, 64))[0] == "FA_OK"
    assert call(q=None, k=None, v=None, o=None, lse=None, shape=(1, 2, 0, 16, 64))[0] == "FA_OK"


def bwd_call(shape=(1, 2, 16, 16, 64), dt=fa.BF16, scale=0.125, causal=0, ws=P, ws_len=None,
             **ptrs):
    names = ["q", "k", "v", "o", "lse", "do", "kvl", "dq", "dk", "dv"]
    vals = {n: P for n in names}
    vals["kvl"] = None
    vals.update(ptrs)
    if ws_len is None:
        ws_len = fa.bwd_workspace_bytes(*shape)
    L = fa.lib()
    st = L.fa_bwd(*[vals[n] for n in names], Shape(*shape), dt, scale, causal, ws, ws_len, None)
    return L.fa_status_str(st).decode(), L.fa_last_error().decode()


def test_bwd_workspace_size():
    # Lg and D per row, rows rounded up to 256
    assert fa.bwd_workspace_bytes(2, 32, 8192, 8192, 128) == 2 * 32 * 8192 * 8
    assert fa.bwd_workspace_bytes(1, 3, 300, 10, 64) == 3 * 512 * 8
    assert fa.bwd_workspace_bytes(1, 1, 0, 10, 64) == 0
    assert fa.bwd_workspace_bytes(1, 1, 16, 16, 64, dtype=fa.F32) == 0


def test_bwd_rejects_before_launch():
    for name in ("q", "o", "lse", "do", "dq", "k", "v", "dk", "dv"):
        assert bwd_call(**{name: None})[0] == "FA_ERR_NULL", name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwd_call(**{name: P + 8})[0] == "FA_ERR_ALIGN", name
    assert bwd_call(lse=P + 2)[0] == "FA_ERR_ALIGN"
    assert bwd_call(kvl=P + 1)[0] == "FA_ERR_ALIGN"
    assert bwd_call(dt=fa.F32)[0] == "FA_ERR_UNSUPPORTED"
    assert bwd_call(shape=(1, 2, 16, 16, 80))[0] == "FA_ERR_UNSUPPORTED"
    assert bwd_call(shape=(1, 2, -3, 16, 64))[0] == "FA_ERR_SHAPE"
    # Q/dO (or K/V) bytes per (batch, head) must stay below 2^31
    assert bwd_call(shape=(1, 1, 1 << 23, 16, 128))[0] == "FA_ERR_UNSUPPORTED"
    assert bwd_call(shape=(1, 1, 16, 1 << 23, 128))[0] == "FA_ERR_UNSUPPORTED"
    for bad in (float("nan"), float("inf"), -1.0):
        assert bwd_call(scale=bad)[0] == "FA_ERR_ARG"
    st, msg = bwd_call(ws=None)
    assert st == "FA_ERR_WORKSPACE" and "workspace" in msg
    need = fa.bwd_workspace_bytes(1, 2, 16, 16, 64)
    assert bwd_call(ws_len=need - 1)[0] == "FA_ERR_WORKSPACE"
    assert bwd_call(ws=P + 16)[0] == "FA_ERR_ALIGN"


def test_bwd_empty_problem_is_a_no_op():
    none = {n: None for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")}
    assert bwd_call(shape=(0, 2, 16, 16, 64), ws=None, **none)[0] == "FA_OK"
    assert bwd_call(shape=(1, 2, 0, 0, 64), ws=None, **none)[0] == "FA_OK"


def test_window_options_checked():
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, window=(-1, 0))
    assert e.value.name == "FA_ERR_ARG"
    L = fa.lib()
    info = fa.PlanInfo()
    bad = Options(0, 0, 2, 0, 0, 0, 0.0, 0.0, 0.0)
    st = L.fa_plan_query(Shape(1, 1, 16, 16, 64), fa.BF16, 0, ctypes.byref(bad), ctypes.byref(info))
    assert L.fa_status_str(st).decode() == "FA_ERR_ARG"
    # a windowed single query runs on the prefill kernel; split-KV has no window
    assert fa.plan(4, 2, 1, 50000, 128, window=(127, 0))["path_name"] == "prefill"
    assert fa.plan(4, 2, 1, 50000, 128)["path_name"] == "splitkv"
    with pytest.raises(fa.FaError) as e:
        fa.plan(4, 2, 1, 50000, 128, path=fa.PATH_SPLITKV, window=(127, 0))
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    assert fa.plan(1, 1, 16, 16, 64, fa.F32, window=(3, 0))["path_name"] == "f32"
    # the backward checks its window the same way
    opt = Options(0, 0, 1, -1, 0, 0, 0.0, 0.0, 0.0)
    st = L.fa_bwd_ex(*([P] * 6), None, P, P, P, Shape(1, 2, 16, 16, 64), fa.BF16, 0.125, 1, P,
                     fa.bwd_workspace_bytes(1, 2, 16, 16, 64), None, ctypes.byref(opt))
    assert L.fa_status_str(st).decode() == "FA_ERR_ARG"


def test_kvouter_plan():
    """The key/value-outer ablation: never chosen by the planner; one or more
    256-query tiles per workgroup; a float32 accumulator workspace."""
    assert fa.plan(2, 32, 8192, 8192, 128, causal=True)["path_name"] == "prefill"
    p = fa.plan(2, 32, 8192, 8192, 128, causal=True, path=fa.PATH_KVOUTER)
    assert p["path_name"] == "kvouter" and p["grid"] == 32 * 64 and p["block_q"] == 256
    assert p["workspace_bytes"] >= 64 * 8192 * 130 * 4
    p = fa.plan(2, 32, 8192, 8192, 128, causal=True, path=fa.PATH_KVOUTER, kvouter_query_tiles=1000)
    assert p["grid"] == 64 and p["block_q"] == 8192
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, path=fa.PATH_KVOUTER, window=(3, 0))
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, path=fa.PATH_KVOUTER, kvouter_query_tiles=-1)
    assert e.value.name == "FA_ERR_ARG"
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, fa.F32, path=fa.PATH_KVOUTER)
    assert e.value.name == "FA_ERR_UNSUPPORTED"


def test_fp8_plan():
    p = fa.plan(2, 32, 8192, 8192, 128, fa.FP8, True)
    assert p["path_name"] == "fp8" and p["threads"] == 512 and p["grid"] == 256   # persistent
    assert fa.plan(2, 32, 8192, 8192, 128, fa.FP8, False)["grid"] == 32 * 64
    assert fa.plan(4, 2, 1, 5000, 64, fa.FP8)["path_name"] == "fp8"   # no split-KV for fp8
    for kw, st in ((dict(window=(3, 0)), "FA_ERR_UNSUPPORTED"),
                   (dict(path=fa.PATH_PREFILL), "FA_ERR_UNSUPPORTED"),
                   (dict(path=fa.PATH_SPLITKV), "FA_ERR_UNSUPPORTED")):
        with pytest.raises(fa.FaError) as e:
            fa.plan(1, 1, 16, 16, 64, fa.FP8, **kw)
        assert e.value.name == st, kw
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, fa.BF16, path=fa.PATH_FP8)
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    L = fa.lib()
    info = fa.PlanInfo()
    bad = Options(0, 0, 0, 0, 0, 0, -1.0, 0.0, 0.0)
    st = L.fa_plan_query(Shape(1, 1, 16, 16, 64), fa.FP8, 0, ctypes.byref(bad), ctypes.byref(info))
    assert L.fa_status_str(st).decode() == "FA_ERR_ARG"


def test_mask_plan():
    """An element mask runs on the prefill path (also for N = 1) and the
    fp32 path; the prefill path then needs workspace for its tile lists,
    tile classes and blocks of mask words."""
    p = fa.plan(2, 32, 8192, 8192, 128, fa.BF16, True, mask_shape=(1, 1))
    assert p["path_name"] == "prefill"
    # 32 lists of 129 int32 (16,512 B -> 16,640), 32 x 128 class bytes, then
    # 32 rows of 1 + 128 blocks of 2 KB, then (causal) the walk order of the
    # 2 x 32 x 32 work items
    assert p["workspace_bytes"] == 16640 + 4096 + 32 * 129 * 2048 + 2048 * 4 == \
        mask_layout(8192, 8192, 1, 1, items=2048)["end"]
    p2 = fa.plan(2, 32, 8192, 8192, 128, fa.BF16, True, mask_shape=(2, 32))
    assert p2["workspace_bytes"] == mask_layout(8192, 8192, 2, 32, items=2048)["end"]
    assert fa.plan(3, 2, 600, 700, 64, fa.BF16, mask_shape=(3, 1))["workspace_bytes"] == \
        mask_layout(600, 700, 3, 1)["end"]
    assert fa.plan(2, 32, 8192, 8192, 128, fa.BF16, True)["workspace_bytes"] == 0
    assert fa.plan(4, 2, 1, 5000, 64, fa.BF16, mask_shape=(4, 1))["path_name"] == "prefill"
    assert fa.plan(4, 2, 5, 50, 64, fa.F32, mask_shape=(1, 2))["workspace_bytes"] == 0
    for kw, st in ((dict(path=fa.PATH_SPLITKV), "FA_ERR_UNSUPPORTED"),
                   (dict(path=fa.PATH_KVOUTER), "FA_ERR_UNSUPPORTED")):
        with pytest.raises(fa.FaError) as e:
            fa.plan(2, 2, 1, 700, 64, fa.BF16, mask_shape=(1, 1), **kw)
        assert e.value.name == st, kw
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 16, 16, 64, fa.FP8, mask_shape=(1, 1))
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    for shape in ((3, 1), (1, 5), (-1, 1)):            # B = 2, H = 4
        with pytest.raises(fa.FaError) as e:
            fa.plan(2, 4, 16, 16, 64, fa.BF16, mask_shape=shape)
        assert e.value.name == "FA_ERR_ARG", shape
    with pytest.raises(fa.FaError) as e:               # the list outgrows LDS
        fa.plan(1, 1, 16, 262144, 64, fa.BF16, mask_shape=(1, 1))
    assert e.value.name == "FA_ERR_UNSUPPORTED"
    assert fa.plan(1, 1, 16, 262080, 64, fa.BF16, mask_shape=(1, 1))["path_name"] == "prefill"


def test_bwd_mask_checks():
    """The backward takes an element mask: its workspace adds both passes'
    tile lists, classes and blocks of mask words; bad mask shapes and sizes
    are rejected before any launch."""
    L = fa.lib()
    base = fa.bwd_workspace_bytes(2, 4, 1000, 1000, 64)
    with_mask = fa.bwd_workspace_bytes(2, 4, 1000, 1000, 64, mask_shape=(2, 1))
    lists = 2 * 1 * 4 * (16 + 1) * 4                    # 4 query tiles, 16 key tiles + count
    stages = 2 * 1 * 4 * (16 + 1) * 4                   # 4 key tiles, 16 query stages + count
    cls = 2 * 4 * 16                                    # one byte per (query tile, key tile)
    a = lambda n: (n + 255) // 256 * 256
    off_blocks = a(base) + a(lists) + a(stages) + a(cls)
    rows = 2 * 4                                        # rows of 1 + 16 blocks, each pass
    assert with_mask == a(off_blocks + rows * 17 * 2048) + a(cls) + rows * 17 * 2048
    assert with_mask == mask_layout(1000, 1000, 2, 1, a(base), stages=True)["end"]
    assert fa.bwd_workspace_bytes(2, 4, 1000, 1000, 64, mask_shape=(3, 1)) == 0
    for mb, mh, shape, st_want in ((3, 1, (2, 4, 16, 16, 64), "FA_ERR_ARG"),
                                   (1, 5, (2, 4, 16, 16, 64), "FA_ERR_ARG"),
                                   (1, 1, (1, 1, 16, 262144, 64), "FA_ERR_UNSUPPORTED"),
                                   (1, 1, (1, 1, 262144, 16, 64), "FA_ERR_UNSUPPORTED")):
        opt = Options(0, 0, 0, 0, 0, 0, 0.0, 0.0, 0.0, P, mb, mh)
        st = L.fa_bwd_ex(*([P] * 10), Shape(*shape), fa.BF16, 0.1, 0, P, 1 << 30, None,
                         ctypes.byref(opt))
        assert L.fa_status_str(st).decode() == st_want, (mb, mh, shape)
    opt = Options(0, 0, 0, 0, 0, 0, 0.0, 0.0, 0.0, P + 2, 1, 1)     # misaligned words
    st = L.fa_bwd_ex(*([P] * 10), Shape(1, 1, 16, 16, 64), fa.BF16, 0.1, 0, P, 1 << 30, None,
                     ctypes.byref(opt))
    assert L.fa_status_str(st).decode() == "FA_ERR_ALIGN"
    opt = Options(0, 0, 0, 0, 0, 0, 0.0, 0.0, 0.0, P, 1, 1)          # workspace too small
    need = fa.bwd_workspace_bytes(1, 1, 16, 16, 64, mask_shape=(1, 1))
    st = L.fa_bwd_ex(*([P] * 10), Shape(1, 1, 16, 16, 64), fa.BF16, 0.1, 0, P, need - 1, None,
                     ctypes.byref(opt))
    assert L.fa_status_str(st).decode() == "FA_ERR_WORKSPACE"


def test_pack_mask_layout():
    """Bit j % 32 of word j / 32 is key j (numpy's little-endian bit packing
    read as little-endian words gives the same words)."""
    import numpy as np
    import torch
    rng = np.random.default_rng(3)
    for M in (1, 31, 32, 33, 100, 130):
        a = rng.random((2, 3, 5, M)) < 0.5
        got = fa.pack_mask(torch.from_numpy(a)).numpy().view(np.uint32)
        W = (M + 31) // 32
        padded = np.zeros((2, 3, 5, W * 32), dtype=bool)
        padded[..., :M] = a
        want = np.packbits(padded, axis=-1, bitorder="little").view("<u4")
        assert got.shape == (2, 3, 5, W) and np.array_equal(got, want), M


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """fa_fwd_noalloc turns away a shape whose workspace exceeds the static
    scratch with FA_ERR_WORKSPACE and a message naming both sizes, before any
    device call (this runs without a GPU).  The limit is the header's."""
    L = fa.lib()
    src = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES
    # split-KV decode: 32 x 32 heads, 2^20 keys -> 2048 splits each, far above 48 MiB
    shape = (32, 32, 1, 1 << 20, 128)
    need = fa.workspace_bytes(*shape)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    st = L.fa_fwd_noalloc(P, P, P, None, P, P, Shape(*shape), fa.BF16, 0.1, 0, None)
    assert L.fa_status_str(st).decode() == "FA_ERR_WORKSPACE"
    msg = L.fa_last_error().decode()
    assert str(need) in msg and str(fa.NOALLOC_SCRATCH_BYTES) in msg
    # the largest decode cache the header quotes fits
    assert fa.workspace_bytes(32, 32, 1, 48000, 128) <= fa.NOALLOC_SCRATCH_BYTES


def test_prefill_key_split_plan():
    """options.split_keys on the prefill path: one workgroup per (query tile,
    chunk of keys), workspace for the float32 partial results and their
    log-sum-exps, no window and no element mask."""
    p = fa.plan(1, 8, 1024, 1024, 64, fa.BF16, True, split_keys=256)
    assert p["path_name"] == "prefill" and p["splits"] == 4 and p["grid"] == 4 * 8 * 4
    rows = 4 * 8 * 1024
    assert p["workspace_bytes"] == (rows * 64 * 4 + 255) // 256 * 256 + rows * 4
    assert fa.plan(1, 8, 1024, 1024, 64, fa.BF16, True)["workspace_bytes"] == 0     # no split: none
    assert fa.plan(2, 2, 300, 0, 128, fa.BF16, False, split_keys=64)["splits"] == 1  # M = 0: one chunk
    assert fa.plan(2, 2, 1, 700, 64, fa.BF16, False, split_keys=256)["path_name"] == "splitkv"
    q = fa.plan(2, 2, 1, 700, 64, fa.BF16, False, split_keys=256, path=fa.PATH_PREFILL)
    assert q["path_name"] == "prefill" and q["splits"] == 3
    for kw in (dict(window=(127, 0)), dict(mask_shape=(1, 1))):
        with pytest.raises(fa.FaError) as e:
            fa.plan(1, 2, 300, 300, 64, fa.BF16, True, split_keys=128, **kw)
        assert e.value.name == "FA_ERR_UNSUPPORTED", kw
