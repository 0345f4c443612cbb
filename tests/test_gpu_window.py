"""GPU parity of local (banded) attention: the HIP kernels with a window
against the fp64 oracle with the same window ("FlashAttention: attention was
never compute-bound", Exact means exact: "a 128-wide local window").

Key j is visible to query i only if i + off - left <= j <= i + off + right
(off = kv_len - N; causal caps right at 0).  Small cases compare every
element across several query and key tiles, with windows narrower than a
tile, wider than a workgroup, two-sided, and with ragged tails; the long
workload is compared on sampled rows.
"""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref, attention_rows
from tests.gpu_helpers import abi_scale, compare, default_scale, host64, sample_picks

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make(seed, B, H, N, M, D, dtype):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, dtype, DEV) for x in (q, k, v))


CASES = [
    # B, H, N, M, D, causal, kv_len, window
    (1, 2, 300, 300, 128, True, None, (127, 0)),      # the pages' 128-wide window
    (1, 2, 300, 300, 64, True, None, (3, 0)),          # narrower than a key block
    (2, 2, 600, 600, 128, True, [600, 333], (300, 0)), # wider than a query tile
    (1, 2, 257, 257, 128, False, None, (64, 64)),      # two-sided
    (1, 1, 200, 500, 64, False, None, (50, 10)),       # N != M, off > 0
    (2, 1, 150, 90, 128, True, None, (20, 5)),         # N > M: early rows see nothing
    (1, 1, 130, 130, 128, False, None, (0, 0)),        # one key per query
    (2, 2, 1, 3000, 128, True, [3000, 1111], (127, 0)),  # single queries on prefill
    (1, 1, 700, 700, 128, True, None, (5000, 0)),      # window wider than the sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}w{}-{}".format(
    *c[:5], "c" if c[5] else "", *c[7]))
def test_window_bf16(case):
    B, H, N, M, D, causal, kvl, win = case
    print(f"[window] case {case}", flush=True)
    q, k, v = make(60 + N, B, H, N, M, D, "bf16")
    kvt = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device=DEV)
    if kvl is not None:
        inputs.poison_tail(k, v, kvl)
    o, l = fa.fwd(q, k, v, scale=default_scale(D), causal=causal, kv_len=kvt, window=win)
    torch.cuda.synchronize()
    kk, vv = host64(k), host64(v)
    kk[np.isnan(kk)] = 0
    vv[np.isnan(vv)] = 0
    Or, Lr = attention_ref(host64(q), kk, vv, default_scale(D), causal,
                           None if kvl is None else np.asarray(kvl), window=win)
    compare(host64(o), host64(l), Or, Lr, "bf16", f"window {case}")


@pytest.mark.parametrize("causal,win", [(True, (7, 0)), (False, (5, 9))])
def test_window_f32(causal, win):
    q, k, v = make(71, 1, 2, 150, 170, 64, "f32")
    o, l = fa.fwd(q, k, v, scale=abi_scale(0.2), causal=causal, window=win)
    torch.cuda.synchronize()
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), abi_scale(0.2), causal, window=win)
    compare(host64(o), host64(l), Or, Lr, "f32", f"f32 window {win}")


@pytest.mark.parametrize("win", [(127, 0), (2047, 0)])
def test_window_long_workload_sampled(win):
    """B=2, H=32, N=M=8192, D=128 causal with a window, as the bench runs it."""
    w = inputs.WORKLOADS["prefill_long_d128"]
    print(f"[window] long workload window={win}", flush=True)
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", torch.device(DEV))
    o, l = fa.fwd(q, k, v, causal=True, window=win)
    torch.cuda.synchronize()
    picks = sample_picks(w.B, w.H, w.N, n_heads=4, seed=3)
    Or, Lr = attention_rows(lambda b, h: host64(q[b, h]), lambda b, h: host64(k[b, h]),
                            lambda b, h: host64(v[b, h]), default_scale(w.D), True, None,
                            picks, window=win)
    og = np.stack([host64(o[b, h, i]) for b, h, i in picks])
    lg = np.array([float(l[b, h, i]) for b, h, i in picks])
    compare(og, lg, Or, Lr, "bf16", f"long window {win}")
