"""GPU parity of the fp8 forward (OCP E4M3 Q, K, V with per-tensor descale
factors) against the fp64 oracle run on the exact dequantized inputs
(descale * E4M3 value), within the elementwise bound derived in
``gpu_helpers.fp8_bound``; LSE within 1e-3."""

import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref
from tests.gpu_helpers import default_scale, fp8_bound, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
AMAX = 448.0


def quantize(x):
    """Per-tensor scaling to the E4M3 range: returns (x8, descale)."""
    d = float(x.abs().max()) / AMAX or 1.0
    return (x / d).to(torch.float8_e4m3fn), d


def check(q8, k8, v8, dq, dk, dv, o, l, scale, causal, kvl, what):
    B, H, N, D = q8.shape
    M = k8.shape[2]
    kvs = [M] * B if kvl is None else list(kvl)
    q = host64(q8) * dq
    k = host64(k8) * dk
    v = host64(v8) * dv
    Or, Lr = attention_ref(q, k, v, scale, causal, None if kvl is None else np.asarray(kvl))
    og, lg = host64(o), host64(l)
    assert not np.isnan(og).any() and not np.isnan(lg).any(), what
    assert np.array_equal(np.isneginf(lg), np.isneginf(Lr)), f"{what}: empty rows"
    worst = 0.0
    for b in range(B):
        for h in range(H):
            bound = fp8_bound(q[b, h], k[b, h], v[b, h], scale, causal, kvs[b])
            err = np.abs(og[b, h] - Or[b, h])
            assert np.all(err <= 2 * bound), (f"{what} b{b} h{h}: {int((err > 2 * bound).sum())} "
                                              f"elements over the bound, max err {err.max():.3e}")
            worst = max(worst, float((err / (2 * bound)).max()))
    fin = np.isfinite(Lr)
    el = float(np.max(np.abs(lg[fin] - Lr[fin]))) if fin.any() else 0.0
    assert el <= 1e-3, f"{what}: LSE {el:.3e}"
    print(f"[fp8] {what}: worst error / allowance {worst:.3f}, LSE {el:.2e}", flush=True)


CASES = [
    # B, H, N, M, D, causal, kv_len
    (1, 2, 256, 256, 128, False, None),
    (1, 2, 300, 300, 128, True, None),
    (2, 2, 200, 333, 64, True, [333, 120]),
    (1, 2, 150, 90, 128, True, None),        # N > M: early rows see nothing
    (2, 1, 1, 700, 128, False, [700, 0]),    # single queries, an empty sequence
    (1, 1, 520, 640, 64, False, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}{}".format(
    *c[:5], "c" if c[5] else "", "kv" if c[6] else ""))
def test_fp8_matches_oracle(case):
    B, H, N, M, D, causal, kvl = case
    print(f"[fp8] case {case}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(90 + N + M)
    q = torch.randn(B, H, N, D, generator=g, device=DEV)
    k = torch.randn(B, H, M, D, generator=g, device=DEV)
    v = torch.randn(B, H, M, D, generator=g, device=DEV)
    (q8, dq), (k8, dk), (v8, dv) = quantize(q), quantize(k), quantize(v)
    kvt = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device=DEV)
    scale = default_scale(D)
    o, l = fa.fwd(q8, k8, v8, scale=scale, causal=causal, kv_len=kvt, descale=(dq, dk, dv))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    check(q8, k8, v8, dq, dk, dv, o, l, scale, causal, kvl, f"{case}")


def test_fp8_long_workload_heads():
    """B=2, H=32, N=M=8192, D=128 causal, as the bench runs it: two whole heads."""
    w = inputs.WORKLOADS["prefill_long_d128"]
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", torch.device(DEV))
    (q8, dq), (k8, dk), (v8, dv) = quantize(q.float()), quantize(k.float()), quantize(v.float())
    scale = default_scale(w.D)
    o, l = fa.fwd(q8, k8, v8, scale=scale, causal=True, descale=(dq, dk, dv))
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 31)):
        check(q8[b:b + 1, h:h + 1].contiguous(), k8[b:b + 1, h:h + 1].contiguous(),
              v8[b:b + 1, h:h + 1].contiguous(), dq, dk, dv, o[b:b + 1, h:h + 1],
              l[b:b + 1, h:h + 1], scale, True, None, f"long b{b} h{h}")
