"""GPU invariants that hold at any size (checked on the HIP path alone)."""
import math

import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def dev(seed, B, H, N, M, D):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, "bf16", DEV) for x in (q, k, v))


@pytest.mark.parametrize("D", [64, 128])
def test_causal_row0_is_v0(D):
    """Causal with N = M: query 0 sees only key 0, so O_0 = v_0 exactly and
    LSE_0 = scale * q_0 . k_0."""
    q, k, v = dev(301, 2, 4, 384, 384, D)
    say(f"row0 D={D}")
    o, l = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) / math.sqrt(D)
    assert torch.max(torch.abs(l[:, :, 0].double() - s00)).item() <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean(causal):
    """Q = 0: O_i is the mean of the visible V rows, LSE_i = ln(#visible)."""
    _, k, v = dev(302, 1, 2, 300, 300, 128)
    q = torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16, device=DEV)
    say(f"zero query causal={causal}")
    o, l = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    vv = v.double()
    if causal:
        mean = torch.cumsum(vv, dim=2) / torch.arange(1, 301, device=DEV).double()[:, None]
        lse = torch.log(torch.arange(1, 301, device=DEV).double())
    else:
        mean = vv.mean(dim=2, keepdim=True).expand_as(vv)
        lse = torch.full((300,), math.log(300), device=DEV, dtype=torch.float64)
    assert torch.max(torch.abs(o.double() - mean)).item() <= 2e-2
    assert torch.max(torch.abs(l.double() - lse)).item() <= 1e-3


def test_run_to_run_bitwise_deterministic():
    q, k, v = dev(303, 2, 3, 700, 700, 128)
    say("determinism prefill")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    qd, kd, vd = dev(304, 3, 2, 1, 4000, 128)
    say("determinism decode")
    o3, l3 = fa.fwd(qd, kd, vd, kv_len=[4000, 17, 2500])
    o4, l4 = fa.fwd(qd, kd, vd, kv_len=[4000, 17, 2500])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_split_count_invariance():
    """Different split sizes and the prefill path give the same decode result
    within rounding (the merge is exact in real arithmetic)."""
    q, k, v = dev(305, 2, 4, 1, 6000, 128)
    kvl = [6000, 3001]
    outs = []
    for kw in (dict(path=fa.PATH_SPLITKV, split_keys=64), dict(path=fa.PATH_SPLITKV, split_keys=4096),
               dict(path=fa.PATH_PREFILL)):
        say(f"split invariance {kw}")
        outs.append(fa.fwd(q, k, v, kv_len=kvl, **kw))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.max(torch.abs(o.float() - outs[0][0].float())).item() <= 1e-2
        assert torch.max(torch.abs(l - outs[0][1])).item() <= 1e-4


def test_shift_invariance():
    """Adding delta to every score of a row (K[:, 0] = 1, Q[:, 0] += delta/scale)
    leaves O unchanged and shifts LSE by delta."""
    q, k, v = dev(306, 1, 2, 256, 256, 64)
    k[..., 0] = 1.0
    scale = 1 / 8
    say("shift invariance")
    o0, l0 = fa.fwd(q, k, v, scale=scale, causal=True)
    q2 = q.clone()
    q2[..., 0] = q2[..., 0].float().add(64.0 / scale).to(torch.bfloat16)  # exact in bf16
    o1, l1 = fa.fwd(q2, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    shift = (q2[..., 0].double() - q[..., 0].double()) * scale
    assert torch.max(torch.abs(o1.float() - o0.float())).item() <= 2e-2
    assert torch.max(torch.abs((l1.double() - l0.double()) - shift)).item() <= 1e-3
