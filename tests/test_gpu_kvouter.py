"""GPU parity of the key/value-outer ablation path (the first version's loop
order: key tiles outside, query tiles inside, the output accumulator and
row statistics read and written back in HBM for every key tile) against the
fp64 oracle -- the same function as every other path."""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref, attention_rows
from tests.gpu_helpers import compare, default_scale, host64, sample_picks

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make(seed, B, H, N, M, D):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, "bf16", DEV) for x in (q, k, v))


CASES = [
    # B, H, N, M, D, causal, kv_len, query tiles per workgroup
    (1, 2, 300, 300, 128, True, None, 0),
    (1, 2, 300, 300, 128, True, None, 100),       # one workgroup per (batch, head)
    (2, 2, 600, 517, 64, False, [517, 200], 2),
    (1, 2, 200, 90, 128, True, None, 0),          # N > M: early rows see nothing
    (2, 1, 130, 260, 128, True, [260, 0], 0),     # an empty sequence
    (1, 1, 1, 700, 128, False, None, 0),          # one query
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}t{}".format(
    *c[:5], "c" if c[5] else "", c[7]))
def test_kvouter_matches_oracle(case):
    B, H, N, M, D, causal, kvl, tpg = case
    print(f"[kvouter] case {case}", flush=True)
    q, k, v = make(80 + N, B, H, N, M, D)
    kvt = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device=DEV)
    if kvl is not None:
        inputs.poison_tail(k, v, kvl)
    o, l = fa.fwd(q, k, v, scale=default_scale(D), causal=causal, kv_len=kvt,
                  path=fa.PATH_KVOUTER, kvouter_query_tiles=tpg)
    torch.cuda.synchronize()
    kk, vv = host64(k), host64(v)
    kk[np.isnan(kk)] = 0
    vv[np.isnan(vv)] = 0
    Or, Lr = attention_ref(host64(q), kk, vv, default_scale(D), causal,
                           None if kvl is None else np.asarray(kvl))
    compare(host64(o), host64(l), Or, Lr, "bf16", f"kvouter {case}")


@pytest.mark.parametrize("tpg", [0, 32])
def test_kvouter_long_workload_sampled(tpg):
    """B=2, H=32, N=M=8192, D=128 causal, as the bench runs it."""
    w = inputs.WORKLOADS["prefill_long_d128"]
    print(f"[kvouter] long workload tiles per group {tpg}", flush=True)
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", torch.device(DEV))
    o, l = fa.fwd(q, k, v, causal=True, path=fa.PATH_KVOUTER, kvouter_query_tiles=tpg)
    torch.cuda.synchronize()
    picks = sample_picks(w.B, w.H, w.N, n_heads=3, seed=5)
    Or, Lr = attention_rows(lambda b, h: host64(q[b, h]), lambda b, h: host64(k[b, h]),
                            lambda b, h: host64(v[b, h]), default_scale(w.D), True, None, picks)
    og = np.stack([host64(o[b, h, i]) for b, h, i in picks])
    lg = np.array([float(l[b, h, i]) for b, h, i in picks])
    compare(og, lg, Or, Lr, "bf16", f"kvouter long tpg={tpg}")
