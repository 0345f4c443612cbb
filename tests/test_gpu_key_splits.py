"""GPU parity of the prefill with key splits (options.split_keys on the
prefill path): each query tile's keys go to separate workgroups in chunks,
and a merge combines the chunks' float32 results through their log-sum-exps.
Every element is compared with the fp64 oracle on ragged shapes, with kv_len
tails poisoned, rows with no visible key, a chunk size past M and the
reference moving inside a chunk."""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref
from tests.gpu_helpers import compare, default_scale, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make(seed, B, H, N, M, D):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, "bf16", DEV) for x in (q, k, v))


def check(q, k, v, scale, causal, kvl, split_keys, what, path=None):
    print(f"[case] key splits {what} split_keys={split_keys}", flush=True)
    p = fa.plan(*q.shape[:3], k.shape[2], q.shape[3], fa.BF16, causal, path=path, split_keys=split_keys)
    assert p["path_name"] == "prefill" and p["splits"] == max(1, -(-k.shape[2] // split_keys))
    o, l = fa.fwd(q, k, v, scale=scale, causal=causal, kv_len=kvl, path=path, split_keys=split_keys)
    torch.cuda.synchronize()
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), scale, causal,
                           None if kvl is None else np.asarray(kvl))
    return compare(host64(o), host64(l), Or, Lr, "bf16", what)


@pytest.mark.parametrize("D,B,H,N,M,causal,kvl,split_keys", [
    (64, 1, 8, 1024, 1024, True, None, 256),       # the small prefill workload, 4 chunks
    (64, 1, 8, 1024, 1024, True, None, 128),
    (128, 2, 3, 300, 333, False, [333, 190], 64),  # chunks past kv_len
    (128, 2, 3, 300, 333, True, [333, 190], 128),
    (64, 1, 2, 520, 200, True, None, 64),          # N > M: early rows see nothing
    (128, 1, 2, 130, 700, True, None, 192),        # three tiles a chunk
    (64, 3, 1, 129, 129, True, [129, 64, 1], 64),
    (128, 1, 2, 700, 700, False, None, 4096),      # one chunk
])
def test_key_splits_match_oracle(D, B, H, N, M, causal, kvl, split_keys):
    q, k, v = make(140 + D, B, H, N, M, D)
    if kvl is not None:
        inputs.poison_tail(k, v, kvl)    # keys past kv_len must never reach O
    check(q, k, v, default_scale(D), causal, kvl, split_keys, f"{B},{H},{N},{M},{D} causal={causal}")


def test_key_splits_one_query_on_the_prefill_path():
    q, k, v = make(150, 1, 2, 1, 1000, 128)
    check(q, k, v, default_scale(128), False, None, 256, "N=1", path=fa.PATH_PREFILL)


@pytest.mark.parametrize("causal", [False, True])
def test_key_splits_reference_moves(causal):
    """Scores that jump by ~29 (base 2) in later key blocks: the reference of
    a chunk moves in the middle of its rows."""
    D = 128
    q, k, v = make(33, 1, 2, 384, 384, D)
    scale = default_scale(D)
    b = torch.zeros(384)
    b[96:128], b[192:224], b[288:320] = 1.0, 2.0, 3.0
    q[..., 0] = torch.tensor(20.0 / scale, dtype=torch.bfloat16)
    k[..., 0] = b.to(device=DEV, dtype=torch.bfloat16)
    check(q, k, v, scale, causal, None, 128, f"reference moves causal={causal}")


def test_key_splits_no_keys_and_empty_sequences():
    q = torch.randn((2, 2, 70, 64), device=DEV).to(torch.bfloat16)
    k = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    o, l = fa.fwd(q, k, k, scale=0.1, split_keys=64)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    q, k, v = make(151, 2, 2, 90, 300, 64)
    inputs.poison_tail(k, v, [300, 0])
    o, l = fa.fwd(q, k, v, scale=0.125, kv_len=[300, 0], split_keys=128)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))
    Or, Lr = attention_ref(host64(q[:1]), host64(k[:1]), host64(v[:1]), 0.125, False, np.asarray([300]))
    compare(host64(o[:1]), host64(l[:1]), Or, Lr, "bf16", "kv_len 0 beside a full sequence")


def test_key_splits_are_deterministic():
    q, k, v = make(152, 1, 4, 600, 900, 128)
    a = fa.fwd(q, k, v, causal=True, split_keys=192)
    b = fa.fwd(q, k, v, causal=True, split_keys=192)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
