"""GPU parity at the largest sizes each path accepts.

The tile kernels address one (batch, head) of K and V with 32-bit byte
offsets against a buffer descriptor that ends at kv_len, and whole heads with
64-bit offsets; the split-KV decode addresses everything with 64-bit offsets;
a masked prefill holds one query tile's list of key tiles in LDS, whose
capacity sets its largest M.  Each case sits on such a limit and is compared
with the fp64 oracle ("Understanding FlashAttention", Attention: the function
softmax(mask(Q K^T / sqrt(d))) V) on the rows the oracle can afford.
"""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref, attention_rows
from tests.gpu_helpers import compare, default_scale, host64
from tests.test_gpu_bwd import _check_head, _run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# the largest M with M * D * 2 < 2^31 at D = 128: K or V of one head is
# 2^31 - 256 bytes
M_PREFILL_MAX = (1 << 23) - 1
# the largest M whose list of 64-key tiles (plus its count) fits the LDS list
M_MASK_MAX = 262080


def say(*a):
    print("[limits]", *a, flush=True)


def _rows_check(q, k, v, o, l, scale, causal, kvl, picks, what, mask=None):
    Or, Lr = attention_rows(lambda b, h: host64(q[b, h]), lambda b, h: host64(k[b, h]),
                            lambda b, h: host64(v[b, h]), scale, causal, kvl, picks, mask=mask)
    og = np.stack([host64(o[b, h, i]) for b, h, i in picks])
    lg = np.array([float(l[b, h, i]) for b, h, i in picks])
    eo, el = compare(og, lg, Or, Lr, "bf16", what)
    say(f"{what}: {len(picks)} rows, O {eo:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("causal,kv_cut", [(True, 0), (False, 37)])
def test_prefill_largest_kv(causal, kv_cut):
    """Three heads of M = 2^23 - 1 keys: the third head's K/V start 4 GiB - 512
    bytes into the tensors and each head ends 256 bytes short of 2^31; the
    last tile is ragged and the loads ahead of it run past the descriptor."""
    B, H, N, M, D = 1, 3, 260, M_PREFILL_MAX, 128
    assert fa.plan(B, H, N, M, D, fa.BF16, causal)["path_name"] == "prefill"
    say(f"generate B{B} H{H} N{N} M{M} D{D} causal={causal} kv_cut={kv_cut}")
    q, k, v = inputs.qkv_device(401, B, H, N, M, D, "bf16", torch.device(DEV))
    kvl = None if kv_cut == 0 else [M - kv_cut]
    kvt = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device=DEV)
    say("fa.fwd")
    o, l = fa.fwd(q, k, v, scale=default_scale(D), causal=causal, kv_len=kvt)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
    heads = [(0, 2)] if kv_cut else [(0, 0), (0, 2)]
    picks = [(b, h, i) for b, h in heads for i in (0, 1, 129, 255, 256, N - 1)]
    _rows_check(q, k, v, o, l, default_scale(D), causal, kvl, picks,
                f"prefill M={M} causal={causal} kv_len={kvl}")


def test_decode_beyond_4gib():
    """Split-KV decode over two heads of 2^23 + 77 keys: the second head's
    keys lie between 2 GiB and past 4 GiB into K and V."""
    B, H, N, M, D = 1, 2, 1, (1 << 23) + 77, 128
    assert fa.plan(B, H, N, M, D, fa.BF16, False)["path_name"] == "splitkv"
    say(f"generate decode B{B} H{H} M{M} D{D}")
    q, k, v = inputs.qkv_device(402, B, H, N, M, D, "bf16", torch.device(DEV))
    say("fa.fwd")
    o, l = fa.fwd(q, k, v, scale=default_scale(D))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
    _rows_check(q, k, v, o, l, default_scale(D), False, None, [(0, 1, 0)],
                f"decode M={M} head 1")


@pytest.mark.parametrize("causal", [False, True])
def test_mask_largest_key_count(causal):
    """M = 262080 under a shared random mask (one pair in two kept), two
    sequences, one cut by kv_len: every query tile's list is as long as the
    list buffer allows."""
    B, H, N, M, D = 2, 1, 300, M_MASK_MAX, 128
    assert fa.plan(B, H, N, M, D, fa.BF16, causal, mask_shape=(1, 1))["path_name"] == "prefill"
    with pytest.raises(fa.FaError):
        fa.plan(B, H, N, M + 64, D, fa.BF16, causal, mask_shape=(1, 1))
    say(f"generate B{B} H{H} N{N} M{M} D{D} causal={causal}")
    q, k, v = inputs.qkv_device(403, B, H, N, M, D, "bf16", torch.device(DEV))
    kvl = [M, 200001]
    inputs.poison_tail(k, v, kvl)
    allowed = inputs.random_mask(404, 1, 1, N, M, 0.5)
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    say("fa.fwd")
    o, l = fa.fwd(q, k, v, scale=default_scale(D), causal=causal,
                  kv_len=torch.tensor(kvl, dtype=torch.int32, device=DEV), mask=words)
    torch.cuda.synchronize()
    kk, vv = host64(k), host64(v)
    kk[np.isnan(kk)] = 0
    vv[np.isnan(vv)] = 0
    Or, Lr = attention_ref(host64(q), kk, vv, default_scale(D), causal, np.asarray(kvl),
                           mask=allowed)
    eo, el = compare(host64(o), host64(l), Or, Lr, "bf16", f"mask M={M} causal={causal}")
    say(f"mask M={M} causal={causal}: O {eo:.2e} LSE {el:.2e}")


def test_bwd_mask_largest_key_count():
    """The backward under a random mask at M = 262080: the dQ pass walks the
    longest key-tile list the LDS holds; every gradient element is checked."""
    B, H, N, M, D = 1, 1, 200, M_MASK_MAX, 64
    allowed = inputs.random_mask(405, 1, 1, N, M, 0.5)
    say(f"bwd B{B} H{H} N{N} M{M} D{D} random mask")
    t = _run(B, H, N, M, D, False, None, seed=406, device=torch.device(DEV), mask=allowed)
    _check_head(t, 0, 0, False, M, f"bwd mask M={M}", allow=allowed[0, 0])
