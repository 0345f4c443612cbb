"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Small cases compare every element; they span several query and key tiles and
end in ragged tails.  The full-size workloads run in the launch configuration
the bench times and are compared element by element on whole heads (prefill)
and on every row (decode).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref
from tests.gpu_helpers import abi_scale, compare, default_scale, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def run(q, k, v, scale, causal, kv_len=None, **kw):
    kvs = None if kv_len is None else (
        kv_len.tolist() if isinstance(kv_len, torch.Tensor) else list(kv_len))[:8]
    say(f"fa.fwd q={tuple(q.shape)} k={tuple(k.shape)} {q.dtype} causal={causal} "
        f"kv_len={kvs} {kw}")
    o, l = fa.fwd(q, k, v, scale=scale, causal=causal, kv_len=kv_len, **kw)
    torch.cuda.synchronize()
    return o, l


def full_check(q, k, v, scale, causal, kv_len, dtype, what, **kw):
    o, l = run(q, k, v, scale, causal, kv_len, **kw)
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), scale, causal,
                           None if kv_len is None else np.asarray(kv_len))
    return compare(host64(o), host64(l), Or, Lr, dtype, what)


def make(seed, B, H, N, M, D, dtype):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return (inputs.to_device(q, dtype, DEV), inputs.to_device(k, dtype, DEV),
            inputs.to_device(v, dtype, DEV))


# ---------------------------------------------------------------- float32 path

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("stress", [1.0, 16.0])
def test_tiny_f32_exactness(causal, stress):
    """B=1, H=1, N=M=128, D=64, fp32; plus the copy with Q x 16 (scores near
    90: overflow safety)."""
    w = inputs.WORKLOADS["tiny_f32"]
    q, k, v = inputs.qkv_host(w.seed, w.B, w.H, w.N, w.M, w.D)
    q = q * np.float32(stress)
    qd, kd, vd = (inputs.to_device(x, "f32", DEV) for x in (q, k, v))
    eo, el = full_check(qd, kd, vd, default_scale(w.D), causal, None, "f32",
                        f"tiny_f32 causal={causal} x{stress}")
    say(f"tiny_f32 causal={causal} x{stress}: O {eo:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("B,H,N,M,D,causal,kvl", [
    (2, 3, 77, 133, 128, True, [133, 40]),
    (1, 2, 200, 150, 64, True, None),      # N > M: first rows see nothing
    (2, 1, 1, 300, 128, False, [300, 0]),  # decode rows, one empty sequence
    (1, 1, 33, 0, 64, False, None),        # no keys at all
])
def test_f32_ragged(B, H, N, M, D, causal, kvl):
    q, k, v = make(17, B, H, N, M, D, "f32")
    full_check(q, k, v, abi_scale(0.11), causal, kvl, "f32", f"f32 {B},{H},{N},{M},{D}")


# --------------------------------------------------------------- bf16 prefill

def test_prefill_small_full():
    """B=1, H=8, N=M=1024, D=64, bf16, causal: every element."""
    w = inputs.WORKLOADS["prefill_small"]
    q, k, v = make(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16")
    eo, el = full_check(q, k, v, default_scale(w.D), True, None, "bf16", "prefill_small")
    say(f"prefill_small: O {eo:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N,M,causal,kvl", [
    (2, 3, 300, 333, False, [333, 190]),
    (2, 3, 300, 333, True, [333, 190]),
    (1, 2, 520, 200, True, None),        # N > M, bottom-right: early rows empty
    (1, 2, 130, 700, True, None),        # N < M: rows see a long prefix
    (3, 1, 129, 129, True, [129, 64, 1]),
    (1, 1, 1, 1000, False, None),         # one query on the prefill path
])
def test_prefill_ragged(D, B, H, N, M, causal, kvl):
    q, k, v = make(100 + D, B, H, N, M, D, "bf16")
    if kvl is not None:
        inputs.poison_tail(k, v, kvl)    # masked rows must never be read into O
    full_check(q, k, v, default_scale(D), causal, kvl, "bf16",
               f"prefill {B},{H},{N},{M},{D} causal={causal}", path=fa.PATH_PREFILL)


def test_prefill_large_scores_no_overflow():
    """Scores of several hundred (Q x 16 at D=128): no overflow, same tolerance."""
    q, k, v = make(31, 1, 2, 256, 256, 128, "bf16")
    q = (q.float() * 16).to(torch.bfloat16)
    full_check(q, k, v, default_scale(128), True, None, "bf16", "prefill x16")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_reference_moves_in_later_blocks(D, causal):
    """Scores that jump by ~29 (base 2) at later 32-key blocks -- in key block
    1 of tile 1, key block 0 of tile 3 and key block 1 of tile 4 -- push the
    weights of rows that already have a reference far above 2^20, so the
    reference has to move in the middle of a row (both rare paths)."""
    q, k, v = make(33, 1, 2, 384, 384, D, "bf16")
    scale = default_scale(D)
    lam = 20.0 / scale                      # q_0 = lam, k_j0 = b_j: score + 20 b_j (natural)
    b = torch.zeros(384)
    b[96:128] = 1.0                         # tile 1, key block 1
    b[192:224] = 2.0                        # tile 3, key block 0
    b[288:320] = 3.0                        # tile 4, key block 1
    q[..., 0] = torch.tensor(lam, dtype=torch.bfloat16)
    k[..., 0] = b.to(device=DEV, dtype=torch.bfloat16)
    full_check(q, k, v, scale, causal, None, "bf16", f"reference moves D={D} causal={causal}")


def test_prefill_scale_zero_is_uniform():
    q, k, v = make(32, 1, 2, 200, 150, 64, "bf16")
    o, l = run(q, k, v, 0.0, False)
    vv = host64(v)
    assert np.max(np.abs(host64(o) - vv.mean(axis=2, keepdims=True))) <= 2e-2
    assert np.max(np.abs(host64(l) - math.log(150))) <= 1e-3


# ------------------------------------------------------------- split-KV decode

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("split_keys", [0, 64, 256, 1024])
def test_decode_splitkv(D, split_keys):
    B, H, M = 4, 3, 5000
    kvl = [5000, 1, 777, 0]
    q, k, v = make(200 + D, B, H, 1, M, D, "bf16")
    inputs.poison_tail(k, v, kvl)
    full_check(q, k, v, default_scale(D), False, kvl, "bf16",
               f"decode D={D} split_keys={split_keys}", path=fa.PATH_SPLITKV,
               split_keys=split_keys)


def test_decode_causal_sees_history():
    """N = 1 with the causal flag sees every cached key (bottom-right)."""
    q, k, v = make(210, 2, 2, 1, 3000, 128, "bf16")
    o1, l1 = run(q, k, v, default_scale(128), True, [3000, 1234])
    o2, l2 = run(q, k, v, default_scale(128), False, [3000, 1234])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------- full workloads
#
# "Understanding FlashAttention", Attention: the check of a streamed form is a
# comparison with the direct calculation.  At the full sizes the oracle still
# affords whole heads (every query row against every key), so each launch the
# bench times is compared element by element on several whole heads.

# Flat (batch * H + head) indices compared in full.  The causal grid is
# persistent: at N = 8192 each XCD walks 8 heads, one per round, and odd
# rounds take the query tiles in reverse; heads 0, 9, 18 and 63 fall on XCDs
# 0, 1, 2 and 7 in rounds 0, 1, 2 and 7 (even and odd).  At N = 4096 a round
# covers two heads: 0, 9, 18, 63 are rounds 0, 0, 1, 3 of XCDs 0, 1, 2, 7.
WHOLE_HEADS = (0, 9, 18, 63)


def _whole_heads(q, k, v, o, l, scale, causal, heads, what):
    H = q.shape[1]
    worst_o = worst_l = 0.0
    for flat in heads:
        b, h = divmod(flat, H)
        say(f"{what}: oracle on whole head b={b} h={h}")
        Or, Lr = attention_ref(host64(q[b, h])[None, None], host64(k[b, h])[None, None],
                               host64(v[b, h])[None, None], scale, causal)
        eo, el = compare(host64(o[b, h])[None, None], host64(l[b, h])[None, None], Or, Lr,
                         "bf16", f"{what} b={b} h={h}")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    return worst_o, worst_l


@pytest.mark.parametrize("name,causal", [("prefill_mid", True), ("prefill_mid", False),
                                         ("prefill_long_d64", True), ("prefill_long_d128", True)])
def test_full_prefill_whole_heads(name, causal):
    w = inputs.WORKLOADS[name]
    say(f"generate {name}")
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", DEV)
    o, l = run(q, k, v, default_scale(w.D), causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
    eo, el = _whole_heads(q, k, v, o, l, default_scale(w.D), causal, WHOLE_HEADS, name)
    say(f"{name} causal={causal}: {len(WHOLE_HEADS)} whole heads, O {eo:.2e} LSE {el:.2e}")


def test_full_decode_every_row():
    """All B * H = 1024 decode rows against the oracle, each over its whole
    KV history (kv_len[b] keys)."""
    w = inputs.WORKLOADS["decode"]
    kvl = inputs.kv_lens(w.kv_seed, w.B, *w.kv_range)
    M = int(kvl.max())
    say(f"generate decode M={M}")
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, 1, M, w.D, "bf16", DEV)
    inputs.poison_tail(k, v, kvl)
    kvl_d = torch.as_tensor(kvl, device=DEV)
    o, l = run(q, k, v, default_scale(w.D), False, kvl_d)
    og, lg = host64(o), host64(l)
    Or = np.zeros_like(og)
    Lr = np.zeros_like(lg)
    for b in range(w.B):
        n = int(kvl[b])
        # one sequence at a time: its keys and values up to kv_len, as bf16 on the host
        kb, vb = k[b, :, :n].cpu(), v[b, :, :n].cpu()
        qb = host64(q[b])
        for h in range(w.H):
            O1, L1 = attention_ref(qb[h][None, None], kb[h].double().numpy()[None, None],
                                   vb[h].double().numpy()[None, None], default_scale(w.D), False)
            Or[b, h], Lr[b, h] = O1[0, 0], L1[0, 0]
    eo, el = compare(og, lg, Or, Lr, "bf16", "decode (every row)")
    say(f"decode: {w.B * w.H} rows, O {eo:.2e} LSE {el:.2e}")


# ------------------------------------------------------ entry points, streams

@pytest.mark.parametrize("N,path", [(1, fa.PATH_SPLITKV), (300, fa.PATH_PREFILL)])
def test_plain_and_extended_entry_points_on_a_side_stream(N, path):
    """The plain fa_fwd (the binding's route when no option is set) against
    the oracle, fa_fwd_ex with the same path forced gives the same bits, and
    so does a call on a stream that is not the current one with kv_len given
    as a host list (the binding's device copy of kv_len and its workspace
    then live on that stream)."""
    B, H, M, D = 3, 2, 2000, 128
    kvl = [2000, 777, 1]
    q, k, v = make(220 + N, B, H, N, M, D, "bf16")
    inputs.poison_tail(k, v, kvl)
    scale = default_scale(D)
    o1, l1 = run(q, k, v, scale, True, kvl)                    # fa_fwd
    o2, l2 = run(q, k, v, scale, True, kvl, path=path)         # fa_fwd_ex
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    side = torch.cuda.Stream(device=DEV)
    say(f"side stream N={N}")
    o3, l3 = fa.fwd(q, k, v, scale=scale, causal=True, kv_len=kvl, stream=side)
    side.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), scale, True, np.asarray(kvl))
    compare(host64(o1), host64(l1), Or, Lr, "bf16", f"plain fa_fwd N={N}")


# ------------------------------------------------------------------ edge cases

def test_empty_inputs():
    for shape in [(0, 2, 16, 16, 64), (1, 2, 0, 16, 64)]:
        B, H, N, M, D = shape
        q = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=DEV)
        k = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=DEV)
        o, l = run(q, k, k, 0.1, True)
        assert o.shape == (B, H, N, D) and l.shape == (B, H, N)


@pytest.mark.parametrize("N,path", [(5, fa.PATH_PREFILL), (1, fa.PATH_SPLITKV)])
def test_no_keys(N, path):
    q = torch.randn((2, 2, N, 128), device=DEV).to(torch.bfloat16)
    k = torch.empty((2, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    o, l = run(q, k, k, 0.1, False, path=path)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
