"""GPU parity of the backward: the HIP kernels through the C ABI against the
fp64 oracle (``oracle.backward``) on the same seeded inputs.

The forward runs first on the GPU; its O and LSE are what the backward is
given.  Each gradient element must lie within twice the elementwise bound
that ``gpu_helpers.bwd_bound`` derives from the kernels' arithmetic; masked
keys get exactly zero gradients and rows with no visible key exactly zero dQ.
"""

import numpy as np
import pytest

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import clamp_kv_len
from oracle.backward import head_backward
from tests.gpu_helpers import bwd_bound, compare_bwd, default_scale, host64

pytestmark = pytest.mark.gpu


def _run(B, H, N, M, D, causal, kv_len, seed, device, poison=True, window=None, mask=None):
    import torch
    words = None if mask is None else fa.pack_mask(torch.from_numpy(mask).to(device))
    q, k, v = inputs.qkv_device(seed, B, H, N, M, D, "bf16", device)
    do = inputs.grad_device(seed + 1000, B, H, N, D, "bf16", device)
    kvt = None
    if kv_len is not None:
        kvt = torch.tensor(kv_len, dtype=torch.int32, device=device)
        if poison:
            inputs.poison_tail(k, v, kv_len)
    scale = default_scale(D)
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal, kv_len=kvt, window=window, mask=words)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal, kv_len=kvt, window=window,
                        mask=words)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, scale=scale)


def _check_head(t, b, h, causal, kvl, what, window=None, allow=None):
    q, k, v, do = (host64(t[n][b, h]) for n in ("q", "k", "v", "do"))
    k = np.where(np.isnan(k), 0.0, k)          # the poisoned tail is never read
    v = np.where(np.isnan(v), 0.0, v)
    O_gpu, L_gpu = host64(t["o"][b, h]), host64(t["lse"][b, h])
    r = head_backward(q, k, v, do, t["scale"], causal, kvl, window, allow)
    # the exact forward's LSE for the same head
    S = t["scale"] * (q @ k[:kvl].T)
    N = q.shape[0]
    from oracle.attention import visible_mask
    S = np.where(visible_mask(N, kvl, causal, window, allow), S, -np.inf)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = S.max(axis=1) if kvl else np.full(N, -np.inf)
        L_ref = np.where(np.isfinite(m), m + np.log(np.sum(np.exp(S - m[:, None]), axis=1)), -np.inf) \
            if kvl else np.full(N, -np.inf)
    bq, bk, bv = bwd_bound(r, q, k, v, do, O_gpu, L_gpu, L_ref, t["scale"])
    dq, dk, dv = (host64(t[n][b, h]) for n in ("dq", "dk", "dv"))
    worst = [compare_bwd(dq, r["dq"], bq, f"{what} dQ"),
             compare_bwd(dk, r["dk"], bk, f"{what} dK"),
             compare_bwd(dv, r["dv"], bv, f"{what} dV")]
    # exact zeros where the definition gives exact zeros
    assert np.all(dk[kvl:] == 0) and np.all(dv[kvl:] == 0), f"{what}: masked keys"
    assert np.all(dq[np.isneginf(L_ref)] == 0), f"{what}: rows with no visible key"
    return max(worst)


CASES = [
    # B, H, N, M, D, causal, kv_len
    (1, 2, 128, 128, 128, False, None),
    (1, 2, 128, 128, 128, True, None),
    (2, 3, 200, 200, 64, True, None),           # ragged: not a multiple of 64
    (1, 2, 70, 300, 128, False, None),          # N != M, both ragged
    (2, 2, 96, 333, 128, True, [333, 150]),     # bottom-right causal with kv_len
    (2, 2, 300, 100, 64, True, None),           # N > M: early rows see no key
    (1, 1, 1, 513, 128, False, None),           # one query
    (2, 2, 257, 257, 128, True, [0, 257]),      # an empty batch
    (1, 1, 600, 700, 64, False, [650]),
    (1, 2, 520, 520, 128, True, None),          # several key tiles and query stages
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}{}".format(
    *c[:5], "c" if c[5] else "", "kv" if c[6] else ""))
def test_bwd_matches_oracle(case):
    import torch
    B, H, N, M, D, causal, kv_len = case
    dev = torch.device("cuda:0")
    print(f"[bwd] case {case}", flush=True)
    t = _run(B, H, N, M, D, causal, kv_len, seed=40 + N + M, device=dev)
    kvs = clamp_kv_len(kv_len, B, M)
    for b in range(B):
        for h in range(H):
            _check_head(t, b, h, causal, kvs[b], f"{case} b{b} h{h}")


WINDOW_CASES = [
    # B, H, N, M, D, causal, kv_len, window
    (1, 2, 300, 300, 128, True, None, (127, 0)),       # the pages' 128-wide window
    (1, 2, 600, 600, 64, True, None, (300, 0)),        # wider than a key tile
    (2, 2, 257, 400, 128, False, [400, 199], (50, 70)),  # two-sided, N != M, kv_len
    (1, 1, 200, 90, 128, True, None, (10, 0)),         # N > M: early rows see nothing
    (1, 2, 130, 130, 64, False, None, (0, 0)),         # one key per query
    (1, 1, 700, 700, 128, True, None, (5000, 0)),      # wider than the sequence
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}w{}-{}".format(
    *c[:5], "c" if c[5] else "", *c[7]))
def test_bwd_window_matches_oracle(case):
    import torch
    B, H, N, M, D, causal, kv_len, win = case
    print(f"[bwd] window case {case}", flush=True)
    t = _run(B, H, N, M, D, causal, kv_len, seed=140 + N + M, device=torch.device("cuda:0"),
             window=win)
    kvs = clamp_kv_len(kv_len, B, M)
    for b in range(B):
        for h in range(H):
            _check_head(t, b, h, causal, kvs[b], f"{case} b{b} h{h}", window=win)


MASK_CASES = [
    # B, H, N, M, D, causal, kv_len, window, mask kind
    (1, 2, 300, 300, 128, False, None, None, "random"),
    (2, 2, 260, 517, 64, True, [517, 200], None, "random_per_head"),
    (1, 2, 700, 700, 128, True, None, None, "documents"),
    (2, 1, 513, 600, 128, False, [600, 333], (200, 50), "blocks_per_batch"),
    (1, 1, 200, 90, 128, True, None, None, "random"),            # N > M
    (1, 1, 1, 700, 128, False, None, None, "random"),            # one query
    (2, 1, 130, 260, 128, True, [260, 0], None, "random"),       # an empty sequence
    (1, 2, 70, 40, 64, False, None, None, "random_per_head"),    # M below one key tile
]


def _mask_of(kind, B, H, N, M):
    if kind == "random":
        return inputs.random_mask(111, 1, 1, N, M, 0.5)
    if kind == "random_per_head":
        m = inputs.random_mask(112, 1, H, N, M, 0.4)
        m[0, 0, ::5] = False                                        # rows the mask empties
        return m
    if kind == "documents":
        return inputs.document_mask(113, N, M, 4)
    if kind == "blocks_per_batch":
        return inputs.block_mask(114, B, 1, N, M, 64, 64, 0.5)
    raise ValueError(kind)


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}-{}".format(
    *c[:5], "c" if c[5] else "", c[8]))
def test_bwd_mask_matches_oracle(case):
    """Element masks: the gradients of the masked forward, hidden entries
    passing none (dQ walks the forward's tile lists; dK/dV applies the bits
    on every stage)."""
    import torch
    from oracle.attention import mask_of_head
    B, H, N, M, D, causal, kv_len, win, kind = case
    print(f"[bwd] mask case {case}", flush=True)
    allowed = _mask_of(kind, B, H, N, M)
    t = _run(B, H, N, M, D, causal, kv_len, seed=170 + N + M, device=torch.device("cuda:0"),
             window=win, mask=allowed)
    kvs = clamp_kv_len(kv_len, B, M)
    for b in range(B):
        for h in range(H):
            _check_head(t, b, h, causal, kvs[b], f"{case} b{b} h{h}", window=win,
                        allow=mask_of_head(allowed, b, h))


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_all_ones_mask_matches_unmasked(D):
    """A mask that keeps every key gives the unmasked gradients bit for bit
    (the same tiles, the same arithmetic on the kept entries; the unmasked
    causal dQ pass runs a stage as one pipeline, the masked one as two plain
    steps)."""
    import torch
    dev = torch.device("cuda:0")
    print(f"[bwd] all-ones mask D={D}", flush=True)
    t = _run(1, 2, 600, 600, D, True, None, seed=91, device=dev)
    words = fa.pack_mask(torch.ones((1, 1, 600, 600), dtype=torch.bool, device=dev))
    dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], causal=True, mask=words)
    torch.cuda.synchronize()
    assert torch.equal(dq, t["dq"]) and torch.equal(dk, t["dk"]) and torch.equal(dv, t["dv"])


def test_bwd_degenerate_sizes():
    """M = 0: dQ = 0; N = 0: dK = dV = 0; both written by the kernels."""
    import torch
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 40, 64, device=dev).to(torch.bfloat16)
    e = torch.empty(1, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    lse = torch.full((1, 2, 40), float("-inf"), device=dev)
    o = torch.zeros_like(q)
    dq, dk, dv = fa.bwd(q, e, e, o, lse, q.clone(), dq=torch.full_like(q, 7.0))
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    kk = torch.randn(1, 2, 50, 64, device=dev).to(torch.bfloat16)
    dq, dk, dv = fa.bwd(e, kk, kk, e, torch.empty(1, 2, 0, device=dev), e,
                        dk=torch.full_like(kk, 7.0), dv=torch.full_like(kk, 7.0))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_is_deterministic():
    import torch
    dev = torch.device("cuda:0")
    t = _run(2, 4, 1000, 1000, 128, True, None, seed=77, device=dev)
    dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, t["dq"]) and torch.equal(dk, t["dk"]) and torch.equal(dv, t["dv"])


@pytest.mark.parametrize("name,causal,heads", [
    ("prefill_small", True, [(0, h) for h in range(8)]),
    ("prefill_mid", True, [(0, 0), (3, 15)]),
    ("prefill_mid", False, [(1, 7)]),
    ("prefill_long_d64", True, [(1, 31)]),
    ("prefill_long_d128", True, [(0, 0)]),
])
def test_bwd_workloads_sampled_heads(name, causal, heads):
    """The prefill workloads at full size; the oracle checks whole heads."""
    import torch
    w = inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"[bwd] workload {name} causal={causal}", flush=True)
    t = _run(w.B, w.H, w.N, w.M, w.D, causal, None, seed=w.seed, device=dev)
    for b, h in heads:
        _check_head(t, b, h, causal, w.M, f"{name} b{b} h{h}")


def test_bwd_long_workload_documents_mask():
    """B=2, H=32, N=M=8192, D=128 causal under the bench's 8-document mask
    (shared by every batch and head), whole heads checked."""
    import torch
    w = inputs.WORKLOADS["prefill_long_d128"]
    dev = torch.device("cuda:0")
    print("[bwd] long workload, documents mask", flush=True)
    allowed = inputs.document_mask(7, w.N, w.M, 8)
    t = _run(w.B, w.H, w.N, w.M, w.D, True, None, seed=w.seed, device=dev, mask=allowed)
    for b, h in [(0, 3), (1, 30)]:
        _check_head(t, b, h, True, w.M, f"documents b{b} h{h}", allow=allowed[0, 0])
