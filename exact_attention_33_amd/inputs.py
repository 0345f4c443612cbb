"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws numbers and shapes.
Both sides of a parity check (the HIP library and the CPU oracle) receive the
same tensors from here.

The pages use only random matrices (i.i.d. standard normal Q, K, V) and one
random row of 32 scores, so every workload is synthetic:

* small cases draw float32 N(0, 1) on the host with ``numpy.random.default_rng``
  and round to bf16 (round-to-nearest-even) where the case is bf16;
* large cases draw N(0, 1) on the device with a seeded ``torch.Generator`` in
  chunks, then round to bf16;
* decode key counts are uniform integers in [lo, hi] from ``default_rng``.
"""
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "normal_f32", "qkv_host", "kv_lens",
           "score_row", "qkv_device", "grad_device", "to_device", "poison_tail"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str            # "f32" or "bf16"
    causal: tuple         # variants to run
    seed: int
    kv_seed: int = 0      # decode only: seed of the per-sequence key counts
    kv_range: tuple = field(default=())   # decode only: (lo, hi) inclusive


WORKLOADS = {
    # B=1, H=1, N=M=128, D=64, fp32: the exactness case.
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 128, 64, "f32", (False, True), 1),
    # B=1, H=8, N=M=1024, D=64, bf16, causal.
    "prefill_small": Workload("prefill_small", 1, 8, 1024, 1024, 64, "bf16", (True,), 2),
    # B=4, H=16, N=M=4096, D=128, bf16, causal and not.
    "prefill_mid": Workload("prefill_mid", 4, 16, 4096, 4096, 128, "bf16", (True, False), 3),
    # B=2, H=32, N=M=8192, D=64 / D=128, bf16, causal.
    "prefill_long_d64": Workload("prefill_long_d64", 2, 32, 8192, 8192, 64, "bf16", (True,), 4),
    "prefill_long_d128": Workload("prefill_long_d128", 2, 32, 8192, 8192, 128, "bf16", (True,), 5),
    # B=32, H=32, N=1, D=128, bf16, per-sequence KV length uniform in [1024, 32768].
    "decode": Workload("decode", 32, 32, 1, 32768, 128, "bf16", (False,), 6,
                       kv_seed=7, kv_range=(1024, 32768)),
}


def normal_f32(seed, shape):
    """float32 N(0, 1) from ``numpy.random.default_rng(seed)``."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def qkv_host(seed, B, H, N, M, D):
    """Q [B,H,N,D], K and V [B,H,M,D] as float32, drawn in that order."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D), dtype=np.float32)
    k = rng.standard_normal((B, H, M, D), dtype=np.float32)
    v = rng.standard_normal((B, H, M, D), dtype=np.float32)
    return q, k, v


def kv_lens(seed, B, lo, hi):
    """int32 [B], uniform on the integers lo..hi inclusive."""
    return np.random.default_rng(seed).integers(lo, hi, size=B,
                                                endpoint=True).astype(np.int32)


def score_row(seed=1, n=32, scale=3.0):
    """A row of ``n`` scores: standard normal times ``scale`` (fp64)."""
    return np.random.default_rng(seed).standard_normal(n) * scale


def to_device(arr, dtype, device):
    """Host float32 array -> torch tensor of ``dtype`` ("f32"/"bf16") on
    ``device``; bf16 rounding is torch's round-to-nearest-even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.to(device).contiguous()


def qkv_device(seed, B, H, N, M, D, dtype, device, chunk_rows=1 << 22):
    """Q, K, V drawn N(0, 1) directly on ``device`` with a seeded generator.

    Each tensor is filled in chunks of ``chunk_rows`` rows of D values so that
    the float32 staging buffer stays small next to multi-GB bf16 tensors.
    """
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = []
    for rows in (B * H * N, B * H * M, B * H * M):
        t = torch.empty((rows, D), dtype=tdt, device=device)
        for r0 in range(0, rows, chunk_rows):
            r1 = min(rows, r0 + chunk_rows)
            t[r0:r1] = torch.randn((r1 - r0, D), generator=gen, device=device,
                                   dtype=torch.float32).to(tdt)
        out.append(t)
    q = out[0].view(B, H, N, D)
    k = out[1].view(B, H, M, D)
    v = out[2].view(B, H, M, D)
    return q, k, v


def grad_device(seed, B, H, N, D, dtype, device, chunk_rows=1 << 22):
    """An upstream gradient dO [B,H,N,D], N(0, 1) drawn on ``device`` with a
    seeded generator (chunked like ``qkv_device``)."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    rows = B * H * N
    t = torch.empty((rows, D), dtype=tdt, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t[r0:r1] = torch.randn((r1 - r0, D), generator=gen, device=device,
                               dtype=torch.float32).to(tdt)
    return t.view(B, H, N, D)


def poison_tail(k, v, kv_len):
    """Fill keys/values at or past kv_len[b] with NaN (in place, torch or
    numpy), so that any read of a masked row shows up in the output."""
    for b, n in enumerate(np.asarray(kv_len).reshape(-1).tolist()):
        k[b, :, int(n):] = float("nan")
        v[b, :, int(n):] = float("nan")
    return k, v


# ---- element masks (boolean [Bm, Hm, N, M], True = key visible) ----
# Synthetic stand-ins for the kinds of masks attention serves besides causal
# and a window: packed documents, a bidirectional prefix, random block
# sparsity and unstructured masks.

def document_mask(seed, N, M, n_docs):
    """Packed sequences: the N queries and M keys are cut at the same
    ``n_docs - 1`` random points (queries scaled to M), and a query sees only
    the keys of its own document.  [1, 1, N, M]."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, M), size=n_docs - 1, replace=False))
    key_doc = np.searchsorted(cuts, np.arange(M), side="right")
    qpos = (np.arange(N) * M) // max(N, 1)
    q_doc = np.searchsorted(cuts, qpos, side="right")
    return (q_doc[:, None] == key_doc[None, :])[None, None]


def prefix_mask(N, M, prefix):
    """A bidirectional prefix of ``prefix`` keys that every query sees, and
    bottom-right causal order after it.  [1, 1, N, M]."""
    i = np.arange(N)[:, None]
    j = np.arange(M)[None, :]
    return ((j < prefix) | (j <= i + (M - N)))[None, None]


def block_mask(seed, Bm, Hm, N, M, block_q, block_k, p_keep):
    """Random blocks of ``block_q`` x ``block_k`` kept whole or dropped whole,
    each with probability ``p_keep``.  [Bm, Hm, N, M]."""
    rng = np.random.default_rng(seed)
    nb_q, nb_k = -(-N // block_q), -(-M // block_k)
    blocks = rng.random((Bm, Hm, nb_q, nb_k)) < p_keep
    return np.repeat(np.repeat(blocks, block_q, axis=2), block_k, axis=3)[:, :, :N, :M]


def random_mask(seed, Bm, Hm, N, M, p_keep):
    """Each (query, key) pair kept independently with probability ``p_keep``."""
    return np.random.default_rng(seed).random((Bm, Hm, N, M)) < p_keep
