"""Shared pieces of the GPU parity tests: run the HIP path, run the oracle on
the exact same tensors, compare to the stated tolerances."""
import math

import numpy as np

# Tolerances (max-abs): bf16 inputs O <= 2e-2, LSE <= 1e-3; float32 path 1e-5.
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}


def host64(t):
    """Exact float64 copy of a device tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(O_gpu, L_gpu, O_ref, L_ref, dtype, what=""):
    """Element-wise comparison; -inf LSE rows must match exactly and have O = 0."""
    tol_o, tol_l = TOL[dtype]
    O = np.asarray(O_gpu, dtype=np.float64)
    L = np.asarray(L_gpu, dtype=np.float64)
    assert O.shape == O_ref.shape and L.shape == L_ref.shape, what
    assert not np.isnan(O).any(), f"{what}: NaN in O"
    assert not np.isnan(L).any(), f"{what}: NaN in LSE"
    empty_ref = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), empty_ref), f"{what}: empty-row pattern differs"
    assert np.all(O[empty_ref] == 0), f"{what}: rows with no visible key must be 0"
    eo = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    fin = ~empty_ref
    el = float(np.max(np.abs(L[fin] - L_ref[fin]))) if fin.any() else 0.0
    assert eo <= tol_o, f"{what}: O max-abs {eo:.3e} > {tol_o}"
    assert el <= tol_l, f"{what}: LSE max-abs {el:.3e} > {tol_l}"
    return eo, el


def sample_picks(B, H, N, n_heads=6, seed=0, extra_rows=6):
    """(b, h, i) picks: the first and last heads and a few random ones; in each,
    rows at both ends, at 128-row tile edges and a few random rows."""
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (B - 1, H - 1)}
    while len(heads) < min(n_heads, B * H):
        heads.add((int(rng.integers(B)), int(rng.integers(H))))
    rows = {0, N - 1}
    for r in (1, 127, 128, 129, N // 2, N - 129, N - 128, N - 2):
        if 0 <= r < N:
            rows.add(r)
    picks = []
    for (b, h) in sorted(heads):
        rr = set(rows) | {int(x) for x in rng.integers(0, N, size=extra_rows)}
        picks += [(b, h, i) for i in sorted(rr)]
    return picks


def default_scale(D):
    return 1.0 / math.sqrt(D)
