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


def abi_scale(s):
    """The scale as the kernels receive it: the C ABI takes a float32, and
    the oracle is handed that same value, upcast exactly."""
    return float(np.float32(s))


def default_scale(D):
    """1/sqrt(D) rounded to float32, the value the C ABI carries."""
    return abi_scale(1.0 / math.sqrt(D))


# ---- backward ----
#
# Elementwise error bound of the bf16 backward for one (batch, head), from
# the arithmetic of the kernels (all in fp64 here):
#   * the kernel forms D_i from the bf16 forward output O^ it is given:
#     |dD_i| <= |sum_d dO_id (O^_id - O_id)| + float32 rounding;
#   * it recomputes P from the float32 LSE the forward returned:
#     relative error |LSE^_i - LSE_i| + float32 slack (scores accumulated in
#     float32, exp2 of a float32 argument);
#   * P and dS are rounded to bf16 (unit roundoff 2^-9, taken as 2^-8)
#     before the products that use them, which accumulate in float32
#     (n terms: n 2^-24 of the absolute sum, worst case), and each output is
#     rounded to bf16 once.
# The test accepts |GPU - oracle| <= 2 * bound elementwise.
U_BWD = 2.0 ** -8
F32 = 2.0 ** -24


def bwd_bound(r, q, k, v, do, O_gpu, lse_gpu, lse_ref, scale):
    """Bounds (bq [N,D], bk [M,D], bv [M,D]) for oracle head result ``r``
    (``oracle.backward.head_backward``) and the exact inputs of that head."""
    P, dP, dS, delta = r["p"], r["dp"], r["ds"], r["delta"]
    N, D = q.shape
    M = k.shape[0]
    kvl = P.shape[1]
    kv, vv = k[:kvl], v[:kvl]
    aq, akv, avv, ado = np.abs(q), np.abs(kv), np.abs(vv), np.abs(do)
    dD = np.abs(np.sum(do * (O_gpu - r["o"]), axis=1)) + 4 * D * F32 * np.sum(np.abs(do * O_gpu), axis=1)
    fin = np.isfinite(lse_ref)
    L_ref = np.where(fin, lse_ref, 0.0)
    dL = np.where(fin, np.abs(np.where(fin, lse_gpu, 0.0) - L_ref), 0.0)
    relP = (dL + 16 * F32 * (1.0 + np.abs(L_ref)))[:, None] + scale * 4 * D * F32 * (aq @ akv.T)
    dP_err = 4 * D * F32 * (ado @ avv.T)
    dS_err = (U_BWD * np.abs(dS) + P * dD[:, None] + relP * P * np.abs(dP - delta[:, None])
              + P * dP_err)
    bv = np.zeros((M, D))
    bk = np.zeros((M, D))
    bv[:kvl] = (((U_BWD + relP) * P).T @ ado + N * F32 * (P.T @ ado) + U_BWD * np.abs(r["dv"][:kvl]))
    bk[:kvl] = (scale * (dS_err.T @ aq) + N * F32 * scale * (np.abs(dS).T @ aq)
                + U_BWD * np.abs(r["dk"][:kvl]))
    bq = scale * (dS_err @ akv) + max(kvl, 1) * F32 * scale * (np.abs(dS) @ akv) + U_BWD * np.abs(r["dq"])
    return bq, bk, bv


def compare_bwd(got, want, bound, what):
    """|got - want| <= 2 * bound elementwise; returns the worst ratio."""
    got = np.asarray(got, dtype=np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN"
    err = np.abs(got - want)
    lim = 2 * bound + 1e-30
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements over the bound; first at "
                             f"{tuple(int(x) for x in idx)}: got {got[tuple(idx)]:.6g} "
                             f"want {want[tuple(idx)]:.6g} bound {lim[tuple(idx)]:.3g}")
    return float(np.max(err / lim)) if err.size else 0.0


# ---- fp8 (E4M3) forward ----
#
# The kernel forms weights w_j = 2^(t_j - m) against a reference m with
# m <= max_j t_j <= m + 8 (t in log2 units), rounds them to E4M3 (round to
# nearest even: relative error <= 2^-4 for w >= 2^-6, absolute <= 2^-10
# below, where E4M3 is subnormal) before P V, and divides by the float32 sum
# of the unrounded weights.  With P the exact softmax and
# l_rel = sum_j exp(s_j - max_k s_k) >= 1, per element:
#   |dO_id| <= 2^-4 sum_j P_ij |v_jd| + 2^-10 sum_(visible j) |v_jd| / l_rel_i
# plus one bf16 rounding of O (2^-8 |O| taken) and float32 slack.  The test
# accepts twice that; LSE keeps the bf16 path's 1e-3 (the sums are float32
# over float32 weights, the scores exact products accumulated in float32).
U_E4M3 = 2.0 ** -4
E4M3_SUB = 2.0 ** -10


def fp8_bound(q, k, v, scale, causal, kvl, window=None):
    """Elementwise bound [N, D] for one head from the exact (dequantized) inputs."""
    from oracle.attention import visible_mask
    N, D = q.shape
    kv, vv = k[:kvl], v[:kvl]
    if kvl == 0:
        return np.full((N, D), 1e-6)
    S = scale * (q @ kv.T)
    vis = visible_mask(N, kvl, causal, window)
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    fin = np.isfinite(m)[:, 0]
    E = np.where(vis & fin[:, None], np.exp(np.where(fin[:, None], S - np.where(fin[:, None], m, 0), -np.inf)), 0.0)
    l_rel = E.sum(axis=1)
    P = E / np.where(l_rel > 0, l_rel, 1.0)[:, None]
    av = np.abs(vv)
    O = P @ vv
    b = U_E4M3 * (P @ av) + E4M3_SUB * (vis.astype(np.float64) @ av) / np.where(l_rel > 0, l_rel, 1.0)[:, None]
    return b + 2.0 ** -8 * np.abs(O) + 1e-6
