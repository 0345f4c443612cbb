"""Pins for the backward oracle: checks against what the mathematics fixes.

Each ``pin_*`` takes a gradient function with the oracle's signature
``bwd(q, k, v, do, scale, causal, kv_len) -> (dQ, dK, dV, D)`` and raises
AssertionError when it disagrees.  The forward used for finite differences
and for the D shortcut is the forward oracle (``oracle.attention``), which is
pinned on its own against 50-digit brute force.

The pages derive the gradients in "Flash Attention: The Hidden Gem", Phase 2:
Backward Pass (Chain Rule Through a Matrix Multiply, The Softmax Jacobian,
The D Shortcut, The Algorithm).
"""
import numpy as np

from oracle.attention import attention_ref


def _rand(seed, B, H, N, M, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, D)), rng.standard_normal((B, H, M, D)),
            rng.standard_normal((B, H, M, D)), rng.standard_normal((B, H, N, D)))


def _loss(q, k, v, do, scale, causal, kv_len, window=None, mask=None):
    """The scalar whose gradient the backward returns: sum(dO * O)."""
    O, _ = attention_ref(q, k, v, scale, causal, kv_len, window=window, mask=mask)
    return float(np.sum(do * O))


def _central_diff(f, x, h):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


FD_CASES = [
    # seed, B, H, N, M, D, scale, causal, kv_len
    (21, 1, 1, 5, 7, 4, 0.6, False, None),
    (22, 1, 1, 6, 6, 3, 0.8, True, None),
    (23, 2, 1, 3, 7, 4, 0.5, True, [7, 4]),      # bottom-right causal, kv_len
    (24, 1, 1, 6, 5, 3, 1.1, True, [3]),         # N > kv_len: three rows see nothing
    (25, 2, 1, 4, 6, 3, 0.9, False, [0, 5]),     # an empty batch
]


def pin_finite_differences(bwd):
    """Central differences of sum(dO * O) match dQ, dK and dV everywhere,
    including zeros for masked keys and for rows with no visible key."""
    h = 1e-5
    for seed, B, H, N, M, D, scale, causal, kvl in FD_CASES:
        q, k, v, do = _rand(seed, B, H, N, M, D)
        dq, dk, dv, _ = bwd(q, k, v, do, scale, causal, kvl)
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            fd = _central_diff(lambda: _loss(q, k, v, do, scale, causal, kvl), x, h)
            err = np.max(np.abs(np.asarray(g) - fd))
            assert err < 1e-7 * max(1.0, np.max(np.abs(fd))), (name, seed, err)


def pin_delta_shortcut(bwd):
    """The D Shortcut: sum_k dP_ik P_ik equals sum_m dO_im O_im."""
    for seed, B, H, N, M, D, scale, causal, kvl in FD_CASES + [
            (26, 1, 2, 16, 16, 8, 0.35, True, None)]:
        q, k, v, do = _rand(seed, B, H, N, M, D)
        _, _, _, delta = bwd(q, k, v, do, scale, causal, kvl)
        O, _ = attention_ref(q, k, v, scale, causal, kvl)
        want = np.sum(do * O, axis=-1)
        assert np.max(np.abs(np.asarray(delta) - want)) < 1e-12 * max(1.0, np.max(np.abs(want))), seed


def pin_single_key(bwd):
    """One visible key: P = 1, so dS = 0 (dQ = dK = 0) and dV_0 = sum_i dO_i."""
    q, k, v, do = _rand(27, 1, 1, 5, 4, 3)
    dq, dk, dv, _ = bwd(q, k, v, do, 0.7, False, [1])
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    assert np.max(np.abs(dv[0, 0, 0] - do[0, 0].sum(axis=0))) < 1e-13
    assert np.max(np.abs(dv[0, 0, 1:])) == 0.0


def pin_uniform_scores(bwd):
    """Q = 0: every visible key gets weight 1/kv_len, so dV_j is the mean of
    dO over the queries and dK = scale * dS^T Q = 0."""
    _, k, v, do = _rand(28, 1, 1, 6, 5, 4)
    q = np.zeros((1, 1, 6, 4))
    dq, dk, dv, _ = bwd(q, k, v, do, 0.9, False, None)
    want = np.broadcast_to(do[0, 0].sum(axis=0) / 5, (5, 4))
    assert np.max(np.abs(dv[0, 0] - want)) < 1e-13
    assert np.max(np.abs(dk)) < 1e-13
    assert np.max(np.abs(dq)) > 1e-3      # Q still has a gradient


def pin_dk_sums_to_zero(bwd):
    """O does not change when the same vector is added to every key (each row
    of scores moves by a constant), so the key gradients sum to zero."""
    for causal in (False, True):
        q, k, v, do = _rand(29, 1, 2, 7, 7, 5)
        _, dk, _, _ = bwd(q, k, v, do, 0.45, causal, None)
        s = np.asarray(dk).sum(axis=2)
        assert np.max(np.abs(s)) < 1e-12 * max(1.0, np.max(np.abs(dk))), causal


def pin_causal_row0(bwd):
    """Causal row 0 sees key 0 only, so its score gradient is zero: dQ_0 = 0."""
    q, k, v, do = _rand(30, 1, 1, 5, 5, 4)
    dq, _, _, _ = bwd(q, k, v, do, 0.5, True, None)
    assert np.max(np.abs(dq[0, 0, 0])) < 1e-14
    assert np.max(np.abs(dq[0, 0, 1])) > 1e-3


def pin_window_finite_differences(bwd):
    """Central differences through the windowed forward oracle: one- and
    two-sided bands, causal and not, with kv_len."""
    h = 1e-5
    for seed, B, H, N, M, D, scale, causal, kvl, win in [
            (51, 1, 1, 6, 6, 3, 0.7, True, None, (2, 0)),
            (52, 1, 1, 5, 7, 3, 0.6, False, [6], (1, 2))]:
        q, k, v, do = _rand(seed, B, H, N, M, D)
        dq, dk, dv, _ = bwd(q, k, v, do, scale, causal, kvl, window=win)
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            fd = _central_diff(lambda: _loss(q, k, v, do, scale, causal, kvl, win), x, h)
            err = np.max(np.abs(np.asarray(g) - fd))
            assert err < 1e-7 * max(1.0, np.max(np.abs(fd))), (name, seed, err)


def pin_mask_finite_differences(bwd):
    """Central differences through the forward oracle under an element mask
    (shared and per-head, with causal and kv_len, a row the mask empties)."""
    h = 1e-5
    for seed, B, H, N, M, D, scale, causal, kvl, mshape in [
            (53, 1, 2, 5, 6, 3, 0.7, False, None, (1, 2, 5, 6)),
            (54, 2, 1, 6, 6, 3, 0.9, True, [6, 4], (1, 1, 6, 6))]:
        q, k, v, do = _rand(seed, B, H, N, M, D)
        mask = np.random.default_rng(seed + 7).random(mshape) < 0.6
        mask[0, 0, 2] = False
        dq, dk, dv, _ = bwd(q, k, v, do, scale, causal, kvl, mask=mask)
        assert not np.asarray(dq)[:, 0, 2].any()     # the emptied row of head 0
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            fd = _central_diff(lambda: _loss(q, k, v, do, scale, causal, kvl, mask=mask), x, h)
            err = np.max(np.abs(np.asarray(g) - fd))
            assert err < 1e-7 * max(1.0, np.max(np.abs(fd))), (name, seed, err)


ALL_BWD_PINS = [pin_finite_differences, pin_window_finite_differences,
                pin_mask_finite_differences, pin_delta_shortcut,
                pin_single_key, pin_uniform_scores, pin_dk_sums_to_zero, pin_causal_row0]
