"""Streamed forms of softmax and attention, written from the pages' derivations.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  These are self-test
helpers: each one is a different route to the result that ``oracle.attention``
defines, and the pins check that the routes agree (and that they reproduce the
numbers the pages print).  GPU parity never uses them.

All arithmetic is fp64 (NumPy / Python floats).
"""
import math

import numpy as np

__all__ = ["online_softmax", "online_normalizer", "per_key_attention",
           "tiled_attention", "split_merge_attention"]


def online_softmax(row, block=8, rescale=True):
    """Softmax of ``row`` with the running max m and running sum l.

    "FlashAttention: attention was never compute-bound", The one formula:
    each block updates m to max(m, block max) and l to
    e^(m_old - m_new) * l_old + sum over the block of e^(x - m_new).
    "Flash Attention: The Hidden Gem", Online Softmax: start from m = -inf,
    l = 0, and at the end the weights are e^(x - m) / l.

    ``rescale=False`` drops the correction factor on l -- the deliberate bug of
    the explainer's "Now break it" section.  The final weights are produced
    with the final m (the second read the pages describe).
    """
    x = np.asarray(row, dtype=np.float64)
    m, l = -np.inf, 0.0
    for start in range(0, x.size, block):
        blk = x[start:start + block]
        m_new = max(m, float(blk.max()))
        if rescale and l != 0.0:
            l *= math.exp(m - m_new)        # e^(m_old - m_new) * l_old
        l += float(np.exp(blk - m_new).sum())
        m = m_new
    return np.exp(x - m) / l


def online_normalizer(x):
    """Running maximum g and running denominator s after one sweep.

    "Understanding FlashAttention", Online softmax: start from the first
    element (g = x_1, s = 1); for each later element g_i = max(g_{i-1}, x_i)
    and s_i = s_{i-1} e^(g_{i-1} - g_i) + e^(x_i - g_i).  At the end g is the
    row maximum and s the safe-softmax denominator.
    """
    vals = [float(t) for t in np.asarray(x, dtype=np.float64).reshape(-1)]
    g, s = vals[0], 1.0
    for xi in vals[1:]:
        g_new = max(g, xi)
        s = s * math.exp(g - g_new) + math.exp(xi - g_new)
        g = g_new
    return g, s


def per_key_attention(q, k, v, scale=1.0):
    """One key at a time, with a normalised accumulator (no mask).

    "Understanding FlashAttention", Optimizing loop (2) and Merging the two
    loops: for each query row keep g (max), s (denominator) and A' (the
    attention result over the keys seen so far).  Each key's score x gives
    g_new = max(g, x), s_new = s e^(g - g_new) + e^(x - g_new) and
    A'_new = (A' s e^(g - g_new) + e^(x - g_new) v) / s_new.
    q [N, D], k/v [M, D]; returns A [N, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros((q.shape[0], v.shape[1]))
    for n in range(q.shape[0]):
        g, s, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        for mi in range(k.shape[0]):
            x = float(scale) * float(q[n] @ k[mi])
            g_new = max(g, x)
            keep = s * math.exp(g - g_new) if s != 0.0 else 0.0
            e = math.exp(x - g_new)
            s_new = keep + e
            acc = (acc * keep + e * v[mi]) / s_new
            g, s = g_new, s_new
        out[n] = acc
    return out


def tiled_attention(q, k, v, scale, Br, Bc, causal=False, kv_len=None,
                    rescale=True):
    """The tiled forward of one head: Q tiles outside, K/V tiles inside.

    "Flash Attention: The Hidden Gem", The Algorithm (the FlashAttention-2
    forward) and The Correction Factor: for each Q tile start from O = 0,
    l = 0, m = -inf; for each K/V tile form the score tile, take
    m_new = max(rowmax(S), m_old), P = exp(S - m_new),
    l = e^(m_old - m_new) l + rowsum(P), O = diag(e^(m_old - m_new)) O + P V;
    after the last tile O = diag(l)^-1 O and L = m + log(l).

    The mask (causal, bottom-right aligned; keys >= kv_len dropped) is applied
    to each score tile before the max.  A correction e^(-inf - (-inf)) is
    taken as 0 ("Understanding FlashAttention", What is left to the
    implementation); a row with no visible key ends with O = 0, L = -inf.
    q [N, D], k/v [M, D]; returns (O [N, D], L [N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, D = q.shape
    kvl = k.shape[0] if kv_len is None else int(kv_len)
    O = np.zeros((N, D))
    L = np.full(N, -np.inf)
    for i0 in range(0, N, Br):
        qi = q[i0:i0 + Br]
        rows = np.arange(i0, i0 + qi.shape[0])[:, None]
        acc = np.zeros((qi.shape[0], D))
        l = np.zeros((qi.shape[0], 1))
        m = np.full((qi.shape[0], 1), -np.inf)
        for j0 in range(0, kvl, Bc):
            kj, vj = k[j0:min(j0 + Bc, kvl)], v[j0:min(j0 + Bc, kvl)]
            cols = np.arange(j0, j0 + kj.shape[0])[None, :]
            s = float(scale) * (qi @ kj.T)
            if causal:
                s = np.where(cols <= rows + (kvl - N), s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1, keepdims=True))
            # rows still without a visible key keep a zero tile
            base = np.where(m_new == -np.inf, 0.0, m_new)
            p = np.exp(s - base)
            if rescale:
                corr = np.where(m == -np.inf, 0.0, np.exp(m - base))
                l = corr * l + p.sum(axis=1, keepdims=True)
                acc = corr * acc + p @ vj
            else:
                l = l + p.sum(axis=1, keepdims=True)
                acc = acc + p @ vj
            m = m_new
        ok = (l[:, 0] > 0)
        O[i0:i0 + qi.shape[0]][ok] = acc[ok] / l[ok]
        L[i0:i0 + qi.shape[0]][ok] = m[ok, 0] + np.log(l[ok, 0])
    return O, L


def split_merge_attention(q, k, v, scale, bounds, causal=False, kv_len=None):
    """Attention of one head from partial results over key ranges.

    Each range [a, b) of keys gives a partial state (L_s, O_s): the attention
    of the visible keys in that range alone, and its log-sum-exp.  The pages
    do not print this merge; it follows from the rescale identity
    e^(a - c) = e^(a - b) e^(b - c) ("FlashAttention: attention was never
    compute-bound", On the maths anxiety) applied to two partial states as in
    "Flash Attention: The Hidden Gem", The Algorithm, step 5:
    L = M* + log sum_s e^(L_s - M*) with M* = max_s L_s, and
    O = sum_s e^(L_s - L) O_s.  Empty ranges (L_s = -inf) get weight 0.
    q [N, D], k/v [M, D]; returns (O [N, D], L [N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, D = q.shape
    kvl = k.shape[0] if kv_len is None else int(kv_len)
    parts = []
    for a, b in bounds:
        a, b = max(a, 0), min(b, kvl)
        Ls = np.full(N, -np.inf)
        Os = np.zeros((N, D))
        if b > a:
            s = float(scale) * (q @ k[a:b].T)
            if causal:
                i = np.arange(N)[:, None]
                j = np.arange(a, b)[None, :]
                s = np.where(j <= i + (kvl - N), s, -np.inf)
            mx = s.max(axis=1)
            has = mx > -np.inf
            e = np.exp(s[has] - mx[has, None])
            Ls[has] = mx[has] + np.log(e.sum(axis=1))
            Os[has] = (e / e.sum(axis=1, keepdims=True)) @ v[a:b]
        parts.append((Ls, Os))
    Lall = np.stack([p[0] for p in parts])          # [S, N]
    Mstar = Lall.max(axis=0)
    L = np.full(N, -np.inf)
    O = np.zeros((N, D))
    has = Mstar > -np.inf
    w = np.exp(Lall[:, has] - Mstar[has])           # e^(L_s - M*), 0 if empty
    L[has] = Mstar[has] + np.log(w.sum(axis=0))
    for s_idx, (Ls, Os) in enumerate(parts):
        coef = np.exp(Ls[has] - L[has])
        O[has] += coef[:, None] * Os[has]
    return O, L
