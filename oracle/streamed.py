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


def _absorb_block(state, block, correct):
    """One step of the online normaliser over a block of scores.

    ``state`` is (m, l): the largest score seen and the running sum of
    e^(x - m) over the scores seen.  "FlashAttention: attention was never
    compute-bound", The one formula: the new maximum is the larger of m and
    the block's maximum, and l becomes e^(m_old - m_new) l + sum of
    e^(x - m_new) over the block.  ``correct=False`` keeps l as it is instead
    of multiplying it by e^(m_old - m_new) (the mistake the same page's
    "Now break it" section makes on purpose).  Starting from (-inf, 0), the
    factor e^(-inf) is 0 and multiplies an empty sum.
    """
    m_old, l_old = state
    m_new = max(m_old, float(np.max(block)))
    factor = math.exp(m_old - m_new) if correct else 1.0
    return m_new, factor * l_old + float(np.exp(block - m_new).sum())


def online_softmax(scores, block_len=8, correct=True):
    """Softmax of a 1-D score vector from a single streamed sweep.

    The scores are cut into consecutive blocks of ``block_len``; the state
    (m, l) starts at (-inf, 0) ("Flash Attention: The Hidden Gem", Online
    Softmax) and absorbs the blocks in order (``_absorb_block``).  A second
    read then turns every score into e^(x - m) / l with the final m and l.
    """
    x = np.asarray(scores, dtype=np.float64).reshape(-1)
    blocks = [x[a:a + block_len] for a in range(0, x.size, block_len)]
    state = (-math.inf, 0.0)
    for blk in blocks:
        state = _absorb_block(state, blk, correct)
    m_fin, l_fin = state
    return np.exp(x - m_fin) / l_fin


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


class _RowBlockState:
    """Running state of one block of query rows: per row the largest visible
    score m, the sum l of e^(s - m) and the unnormalised output acc, all
    relative to the same m ("FlashAttention: attention was never
    compute-bound", The one formula: O is rescaled alongside l because its
    weights moved)."""

    def __init__(self, rows, d, correct):
        self.m = np.full(rows, -np.inf)
        self.l = np.zeros(rows)
        self.acc = np.zeros((rows, d))
        self.correct = correct

    def absorb(self, s, v_tile):
        """Fold in one score tile s [rows, keys] (masked entries -inf) and the
        matching value rows.  Rows that still see no key keep m = -inf and
        add nothing; their correction factor is taken as 0 instead of
        e^(-inf - (-inf)) ("Understanding FlashAttention", What is left to
        the implementation)."""
        m_new = np.maximum(self.m, s.max(axis=1))
        seen = m_new > -np.inf
        ref = np.where(seen, m_new, 0.0)                 # finite baseline per row
        w = np.exp(s - ref[:, None])                     # e^(S - m_new); 0 where masked
        if self.correct:
            alpha = np.where(self.m > -np.inf, np.exp(self.m - ref), 0.0)
        else:
            alpha = np.ones_like(self.l)
        self.l = alpha * self.l + w.sum(axis=1)
        self.acc = alpha[:, None] * self.acc + w @ v_tile
        self.m = m_new

    def finish(self):
        """O = acc / l and L = m + ln l; rows that saw no key give 0 and -inf
        ("Flash Attention: The Hidden Gem", The Algorithm, the last step)."""
        live = self.l > 0
        O = np.zeros_like(self.acc)
        L = np.full(self.l.shape, -np.inf)
        O[live] = self.acc[live] / self.l[live, None]
        L[live] = self.m[live] + np.log(self.l[live])
        return O, L


def tiled_attention(q, k, v, scale, Br, Bc, causal=False, kv_len=None, correct=True):
    """The tiled forward of one head: blocks of Br query rows, each sweeping
    the keys in tiles of Bc.

    "Flash Attention: The Hidden Gem", The Algorithm and The Correction
    Factor: for every query block and every key tile, form the score tile,
    move the running maximum, rescale l and the output accumulator by
    e^(m_old - m_new) and add the tile's weights and weighted values; divide
    once at the end.  The mask -- keys >= kv_len dropped, and with ``causal``
    key j visible to query i iff j <= i + (kv_len - N) -- is applied to each
    score tile before it is absorbed.  ``correct=False`` omits the rescale.
    q [N, D], k/v [M, D]; returns (O [N, D], L [N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    n_k = k.shape[0] if kv_len is None else int(kv_len)
    O = np.zeros((n_q, d))
    L = np.full(n_q, -np.inf)
    for r0 in range(0, n_q, Br):
        r1 = min(r0 + Br, n_q)
        state = _RowBlockState(r1 - r0, d, correct)
        qi = np.arange(r0, r1)
        for c0 in range(0, n_k, Bc):
            c1 = min(c0 + Bc, n_k)
            s = float(scale) * (q[r0:r1] @ k[c0:c1].T)
            if causal:
                kj = np.arange(c0, c1)
                s = np.where(kj[None, :] <= qi[:, None] + (n_k - n_q), s, -np.inf)
            state.absorb(s, v[c0:c1])
        O[r0:r1], L[r0:r1] = state.finish()
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
