"""The definition of exact attention, written out plainly in fp64.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  No blocking, fusion,
streaming or reordering: the full score matrix of each head is materialised,
masked, passed through a three-pass safe softmax and multiplied by V.

Sources (page title, section):
  * "Flash Attention: The Hidden Gem" -- Background (the attention formula
    softmax(Q K^T / sqrt(d_k)) V and the three-step standard computation:
    score matrix, row softmax, multiply by V) and Safe Softmax (subtract the
    row maximum before exponentiating).
  * "Understanding FlashAttention" -- Safe softmax (three logical passes: max,
    sum, divide) and Attention (shapes Q [N,D], K [M,D], V [M,D]; N = 1 for
    decoding against a KV cache of M keys; mask() is elementwise and does not
    depend on the scores; batch and heads only repeat independent problems).
  * "Flash Attention: The Hidden Gem" -- The Algorithm, step 6: the
    log-sum-exp L = m + log(l) that the forward pass also returns.

Readings where the pages leave a step open (each listed in the design notes):
  * causal mask alignment: key j is visible to query i iff j <= i + (kv_len - N)
    ("bottom-right").  With N == kv_len this is the usual j <= i; with N = 1
    the query sees its whole KV-cache history.
  * ``kv_len[b]`` masks keys j >= kv_len[b] of batch b; queries are never
    masked.  ``kv_len=None`` means every batch uses all M keys.
  * a row with no visible key returns O = 0 and LSE = -inf (the pages only
    warn that -inf - (-inf) is undefined).
  * LSE uses the natural logarithm of the sum over visible keys of
    exp(scale * q.k).
  * ``scale`` multiplies the score matrix; the value passed in is upcast to
    fp64 exactly, as are the inputs.
  * local window ("FlashAttention: attention was never compute-bound", Exact
    means exact, compares with "a 128-wide local window" without defining it):
    ``window = (left, right)`` keeps key j for query i only if
    i + off - left <= j <= i + off + right (off = kv_len - N, the causal
    alignment); with ``causal`` the right bound is min(right, 0).  A causal
    128-wide window is ``(127, 0)``: each query sees its 128 most recent keys.
    It is an elementwise mask that does not depend on the scores, the kind
    "Understanding FlashAttention", Attention, allows.
  * any other elementwise mask (the same section: mask() covers causal
    masking "and other kinds", each a constant that does not depend on the
    scores): ``mask`` is a boolean array [Bm, Hm, N, M] (Bm in {1, B}, Hm in
    {1, H}; size 1 means shared by every batch or head); key j is visible to
    query i of (b, h) only if ``mask[b or 0, h or 0, i, j]`` is true, on top of
    kv_len, causal and the window.
"""
import numpy as np

__all__ = ["visible_mask", "safe_softmax", "attention_ref", "attention_rows",
           "clamp_kv_len", "mask_of_head"]


def clamp_kv_len(kv_len, B, M):
    """Per-batch key counts as Python ints in [0, M]; ``None`` -> M for all."""
    if kv_len is None:
        return [M] * B
    kv = np.asarray(kv_len).reshape(-1)
    if kv.shape[0] != B:
        raise ValueError("kv_len must have one entry per batch")
    return [int(min(max(int(x), 0), M)) for x in kv]


def visible_mask(N, kv_len_b, causal, window=None, allow=None):
    """Boolean [N, kv_len_b]: is key j visible to query i.

    Keys at or past ``kv_len_b`` are not part of the matrix at all.  With
    ``causal`` the bottom-right alignment applies: j <= i + (kv_len_b - N).
    ``window = (left, right)`` further keeps only
    i + off - left <= j <= i + off + right.  ``allow`` (boolean [N, >= kv_len_b])
    further keeps only the pairs it marks true.
    """
    i = np.arange(N)[:, None]
    j = np.arange(kv_len_b)[None, :]
    off = kv_len_b - N
    vis = np.ones((N, kv_len_b), dtype=bool)
    if causal:
        vis &= j <= i + off
    if window is not None:
        left, right = (int(x) for x in window)
        if left < 0 or right < 0:
            raise ValueError("window bounds must be >= 0")
        vis &= (j >= i + off - left) & (j <= i + off + right)
    if allow is not None:
        allow = np.asarray(allow, dtype=bool)
        if allow.shape[0] != N or allow.shape[1] < kv_len_b:
            raise ValueError("allow must be [N, >= kv_len] booleans")
        vis &= allow[:, :kv_len_b]
    return vis


def safe_softmax(x):
    """Softmax of a 1-D fp64 vector in three logical passes.

    Pass 1 finds the maximum, pass 2 sums exp(x - max), pass 3 divides.
    Entries equal to -inf (masked) get weight 0.  Returns (weights, max, sum);
    an all -inf row returns zeros with max = -inf and sum = 0.
    """
    x = np.asarray(x, dtype=np.float64)
    m = x.max() if x.size else -np.inf          # pass 1
    if m == -np.inf:
        return np.zeros_like(x), -np.inf, 0.0
    e = np.exp(x - m)                           # exp(-inf - m) = 0 for masked
    l = e.sum()                                 # pass 2
    return e / l, m, l                          # pass 3


def _scores(q, k, scale):
    """Full scaled score matrix S = scale * Q K^T (fp64)."""
    return np.float64(scale) * (q @ k.T)


def _head(q, k, v, scale, causal, kvl, rows=None, window=None, allow=None):
    """One (batch, head) problem.  q [N,D], k/v [M,D] fp64.

    Returns O [len(rows), D] and LSE [len(rows)] for the requested query rows
    (all rows when ``rows`` is None).
    """
    N, D = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    k = k[:kvl]
    v = v[:kvl]
    O = np.zeros((rows.size, D))
    LSE = np.full(rows.size, -np.inf)
    if kvl == 0 or rows.size == 0:
        return O, LSE
    S = _scores(q[rows], k, scale)                      # step 1: materialise S
    vis = visible_mask(N, kvl, causal, window, allow)[rows]
    S = np.where(vis, S, -np.inf)                       # step 2: mask
    for r in range(rows.size):                          # steps 3-5: softmax
        p, m, l = safe_softmax(S[r])
        if m == -np.inf:
            continue                                    # no visible key
        O[r] = p @ v                                    # step 6: P V
        LSE[r] = m + np.log(l)                          # step 7: L = m + log l
    return O, LSE


def mask_of_head(mask, b, h):
    """The [N, M] slice of an elementwise mask [Bm, Hm, N, M] that applies to
    (batch b, head h); a size-1 batch or head axis is shared.  None -> None."""
    if mask is None:
        return None
    mask = np.asarray(mask, dtype=bool)
    if mask.ndim != 4:
        raise ValueError("mask must be [Bm, Hm, N, M]")
    return mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]


def attention_ref(q, k, v, scale, causal=False, kv_len=None, window=None, mask=None):
    """Exact attention forward for [B, H, N, D] / [B, H, M, D] inputs.

    Returns (O [B,H,N,D] fp64, LSE [B,H,N] fp64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    M = k.shape[2]
    if k.shape != (B, H, M, D) or v.shape != (B, H, M, D):
        raise ValueError("K and V must be [B, H, M, D] matching Q [B, H, N, D]")
    kvs = clamp_kv_len(kv_len, B, M)
    O = np.zeros((B, H, N, D))
    LSE = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = _head(q[b, h], k[b, h], v[b, h], scale,
                                       causal, kvs[b], window=window,
                                       allow=mask_of_head(mask, b, h))
    return O, LSE


def attention_rows(q, k, v, scale, causal, kv_len, picks, window=None, mask=None):
    """The same definition evaluated only for selected outputs.

    ``picks`` is a sequence of (b, h, i).  ``q`` may be [B,H,N,D] or a callable
    ``q(b, h) -> [N, D]`` (likewise ``k``, ``v`` with [M, D]) so that large
    device tensors can be copied back one head at a time.  Returns
    (O [P, D], LSE [P]) in fp64.  ``mask`` is as in ``attention_ref``.
    """
    def head_of(t, b, h):
        return np.asarray(t(b, h) if callable(t) else t[b, h], dtype=np.float64)

    picks = [tuple(int(x) for x in p) for p in picks]
    by_head = {}
    for idx, (b, h, i) in enumerate(picks):
        by_head.setdefault((b, h), []).append((idx, i))
    outO, outL = None, np.full(len(picks), -np.inf)
    for (b, h), lst in by_head.items():
        qh, kh, vh = head_of(q, b, h), head_of(k, b, h), head_of(v, b, h)
        N, D = qh.shape
        M = kh.shape[0]
        if outO is None:
            outO = np.zeros((len(picks), D))
        kvl = min(max(int(M if kv_len is None else np.asarray(kv_len).reshape(-1)[b]), 0), M)
        rows = [i for _, i in lst]
        O, L = _head(qh, kh, vh, scale, causal, kvl, rows, window=window,
                     allow=mask_of_head(mask, b, h))
        for r, (idx, _) in enumerate(lst):
            outO[idx] = O[r]
            outL[idx] = L[r]
    if outO is None:
        outO = np.zeros((0, 0))
    return outO, outL

