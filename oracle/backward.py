"""Gradients of exact attention, written out plainly in fp64.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Every matrix of a
head is materialised: the probabilities P, the upstream gradient of P, the
row statistic D and the gradient of the scores.  No tiling, no recomputation
from a saved log-sum-exp, no streaming.

Sources (page title, section):
  * "Flash Attention: The Hidden Gem" -- Phase 2: Backward Pass:
      - Chain Rule Through a Matrix Multiply: from O = P V, the gradients are
        dV = P^T dO and dP = dO V^T;
      - The Softmax Jacobian: per row, J_i = diag(P_i) - P_i P_i^T, which
        gives dS_ij = P_ij (dP_ij - D_i) with D_i = sum_k dP_ik P_ik;
      - The D Shortcut: the same D_i equals sum_m dO_im O_im (that identity
        is checked by the tests, not used here);
      - The Algorithm, steps 15 and 16: from S = Q K^T, dQ = dS K and
        dK = dS^T Q.
  * "FlashAttention: attention was never compute-bound" -- The backward pass:
    pay flops, save bytes (what the fused backward stores and recomputes;
    the counting forms live in ``oracle/counting.py``).

Readings where the pages leave a step open (each listed in the design notes):
  * the pages write S = Q K^T without the softmax scale.  With the forward's
    S = scale * Q K^T the chain rule puts the same factor on both score
    gradients: dQ = scale * dS K and dK = scale * dS^T Q.
  * a masked entry has P = 0 and therefore dS = 0: it passes no gradient.
    Keys at or past kv_len[b] get dK = dV = 0; a query row with no visible key
    gets dQ = 0 and D = 0.
  * an element mask (``oracle.attention``: a constant that does not depend
    on the scores) enters only through which entries are visible, so it
    changes nothing in the chain rule: its hidden entries pass no gradient.
  * dO is the gradient of the loss with respect to O, same shape as O; the
    gradient with respect to LSE is not an input (the pages keep L for the
    backward pass only, never as a result of the layer).
"""
import numpy as np

from .attention import clamp_kv_len, mask_of_head, safe_softmax, visible_mask

__all__ = ["head_backward", "attention_bwd_ref"]


def head_backward(q, k, v, do, scale, causal, kvl, window=None, allow=None):
    """One (batch, head) problem in fp64: q, do [N,D]; k, v [M,D]; ``allow``
    an optional boolean [N, M] element mask.

    Returns a dict with the gradients ``dq`` [N,D], ``dk`` [M,D], ``dv``
    [M,D], the row statistic ``delta`` [N] and the intermediates ``p``,
    ``dp``, ``ds`` (each [N, kvl]) and ``o`` [N,D].
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    N, D = q.shape
    M = k.shape[0]
    kvl = int(min(max(kvl, 0), M))
    kv, vv = k[:kvl], v[:kvl]
    # forward, as defined: scores, mask, row softmax, weighted sum of V
    S = np.float64(scale) * (q @ kv.T)
    S = np.where(visible_mask(N, kvl, causal, window, allow), S, -np.inf)
    P = np.zeros((N, kvl))
    for i in range(N):
        P[i] = safe_softmax(S[i])[0]      # a row with no visible key stays 0
    O = P @ vv
    # chain rule through O = P V
    dV = P.T @ do                          # dV = P^T dO
    dP = do @ vv.T                         # dP = dO V^T
    # softmax Jacobian, row by row: dS_i = dP_i J_i with J_i = diag(P_i) - P_i P_i^T
    delta = np.einsum("ij,ij->i", dP, P)   # D_i = sum_k dP_ik P_ik
    dS = P * (dP - delta[:, None])
    # chain rule through S = scale * Q K^T
    dQ = np.float64(scale) * (dS @ kv)
    dK = np.zeros((M, D))
    dVf = np.zeros((M, D))
    dK[:kvl] = np.float64(scale) * (dS.T @ q)
    dVf[:kvl] = dV
    return {"dq": dQ, "dk": dK, "dv": dVf, "delta": delta,
            "p": P, "dp": dP, "ds": dS, "o": O}


def attention_bwd_ref(q, k, v, do, scale, causal=False, kv_len=None, window=None, mask=None):
    """Gradients of O = attention(Q, K, V) for the upstream gradient dO.

    q, do [B,H,N,D]; k, v [B,H,M,D]; ``mask`` as in
    ``oracle.attention.attention_ref``.  Returns (dQ, dK, dV, D) in fp64 with
    D [B,H,N] the row statistic sum_k dP_ik P_ik.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, D = q.shape
    M = k.shape[2]
    if k.shape != (B, H, M, D) or v.shape != (B, H, M, D) or do.shape != q.shape:
        raise ValueError("shapes: q, do [B,H,N,D]; k, v [B,H,M,D]")
    kvs = clamp_kv_len(kv_len, B, M)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    delta = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            r = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, kvs[b], window,
                              mask_of_head(mask, b, h))
            dQ[b, h], dK[b, h], dV[b, h], delta[b, h] = r["dq"], r["dk"], r["dv"], r["delta"]
    return dQ, dK, dV, delta
