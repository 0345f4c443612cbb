"""The backward oracle against its pins, an independent fp64 autograd, and
planted mistakes (all on the CPU)."""
import os
import types

import numpy as np
import pytest

from oracle.backward import attention_bwd_ref, head_backward
from tests import pins_bwd


@pytest.mark.parametrize("pin", pins_bwd.ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin):
    pin(attention_bwd_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_oracle_matches_torch_autograd_fp64(causal):
    """torch's autograd of a plain fp64 softmax attention on the CPU (another
    code path for the same derivative: masked_fill, softmax's own backward)."""
    import torch
    rng = np.random.default_rng(31)
    B, H, N, M, D, scale = 2, 2, 9, 11, 6, 0.4
    kvl = [11, 7]
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(B, H, N, D), (B, H, M, D), (B, H, M, D), (B, H, N, D)])
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    i = torch.arange(N)[:, None]
    j = torch.arange(M)[None, :]
    vis = torch.stack([(j < kvl[b]) & ((j <= i + kvl[b] - N) if causal else True)
                       for b in range(B)])[:, None]
    p = torch.softmax(s.masked_fill(~vis, float("-inf")), dim=-1)
    p = torch.nan_to_num(p, nan=0.0)        # rows with no visible key
    (p @ tv).backward(torch.tensor(do))
    dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, scale, causal, kvl)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(got - want.numpy())) < 1e-12


def test_bwd_oracle_softmax_jacobian_rows():
    """Each row of dS sums to zero (J_i has zero row sums), and dS = dP J_i
    with the Jacobian built entry by entry from its two cases."""
    rng = np.random.default_rng(32)
    q, k, v, do = (rng.standard_normal(s) for s in [(6, 4), (8, 4), (8, 4), (6, 4)])
    r = head_backward(q, k, v, do, 0.7, True, 8)
    assert np.max(np.abs(r["ds"].sum(axis=1))) < 1e-13
    for i in range(6):
        p = r["p"][i]
        J = np.array([[p[a] * (1 - p[a]) if a == c else -p[a] * p[c]
                       for c in range(8)] for a in range(8)])
        assert np.max(np.abs(r["dp"][i] @ J - r["ds"][i])) < 1e-13


SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "backward.py")

MUTANTS = {
    "delta_dropped": ("dS = P * (dP - delta[:, None])", "dS = P * dP"),
    "delta_sign": ("dS = P * (dP - delta[:, None])", "dS = P * (dP + delta[:, None])"),
    "jacobian_diagonal_only": ("dS = P * (dP - delta[:, None])", "dS = P * (1 - P) * dP"),
    "dq_scale_dropped": ("dQ = np.float64(scale) * (dS @ kv)", "dQ = dS @ kv"),
    "dk_scale_dropped": ("dK[:kvl] = np.float64(scale) * (dS.T @ q)", "dK[:kvl] = dS.T @ q"),
    "dq_uses_v": ("dQ = np.float64(scale) * (dS @ kv)", "dQ = np.float64(scale) * (dS @ vv)"),
    "dk_uses_do": ("dK[:kvl] = np.float64(scale) * (dS.T @ q)",
                   "dK[:kvl] = np.float64(scale) * (dS.T @ do)"),
    "dv_uses_q": ("dV = P.T @ do", "dV = P.T @ q"),
    "dp_uses_k": ("dP = do @ vv.T", "dP = do @ kv.T"),
    "delta_from_dp_only": ('delta = np.einsum("ij,ij->i", dP, P)', "delta = dP.sum(axis=1)"),
    "top_left_causal": ("S = np.where(visible_mask(N, kvl, causal, window, allow), S, -np.inf)",
                        "S = np.where(visible_mask(N, N, causal)[:, :kvl] if kvl <= N else "
                        "visible_mask(N, kvl, causal), S, -np.inf)"),
    "mask_ignored": ("visible_mask(N, kvl, causal, window, allow)", "visible_mask(N, kvl, causal, window)"),
}


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_mutant(name):
    mod = _load_mutant(*MUTANTS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins_bwd.ALL_BWD_PINS:
            try:
                pin(mod.attention_bwd_ref)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"no pin fails for mutant {name}"
