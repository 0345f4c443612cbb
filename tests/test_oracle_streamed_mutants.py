"""Plant one mistake at a time in a copy of the streamed forms (online
softmax, tiled forward) and check that their pins catch each (CPU only)."""
import math
import os
import types

import numpy as np
import pytest

from oracle import attention as A
from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "streamed.py")

MUTANTS = {
    "correction_inverted": ("factor = math.exp(m_old - m_new) if correct else 1.0",
                            "factor = math.exp(m_new - m_old) if correct else 1.0"),
    "correction_dropped": ("factor = math.exp(m_old - m_new) if correct else 1.0",
                           "factor = 1.0"),
    "block_sum_old_max": ("float(np.exp(block - m_new).sum())",
                          "float(np.exp(block - m_old).sum())"),
    "no_final_division": ("return np.exp(x - m_fin) / l_fin", "return np.exp(x - m_fin)"),
    "tiled_output_not_rescaled": ("self.acc = alpha[:, None] * self.acc + w @ v_tile",
                                  "self.acc = self.acc + w @ v_tile"),
    "tiled_top_left_causal": ("kj[None, :] <= qi[:, None] + (n_k - n_q)",
                              "kj[None, :] <= qi[:, None]"),
}


def load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("streamed_mutant")
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def pin_online_row(mod):
    pins.pin_p2_online_row(A.safe_softmax, mod.online_softmax)


def pin_tiled(mod):
    rng = np.random.default_rng(7)
    N, D = 160, 32
    q, k, v = (rng.standard_normal((N, D)), rng.standard_normal((N, D)),
               rng.standard_normal((N, D)))
    for causal, kvl in ((False, None), (True, 150)):
        O, L = mod.tiled_attention(q, k, v, 1 / math.sqrt(D), 16, 48, causal, kvl)
        Or, Lr = A.attention_ref(q[None, None], k[None, None], v[None, None], 1 / math.sqrt(D),
                                 causal, None if kvl is None else [kvl])
        assert np.max(np.abs(O - Or[0, 0])) <= 1e-14


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_streamed_pins_catch_mutant(name):
    mod = load_mutant(*MUTANTS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in (pin_online_row, pin_tiled):
            try:
                pin(mod)
            except (AssertionError, ValueError, FloatingPointError, OverflowError, ZeroDivisionError):
                caught.append(pin.__name__)
    assert caught, f"no pin fails for mutant {name}"


def test_unmutated_streamed_forms_pass():
    import oracle.streamed as S
    pin_online_row(S)
    pin_tiled(S)
