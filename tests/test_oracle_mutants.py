"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and check that the pins catch every one of them."""
import importlib.util
import os
import types

import numpy as np
import pytest

from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "lse_sign": ("LSE[r] = m + np.log(l)", "LSE[r] = m - np.log(l)"),
    "no_max_shift": ("e = np.exp(x - m)", "e = np.exp(x)"),
    "no_divide": ("return e / l, m, l", "return e, m, l"),
    "top_left_causal": ("        vis &= j <= i + off\n", "        vis &= j <= i\n"),
    "strict_causal": ("        vis &= j <= i + off\n", "        vis &= j < i + off\n"),
    "window_lower_strict": ("vis &= (j >= i + off - left)", "vis &= (j > i + off - left)"),
    "window_top_left": ("vis &= (j >= i + off - left) & (j <= i + off + right)",
                        "vis &= (j >= i - left) & (j <= i + right)"),
    "window_ignored": ("vis &= (j >= i + off - left) & (j <= i + off + right)", "pass"),
    "mask_ignored": ("        vis &= allow[:, :kv_len_b]\n", "        pass\n"),
    "mask_inverted": ("        vis &= allow[:, :kv_len_b]\n", "        vis &= ~allow[:, :kv_len_b]\n"),
    "mask_transposed_broadcast": ("mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]",
                                  "mask[h if mask.shape[0] > 1 else 0, b if mask.shape[1] > 1 else 0]"),
    "mask_shared_by_heads": ("mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]",
                             "mask[b if mask.shape[0] > 1 else 0, 0]"),
    "scale_twice": ("return np.float64(scale) * (q @ k.T)",
                    "return np.float64(scale) ** 2 * (q @ k.T)"),
    "scale_dropped": ("return np.float64(scale) * (q @ k.T)", "return (q @ k.T)"),
    "k_for_v": ("O[r] = p @ v", "O[r] = p @ k"),
    "kv_len_ignored": ("k = k[:kvl]\n    v = v[:kvl]", "k = k\n    v = v"),
    "log2_lse": ("LSE[r] = m + np.log(l)", "LSE[r] = m + np.log2(l)"),
}


def load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = load_mutant(*MUTANTS[name])

    def attn(q, k, v, scale, causal, kv_len, window=None, mask=None):
        return mod.attention_ref(q, k, v, scale, causal, kv_len, window=window, mask=mask)

    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_ATTN_PINS:
            try:
                pin(attn)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"no pin fails for mutant {name}"
