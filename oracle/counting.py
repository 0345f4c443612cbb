"""HBM-byte and FLOP counting model of the explainer page, as closed forms.

TEST INFRASTRUCTURE AND REPORTING ONLY -- see ``oracle/__init__.py``.

"FlashAttention: attention was never compute-bound" counts, for one head with
sequence length n and head dim d, every element that crosses between slow and
fast memory and every multiply-add (sections Where the time actually goes,
Tiling: same answer, flat memory, How big should a tile be?, The backward
pass: pay flops, save bytes, And no, it is not doing less arithmetic).  Its
script is not available; the forms below are read off the tiled forward it
prints (one Q tile load per row block, one K and one V tile load per pair of
blocks, one O write per row block; the working set of one Q tile, one K and
one V tile, one score tile and two running statistics) and off the standard
three-kernel computation (read Q and K, write S, read S, write P, read P,
read V, write O).  Every printed row of its tables follows from them exactly
(``tests/test_counting_model.py``).  "MB" on the page is 2**20 bytes.

``elem`` is the element size in bytes: 4 on the page (float32); 2 for bf16.
"""
import math

__all__ = ["naive_elems", "naive_bytes", "flash_elems", "flash_bytes",
           "working_set_elems", "std_peak_elems", "attention_flops",
           "bwd_std_stored_elems", "bwd_flash_stored_elems",
           "bwd_std_flops", "bwd_flash_flops", "MiB"]

MiB = float(1 << 20)


def naive_elems(n, d):
    """Standard attention: Q, K read (2nd); S written and read, P written and
    read (4n^2); V read and O written (2nd)."""
    return 4 * n * n + 4 * n * d


def naive_bytes(n, d, elem=4):
    return elem * naive_elems(n, d)


def flash_elems(n, d, Br):
    """Tiled forward: Q read once and O written once (2nd) plus all of K and V
    once per Q row block (2nd per block, ceil(n / Br) blocks)."""
    return 2 * n * d + 2 * n * d * math.ceil(n / Br)


def flash_bytes(n, d, Br, elem=4):
    return elem * flash_elems(n, d, Br)


def working_set_elems(d, Br, Bc):
    """On-chip working set: one Q tile, one K and one V tile, one score tile,
    two running statistics per row."""
    return Br * d + 2 * Bc * d + Br * Bc + 2 * Br


def std_peak_elems(n):
    """Standard attention keeps the n x n score matrix."""
    return n * n


def attention_flops(n, d):
    """Two n x n x d products at 2 flops per multiply-add: 4 n^2 d."""
    return 4 * n * n * d


def bwd_std_stored_elems(n, d):
    """Backward of standard attention stores P (n^2) plus Q, K, V (3nd)."""
    return n * n + 3 * n * d


def bwd_flash_stored_elems(n, d):
    """Backward of the fused kernel stores Q, K, V and two statistics per row."""
    return 3 * n * d + 2 * n


def bwd_std_flops(n, d):
    """Counted backward flops of standard attention (the page prints 10 n^2 d
    worth without breaking it down)."""
    return 10 * n * n * d


def bwd_flash_flops(n, d):
    """Backward with the score tile recomputed: one extra n x n x d product."""
    return 12 * n * n * d
