"""The oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import streamed as S
from tests import pins


def oracle_attn(q, k, v, scale, causal, kv_len, window=None, mask=None):
    return A.attention_ref(q, k, v, scale, causal, kv_len, window=window, mask=mask)


@pytest.mark.parametrize("pin", pins.ALL_ATTN_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_attn)


def test_p2_online_softmax_row():
    """Printed: online vs ordinary max-abs 0.00e+00; no-rescale 6.53e-01 with
    weights summing to 0.190131; the first six weights of each."""
    row, ordinary, online, broken = pins.pin_p2_online_row(A.safe_softmax, S.online_softmax)
    # the page calls the agreement exact; with this row and block it is bit-zero
    assert np.max(np.abs(online - ordinary)) <= 1e-15
    # only l differs without the rescale, so every weight is off by one factor
    assert np.allclose(broken / ordinary, broken.sum(), rtol=1e-12, atol=0)


def test_p3_online_normalizer():
    """"Understanding FlashAttention", Online softmax: after one sweep the
    running max equals the row max exactly and the running sum matches the
    safe-softmax denominator (the page asserts isclose)."""
    for seed in range(5):
        x = np.random.default_rng(100 + seed).random(8)
        g, s = S.online_normalizer(x)
        _, m, l = A.safe_softmax(x)
        assert g == m
        assert math.isclose(s, l, rel_tol=1e-13)


def test_p3_per_key_recurrence_matches_definition():
    """"Understanding FlashAttention", Merging the two loops: the per-key
    recurrence with a normalised accumulator equals the direct calculation."""
    rng = np.random.default_rng(5)
    q, k, v = rng.random((8, 4)), rng.random((6, 4)), rng.random((6, 4))
    out = S.per_key_attention(q, k, v)
    O, _ = A.attention_ref(q[None, None], k[None, None], v[None, None], 1.0)
    assert np.max(np.abs(out - O[0, 0])) <= 1e-14


@pytest.mark.parametrize("Br,Bc", [(2, 2), (64, 64), (16, 48), (128, 32), (7, 5)])
@pytest.mark.parametrize("causal,kvl", [(False, None), (True, None), (True, 150), (False, 77)])
def test_tiled_forward_equals_definition(Br, Bc, causal, kvl):
    """"Flash Attention: The Hidden Gem", The Algorithm (worked example
    N = 8, d = 128, Br = Bc = 2 among the tile sizes) and "FlashAttention:
    attention was never compute-bound", Tiling: the tiled recurrence returns
    the same O and L as the materialised definition (the page prints
    max-abs 8e-17 .. 2.5e-16 in fp64)."""
    rng = np.random.default_rng(7)
    N, M, D = 160, 160, 64
    q, k, v = (rng.standard_normal((N, D)), rng.standard_normal((M, D)),
               rng.standard_normal((M, D)))
    scale = 1 / math.sqrt(D)
    O, L = S.tiled_attention(q, k, v, scale, Br, Bc, causal, kvl)
    Or, Lr = A.attention_ref(q[None, None], k[None, None], v[None, None], scale,
                             causal, None if kvl is None else [kvl])
    assert np.array_equal(np.isneginf(L), np.isneginf(Lr[0, 0]))
    fin = np.isfinite(L)
    assert np.max(np.abs(O - Or[0, 0])) <= 1e-14
    assert np.max(np.abs(L[fin] - Lr[0, 0][fin])) <= 1e-13


def test_tiled_forward_without_rescale_is_wrong():
    """"Now break it": dropping the correction gives a visibly wrong output."""
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((64, 16)) * 2, rng.standard_normal((64, 16)),
               rng.standard_normal((64, 16)))
    O, _ = S.tiled_attention(q, k, v, 1.0, 16, 8, correct=False)
    Or, _ = A.attention_ref(q[None, None], k[None, None], v[None, None], 1.0)
    assert np.max(np.abs(O - Or[0, 0])) > 1e-2


def test_p1_worked_example_first_tile():
    """"Flash Attention: The Hidden Gem", The Algorithm, inner step j = 1:
    with one K/V tile the running state is exactly P_11 V_1 with
    l = rowsum(P_11) and no correction, so the tiled result over a single
    tile of two keys equals the definition over those two keys."""
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((8, 128)), rng.standard_normal((2, 128)), rng.standard_normal((2, 128))
    O, L = S.tiled_attention(q, k, v, 1.0, 2, 2)
    s = q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    assert np.max(np.abs(O - (p @ v) / p.sum(axis=1, keepdims=True))) <= 1e-14


@pytest.mark.parametrize("bounds", [[(0, 300)], [(0, 100), (100, 200), (200, 300)],
                                    [(0, 1), (1, 257), (257, 300)],
                                    [(0, 64), (64, 128), (128, 192), (192, 256), (256, 320)]])
@pytest.mark.parametrize("causal,kvl,N", [(False, None, 1), (False, 173, 1), (True, 200, 1),
                                          (False, None, 5), (True, None, 300)])
def test_split_merge_equals_definition(bounds, causal, kvl, N):
    """Partial states over key ranges merged through the log-sum-exp give the
    definition; empty ranges (past kv_len) carry weight 0."""
    rng = np.random.default_rng(10)
    M, D = 300, 32
    q, k, v = (rng.standard_normal((N, D)), rng.standard_normal((M, D)),
               rng.standard_normal((M, D)))
    O, L = S.split_merge_attention(q, k, v, 0.2, bounds, causal, kvl)
    Or, Lr = A.attention_ref(q[None, None], k[None, None], v[None, None], 0.2,
                             causal, None if kvl is None else [kvl])
    fin = np.isfinite(Lr[0, 0])
    assert np.array_equal(fin, np.isfinite(L))
    assert np.max(np.abs(O - Or[0, 0])) <= 1e-14
    assert np.max(np.abs(L[fin] - Lr[0, 0][fin])) <= 1e-13


def test_p3_loop_interchange_is_exact():
    """"Understanding FlashAttention", How to understand it: swapping the d and
    m loops of a matrix product keeps the order over m, so the result is
    bit-identical."""
    rng = np.random.default_rng(11)
    y, v = rng.random((8, 6)).tolist(), rng.random((6, 4)).tolist()
    a = [[0.0] * 4 for _ in range(8)]
    for n in range(8):
        for d in range(4):
            for m in range(6):
                a[n][d] += y[n][m] * v[m][d]
    a2 = [[0.0] * 4 for _ in range(8)]
    for n in range(8):
        for m in range(6):
            for d in range(4):
                a2[n][d] += y[n][m] * v[m][d]
    assert a == a2


def test_attention_rows_matches_full():
    """The sampled-row entry used at large sizes is the same definition."""
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((2, 3, 20, 8)), rng.standard_normal((2, 3, 25, 8)),
               rng.standard_normal((2, 3, 25, 8)))
    kvl = [25, 11]
    O, L = A.attention_ref(q, k, v, 0.3, True, kvl)
    picks = [(0, 0, 0), (1, 2, 19), (1, 0, 3), (0, 1, 10), (1, 1, 9)]
    Os, Ls = A.attention_rows(q, k, v, 0.3, True, kvl, picks)
    for r, (b, h, i) in enumerate(picks):
        # a subset of rows may take another BLAS summation order
        assert np.max(np.abs(Os[r] - O[b, h, i])) <= 1e-15
        assert (np.isneginf(Ls[r]) and np.isneginf(L[b, h, i])) or abs(Ls[r] - L[b, h, i]) <= 1e-15
    # callable form (one head copied at a time)
    Os2, Ls2 = A.attention_rows(lambda b, h: q[b, h], lambda b, h: k[b, h],
                                lambda b, h: v[b, h], 0.3, True, kvl, picks)
    assert np.array_equal(Os, Os2) and np.array_equal(Ls, Ls2)


@pytest.mark.parametrize("window,with_mask", [((5, 0), False), ((3, 2), False), (None, True),
                                              ((6, 1), True)])
def test_attention_rows_with_window_and_mask(window, with_mask):
    """The sampled-row entry under a local window and an element mask equals
    the matching rows of the whole-tensor definition (the large-size window
    and mask parity checks rest on this).  The mask is shared over heads
    (size-1 head axis) so the broadcast path is covered too."""
    rng = np.random.default_rng(14)
    B, H, N, M, D = 2, 3, 20, 25, 8
    q, k, v = (rng.standard_normal((B, H, N, D)), rng.standard_normal((B, H, M, D)),
               rng.standard_normal((B, H, M, D)))
    kvl = [25, 13]
    mask = rng.random((B, 1, N, M)) < 0.6 if with_mask else None
    O, L = A.attention_ref(q, k, v, 0.3, True, kvl, window=window, mask=mask)
    picks = [(b, h, i) for b in range(B) for h in range(H) for i in (0, 3, 9, 19)]
    Os, Ls = A.attention_rows(q, k, v, 0.3, True, kvl, picks, window=window, mask=mask)
    for r, (b, h, i) in enumerate(picks):
        assert np.max(np.abs(Os[r] - O[b, h, i])) <= 1e-15
        assert (np.isneginf(Ls[r]) and np.isneginf(L[b, h, i])) or abs(Ls[r] - L[b, h, i]) <= 1e-15
    # the window and the mask change the answer on these rows (not a vacuous check)
    O0, _ = A.attention_ref(q, k, v, 0.3, True, kvl)
    assert np.max(np.abs(O - O0)) > 1e-3


def test_oracle_float32_inputs_upcast_exactly():
    """Inputs are upcast exactly: float32 data gives the same result as the
    same values already in float64."""
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, 1, 9, 8)).astype(np.float32) for _ in range(3))
    O32, L32 = A.attention_ref(q, k, v, np.float32(0.125), False)
    O64, L64 = A.attention_ref(q.astype(np.float64), k.astype(np.float64),
                               v.astype(np.float64), 0.125, False)
    assert np.array_equal(O32, O64) and np.array_equal(L32, L64)


def test_e4m3_decoding_used_by_the_fp8_tests():
    """torch's float8_e4m3fn -> float conversion, which the fp8 tests use to
    hand the oracle the exact input values, against the OCP E4M3 definition:
    sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at exponent
    0, NaN for S.1111.111 and no infinities."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(got[c]), c
            continue
        val = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert got[c] == (-val if s else val), (c, got[c])
