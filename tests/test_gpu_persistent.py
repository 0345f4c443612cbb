"""GPU parity of the causal prefill's persistent walk run as one pipeline.

With causal or windowed attention (or causal with an element mask), no
kv_len, M >= N >= 256 and more work items than workgroups, each persistent
workgroup walks several items (256-query tiles of some
(batch, head)) and its iterations on the last tiles of one item already load,
score and weigh the first tiles of the next ("Understanding FlashAttention",
From loops to tiling: the tiles of one query block are independent of every
other block's, so the order of the blocks is free).  These cases give every
workgroup two or three items, end items in ragged query tiles, move the row
reference on an item's first tile, and compare every element with the fp64
oracle -- and bit for bit with the same launch given kv_len = M, which runs
each item on its own (same arithmetic, same order).
"""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref
from tests.gpu_helpers import compare, default_scale, host64
from tests.mask_layout import mask_layout

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def make(seed, B, H, N, M, D):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, "bf16", DEV) for x in (q, k, v))


def check_walk(q, k, v, scale, what, rel_o=0.0, causal=True, window=None, allowed=None):
    B, H, N, D = q.shape
    M = k.shape[2]
    items = B * H * ((N + 255) // 256)
    say(f"{what}: B={B} H={H} N={N} M={M} D={D} causal={causal} window={window} "
        f"mask={None if allowed is None else allowed.shape}, {items} work items over 256 workgroups")
    words = None if allowed is None else fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    o, l = fa.fwd(q, k, v, scale=scale, causal=causal, window=window, mask=words)
    torch.cuda.synchronize()
    say(f"{what}: same launch item by item (kv_len = M)")
    o2, l2 = fa.fwd(q, k, v, scale=scale, causal=causal, window=window, mask=words, kv_len=[M] * B)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), f"{what}: output differs from the item-by-item walk"
    assert torch.equal(l, l2), f"{what}: LSE differs from the item-by-item walk"
    say(f"{what}: oracle")
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), scale, causal, window=window, mask=allowed)
    O = host64(o)
    if rel_o:
        # the part of the output error that scales with |O|: bf16 rounding
        # of the output itself, at most half an ulp, 2^-8 |O|
        excess = np.abs(O - Or) - rel_o * np.abs(Or)
        say(f"{what}: O error beyond {rel_o:g} |O|: {float(excess.max()):.2e}")
        O = Or + np.sign(O - Or) * np.maximum(excess, 0.0)
    eo, el = compare(O, host64(l), Or, Lr, "bf16", what)
    say(f"{what}: O {eo:.2e} LSE {el:.2e}")


@pytest.mark.parametrize("D", [64, 128])
def test_walk_several_items_per_workgroup(D):
    """600 items of 2 query tiles: workgroups run 2 or 3 items back to back."""
    q, k, v = make(400 + D, 2, 150, 512, 512, D)
    check_walk(q, k, v, default_scale(D), f"walk D={D}")


@pytest.mark.parametrize("N,M,D", [(700, 700, 128), (300, 333, 64), (256, 256, 128)])
def test_walk_ragged_and_shortest_items(N, M, D):
    """A partial last query tile (700), more keys than queries (333 > 300), and
    items of exactly four key tiles (256, the fewest the walk takes)."""
    B = 2
    H = 600 // (B * ((N + 255) // 256))
    q, k, v = make(410 + N, B, H, N, M, D)
    check_walk(q, k, v, default_scale(D), f"walk N={N} M={M} D={D}")


def test_walk_reference_moves_on_an_item_first_tile():
    """Scores that jump by ~29 (base 2) in key block 1 of tile 0 and in key
    block 0 of tile 4: the first tile of every item moves its rows' reference
    inside the tile -- in the iteration that still finishes the previous
    item's output -- and the rows of the second query tile move it again."""
    D, N = 128, 512
    q, k, v = make(420, 2, 150, N, N, D)
    scale = default_scale(D)
    lam = 20.0 / scale
    b = torch.zeros(N)
    b[32:64] = 1.0      # tile 0, key block 1
    b[256:288] = 2.0    # tile 4, key block 0
    q[..., 0] = torch.tensor(lam, dtype=torch.bfloat16)
    k[..., 0] = b.to(device=DEV, dtype=torch.bfloat16)
    check_walk(q, k, v, scale, "walk reference moves")


def test_walk_large_scores():
    """Q x 16 (scores of several hundred): no overflow across item changes.
    Rows this peaked take O from one or two values of V, up to about 4.5 in
    magnitude, where half an ulp of bf16 is 2^-6: the output's own rounding
    is allowed on top of the absolute bound."""
    q, k, v = make(430, 2, 150, 512, 512, 128)
    q = (q.float() * 16).to(torch.bfloat16)
    check_walk(q, k, v, default_scale(128), "walk x16", rel_o=2.0 ** -8)


@pytest.mark.parametrize("N,M,D,causal,window", [
    (512, 512, 128, True, (127, 0)),    # the pages' 128-wide window
    (700, 700, 64, True, (300, 0)),     # ragged last query tile
    (512, 512, 128, True, (0, 0)),      # the diagonal only: items of 4-5 tiles
    (512, 512, 128, False, (100, 200)),
    (512, 600, 128, False, (100, 150)),  # more keys than queries (offset 88)
    (300, 333, 64, False, (50, 50)),    # a last item of 3 tiles: item by item
    (512, 512, 64, True, (5000, 0)),    # wider than the sequence: plain causal
])
def test_walk_windows(N, M, D, causal, window):
    """Local windows: items of a few tiles that start at the window's first
    tile, each workgroup walking two or three of them."""
    B = 2
    H = 600 // (B * ((N + 255) // 256))
    q, k, v = make(440 + N + D, B, H, N, M, D)
    check_walk(q, k, v, default_scale(D), f"walk window {window} N={N} M={M} D={D}",
               causal=causal, window=window)


@pytest.mark.parametrize("kind,N,D", [
    ("documents", 512, 128),       # random document cuts: short lists filled up to 4 tiles
    ("documents", 700, 64),        # ragged last query tile
    ("random_per_head", 512, 64),  # long lists, one mask per head
    ("blocks", 512, 128),          # 64 x 64 blocks kept with p = 0.3: items with no tile at all
])
def test_walk_masks(kind, N, D):
    """Causal with an element mask: each workgroup's items' tile lists run as
    one stream; the pre-pass cuts the lists at the causal limit and fills the
    short ones up to four tiles with fully masked ones (their weights are
    exactly 0, so the bits agree with the item-by-item walk)."""
    B = 2
    H = 600 // (B * ((N + 255) // 256))
    if kind == "documents":
        allowed = inputs.document_mask(450 + N, N, N, 7)
    elif kind == "random_per_head":
        allowed = inputs.random_mask(451, 1, H, N, N, 0.5)
    else:
        allowed = inputs.block_mask(452, B, H, N, N, 64, 64, 0.3)
    q, k, v = make(460 + N + D, B, H, N, N, D)
    check_walk(q, k, v, default_scale(D), f"walk mask {kind} N={N} D={D}", allowed=allowed)


def test_walk_mask_prepass_lists_and_order():
    """The pre-pass output the masked walk runs on, read back from the
    workspace: each query tile's list is the mask's tiles below the causal
    limit (the tile after the tile's last query's last key), a list shorter
    than four tiles is filled with tiles the mask does not touch, in tile
    order and flagged with all-zero words, and each XCD's range of work
    items is ordered by tile count, most first, ties by item."""
    B, H, N, D = 2, 150, 512, 64
    M = N
    allowed = np.zeros((1, 1, N, M), dtype=bool)
    allowed[0, 0, 130:140, 140:150] = True    # query tile 0: one tile kept in part, three fillers
    allowed[0, 0, 256:, :384] = True          # query tile 1: six whole tiles, none past them
    q, k, v = make(471, B, H, N, M, D)
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    n_qt, n_kt = (N + 255) // 256, (M + 63) // 64
    items = B * H * n_qt
    assert items > 256
    ws = torch.zeros(fa.workspace_bytes(B, H, N, M, D, causal=True, mask_shape=(1, 1)),
                     dtype=torch.uint8, device=DEV)
    say(f"pre-pass of the masked walk: {items} items, mask [1, 1, {N}, {M}]")
    fa.fwd(q, k, v, causal=True, mask=words, workspace=ws)
    torch.cuda.synchronize()
    lay = mask_layout(N, M, 1, 1, items=items)
    wsb = ws.cpu().numpy()
    w32 = wsb.view(np.uint32)
    stride = n_kt + 1
    sizes = []
    for qt in range(n_qt):
        row = w32[lay["lists"] // 4 + qt * stride:][:stride]
        got = [int(x) for x in row[1:1 + int(row[0])]]
        blk = allowed[0, 0, qt * 256:(qt + 1) * 256]
        t_end = (min(M, min(qt * 256 + 256, N) + (M - N)) + 63) // 64
        cls = [0 if not blk[:, t * 64:(t + 1) * 64].any() else (1 if blk[:, t * 64:(t + 1) * 64].all() else 2)
               for t in range(t_end)]
        want = [t | (1 << 31) if cls[t] == 2 else t for t in range(t_end) if cls[t]]
        if len(want) < 4:
            pads = [t for t in range(t_end) if cls[t] == 0][:4 - len(want)]
            want = sorted(want + [t | (1 << 31) for t in pads], key=lambda e: e & 0x7FFFFFFF)
            for t in pads:   # the filler tile's words: all zero
                at = lay["blocks"] + (qt * stride + t + 1) * 2048
                assert not wsb[at:at + 2048].any(), f"query tile {qt}: filler tile {t} has mask words"
        assert got == want, f"query tile {qt}: list {got} != {want}"
        sizes.append(len(want))
    order = w32[lay["order"] // 4:][:items].astype(np.int64)
    qx, rx = divmod(items, 8)
    for x in range(8):
        start, cnt = x * qx + min(x, rx), qx + (1 if x < rx else 0)
        size = [sizes[n_qt - 1 - (start + j) % n_qt] for j in range(cnt)]
        want = sorted(range(cnt), key=lambda j: (-size[j], j))
        assert order[start:start + cnt].tolist() == want, f"XCD {x}: walk order"
    say("lists, filler words and walk order as expected")
    # and the output: rows that see no key at all (O = 0, LSE = -inf) beside
    # items that start on filler tiles
    check_walk(q, k, v, default_scale(D), "walk mask with fillers", allowed=allowed)
