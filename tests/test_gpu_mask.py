"""GPU parity of element masks: the HIP kernels with a packed bitmask against
the fp64 oracle with the same boolean mask ("Understanding FlashAttention",
Attention: mask() covers causal masking and other kinds, each an elementwise
constant that does not depend on the scores).

Key j is visible to query i of (b, h) only if the mask keeps it, on top of
kv_len, the causal rule and the window.  Cases cover masks shared by every
batch and head and per-head masks; tiles the mask drops whole (skipped),
keeps whole and keeps in part; rows the mask empties; N != M, ragged tails,
single queries and the fp32 path.  The long workload is compared on sampled
rows.
"""
import numpy as np
import pytest
import torch

import exact_attention_33_amd as fa
from exact_attention_33_amd import inputs
from oracle.attention import attention_ref, attention_rows
from tests.gpu_helpers import abi_scale, compare, default_scale, host64, sample_picks
from tests.mask_layout import mask_layout

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make(seed, B, H, N, M, D, dtype):
    q, k, v = inputs.qkv_host(seed, B, H, N, M, D)
    return tuple(inputs.to_device(x, dtype, DEV) for x in (q, k, v))


def mask_for(kind, B, H, N, M):
    if kind == "random":
        return inputs.random_mask(91, 1, 1, N, M, 0.5)
    if kind == "random_per_head":
        return inputs.random_mask(92, 1, H, N, M, 0.3)
    if kind == "per_batch_head_blocks":
        return inputs.block_mask(93, B, H, N, M, 64, 64, 0.5)
    if kind == "documents":
        return inputs.document_mask(94, N, M, 5)
    if kind == "prefix":
        return inputs.prefix_mask(N, M, M // 3)
    if kind == "blocks_ragged":
        return inputs.block_mask(95, 1, 1, N, M, 100, 37, 0.4)
    if kind == "empty_rows":
        m = inputs.random_mask(96, 1, 1, N, M, 0.6)
        m[0, 0, ::7] = False
        return m
    raise ValueError(kind)


CASES = [
    # B, H, N, M, D, causal, kv_len, window, mask kind
    (1, 2, 300, 300, 128, False, None, None, "random"),
    (2, 2, 300, 517, 64, True, [517, 200], None, "random_per_head"),
    (2, 2, 600, 640, 128, False, None, None, "per_batch_head_blocks"),
    (1, 2, 1000, 1000, 128, True, None, None, "documents"),
    (1, 1, 700, 700, 64, False, None, None, "prefix"),
    (1, 2, 513, 900, 128, False, [650], (200, 50), "blocks_ragged"),
    (2, 1, 260, 260, 128, True, None, None, "empty_rows"),
    (2, 2, 1, 3000, 128, False, [3000, 1111], None, "random"),      # single queries
    (1, 1, 150, 90, 128, True, None, None, "random"),                # N > M
    (2, 1, 130, 260, 128, True, [260, 0], None, "random"),           # an empty sequence
    (1, 2, 70, 40, 64, False, None, None, "random_per_head"),        # M below one key tile
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}M{}D{}{}-{}".format(
    *c[:5], "c" if c[5] else "", c[8]))
def test_mask_bf16(case):
    B, H, N, M, D, causal, kvl, win, kind = case
    print(f"[mask] case {case}", flush=True)
    q, k, v = make(70 + N, B, H, N, M, D, "bf16")
    kvt = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device=DEV)
    if kvl is not None:
        inputs.poison_tail(k, v, kvl)
    allowed = mask_for(kind, B, H, N, M)
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    o, l = fa.fwd(q, k, v, scale=default_scale(D), causal=causal, kv_len=kvt, window=win,
                  mask=words)
    torch.cuda.synchronize()
    kk, vv = host64(k), host64(v)
    kk[np.isnan(kk)] = 0
    vv[np.isnan(vv)] = 0
    Or, Lr = attention_ref(host64(q), kk, vv, default_scale(D), causal,
                           None if kvl is None else np.asarray(kvl), window=win, mask=allowed)
    compare(host64(o), host64(l), Or, Lr, "bf16", f"mask {case}")


def test_all_ones_mask_matches_unmasked_bitwise():
    """A mask that keeps every key lists every tile as whole: the same tiles
    in the same order as without a mask, so the results are identical."""
    q, k, v = make(97, 1, 2, 700, 700, 128, "bf16")
    words = fa.pack_mask(torch.ones((1, 1, 700, 700), dtype=torch.bool, device=DEV))
    for causal in (False, True):
        o1, l1 = fa.fwd(q, k, v, causal=causal)
        o2, l2 = fa.fwd(q, k, v, causal=causal, mask=words)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), causal


def test_mask_is_deterministic():
    q, k, v = make(98, 1, 2, 500, 500, 128, "bf16")
    words = fa.pack_mask(torch.from_numpy(inputs.random_mask(99, 1, 2, 500, 500, 0.5)).to(DEV))
    o1, l1 = fa.fwd(q, k, v, mask=words)
    o2, l2 = fa.fwd(q, k, v, mask=words)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_mask_f32(causal):
    q, k, v = make(72, 1, 2, 150, 170, 64, "f32")
    allowed = inputs.random_mask(73, 1, 2, 150, 170, 0.4)
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    o, l = fa.fwd(q, k, v, scale=abi_scale(0.2), causal=causal, mask=words)
    torch.cuda.synchronize()
    Or, Lr = attention_ref(host64(q), host64(k), host64(v), abi_scale(0.2), causal, mask=allowed)
    compare(host64(o), host64(l), Or, Lr, "f32", f"f32 mask causal={causal}")


@pytest.mark.parametrize("kind", ["documents8", "random50"])
def test_mask_long_workload_sampled(kind):
    """B=2, H=32, N=M=8192, D=128 causal with the bench's masks (8 packed
    documents; each pair kept with p = 1/2), shared by every batch and head."""
    w = inputs.WORKLOADS["prefill_long_d128"]
    print(f"[mask] long workload, {kind}", flush=True)
    q, k, v = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", torch.device(DEV))
    allowed = (inputs.document_mask(7, w.N, w.M, 8) if kind == "documents8"
               else inputs.random_mask(11, 1, 1, w.N, w.M, 0.5))
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    o, l = fa.fwd(q, k, v, causal=True, mask=words)
    torch.cuda.synchronize()
    picks = sample_picks(w.B, w.H, w.N, n_heads=4, seed=8)
    Or, Lr = attention_rows(lambda b, h: host64(q[b, h]), lambda b, h: host64(k[b, h]),
                            lambda b, h: host64(v[b, h]), default_scale(w.D), True, None,
                            picks, mask=allowed)
    og = np.stack([host64(o[b, h, i]) for b, h, i in picks])
    lg = np.array([float(l[b, h, i]) for b, h, i in picks])
    compare(og, lg, Or, Lr, "bf16", f"long {kind}")


def _expected_lists(allowed, rows_per, cols_per, transpose=False):
    """Per (mask batch, mask head, tile of `rows_per` rows): the ascending
    tiles of `cols_per` columns holding a True, bit 31 set where not all are
    True (rows past the end and columns past the end do not count)."""
    Bm, Hm, N, M = allowed.shape
    a = allowed.transpose(0, 1, 3, 2) if transpose else allowed
    R, C = (M, N) if transpose else (N, M)
    out = []
    for bm in range(Bm):
        for hm in range(Hm):
            for r0 in range(0, R, rows_per):
                lst = []
                for ci, c0 in enumerate(range(0, C, cols_per)):
                    blk = a[bm, hm, r0:r0 + rows_per, c0:c0 + cols_per]
                    if blk.any():
                        lst.append(ci if blk.all() else ci | (1 << 31))
                out.append(lst)
    return out


def _read_lists(ws_words, n_lists, stride):
    got = []
    for i in range(n_lists):
        cnt = int(ws_words[i * stride])
        got.append([int(x) & 0xFFFFFFFF for x in ws_words[i * stride + 1:i * stride + 1 + cnt]])
    return got


def test_tile_lists_match_the_mask():
    """The pre-passes' lists, read back from the workspace: the forward's key
    tiles per query tile and the backward's query stages per key tile, with
    the partial-tile flags, equal a NumPy classification of the mask."""
    B, H, N, M, D = 2, 2, 600, 700, 64
    allowed = inputs.block_mask(120, B, 1, N, M, 32, 32, 0.5)     # whole, partial and empty tiles
    allowed[1, 0, :, 640:] = True                                  # a ragged last tile kept whole
    q, k, v = make(121, B, H, N, M, D, "bf16")
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    ws = torch.zeros(fa.workspace_bytes(B, H, N, M, D, mask_shape=(B, 1)), dtype=torch.uint8, device=DEV)
    o, l = fa.fwd(q, k, v, mask=words, workspace=ws)
    torch.cuda.synchronize()
    stride = (M + 63) // 64 + 1
    n_qt = (N + 255) // 256
    got = _read_lists(ws.view(torch.int32).cpu().numpy(), B * n_qt, stride)
    assert got == _expected_lists(allowed, 256, 64)
    # the backward's dK/dV stage lists sit after its statistics and dQ lists
    g = inputs.to_device(inputs.normal_f32(122, (B, H, N, D)), "bf16", DEV)
    wsb = torch.zeros(fa.bwd_workspace_bytes(B, H, N, M, D, mask_shape=(B, 1)), dtype=torch.uint8,
                      device=DEV)
    fa.bwd(q, k, v, o, l, g, mask=words, workspace=wsb)
    torch.cuda.synchronize()
    npad = (N + 255) // 256 * 256
    stats = B * H * npad * 2 * 4
    off = (stats + 255) // 256 * 256
    dq_lists = B * n_qt * stride * 4
    off_st = off + (dq_lists + 255) // 256 * 256
    words_b = wsb.view(torch.int32).cpu().numpy()
    assert _read_lists(words_b[off // 4:], B * n_qt, stride) == _expected_lists(allowed, 256, 64)
    n_kt = (M + 255) // 256
    stride_s = (N + 63) // 64 + 1
    assert _read_lists(words_b[off_st // 4:], B * n_kt, stride_s) == \
        _expected_lists(allowed, 256, 64, transpose=True)


def _tile_classes(allowed, rows_per, cols_per, transpose=False):
    """[Bm * Hm, row tiles, column tiles] of 0 (nothing kept), 1 (all kept),
    2 (some kept), over the real rows and columns of each tile."""
    a = allowed.transpose(0, 1, 3, 2) if transpose else allowed
    Bm, Hm, R, C = a.shape
    out = np.zeros((Bm * Hm, -(-R // rows_per), -(-C // cols_per)), dtype=np.uint8)
    for g in range(Bm * Hm):
        for i, r0 in enumerate(range(0, R, rows_per)):
            for j, c0 in enumerate(range(0, C, cols_per)):
                blk = a[g // Hm, g % Hm, r0:r0 + rows_per, c0:c0 + cols_per]
                out[g, i, j] = 1 if blk.all() else (2 if blk.any() else 0)
    return out


@pytest.mark.parametrize("N,M", [(600, 700), (300, 2100)])
def test_mask_blocks_hold_the_words(N, M):
    """The pre-passes' class bytes and blocks of mask words, read back from
    the workspace (layout of include/fa_mi355x.h): a block for every tile
    (and, in the backward, every dK/dV stage) the mask keeps in part, each
    word where the kernels' wave loads expect it (rows past N copy row N - 1;
    words past the row are 0), and an all-ones block 0 in every row of
    blocks."""
    B, H, D = 2, 2, 64
    allowed = inputs.block_mask(123, B, 1, N, M, 32, 32, 0.5)
    allowed[1, 0, :, M - 300:] = True       # tiles (and 256-key tiles) kept whole
    allowed[0, 0, :256, 64:320] = False     # tiles kept nowhere
    q, k, v = make(124, B, H, N, M, D, "bf16")
    words = fa.pack_mask(torch.from_numpy(allowed).to(DEV))
    wn = words.cpu().numpy().view(np.uint32).reshape(B, N, -1)
    lay = mask_layout(N, M, B, 1)
    n_qt, n_kt, n_kt256, n_st = lay["n_qt"], lay["n_kt"], lay["n_kt256"], lay["n_st"]
    # the words the kernels load: rows padded by copies of row N - 1, columns by 0
    cols = max(2 * n_kt, 8 * n_kt256)
    P = np.zeros((B, n_qt * 256, cols), dtype=np.uint32)
    P[:, :N, :wn.shape[2]] = wn
    P[:, N:, :wn.shape[2]] = wn[:, N - 1:N, :]

    def fwd_block(g, qt, kt):   # [wave][word][row of the wave]
        return P[g, qt * 256:(qt + 1) * 256, 2 * kt:2 * kt + 2].reshape(4, 64, 2).transpose(0, 2, 1).ravel()

    def stage_block(g, kt, st):  # [word][row]
        return P[g, st * 64:st * 64 + 64, 8 * kt:8 * kt + 8].T.ravel()

    cls = _tile_classes(allowed, 256, 64)
    scls = _tile_classes(allowed, 256, 64, transpose=True)
    assert (cls == 1).any() and (cls == 2).any() and (cls == 0).any()

    def check_fwd(wsb, lay):
        got_cls = wsb[lay["cls"]:lay["cls"] + B * n_qt * n_kt].reshape(B, n_qt, n_kt)
        assert np.array_equal(got_cls, cls)
        blocks = wsb[lay["blocks"]:lay["blocks"] + B * n_qt * (n_kt + 1) * 2048].view(np.uint32)
        blocks = blocks.reshape(B, n_qt, n_kt + 1, 512)
        assert (blocks[:, :, 0] == 0xFFFFFFFF).all()
        for g, qt, kt in zip(*np.nonzero(cls == 2)):
            assert np.array_equal(blocks[g, qt, kt + 1], fwd_block(g, qt, kt)), (g, qt, kt)

    ws = torch.zeros(fa.workspace_bytes(B, H, N, M, D, mask_shape=(B, 1)), dtype=torch.uint8, device=DEV)
    assert ws.numel() == lay["end"]
    o, l = fa.fwd(q, k, v, mask=words, workspace=ws)
    torch.cuda.synchronize()
    check_fwd(ws.cpu().numpy(), lay)

    g_ = inputs.to_device(inputs.normal_f32(125, (B, H, N, D)), "bf16", DEV)
    base = (B * H * ((N + 255) // 256 * 256) * 8 + 255) // 256 * 256
    layb = mask_layout(N, M, B, 1, base, stages=True)
    wsb = torch.zeros(fa.bwd_workspace_bytes(B, H, N, M, D, mask_shape=(B, 1)), dtype=torch.uint8,
                      device=DEV)
    assert wsb.numel() == layb["end"]
    fa.bwd(q, k, v, o, l, g_, mask=words, workspace=wsb)
    torch.cuda.synchronize()
    wb = wsb.cpu().numpy()
    check_fwd(wb, layb)
    got_s = wb[layb["stage_cls"]:layb["stage_cls"] + B * n_kt256 * n_st].reshape(B, n_kt256, n_st)
    assert np.array_equal(got_s, scls)
    sblocks = wb[layb["stage_blocks"]:layb["stage_blocks"] + B * n_kt256 * (n_st + 1) * 2048].view(np.uint32)
    sblocks = sblocks.reshape(B, n_kt256, n_st + 1, 512)
    assert (sblocks[:, :, 0] == 0xFFFFFFFF).all()
    assert (scls == 2).any() and (scls == 1).any()
    for g, kt, st in zip(*np.nonzero(scls == 2)):
        assert np.array_equal(sblocks[g, kt, st + 1], stage_block(g, kt, st)), (g, kt, st)
