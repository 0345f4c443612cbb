"""Byte layout of the element-mask pre-pass output inside a workspace, as
include/fa_mi355x.h documents it: per (mask batch, mask head) the forward's
tile lists (one per 256-query tile, ceil(M / 64) + 1 int32 each), with the
backward the dK/dV pass's stage lists (one per 256-key tile, ceil(N / 64) + 1
int32 each), then one class byte per (query tile, 64-key tile) and per query
tile a row of 1 + ceil(M / 64) blocks of 2 KB, then (backward) one class
byte per (256-key tile, 64-query stage) and per key tile a row of
1 + ceil(N / 64) blocks, or (forward, causal) one int32 per work item, the
order of the pipelined walk.  Block 0 of a row is all ones; tile t of the row
has block t + 1.  Every region starts on 256 bytes."""


def _a(n):
    return (n + 255) // 256 * 256


def mask_layout(N, M, mb, mh, base=0, stages=False, items=0):
    mbh = mb * mh
    n_qt, n_kt = (N + 255) // 256, (M + 63) // 64
    n_kt256, n_st = (M + 255) // 256, (N + 63) // 64
    w = {"lists": base, "n_qt": n_qt, "n_kt": n_kt, "n_kt256": n_kt256, "n_st": n_st}
    w["stage_lists"] = _a(base + mbh * n_qt * (n_kt + 1) * 4)
    w["cls"] = _a(w["stage_lists"] + mbh * n_kt256 * (n_st + 1) * 4) if stages else w["stage_lists"]
    w["blocks"] = _a(w["cls"] + mbh * n_qt * n_kt)
    w["stage_cls"] = _a(w["blocks"] + mbh * n_qt * (n_kt + 1) * 2048)
    w["stage_blocks"] = _a(w["stage_cls"] + mbh * n_kt256 * n_st) if stages else w["stage_cls"]
    w["end"] = w["stage_blocks"] + mbh * n_kt256 * (n_st + 1) * 2048 if stages else w["stage_cls"]
    if not stages and items:
        w["order"] = _a(w["stage_cls"])
        w["end"] = w["order"] + items * 4
    return w
