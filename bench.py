#!/usr/bin/env python3
"""Benchmark of the fused exact-attention forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. the fused prefill forward (bf16, causal) on B=2, H=32, N=M=8192, D=128;
  2. the split-KV decode (partial + merge kernels) on B=32 sequences, H=32,
     N=1, D=128, per-sequence KV length uniform in [1024, 32768].
After the timed steps, the wider rows are timed one by one on the same
tensors (each with its own warmup), so they never share a timed region with
the hot path:
  3. the backward of the prefill (row statistic, dK/dV and dQ kernels) for an
     upstream gradient dO ~ N(0, 1), reported beside the forward;
  4. the same prefill with a causal local window of 128 keys per query (the
     pages' 128-wide window) and of 2048 keys, reported beside it;
  5. the key/value-outer ablation of the same prefill (the first version's
     loop order), one query tile per workgroup and one workgroup per head;
  6. the same prefill on E4M3 inputs (the prefill's tensors quantized per
     tensor) on the fp8 matrix cores;
  7. the same prefill with an element mask shared by every batch and head:
     8 packed documents (a query sees its own document's keys), and an
     unstructured mask keeping each (query, key) pair with probability 1/2
     (every tile applies bits); the tile-list pre-pass is inside the timing;
     the backward under the 8-document mask is timed beside them;
  8. the other prefill shapes of the workload list, each on its own tensors:
     B=1 H=8 N=M=1024 D=64 causal (a latency: one launch is a few
     microseconds), B=4 H=16 N=M=4096 D=128 causal and non-causal, and
     B=2 H=32 N=M=8192 D=64 causal (the pages' n=8192, d=64 example).
Inputs are N(0, 1) drawn on the device from fixed seeds and are resident in
HBM before timing starts.  Beside the long prefill the bench prints the HBM
bytes that the naive (unfused) computation would move for the same shapes
under the pages' counting model (score and weight matrices written and read
back once each, Q, K, V read and O written once), in float32 and bf16.

`value` is the prefill throughput in TFLOP/s with the FLOP convention
4*B*H*N*M*D, halved for causal; the decode throughput (KV-cache bytes read
per second) is reported beside it.  Each launch is timed with HIP events on
the stream it runs on.  The CPU oracle (fp64 NumPy) is timed on a bounded
sample of the same tensors on this host, and its results double as a parity
check of the sampled heads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time
from statistics import median

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak; decode KV GB/s & % HBM peak"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_attention_33_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


SOURCES = {"prefill": ["prefill_bf16.hip", "device_common.h", "fa_internal.h"],
           "decode": ["decode_bf16.hip", "device_common.h", "fa_internal.h"],
           "backward": ["bwd_bf16.hip", "device_common.h", "fa_internal.h", "mfma_asm.h"],
           "fp8": ["prefill_fp8.hip", "device_common.h", "fa_internal.h"],
           "kvouter": ["kvouter_bf16.hip", "device_common.h", "fa_internal.h", "mfma_asm.h"]}
SOURCES["window"] = SOURCES["configs"] = SOURCES["prefill"]
SOURCES["mask"] = SOURCES["prefill"] + ["mask_prep.hip"]


def measured_traffic(kind, case=None):
    """HBM bytes per launch (per call for several launches) from the committed
    counter profile, or None when the kernel sources changed since the
    counters were taken.  ``case`` picks one configuration of a leg that
    times several (a window width, a mask)."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(SOURCES[kind]):
        return None
    if case is not None:
        rec = rec.get("cases", {}).get(case)
        if not rec:
            return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward", "window", "kvouter",
                                       "fp8", "mask", "configs", "copy"],
                    default="all",
                    help="run one leg only (for counter runs); 'copy' runs a plain "
                         "device copy of known size for counter calibration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8, help="prefill heads the oracle times")
    ap.add_argument("--cpu-decode-heads", type=int, default=1024)
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 output under DIR "
                         "(see summarize_profiles) and exit; needs no GPU")
    return ap.parse_args()


def main():
    args = parse()
    if args.profile_summary:
        summarize_profiles(args.profile_summary)
        return 0
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs on one GPU "
              "only (no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_33_amd as fa
    from exact_attention_33_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa.lib()  # fail loudly if the HIP library is missing
    stream = torch.cuda.Stream(device=dev)

    if args.only == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": args.steps}))
        return 0

    wp = inputs.WORKLOADS["prefill_long_d128"]
    wd = inputs.WORKLOADS["decode"]
    do_p = args.only in ("all", "prefill")
    do_d = args.only in ("all", "decode")
    do_b = args.only in ("all", "backward")
    do_w = args.only in ("all", "window")
    do_k = args.only in ("all", "kvouter")
    do_8 = args.only in ("all", "fp8")
    do_m = args.only in ("all", "mask")
    do_c = args.only in ("all", "configs")
    # the other prefill shapes: (workload, causal, label)
    CONFIGS = (("prefill_small", True, "B1_H8_N1024_D64_causal"),
               ("prefill_mid", True, "B4_H16_N4096_D128_causal"),
               ("prefill_mid", False, "B4_H16_N4096_D128_noncausal"),
               ("prefill_long_d64", True, "B2_H32_N8192_D64_causal"))
    # the small prefill once more with its keys in chunks of 256 (four
    # workgroups per query tile instead of one: 128 of the 256 CUs)
    SPLIT_SMALL, SPLIT_LABEL = 256, "B1_H8_N1024_D64_causal_split_keys256"
    KVO = (("tile_per_group", 1), ("head_per_group", 1 << 20))  # 256-query tiles per workgroup
    WINDOWS = (128, 2048)  # keys per query (causal band: window_left = W - 1)

    # ---- inputs, resident in HBM before timing ----
    if do_p or do_b or do_w or do_k or do_8 or do_m:
        # the long prefill's Q, K, V, shared by every prefill leg
        qp, kp, vp = inputs.qkv_device(wp.seed, wp.B, wp.H, wp.N, wp.M, wp.D, "bf16", dev)
        scale_p = 1.0 / math.sqrt(wp.D)
    if do_p:
        op = torch.empty_like(qp)
        lp = torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
        flop_p = 4.0 * wp.B * wp.H * wp.N * wp.M * wp.D / 2.0   # causal convention
    if do_d:
        kvl_h = inputs.kv_lens(wd.kv_seed, wd.B, *wd.kv_range)
        Md = int(kvl_h.max())
        qd, kd, vd = inputs.qkv_device(wd.seed, wd.B, wd.H, 1, Md, wd.D, "bf16", dev)
        kvl_d = torch.as_tensor(kvl_h, device=dev)
        od = torch.empty_like(qd)
        ld = torch.empty((wd.B, wd.H, 1), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, fa.workspace_bytes(wd.B, wd.H, 1, Md, wd.D)), dtype=torch.uint8,
                         device=dev)
        scale_d = 1.0 / math.sqrt(wd.D)
        kv_bytes = float(kvl_h.astype(np.int64).sum()) * wd.H * wd.D * 2 * 2
        plan_d = fa.plan(wd.B, wd.H, 1, Md, wd.D)
    if do_b:
        # backward of the same causal prefill: the forward's O and LSE, an
        # upstream gradient dO ~ N(0, 1), and the gradient buffers
        ob, lb = fa.fwd(qp, kp, vp, scale=scale_p, causal=True)
        gb = inputs.grad_device(wp.seed + 1000, wp.B, wp.H, wp.N, wp.D, "bf16", dev)
        dqb, dkb, dvb = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
        wsb = torch.empty(fa.bwd_workspace_bytes(wp.B, wp.H, wp.N, wp.M, wp.D), dtype=torch.uint8,
                          device=dev)
        # five tile products (S recomputed, dP, dV, dK, dQ) of 2 N M D each,
        # halved for causal: 2.5 x the forward's count
        flop_b = 10.0 * wp.B * wp.H * wp.N * wp.M * wp.D / 2.0
    if do_8:
        # the prefill's tensors quantized per tensor to E4M3 (scale = amax / 448)
        q8s, d8 = [], []
        for t in (qp, kp, vp):
            d = float(t.abs().max()) / 448.0
            q8s.append((t.float() / d).to(torch.float8_e4m3fn))
            d8.append(d)
        o8 = torch.empty_like(qp)
        l8 = torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
        flop_8 = 4.0 * wp.B * wp.H * wp.N * wp.M * wp.D / 2.0
    if do_k:
        ok_, lk_ = torch.empty_like(qp), torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
        wsk = torch.empty(fa.workspace_bytes(wp.B, wp.H, wp.N, wp.M, wp.D, causal=True,
                                             path=fa.PATH_KVOUTER), dtype=torch.uint8, device=dev)
        flop_k = 4.0 * wp.B * wp.H * wp.N * wp.M * wp.D / 2.0
    if do_w:
        ow, lw = torch.empty_like(qp), torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
        # visible (query, key) pairs per head of a causal band of W keys
        pairs_w = {W: W * wp.N - W * (W - 1) // 2 for W in WINDOWS}
        bytes_w = (4.0 * wp.N * wp.D * 2 + wp.N * 4) * wp.B * wp.H   # Q, K, V read, O and LSE written
    if do_m:
        om, lm = torch.empty_like(qp), torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
        masks = {"documents8": inputs.document_mask(7, wp.N, wp.M, 8),
                 "random50": inputs.random_mask(11, 1, 1, wp.N, wp.M, 0.5)}
        causal_pairs = np.tril(np.ones((wp.N, wp.M), dtype=bool), wp.M - wp.N)
        # visible (query, key) pairs per head: the mask and the causal rule
        pairs_m = {k: int(np.count_nonzero(m[0, 0] & causal_pairs)) for k, m in masks.items()}
        words_m = {k: fa.pack_mask(torch.from_numpy(m).to(dev)) for k, m in masks.items()}
        del masks, causal_pairs
        wsm = torch.empty(fa.workspace_bytes(wp.B, wp.H, wp.N, wp.M, wp.D, causal=True,
                                             mask_shape=(1, 1)), dtype=torch.uint8, device=dev)
        # backward under the document mask: the forward's O and LSE, dO ~ N(0, 1)
        omb, lmb = fa.fwd(qp, kp, vp, scale=scale_p, causal=True, mask=words_m["documents8"])
        gmb = inputs.grad_device(wp.seed + 1000, wp.B, wp.H, wp.N, wp.D, "bf16", dev)
        dqm, dkm, dvm = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
        wsmb = torch.empty(fa.bwd_workspace_bytes(wp.B, wp.H, wp.N, wp.M, wp.D, mask_shape=(1, 1)),
                           dtype=torch.uint8, device=dev)
    if do_c:
        cfg_t = {}
        for name in sorted({c[0] for c in CONFIGS}):
            w = inputs.WORKLOADS[name]
            q_, k_, v_ = inputs.qkv_device(w.seed, w.B, w.H, w.N, w.M, w.D, "bf16", dev)
            cfg_t[name] = (w, q_, k_, v_, torch.empty_like(q_),
                           torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    def main_step(evs=None):
        """One pass of the hot path: the causal prefill and the split-KV decode."""
        with torch.cuda.stream(stream):
            if do_p:
                if evs: evs[0].record(stream)
                fa.fwd(qp, kp, vp, scale=scale_p, causal=True, out=op, lse=lp, stream=stream)
                if evs: evs[1].record(stream)
            if do_d:
                if evs: evs[2].record(stream)
                fa.fwd(qd, kd, vd, scale=scale_d, causal=False, kv_len=kvl_d, out=od, lse=ld,
                       workspace=ws, stream=stream)
                if evs: evs[3].record(stream)

    def timed(fn, steps, warmup):
        """HIP events on the library's stream around each of `steps` calls."""
        for _ in range(warmup):
            with torch.cuda.stream(stream):
                fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            with torch.cuda.stream(stream):
                a.record(stream)
                fn()
                b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    # ---- the timed region of the hot path ----
    for _ in range(args.warmup):
        main_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        main_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_p = [e[0].elapsed_time(e[1]) for e in events] if do_p else []
    ms_d = [e[2].elapsed_time(e[3]) for e in events] if do_d else []

    # ---- the wider rows, each timed on its own after the hot path ----
    ms_b = timed(lambda: fa.bwd(qp, kp, vp, ob, lb, gb, scale=scale_p, causal=True, dq=dqb,
                                dk=dkb, dv=dvb, workspace=wsb, stream=stream),
                 args.steps, args.warmup) if do_b else []
    ms_w = {W: timed(lambda W=W: fa.fwd(qp, kp, vp, scale=scale_p, causal=True, out=ow, lse=lw,
                                        window=(W - 1, 0), stream=stream),
                     args.steps, args.warmup) for W in WINDOWS} if do_w else {}
    ms_8 = timed(lambda: fa.fwd(q8s[0], q8s[1], q8s[2], scale=scale_p, causal=True, out=o8, lse=l8,
                                descale=tuple(d8), stream=stream),
                 args.steps, args.warmup) if do_8 else []
    ms_m = {name: timed(lambda name=name: fa.fwd(qp, kp, vp, scale=scale_p, causal=True, out=om,
                                                 lse=lm, mask=words_m[name], workspace=wsm,
                                                 stream=stream),
                        args.steps, args.warmup) for name in words_m} if do_m else {}
    ms_mb = timed(lambda: fa.bwd(qp, kp, vp, omb, lmb, gmb, scale=scale_p, causal=True, dq=dqm,
                                 dk=dkm, dv=dvm, workspace=wsmb, mask=words_m["documents8"],
                                 stream=stream),
                  args.steps, args.warmup) if do_m else []
    ms_k = {name: timed(lambda tpg=tpg: fa.fwd(qp, kp, vp, scale=scale_p, causal=True, out=ok_,
                                               lse=lk_, workspace=wsk, path=fa.PATH_KVOUTER,
                                               kvouter_query_tiles=tpg, stream=stream),
                        max(2, args.steps // 4), 1) for name, tpg in KVO} if do_k else {}
    ms_c = {}
    if do_c:
        for name, causal, label in CONFIGS:
            w, q_, k_, v_, o_, l_ = cfg_t[name]
            ms_c[label] = timed(lambda w=w, q_=q_, k_=k_, v_=v_, o_=o_, l_=l_, causal=causal:
                                fa.fwd(q_, k_, v_, scale=1.0 / math.sqrt(w.D), causal=causal,
                                       out=o_, lse=l_, stream=stream),
                                args.steps, args.warmup)
        w, q_, k_, v_, o_, l_ = cfg_t["prefill_small"]
        wsc = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.M, w.D, causal=True, split_keys=SPLIT_SMALL),
                          dtype=torch.uint8, device=dev)
        ms_c[SPLIT_LABEL] = timed(lambda: fa.fwd(q_, k_, v_, scale=1.0 / math.sqrt(w.D), causal=True, out=o_,
                                                 lse=l_, split_keys=SPLIT_SMALL, workspace=wsc, stream=stream),
                                  args.steps, args.warmup)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": 1e3 * wall / max(1, args.steps), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: Q/K/V i.i.d. N(0,1) from fixed seeds (device generator), "
                   "decode KV lengths uniform [1024, 32768] from seed 7"}
    cfg = {"workload": "causal prefill B=2 H=32 N=M=8192 D=128 bf16 + split-KV decode "
                       "B=32 H=32 N=1 D=128 bf16 kv_len~U[1024,32768]",
           "prefill": {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True},
           "decode": {"B": wd.B, "H": wd.H, "N": 1, "D": wd.D, "kv_seed": wd.kv_seed,
                      "kv_range": list(wd.kv_range)}}
    if do_p:
        avg_p = sum(ms_p) / len(ms_p)
        tfs = flop_p / (avg_p * 1e-3) / 1e12
        out.update({"value": tfs, "unit": "TFLOP/s"})
        out["prefill"] = {"ms_mean": avg_p, "ms_min": min(ms_p), "ms_median": median(ms_p), "tflops": tfs,
                          "frac_bf16_peak": tfs / PEAK_BF16_TFLOPS, "flop_per_launch": flop_p}
        traffic = measured_traffic("prefill")
        out["roofline"] = {"bound": "mfma", "kernel": "prefill_cont_kernel<128, true, false, false>",
                           "achieved": tfs, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tfs / PEAK_BF16_TFLOPS, "traffic": traffic}
    if do_d:
        avg_d = sum(ms_d) / len(ms_d)
        gbs = kv_bytes / (avg_d * 1e-3) / 1e9
        out["decode"] = {"ms_mean": avg_d, "ms_min": min(ms_d), "ms_median": median(ms_d), "kv_bytes": kv_bytes,
                         "value": gbs, "unit": "GB/s", "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                         "splits": plan_d["splits"], "split_keys": plan_d["block_k"],
                         "roofline": {"bound": "hbm", "kernel": "splitkv partial + merge",
                                      "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": measured_traffic("decode")}}
        if not do_p:
            out.update({"value": gbs, "unit": "GB/s"})
    if do_b:
        avg_b = sum(ms_b) / len(ms_b)
        tfb = flop_b / (avg_b * 1e-3) / 1e12
        out["backward"] = {"ms_mean": avg_b, "ms_min": min(ms_b), "ms_median": median(ms_b), "value": tfb, "unit": "TFLOP/s",
                           "frac_bf16_peak": tfb / PEAK_BF16_TFLOPS, "flop_per_call": flop_b,
                           "flop_convention": "10 B H N M D / 2 (S recomputed, dP, dV, dK, dQ; "
                                              "causal halved)",
                           "roofline": {"bound": "mfma",
                                        "kernel": "fa_bwd: rowstat + dkdv + dq (whole call)",
                                        "achieved": tfb, "peak": PEAK_BF16_TFLOPS,
                                        "unit": "TFLOP/s", "frac": tfb / PEAK_BF16_TFLOPS,
                                        "traffic": measured_traffic("backward")}}
        cfg["backward"] = {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True,
                           "dO": "N(0,1), seed %d" % (wp.seed + 1000)}
        if not do_p and not do_d:
            out.update({"value": tfb, "unit": "TFLOP/s"})
    if do_w:
        res = {}
        for W in WINDOWS:
            avg = sum(ms_w[W]) / len(ms_w[W])
            flop = 4.0 * wp.D * pairs_w[W] * wp.B * wp.H
            tf = flop / (avg * 1e-3) / 1e12
            gbs = bytes_w / (avg * 1e-3) / 1e9
            # the bound is the resource with the longer time at its peak
            mfma_bound = flop / (PEAK_BF16_TFLOPS * 1e12) >= bytes_w / (PEAK_HBM_GBS * 1e9)
            roof = ({"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS} if mfma_bound else
                    {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS})
            roof.update({"kernel": "prefill_cont_kernel<128, true, true, false>",
                         "traffic": measured_traffic("window", f"w{W}")})
            res[f"w{W}"] = {"window": [W - 1, 0], "ms_mean": avg, "ms_min": min(ms_w[W]), "ms_median": median(ms_w[W]),
                            "tflops": tf, "gbs": gbs, "flop_per_launch": flop,
                            "bytes_per_launch": bytes_w, "roofline": roof}
        out["window"] = dict(res, flop_convention="4 D x visible (query, key) pairs per head "
                                                  "(exact count), B H heads")
        cfg["window"] = {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True,
                         "keys_per_query": list(WINDOWS)}
        if not (do_p or do_d or do_b):
            out.update({"value": res[f"w{WINDOWS[0]}"]["gbs"], "unit": "GB/s"})
    if do_m:
        res = {}
        for name in ms_m:
            avg = sum(ms_m[name]) / len(ms_m[name])
            flop = 4.0 * wp.D * pairs_m[name] * wp.B * wp.H
            tf = flop / (avg * 1e-3) / 1e12
            res[name] = {"ms_mean": avg, "ms_min": min(ms_m[name]), "ms_median": median(ms_m[name]), "tflops": tf,
                         "visible_pairs_per_head": pairs_m[name],
                         "visible_fraction_of_causal": pairs_m[name] / (wp.N * (wp.N + 1) / 2),
                         "speedup_vs_unmasked_causal": ((sum(ms_p) / len(ms_p)) / avg) if do_p else None,
                         "roofline": {"bound": "mfma",
                                      "kernel": "mask_blocks_kernel + mask_lists_kernel + mask_order_kernel + prefill_cont_kernel<128, true, false, true>",
                                      "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": tf / PEAK_BF16_TFLOPS,
                                      "traffic": measured_traffic("mask", name)}}
        avg_b = sum(ms_mb) / len(ms_mb)
        flop_mb = 10.0 * wp.D * pairs_m["documents8"] * wp.B * wp.H
        tf_mb = flop_mb / (avg_b * 1e-3) / 1e12
        res["backward_documents8"] = {
            "ms_mean": avg_b, "ms_min": min(ms_mb), "ms_median": median(ms_mb), "tflops": tf_mb,
            "speedup_vs_unmasked_backward": ((sum(ms_b) / len(ms_b)) / avg_b) if do_b else None,
            "roofline": {"bound": "mfma", "kernel": "fa_bwd with a mask: rowstat + dkdv + dq (whole call)",
                         "achieved": tf_mb, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf_mb / PEAK_BF16_TFLOPS, "traffic": None}}
        out["mask"] = dict(res, flop_convention="forward 4 D, backward 10 D x visible (query, key) "
                                                "pairs per head (exact count), B H heads")
        cfg["mask"] = {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True,
                       "masks": {"documents8": "8 packed documents (seed 7), shared by all heads",
                                 "random50": "each pair kept with p = 1/2 (seed 11), shared"}}
        if not (do_p or do_d or do_b or do_w):
            out.update({"value": res["documents8"]["tflops"], "unit": "TFLOP/s"})
    if do_8:
        avg8 = sum(ms_8) / len(ms_8)
        tf8 = flop_8 / (avg8 * 1e-3) / 1e12
        out["fp8"] = {"ms_mean": avg8, "ms_min": min(ms_8), "ms_median": median(ms_8), "value": tf8, "unit": "TFLOP/s",
                      "frac_fp8_peak": tf8 / PEAK_FP8_TFLOPS, "flop_per_launch": flop_8,
                      "speedup_vs_bf16_prefill": ((sum(ms_p) / len(ms_p)) / avg8) if do_p else None,
                      "roofline": {"bound": "mfma", "kernel": "prefill_fp8_kernel<128, true>",
                                   "achieved": tf8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                   "frac": tf8 / PEAK_FP8_TFLOPS, "traffic": measured_traffic("fp8")}}
        cfg["fp8"] = {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True,
                      "inputs": "E4M3, per-tensor scale amax/448 of the prefill's tensors"}
        if not (do_p or do_d):
            out.update({"value": tf8, "unit": "TFLOP/s"})
    if do_k:
        res = {}
        for name, tpg in KVO:
            avg = sum(ms_k[name]) / len(ms_k[name])
            tf = flop_k / (avg * 1e-3) / 1e12
            res[name] = {"query_tiles_per_group": min(tpg, -(-wp.N // 256)), "ms_mean": avg,
                         "ms_min": min(ms_k[name]), "ms_median": median(ms_k[name]), "tflops": tf,
                         "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
                         "slowdown_vs_prefill": (avg / (sum(ms_p) / len(ms_p))) if do_p else None,
                         "traffic": measured_traffic("kvouter", name)}
        out["kvouter"] = dict(res, note="ablation: key/value tiles outside, output accumulator "
                                        "and m, l read and written back per key tile (float32 "
                                        "workspace); same FLOP convention as the prefill")
        cfg["kvouter"] = {"B": wp.B, "H": wp.H, "N": wp.N, "M": wp.M, "D": wp.D, "causal": True}
        if not (do_p or do_d or do_b or do_w):
            out.update({"value": res["tile_per_group"]["tflops"], "unit": "TFLOP/s"})
    if do_c:
        res = {}
        for name, causal, label in CONFIGS:
            w = cfg_t[name][0]
            avg = sum(ms_c[label]) / len(ms_c[label])
            flop = 4.0 * w.B * w.H * w.N * w.M * w.D / (2.0 if causal else 1.0)
            tf = flop / (avg * 1e-3) / 1e12
            res[label] = {"B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D, "causal": causal,
                          "seed": w.seed, "ms_mean": avg, "ms_min": min(ms_c[label]), "ms_median": median(ms_c[label]),
                          "tflops": tf, "flop_per_launch": flop,
                          "roofline": {"bound": "mfma",
                                       "kernel": prefill_kernel_name(w, causal),
                                       "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                       "frac": tf / PEAK_BF16_TFLOPS,
                                       "traffic": measured_traffic("configs", label)}}
        res["B1_H8_N1024_D64_causal"]["note"] = (
            "latency: 32 workgroups (1/8 of the CUs) and a few microseconds per launch; "
            "the TFLOP/s figure is not a throughput claim")
        w = cfg_t["prefill_small"][0]
        avg = sum(ms_c[SPLIT_LABEL]) / len(ms_c[SPLIT_LABEL])
        flop = 4.0 * w.B * w.H * w.N * w.M * w.D / 2.0
        tf = flop / (avg * 1e-3) / 1e12
        res[SPLIT_LABEL] = {
            "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D, "causal": True, "seed": w.seed,
            "split_keys": SPLIT_SMALL, "ms_mean": avg, "ms_min": min(ms_c[SPLIT_LABEL]),
            "ms_median": median(ms_c[SPLIT_LABEL]), "tflops": tf, "flop_per_launch": flop,
            "speedup_vs_no_split": (sum(ms_c["B1_H8_N1024_D64_causal"]) / len(ms_c["B1_H8_N1024_D64_causal"])) / avg,
            "roofline": {"bound": "mfma", "kernel": "prefill_split_kernel<64, true> + prefill_merge_kernel<64>",
                         "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("configs", SPLIT_LABEL)},
            "note": "the same latency case with each query tile's keys in chunks of 256 (128 workgroups), "
                    "merged by log-sum-exp in a second launch"}
        out["configs"] = dict(res, flop_convention="4 B H N M D, halved for causal")
        cfg["configs"] = dict({label: name for name, _, label in CONFIGS},
                              **{SPLIT_LABEL: f"prefill_small, split_keys={SPLIT_SMALL}"})
    if do_p:
        out["naive_hbm_bytes"] = naive_traffic_report(wp)
    out["config"] = cfg

    if not args.no_cpu_baseline and args.only == "all":
        out["cpu_baseline"] = cpu_baseline(args, np, torch, qp, kp, vp, op, lp, scale_p, wp,
                                           qd, kd, vd, od, ld, kvl_h, scale_d, wd)
        out["cpu_baseline"]["backward"] = cpu_baseline_bwd(np, qp, kp, vp, gb, dqb, dkb, dvb,
                                                           scale_p, wp)
        out["cpu_baseline"]["configs"] = cpu_baseline_configs(np, CONFIGS, cfg_t)
    print(json.dumps(out), flush=True)
    return 0


def naive_traffic_report(wp):
    """HBM bytes of the naive (unfused) forward for the long prefill's batch
    and heads at D = 64 and 128, from the counting model of "FlashAttention:
    attention was never compute-bound", Where the time actually goes: per
    head, Q and K read, the n x n score matrix written and read, the weight
    matrix written and read, V read and O written, i.e. 4 n^2 + 4 n d
    elements (float32 on the page: 1032 MB per head at n = 8192, d = 64)."""
    n, heads = wp.N, wp.B * wp.H
    rep = {"model": "per head (4 n^2 + 4 n d) elements; MiB = 2^20 bytes", "n": n,
           "heads": heads}
    for d in (64, 128):
        elems = 4 * n * n + 4 * n * d
        for name, size in (("fp32", 4), ("bf16", 2)):
            rep[f"d{d}_{name}_bytes"] = heads * elems * size
            rep[f"d{d}_{name}_mib_per_head"] = elems * size / float(1 << 20)
    return rep


def host_description(blas_threads):
    """The host the oracle runs on: logical CPUs, the CPUs this process may
    use, BLAS threads and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = None
    return {"os_cpu_count": os.cpu_count(), "usable_cpus": usable,
            "blas_threads": blas_threads, "cpu_model": model}


def cpu_baseline_configs(np, configs, tensors, heads_per_config=(8, 1, 1, 1)):
    """The oracle on whole heads of each other prefill shape's tensors (all
    8 heads of the small one, one head of the others); their outputs are
    compared with the GPU's (the bench's launches, element by element)."""
    import torch

    import exact_attention_33_amd as fa
    from oracle.attention import attention_ref
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    res = {}
    for (name, causal, label), n_heads in zip(configs, heads_per_config):
        w, q_, k_, v_, o_, l_ = tensors[name]
        # the causal and non-causal legs of one shape share o_, l_: launch this
        # leg once more so that they hold its output
        fa.fwd(q_, k_, v_, scale=1.0 / math.sqrt(w.D), causal=causal, out=o_, lse=l_)
        torch.cuda.synchronize()
        scale = float(np.float32(1.0 / math.sqrt(w.D)))
        t_cpu, eo, el = 0.0, 0.0, 0.0
        heads = [divmod(i, w.H) for i in range(n_heads)]
        for b, h in heads:
            q, k, v = f64(q_[b, h])[None, None], f64(k_[b, h])[None, None], f64(v_[b, h])[None, None]
            t0 = time.perf_counter()
            O, L = attention_ref(q, k, v, scale, causal)
            t_cpu += time.perf_counter() - t0
            eo = max(eo, float(np.max(np.abs(f64(o_[b, h]) - O[0, 0]))))
            el = max(el, float(np.max(np.abs(f64(l_[b, h]) - L[0, 0]))))
        flop = len(heads) * 4.0 * w.N * w.M * w.D / (2.0 if causal else 1.0)
        res[label] = {"value": flop / t_cpu / 1e12, "unit": "TFLOP/s", "seconds": t_cpu,
                      "sample": f"{len(heads)} whole head(s) of this shape's tensors, fp64 NumPy, "
                                "same FLOP convention",
                      "parity_vs_gpu": {"O_max_abs": eo, "LSE_max_abs": el, "tol": [2e-2, 1e-3]}}
    return res


def cpu_baseline(args, np, torch, qp, kp, vp, op, lp, scale_p, wp, qd, kd, vd, od, ld, kvl_h,
                 scale_d, wd):
    """The oracle as it stands, timed on this host on a bounded sample of the
    same tensors; its outputs are also compared with the GPU's."""
    from oracle.attention import attention_ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    # the scales as the C ABI carries them (float32), upcast exactly
    scale_p, scale_d = float(np.float32(scale_p)), float(np.float32(scale_d))
    rng = np.random.default_rng(0)
    # prefill sample: whole heads (every query row, all keys)
    heads = [(0, 0), (wp.B - 1, wp.H - 1)] + [
        (int(rng.integers(wp.B)), int(rng.integers(wp.H))) for _ in range(max(0, args.cpu_heads - 2))]
    t_cpu, eo, el = 0.0, 0.0, 0.0
    for b, h in heads:
        q, k, v = f64(qp[b, h])[None, None], f64(kp[b, h])[None, None], f64(vp[b, h])[None, None]
        t0 = time.perf_counter()
        O, L = attention_ref(q, k, v, scale_p, True)
        t_cpu += time.perf_counter() - t0
        eo = max(eo, float(np.max(np.abs(f64(op[b, h]) - O[0, 0]))))
        el = max(el, float(np.max(np.abs(f64(lp[b, h]) - L[0, 0]))))
    flop = len(heads) * 4.0 * wp.N * wp.M * wp.D / 2.0
    res = {"value": flop / t_cpu / 1e12, "unit": "TFLOP/s", "cores": blas_threads,
           "kind": "oracle", "seconds": t_cpu, "host": host_description(blas_threads),
           "sample": f"{len(heads)} whole heads (N=M=8192, D=128, causal) of the bench's "
                     f"prefill tensors, fp64 NumPy, same FLOP convention",
           "parity_vs_gpu": {"O_max_abs": eo, "LSE_max_abs": el, "tol": [2e-2, 1e-3]}}
    # decode sample
    dh = [(0, 0), (wd.B - 1, wd.H - 1)] + [
        (int(rng.integers(wd.B)), int(rng.integers(wd.H))) for _ in range(max(0, args.cpu_decode_heads - 2))]
    t_cpu, eo, el, nbytes = 0.0, 0.0, 0.0, 0.0
    for b, h in dh:
        n = int(kvl_h[b])
        q, k, v = f64(qd[b, h])[None, None], f64(kd[b, h, :n])[None, None], f64(vd[b, h, :n])[None, None]
        t0 = time.perf_counter()
        O, L = attention_ref(q, k, v, scale_d, False)
        t_cpu += time.perf_counter() - t0
        nbytes += n * wd.D * 2 * 2
        eo = max(eo, float(np.max(np.abs(f64(od[b, h]) - O[0, 0]))))
        el = max(el, float(np.max(np.abs(f64(ld[b, h]) - L[0, 0]))))
    res["decode"] = {"value": nbytes / t_cpu / 1e9, "unit": "GB/s", "seconds": t_cpu,
                     "sample": f"{len(dh)} (batch, head) pairs of the bench's decode tensors",
                     "parity_vs_gpu": {"O_max_abs": eo, "LSE_max_abs": el, "tol": [2e-2, 1e-3]}}
    return res


def cpu_baseline_bwd(np, qp, kp, vp, gb, dqb, dkb, dvb, scale_p, wp, heads=((0, 0),)):
    """The backward oracle timed on whole heads of the bench's tensors."""
    from oracle.backward import head_backward
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    scale_p = float(np.float32(scale_p))  # as the C ABI carries it
    t_cpu, err = 0.0, {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in heads:
        q, k, v, g = f64(qp[b, h]), f64(kp[b, h]), f64(vp[b, h]), f64(gb[b, h])
        t0 = time.perf_counter()
        r = head_backward(q, k, v, g, scale_p, True, wp.M)
        t_cpu += time.perf_counter() - t0
        for n, t in (("dq", dqb), ("dk", dkb), ("dv", dvb)):
            err[n] = max(err[n], float(np.max(np.abs(f64(t[b, h]) - r[n]))))
    flop = len(heads) * 10.0 * wp.N * wp.M * wp.D / 2.0
    return {"value": flop / t_cpu / 1e12, "unit": "TFLOP/s", "seconds": t_cpu,
            "sample": f"{len(heads)} whole head(s) (N=M=8192, D=128, causal) of the bench's "
                      "backward tensors, fp64 NumPy, same FLOP convention",
            "max_abs_vs_gpu": err}


# ---------------------------------------------------------------------------
# profiles/ summaries from rocprofv3 output (no GPU needed)
# ---------------------------------------------------------------------------
# The runs that produce DIR, all on committed files, from /tmp (TMPDIR=/tmp):
#   rocprofv3 --kernel-trace --stats --output-format csv -d DIR/ktrace -o run --
#       python3 <repo>/bench.py --steps 10 --warmup 3 --no-cpu-baseline
#   for leg in copy prefill decode backward window mask fp8 kvouter configs,
#   c in FETCH_SIZE WRITE_SIZE (one counter per run):
#     rocprofv3 --pmc c --output-format csv -d DIR/pmc_c_leg -o run --
#       python3 <repo>/bench.py --only leg --steps 2 --warmup 0 --no-cpu-baseline
#   for leg in prefill backward fp8:
#     rocprofv3 --pmc <UTIL_COUNTERS> --output-format csv -d DIR/pmc_util_leg -o run -- (same)
UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CU_CYCLES",
                 "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")
KTRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/ktrace -o run -- "
              "python3 <repo>/bench.py --steps 10 --warmup 3 --no-cpu-baseline")
PMC_CMD = ("cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_{c}_{leg} -o run -- "
           "python3 <repo>/bench.py --only {leg} --steps 2 --warmup 0 --no-cpu-baseline")
# leg: (case, first kernel of a call of that case, calls averaged), in the
# order the bench makes them; the last calls of each kind belong to the last case
COUNTER_LEGS = {
    "prefill": [(None, "prefill_cont", 2)],
    "decode": [(None, "splitkv_partial", 2)],
    "backward": [(None, "bwd_rowstat", 2)],
    "window": [("w128", "prefill_cont", 2), ("w2048", "prefill_cont", 2)],
    "mask": [("documents8", "mask_blocks", 2), ("random50", "mask_blocks", 2),
             ("backward_documents8", "bwd_rowstat", 2)],
    "configs": [("B1_H8_N1024_D64_causal", "prefill_bf16", 2), ("B4_H16_N4096_D128_causal", "prefill_cont", 2),
                ("B4_H16_N4096_D128_noncausal", "prefill_bf16", 2), ("B2_H32_N8192_D64_causal", "prefill_cont", 2),
                ("B1_H8_N1024_D64_causal_split_keys256", "prefill_split", 2)],
    "fp8": [(None, "prefill_fp8", 2)],
    "kvouter": [("tile_per_group", "kvouter", 3), ("head_per_group", "kvouter", 3)],
}


def prefill_kernel_name(w, causal):
    """The kernel the library runs for a prefill without window, mask or
    kv_len: causal with more 256-query work items than the 256 persistent
    workgroups runs the walk as one pipeline."""
    if causal and w.N >= 256 and w.M >= w.N and w.B * w.H * ((w.N + 255) // 256) > 256:
        return f"prefill_cont_kernel<{w.D}, true, false, false>"
    return f"prefill_bf16_kernel<{w.D}, {str(causal).lower()}, false, false>"


def _short_kernel(name):
    """'prefill_bf16_kernel<128, true, false, false>' for the library's kernels,
    '__amd_rocclr_copyBuffer' for the calibration copy, else None."""
    if "__amd_rocclr_copyBuffer" in name:
        return "__amd_rocclr_copyBuffer"
    if "fa::" not in name or "(anonymous namespace)::" not in name:
        return None
    return name.split("(anonymous namespace)::")[1].split("(")[0]


def _leg_of_dispatches(rows):
    """Label the library's launches of the default bench sequence by leg, from
    their order (the bench's call order is fixed)."""
    seen_kvo, n = False, {"win": 0, "maskp": 0, "kvo": 0}
    out = []
    for i, (_, s, ns) in enumerate(rows):
        nxt = rows[i + 1][1] if i + 1 < len(rows) else ""
        seen_kvo |= s.startswith("kvouter")
        if s == "prefill_cont_kernel<128, true, false, false>":
            leg = ("prefill B2 H32 N8192 D128 causal (bench step)" if nxt.startswith("splitkv_partial") else
                   "configs B4 H16 N4096 D128 causal" if seen_kvo else
                   "setup (untimed forward for the backward's O, LSE)")
        elif s.startswith("splitkv"):
            leg = "decode B32 H32 D128 (bench step)"
        elif s.startswith("bwd_rowstat"):
            leg = "backward (rowstat, both legs)"
        elif s.startswith("bwd_"):
            leg = "backward B2 H32 N8192 D128 causal" if s.endswith("false>") else "backward under the 8-document mask"
        elif s == "prefill_cont_kernel<128, true, true, false>":
            n["win"] += 1
            leg = "window 128 keys" if n["win"] <= 13 else "window 2048 keys"
        elif s == "prefill_cont_kernel<128, true, false, true>" or s.startswith("mask_"):
            if s.startswith("prefill"):
                n["maskp"] += 1
            k = n["maskp"] if s.startswith("prefill") else n["maskp"] + 1   # a pre-pass precedes its prefill
            leg = ("setup (untimed masked forward for the masked backward)" if k == 1 else
                   "mask, 8 documents" if k <= 14 else
                   "mask, unstructured p = 1/2" if k <= 27 else "backward under the 8-document mask")
        elif s.startswith("prefill_fp8"):
            leg = "fp8 B2 H32 N8192 D128 causal"
        elif s.startswith("kvouter"):
            n["kvo"] += 1
            leg = "kvouter, one query tile per group" if n["kvo"] <= 3 else "kvouter, one head per group"
        elif s == "prefill_bf16_kernel<64, true, false, false>":
            leg = "configs B1 H8 N1024 D64 causal"
        elif s == "prefill_cont_kernel<64, true, false, false>":
            leg = "configs B2 H32 N8192 D64 causal"
        elif s == "prefill_bf16_kernel<128, false, false, false>":
            leg = "configs B4 H16 N4096 D128 non-causal"
        elif s.startswith(("prefill_split", "prefill_merge")):
            leg = "configs B1 H8 N1024 D64 causal, keys in chunks of 256"
        else:
            leg = "other"
        out.append((leg, s, ns))
    return out


def summarize_profiles(d):
    """Write the profiles/ summaries (kernel durations, HBM traffic per leg
    with the copy calibration, matrix-pipe counters) from rocprofv3 output."""
    import csv
    import statistics
    from collections import defaultdict
    prof = os.path.join(ROOT, "profiles")

    def write(name, lines):
        lines = lines[:2] + ["# summarised by: python3 <repo>/bench.py --profile-summary <out>"] + lines[2:]
        with open(os.path.join(prof, name), "w") as f:
            f.write("\n".join(lines) + "\n")

    # kernel durations: rocprofv3 --stats, and the same trace split by leg
    lines = ["# rocprofv3 --stats kernel summary of the default bench sequence (durations in ns), the library's kernels",
             f"# command: {KTRACE_CMD}",
             "# rows aggregate by kernel name: prefill_cont_kernel<128, true, false, false> serves the bench step (N = 8192),",
             "# the configs leg (N = 4096) and one untimed setup call;",
             "# kernel_trace_by_leg_default_bench.txt splits the same trace by leg", "#",
             "# kernel, calls, average_ns, min_ns, max_ns, stddev_ns"]
    for r in csv.DictReader(open(os.path.join(d, "ktrace", "run_kernel_stats.csv"))):
        s = _short_kernel(r["Name"])
        if s and s != "__amd_rocclr_copyBuffer":
            lines.append(f"{s}, {r['Calls']}, {float(r['AverageNs']):.0f}, {r['MinNs']}, {r['MaxNs']}, "
                         f"{float(r['StdDev']):.0f}")
    write("kernel_stats_default_bench.txt", lines)
    rows = []
    for r in csv.DictReader(open(os.path.join(d, "ktrace", "run_kernel_trace.csv"))):
        s = _short_kernel(r["Kernel_Name"])
        if s and s != "__amd_rocclr_copyBuffer":
            rows.append((int(r["Dispatch_Id"]), s, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    agg, order = defaultdict(list), []
    for leg, s, ns in _leg_of_dispatches(rows):
        if (leg, s) not in agg:
            order.append((leg, s))
        agg[(leg, s)].append(ns)
    lines = ["# rocprofv3 kernel trace of the default bench sequence, split by leg (durations in ns)",
             f"# command: {KTRACE_CMD}",
             "# each leg's launches are told apart by their place in the bench's fixed call order (run_kernel_trace.csv);",
             "# every leg runs 3 warmup + 10 timed calls (kvouter 1 + 2); averages include the warmup calls", "#",
             "# leg, kernel, calls, average_ns, min_ns, max_ns, stddev_ns"]
    for leg, s in order:
        v = agg[(leg, s)]
        lines.append(f"{leg}, {s}, {len(v)}, {statistics.mean(v):.0f}, {min(v)}, {max(v)}, {statistics.pstdev(v):.0f}")
    write("kernel_trace_by_leg_default_bench.txt", lines)

    # HBM traffic: per leg, the last calls of each case, calibrated by a copy
    def dispatches(leg, ctr):
        out = []
        for r in csv.DictReader(open(os.path.join(d, f"pmc_{ctr}_{leg}", "run_counter_collection.csv"))):
            s = _short_kernel(r["Kernel_Name"])
            if s:
                out.append((int(r["Dispatch_Id"]), s, float(r["Counter_Value"])))
        return sorted(out)

    def calls_of(rows):
        calls = []
        for _, k, v in rows:
            first = calls[-1][0][0] if calls else ""
            if not calls or k.startswith("bwd_rowstat"):
                start = True
            elif first.startswith("bwd_rowstat") or k.startswith(("splitkv_merge", "prefill_merge")):
                start = False   # a backward call runs to the next rowstat; split calls end with their merge
            elif first.startswith("mask_blocks") and not k.startswith("mask_blocks") and (
                    k.startswith("mask_") or (k.startswith("prefill") and calls[-1][-1][0].startswith("mask_"))):
                start = False   # the forward's pre-pass (three launches), then its prefill
            else:
                start = True
            if start:
                calls.append([])
            calls[-1].append((k, v))
        return calls

    def copy_kib(ctr):
        v = [x for _, s, x in dispatches("copy", ctr) if s == "__amd_rocclr_copyBuffer"]
        return sum(v) / len(v)
    cf, cw = copy_kib("FETCH_SIZE"), copy_kib("WRITE_SIZE")
    copy_bytes = 1 << 30
    ff, wf = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    traffic = {"calibration": {"copy_bytes": copy_bytes, "fetch_factor": ff, "write_factor": wf,
                               "copy_fetch_kib": cf, "copy_write_kib": cw}}
    lines = []
    for leg, spec in COUNTER_LEGS.items():
        per = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            kinds = {}
            for c in calls_of([r for r in dispatches(leg, ctr) if r[1] != "__amd_rocclr_copyBuffer"]):
                kinds.setdefault(c[0][0].split("<")[0].split("_kernel")[0], []).append(c)
            used = {}
            for case, kind, n in reversed(spec):
                pool = [c for key, cs in kinds.items() if key.startswith(kind) for c in cs]
                k0 = used.get(kind, 0)
                kern = defaultdict(float)
                for c in pool[len(pool) - k0 - n:len(pool) - k0]:
                    for k, v in c:
                        kern[k] += v / n
                used[kind] = k0 + n
                per.setdefault(case, {})[ctr] = dict(kern)
        rec = {"source_sha": kernel_source_sha(SOURCES[leg])}
        for case, _, _ in spec:
            kerns, tot = {}, 0.0
            for k, f in per[case]["FETCH_SIZE"].items():
                w = per[case]["WRITE_SIZE"].get(k, 0.0)
                fb, wb = f * 1024 * ff, w * 1024 * wf
                kerns[k] = {"fetch_kib": f, "write_kib": w, "fetch_bytes": fb, "write_bytes": wb}
                tot += fb + wb
                lines.append(f"{leg}{'/' + case if case else ''}, {k}, {f:.0f}, {w:.0f}, {fb:.4g}, {wb:.4g}")
            body = {"bytes_per_launch": tot, "kernels": kerns}
            if case is None:
                rec.update(body)
            else:
                rec.setdefault("cases", {})[case] = body
        traffic[leg] = rec
    head = ["# HBM traffic per library call from rocprofv3 --pmc (KiB per dispatch of each kernel the call launches, "
            "averaged over the timed calls)",
            "# calibration: a 1 GiB device-to-device copy (__amd_rocclr_copyBuffer) reads",
            f"#   FETCH_SIZE {cf:.0f} KiB -> factor {ff:.4f}; WRITE_SIZE {cw:.0f} KiB -> factor {wf:.4f}",
            "# commands, for leg in copy " + " ".join(COUNTER_LEGS) + " and c in FETCH_SIZE WRITE_SIZE:",
            "#   " + PMC_CMD, "#",
            "# leg[/case], kernel, FETCH_SIZE KiB, WRITE_SIZE KiB, scaled fetch bytes, scaled write bytes"]
    write("hbm_traffic_all_legs_n8192_d128.txt", head + lines)
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(traffic, f, indent=1)

    # matrix pipe and LDS
    lines = ["# MFMA utilisation and LDS counters per dispatch (rocprofv3 --pmc, one pass)",
             "# command: " + PMC_CMD.replace("pmc_{c}", "pmc_util").replace("{c}", " ".join(UTIL_COUNTERS))
             + "   (leg in prefill backward fp8)",
             "# GRBM_GUI_ACTIVE is summed over the 8 XCDs; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(256 CUs x 4 SIMDs x GUI cycles per XCD)", "#"]
    for leg in ("prefill", "backward", "fp8"):
        agg, calls = defaultdict(lambda: defaultdict(float)), defaultdict(set)
        for r in csv.DictReader(open(os.path.join(d, f"pmc_util_{leg}", "run_counter_collection.csv"))):
            s = _short_kernel(r["Kernel_Name"])
            if s and s != "__amd_rocclr_copyBuffer":
                agg[s][r["Counter_Name"]] += float(r["Counter_Value"])
                calls[s].add(r["Dispatch_Id"])
        for s, c in agg.items():
            n = len(calls[s])
            g = c["GRBM_GUI_ACTIVE"] / n / 8
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / n / (256 * 4 * g)
            lines.append(f"{s}, dispatches {n}, GRBM_GUI_ACTIVE/XCD {g:.4g} cycles, MFMA busy {busy:.3f} of SIMD-cycles, "
                         f"LDS bank conflicts / LDS active {c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.4f}, "
                         f"wait-inst fraction of wave cycles {c['SQ_WAIT_INST_ANY'] / max(c['SQ_WAVE_CYCLES'], 1):.3f}, "
                         f"VALU insts {c['SQ_INSTS_VALU'] / n:.4g} per dispatch; raw per dispatch: "
                         + ", ".join(f"{k} {v / n:.4g}" for k, v in sorted(c.items())))
    write("counters_mfma_lds_prefill_backward_fp8_n8192_d128.txt", lines)


if __name__ == "__main__":
    sys.exit(main())
