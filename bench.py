"""Benchmark of block-sparse decode on one MI355X.

Workload (default): batch 8, 16 heads, head dim 128, 128K context per
sequence, blocks of 32 keys, z = 1, bfloat16 KV cache, dynamic per-head
threshold tau = w_h.q + c_h with c_h calibrated (on the GPU, by the library's
calibration routine) to an admitted density of 38%.  A step is the whole
decode path for one new query per sequence: threshold (eta_predict_tau),
screen (eta_screen) and split-K attention with its combine (eta_decode).
Inputs are resident in HBM before timing starts.

Printed: one JSON line with dense-equivalent KV tokens/s (sum_b T_b per step
/ step time), the decode kernel's roofline against 8 TB/s, a density sweep
(10/38/70/100%) with the in-house dense HIP decode at the same shape, and the
fp64 oracle timed on the host on a bounded sample of the same workload.  A
grouped-query section follows (32 sequences x 128K, 32 query heads on 4 KV
heads, d 64, b 64: eta_screen_gqa + eta_decode_gqa against the grouped dense
decode at 38/25/10% head density) and a gated prefill section (8 x 2048, the
pages' training shape: eta_gated_prefill against the bf16 matrix-core peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")
GQA_COUNTERS = os.path.join(ROOT, "profiles", "gqa_decode_counters.json")
# the decode kernels and the host code that picks their launch path
CSRC = os.path.join(ROOT, "long_context_decode_eta_amd", "csrc")
DECODE_SRC = [os.path.join(CSRC, f) for f in ("kernels_decode.hip", "eta_api.hip", "eta_internal.h")]
GQA_SRC = [os.path.join(CSRC, f) for f in ("kernels_gqa.hip", "eta_api.hip", "eta_internal.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ctx128k",
                    choices=["ctx128k", "ctx32k", "ctx512k", "ragged"])
    ap.add_argument("--rho", type=float, default=None,
                    help="headline admitted density (default: the workload's target, 38%% for "
                         "the density-swept 128K workload)")
    ap.add_argument("--split", type=int, default=0, help="blocks per split (0: auto)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gqa", action="store_true",
                    help="skip the grouped-query section (32 x 128K, 32 query / 4 KV heads)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the gated prefill section (8 x 2048, 32 query / 4 KV heads)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the gated prefill section and print its JSON")
    ap.add_argument("--gqa-only", action="store_true",
                    help="run only the grouped-query section and print its JSON")
    ap.add_argument("--gqa-rho", default="0.38,0.25,0.10",
                    help="head densities of the grouped-query section")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times "
                         "(reference dispatches for calibrating HBM byte counters)")
    return ap.parse_args()


def copy_reference(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": n, "dispatches": 5}), flush=True)


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def around(self, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        return sum(s.elapsed_time(e) for s, e in self.pairs) / max(1, len(self.pairs))


def kernel_hash(files=DECODE_SRC) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def counters_traffic(path, files, workload):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the same kernel sources and workload."""
    if not os.path.exists(path):
        return None
    cj = json.load(open(path))
    if cj.get("kernel_hash") == kernel_hash(files) and cj.get("workload") == workload:
        return cj.get("hbm_bytes_per_launch")
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path runs on a single GPU; see the sharding notes in the design).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    import numpy as np
    import torch

    from long_context_decode_eta_amd import binding as eb
    from long_context_decode_eta_amd import synth

    if args.rho is None:
        target = synth.CONFIGS[args.workload].get("rho", 0.38)
        args.rho = target if isinstance(target, float) else 0.38
    dev = "cuda"
    torch.cuda.set_device(0)
    gqa_rhos = [float(x) for x in args.gqa_rho.split(",")]
    if args.prefill_only:
        print(json.dumps(prefill_bench(torch, eb, synth, args.steps, args.warmup, args.seed)),
              flush=True)
        return
    if args.gqa_only:
        print(json.dumps(gqa_bench(torch, np, eb, synth, args.steps, args.warmup, args.seed,
                                   gqa_rhos)), flush=True)
        return
    t0 = time.time()
    blk = synth.CONFIGS[args.workload]["block"]
    Tmax = synth.CONFIGS[args.workload]["T"]
    Tmax = Tmax[1] if isinstance(Tmax, tuple) else Tmax
    # room for the appends of the upkeep measurement (4 blocks per stream)
    w = synth.make(args.workload, seed=args.seed, device=dev, cap=Tmax + 4 * blk)
    B, H, D, bs = w.B, w.H, w.D, w.block
    cache = eb.KVCache(B, H, D, bs, w.cap, w.kv_dtype, device=dev, k=w.k, v=w.v)
    cache.seq_len.copy_(w.seq_len)
    eb.build_block_meta(cache)
    sl = w.seq_len.cpu().numpy().astype(np.int64)
    sumT = int(sl.sum())
    dec = eb.Decoder(cache, z=w.z, scale=w.scale, blocks_per_split=args.split or None)
    split = dec.split
    print(f"[bench] workload {args.workload}: B={B} H={H} D={D} b={bs} sumT={sumT} "
          f"split={split} dense split={dec.dense_split} ({time.time() - t0:.1f}s setup)",
          file=sys.stderr, flush=True)
    W = w.W
    # Per-head constants for each target density, from the library's calibration.
    if w.tau_kind == "dynamic":
        tau0 = torch.zeros((B, H), device=dev)
        tmp = torch.zeros_like(tau0)
        eb.predict_tau(w.q, W, torch.zeros(H, device=dev), 0.0, tau0, tmp)
        qs, t0s = w.q[None].contiguous(), tau0[None].contiguous()
    else:
        qs, t0s = w.q_cal.contiguous(), None
    cws = eb.workspace(eb.calibrate_workspace_bytes(qs.shape[0], B, H, cache.cap_blocks))
    rhos = sorted(set([args.rho] + ([] if args.no_sweep else [0.10, 0.38, 0.70, 1.0])))
    consts = {}
    for rho in rhos:
        c = torch.zeros(H, device=dev)
        eb.calibrate_threshold(cache, qs, t0s, w.z, w.scale, rho, cws, c)
        consts[rho] = c
    del cws
    frozen = W is None
    if frozen:
        # frozen constants: no predictor in the timed step; tau is the broadcast
        def set_tau(c):
            dec.predict(w.q, None, c)
    torch.cuda.synchronize()

    kv_bytes = 2 * w.k.numel() * w.k.element_size()
    flush = (torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
             if kv_bytes < (2 << 30) else None)

    def run(rho, steps, warmup):
        """Eager steps timed per kernel with HIP events, then the same step
        captured once in a HIP graph (checked bit for bit against the eager
        output) and timed over `steps` replays."""
        c = consts[rho]
        if frozen:
            set_tau(c)

        def step():
            if not frozen:
                dec.predict(w.q, W, c)
            dec.screen(w.q)
            dec.attend(w.q)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ctr0 = int(dec.density_ctr.item())
        tdec, tscr = Timer(torch), Timer(torch)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(steps):
            if not frozen:
                dec.predict(w.q, W, c)
            tscr.around(lambda: dec.screen(w.q))
            tdec.around(lambda: dec.attend(w.q))
        torch.cuda.synchronize()
        eager = time.perf_counter() - a
        toks = (int(dec.density_ctr.item()) - ctr0) // steps
        # Per-step latency distribution (HIP events around each whole step); for
        # a cache that could sit in the 256 MB last-level cache, 512 MiB of
        # scratch is written before every timed step so no step reads KV from it.
        per_step = []
        for _ in range(steps):
            if flush is not None:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            per_step.append((e0, e1))
        torch.cuda.synchronize()
        lat = sorted(s0.elapsed_time(s1) for s0, s1 in per_step)
        cnt = dec.active_cnt.cpu().numpy().astype(np.int64)
        ref = dec.out.clone()

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):  # every replay must reproduce the eager result exactly
            dec.out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(dec.out, ref), "graph replay differs from eager decode"
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - a
        del graph
        pct = lambda f: lat[min(len(lat) - 1, int(f * (len(lat) - 1) + 0.5))]
        return dict(ms=wall * 1e3 / steps, eager_ms=eager * 1e3 / steps,
                    step_ms_median=pct(0.5), step_ms_p10=pct(0.1), step_ms_p90=pct(0.9),
                    decode_ms=tdec.mean_ms(), screen_ms=tscr.mean_ms(),
                    density=toks / (H * sumT), tokens=toks, cnt=cnt)

    def run_dense(steps, warmup):
        """The in-house dense decode at the same shape, captured in a HIP graph
        like the sparse step."""
        graph = torch.cuda.CUDAGraph()
        dec.dense(w.q)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            dec.dense(w.q)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - a) * 1e3 / steps

    elt = 2 if w.kv_dtype == torch.bfloat16 else 4
    nbc = sl // bs
    meta_bytes = int(H * (nbc * (2 * D + 1) * 4).sum())

    def decode_bytes(r):
        # algorithmic bytes of one eta_decode call: admitted K+V, q, the active
        # list, partial (m, l, acc) write + read for multi-chunk streams, output
        chunks = -(-r["cnt"] // split)
        part = int((np.where(chunks > 1, chunks, 0) * (D + 2) * 4 * 2).sum())
        return r["tokens"] * D * 2 * elt + B * H * D * 4 * 2 + int(r["cnt"].sum()) * 4 + part

    def step_bytes(r):
        pred = 0 if frozen else B * H * D * 4 + H * D * H * 4 + 2 * B * H * 4
        screen = meta_bytes + B * H * D * 4 + int(r["cnt"].sum()) * 4 + B * H * 4
        return pred + screen + decode_bytes(r)

    sweep = {}
    main = None
    for rho in rhos:
        r = run(rho, args.steps, args.warmup)
        r["step_bytes"] = step_bytes(r)
        r["decode_bytes"] = decode_bytes(r)
        sweep[rho] = r
        print(f"[bench] rho={rho:.2f}: density {r['density']:.4f} step {r['ms']:.4f} ms "
              f"(eager {r['eager_ms']:.4f}; screen {r['screen_ms']:.4f}, "
              f"decode {r['decode_ms']:.4f}) "
              f"{r['step_bytes'] / r['ms'] / 1e6:.0f} GB/s", file=sys.stderr, flush=True)
        if rho == args.rho:
            main = r
    dense_ms = run_dense(args.steps, args.warmup)
    dense_bytes = sumT * H * D * 2 * elt
    print(f"[bench] dense: {dense_ms:.4f} ms ({dense_bytes / dense_ms / 1e6:.0f} GB/s)",
          file=sys.stderr, flush=True)

    # Headline run: exactly `steps` timed steps at the headline density.
    r = run(args.rho, args.steps, args.warmup)
    r["step_bytes"] = step_bytes(r)
    r["decode_bytes"] = decode_bytes(r)
    main = r
    value = sumT / (r["ms"] * 1e-3)
    achieved = r["decode_bytes"] / (r["decode_ms"] * 1e-3) / 1e9
    traffic = counters_traffic(COUNTERS, DECODE_SRC, args.workload)
    # The measured streaming peak beside the spec: the dense decode reads every
    # K and V byte of the same cache in long contiguous runs.
    stream_gbs = dense_bytes / dense_ms / 1e6
    roofline = {"bound": "hbm", "kernel": "eta_decode (balanced decode + combine kernels)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(r["decode_bytes"]),
                "avg_launch_ms": round(r["decode_ms"], 5),
                "measured_stream_gbs": round(stream_gbs, 1),
                "frac_of_measured_stream": round(achieved / stream_gbs, 4)}

    offsets = None if args.no_sweep else offset_sweep(torch, np, eb, w, dec, consts[args.rho],
                                                       frozen, sumT, args.steps, args.warmup)
    upkeep = measure_upkeep(torch, eb, w, cache, dec, consts[args.rho], frozen, sumT)
    print(f"[bench] upkeep: {json.dumps(upkeep)}", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_baseline(w, consts[args.rho], args.rho)
    gqa = None
    if not args.no_gqa:
        gqa = gqa_bench(torch, np, eb, synth, args.steps, args.warmup, args.seed, gqa_rhos)
    prefill = None
    if not args.no_prefill:
        prefill = prefill_bench(torch, eb, synth, args.steps, args.warmup, args.seed)

    out = {
        "metric": "dense-equiv KV tokens/s + achieved HBM GB/s (active bytes) at 128K ctx",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "eager_ms_per_step": round(r["eager_ms"], 5),
        "eager_step_ms": {"median": round(r["step_ms_median"], 5),
                          "p10": round(r["step_ms_p10"], 5), "p90": round(r["step_ms_p90"], 5),
                          "llc_flushed": flush is not None},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: batch {B}, {H} heads, head dim {D}, "
                        f"context {int(sl.max())} (sum {sumT}), block {bs}, z {w.z}, "
                        f"{'bf16' if elt == 2 else 'fp32'} KV, "
                        f"{'frozen calibrated' if frozen else 'dynamic linear'} tau at "
                        f"{args.rho:.0%} target density",
            "global_batch": B, "seq_len": int(sl.max()), "parallelism": "single GPU",
            "kv_dtype": "bf16" if elt == 2 else "f32", "blocks_per_split": split,
            "dense_blocks_per_split": dec.dense_split,
        },
        "density": round(r["density"], 4),
        "step_hbm_gbs": round(r["step_bytes"] / r["ms"] / 1e6, 1),
        "step_roofline_frac": round(r["step_bytes"] / r["ms"] / 1e6 / HBM_PEAK_GBS, 4),
        "dense_ms": round(dense_ms, 5),
        "speedup_vs_dense": round(dense_ms / r["ms"], 3),
        "sweep": {f"{k:.2f}": {"density": round(v["density"], 4), "ms": round(v["ms"], 5),
                               "eager_ms": round(v["eager_ms"], 5),
                               "tokens_per_s": round(sumT / (v["ms"] * 1e-3), 1),
                               "step_gbs": round(v["step_bytes"] / v["ms"] / 1e6, 1),
                               "decode_gbs": round(v["decode_bytes"] / v["decode_ms"] / 1e6, 1),
                               "screen_ms": round(v["screen_ms"], 5),
                               "decode_ms": round(v["decode_ms"], 5),
                               "speedup_vs_dense": round(dense_ms / v["ms"], 3),
                               "ideal_speedup": round(dense_bytes / v["step_bytes"], 3)}
                  for k, v in sweep.items()},
        "roofline": roofline,
        "offset_sweep": offsets,
        "upkeep": upkeep,
        "cpu_baseline": cpu,
        "gqa": gqa,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


def offset_sweep(torch, np, eb, w, dec, c, frozen, sumT, steps, warmup):
    """Threshold-offset sweep on the synthetic workload (a Pareto curve in the
    manner of the pages' offset tables): per-head constants fixed at the
    headline density, screening threshold tau - a for several offsets a.  For
    each a: admitted density, recall of the generator's needle blocks, the
    output's relative L2 distance to the same gated attention with every block
    admitted (a = +inf), and the step time (eager, HIP events)."""
    W = None if frozen else w.W
    H = w.H

    def step(a):
        dec.a = a
        dec.predict(w.q, W, c)
        dec.screen(w.q)
        dec.attend(w.q)

    step(math.inf)
    torch.cuda.synchronize()
    full = dec.out.clone()
    out = {}
    for a in (-1.0, -0.5, 0.0, 0.25, 0.5, 1.0, 2.0):
        for _ in range(warmup):
            step(a)
        torch.cuda.synchronize()
        ctr0 = int(dec.density_ctr.item())
        s0 = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(steps):
            step(a)
        e0.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(e0) / steps
        toks = (int(dec.density_ctr.item()) - ctr0) // steps
        idx = dec.active_idx.cpu().numpy()
        cnt = dec.active_cnt.cpu().numpy()
        hit = tot = 0
        for u, nd in enumerate(w.needle_blocks):
            b, h = divmod(u, H)
            if nd.numel():
                sel = idx[b, h, :cnt[b, h]]
                hit += int(np.isin(nd.cpu().numpy(), sel).sum())
                tot += int(nd.numel())
        err = float(torch.linalg.vector_norm(dec.out - full) / torch.linalg.vector_norm(full))
        out[f"{a:+.2f}"] = {"density": round(toks / (H * sumT), 4),
                            "needle_recall": round(hit / max(1, tot), 4),
                            "rel_l2_vs_all_admitted": float(f"{err:.3e}"),
                            "eager_ms": round(ms, 5)}
        print(f"[bench] offset a={a:+.2f}: {json.dumps(out[f'{a:+.2f}'])}", file=sys.stderr,
              flush=True)
    dec.a = 0.0
    return out


def measure_upkeep(torch, eb, w, cache, dec, c, frozen, sumT):
    """Cache upkeep, timed apart from the step: the bulk statistics build that
    follows a prefill, single-token appends (which compute the statistics of
    every block they complete), and the whole per-token loop (append, then
    threshold, screen and decode) run across block boundaries.  Each is timed
    over 2 blocks' worth of tokens so block completions are included at their
    real rate.  Leaves every sequence 4 blocks longer."""
    B, H, D, bs = w.B, w.H, w.D, w.block

    def ev():
        return torch.cuda.Event(enable_timing=True)

    s0, e0 = ev(), ev()
    s0.record()
    for _ in range(3):
        eb.build_block_meta(cache)
    e0.record()
    torch.cuda.synchronize()
    meta_ms = s0.elapsed_time(e0) / 3
    elt = cache.k.element_size()
    meta_bytes = sumT * H * D * elt + (sumT // bs) * H * (2 * D + 1) * 4

    g = torch.Generator(device="cuda").manual_seed(99)
    kn = torch.randn((B, H, D), generator=g, device="cuda").to(cache.kv_dtype)
    vn = torch.randn((B, H, D), generator=g, device="cuda").to(cache.kv_dtype)
    n = 2 * bs
    torch.cuda.synchronize()
    s1, e1 = ev(), ev()
    s1.record()
    for _ in range(n):
        eb.append_kv(cache, kn, vn)
    e1.record()
    torch.cuda.synchronize()
    append_us = s1.elapsed_time(e1) * 1e3 / n

    if frozen:
        dec.predict(w.q, None, c)
    s2, e2 = ev(), ev()
    s2.record()
    for _ in range(n):
        eb.append_kv(cache, kn, vn)
        if not frozen:
            dec.predict(w.q, w.W, c)
        dec.screen(w.q)
        dec.attend(w.q)
    e2.record()
    torch.cuda.synchronize()
    loop_ms = s2.elapsed_time(e2) / n
    s3, e3 = ev(), ev()
    s3.record()
    for _ in range(n):
        if not frozen:
            dec.predict(w.q, w.W, c)
    e3.record()
    torch.cuda.synchronize()
    pred_us = s3.elapsed_time(e3) * 1e3 / n
    return {"meta_build_ms": round(meta_ms, 4),
            "meta_build_gbs": round(meta_bytes / meta_ms / 1e6, 1),
            "append_us": round(append_us, 2),
            "predict_us": round(pred_us, 2) if not frozen else 0.0,
            "loop_ms_per_token": round(loop_ms, 5),
            "tokens_timed": n}


def gqa_bench(torch, np, eb, synth, steps, warmup, seed, rhos=(0.38, 0.25, 0.10)):
    """Grouped-query decode at the pages' benchmark shape (32 sequences x
    128K, 32 query heads on 4 KV heads, d 64, b 64, bf16): dynamic Eq. 1
    thresholds over the query heads with constants calibrated per query head
    (the library's calibration, one call per head position in the group) to
    38%, 25% and 10% head density; step = predict + screen_gqa + decode_gqa,
    graph-captured; the grouped dense decode at the same shape alongside.
    Decode bytes: union K+V rows, q, head masks and union lists, chunk
    partials, outputs."""
    dev = "cuda"
    w = synth.make("gqa128k", seed=seed, device=dev)
    B, Hkv, G, D, bs = w.B, w.H, w.G, w.D, w.block
    Hq = Hkv * G
    cache = eb.KVCache(B, Hkv, D, bs, w.cap, w.kv_dtype, device=dev, k=w.k, v=w.v)
    cache.seq_len.copy_(w.seq_len)
    eb.build_block_meta(cache)
    sumT = int(w.seq_len.sum().item())
    dec = eb.GqaDecoder(cache, G, z=w.z, scale=w.scale)
    tau0 = torch.zeros((B, Hq), device=dev)
    tmp = torch.zeros_like(tau0)
    eb.predict_tau(w.q, w.W, torch.zeros(Hq, device=dev), 0.0, tau0, tmp)
    q4 = w.q.view(B, Hkv, G, D)
    t4 = tau0.view(B, Hkv, G)
    cws = eb.workspace(eb.calibrate_workspace_bytes(1, B, Hkv, cache.cap_blocks))
    res = {}
    for rho in rhos:
        c = torch.zeros((Hkv, G), device=dev)
        cg = torch.zeros(Hkv, device=dev)
        for g in range(G):
            eb.calibrate_threshold(cache, q4[:, :, g].contiguous()[None],
                                   t4[:, :, g].contiguous()[None], w.z, w.scale, rho, cws, cg)
            c[:, g] = cg
        c = c.reshape(Hq).contiguous()

        def step():
            dec.predict(w.q, w.W, c)
            dec.screen(w.q)
            dec.attend(w.q)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ctr0 = dec.density_ctr.clone()
        tscr, tdec = Timer(torch), Timer(torch)
        for _ in range(steps):
            dec.predict(w.q, w.W, c)
            tscr.around(lambda: dec.screen(w.q))
            tdec.around(lambda: dec.attend(w.q))
        torch.cuda.synchronize()
        ctr = ((dec.density_ctr - ctr0) // steps).cpu().numpy()
        ucnt = dec.union_cnt.cpu().numpy().astype(np.int64)
        ref = dec.out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            dec.out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(dec.out, ref), "graph replay differs from eager decode"
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - a) * 1e3 / steps
        del graph
        union_tok = int(ctr[1])
        chunks = -(-ucnt // dec.split)
        part = int((np.where(chunks > 1, chunks, 0) * G * (D + 2) * 4 * 2).sum())
        dbytes = union_tok * D * 2 * 2 + 2 * B * Hq * D * 4 + int(ucnt.sum()) * 8 + part
        res[f"{rho:.2f}"] = {
            "decode_bytes": int(dbytes),
            "d_head": round(int(ctr[0]) / (sumT * Hq), 4),
            "d_union": round(union_tok / (sumT * Hkv), 4),
            "ms": round(ms, 5), "screen_ms": round(tscr.mean_ms(), 5),
            "decode_ms": round(tdec.mean_ms(), 5),
            "decode_gbs": round(dbytes / tdec.mean_ms() / 1e6, 1),
            "tokens_per_s": round(sumT / (ms * 1e-3), 1)}
        print(f"[bench] gqa rho={rho:.2f}: {json.dumps(res[f'{rho:.2f}'])}", file=sys.stderr,
              flush=True)
    graph = torch.cuda.CUDAGraph()
    dec.dense(w.q)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dec.dense(w.q)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    a = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    dense_ms = (time.perf_counter() - a) * 1e3 / steps
    dense_bytes = sumT * Hkv * D * 2 * 2
    for v in res.values():
        v["speedup_vs_dense"] = round(dense_ms / v["ms"], 3)
    roofline = None
    if "0.38" in res:
        r = res["0.38"]
        ach = r["decode_bytes"] / (r["decode_ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "eta_decode_gqa (balanced decode + combine kernels), 38% head",
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": counters_traffic(GQA_COUNTERS, GQA_SRC, "gqa128k"),
                    "algorithmic_bytes_per_launch": r["decode_bytes"],
                    "avg_launch_ms": r["decode_ms"],
                    "measured_stream_gbs": round(dense_bytes / dense_ms / 1e6, 1),
                    "frac_of_measured_stream": round(ach / (dense_bytes / dense_ms / 1e6), 4)}
    out = {"workload": f"gqa128k: batch {B}, {Hq} query heads on {Hkv} KV heads, head dim {D}, "
                       f"context {int(w.seq_len.max())}, block {bs}, z {w.z}, bf16 KV, "
                       "dynamic linear tau",
           "roofline": roofline,
           "blocks_per_split": dec.split, "dense_blocks_per_split": dec.dense_split,
           "dense_ms": round(dense_ms, 5),
           "dense_gbs": round(dense_bytes / dense_ms / 1e6, 1),
           "by_head_density": res}
    print(f"[bench] gqa dense: {dense_ms:.4f} ms", file=sys.stderr, flush=True)
    del dec, cache, w
    torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFS = 2500.0


def prefill_bench(torch, eb, synth, steps, warmup, seed):
    """Gated causal attention forward at the pages' training shape (8 x 2048,
    32 query heads on 4 KV heads, d 64, bf16): one eta_gated_prefill call per
    step, graph-captured and checked against eager.  Algorithmic flops: 4 d
    per (query, causal key) pair (the score and value products)."""
    w = synth.make_prefill(seed=seed, device="cuda")
    out = torch.zeros((w.B, w.Hq, w.T, w.D), device="cuda")
    dens = torch.zeros((w.B, w.Hq, w.T), device="cuda")

    def step():
        eb.gated_prefill(w.q, w.k, w.v, w.tau, w.G, 5.0, w.scale, out, dens)

    # Clocks settle only after some tens of milliseconds of matrix-core work:
    # at least 100 warm-up launches (about 40 ms) before each timed loop.
    warmup = max(warmup, 100)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = Timer(torch)
    for _ in range(steps):
        ev.around(step)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "graph replay differs from eager prefill"
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    a = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - a) * 1e3 / steps
    del graph
    pairs = w.B * w.Hq * w.T * (w.T + 1) // 2
    flops = 4 * w.D * pairs
    tfs = flops / (ev.mean_ms() * 1e-3) / 1e12
    res = {"workload": f"prefill: batch {w.B}, {w.Hq} query heads on {w.H} KV heads, head dim "
                       f"{w.D}, context {w.T}, bf16 q/k/v, beta 5",
           "ms": round(ms, 5), "kernel_ms": round(ev.mean_ms(), 5),
           "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
           "mean_density": round(float(dens.mean()), 4),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 1),
                        "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                        "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                        "algorithmic_flops_per_launch": int(flops)}}
    print(f"[bench] prefill: {json.dumps(res)}", file=sys.stderr, flush=True)
    return res


def cpu_baseline(w, c_gpu, rho):
    """The fp64 oracle on the host: threshold + screen + attention for the
    streams of one sequence (all heads, full context), metadata prebuilt and
    not timed, per-head constants from the oracle's own calibration on that
    sample.  Repeated until about 10 s of CPU work; scaled to tokens/s as
    T_0 / (time per repetition)."""
    import numpy as np

    import oracle
    from long_context_decode_eta_amd import synth

    b0 = 0
    K = synth.kv_numpy(w.k[b0:b0 + 1])
    V = synth.kv_numpy(w.v[b0:b0 + 1])
    q = w.q[b0:b0 + 1].cpu().numpy()
    sl = w.seq_len[b0:b0 + 1].cpu().numpy().astype(np.int32)
    meta = oracle.meta_batch(K, sl, w.block)
    H = w.H
    if w.W is not None:
        Wn = w.W.cpu().numpy()
        tau0, _ = oracle.predict_tau(q, Wn, np.zeros(H, np.float32))
        c, _ = oracle.calibrate(q[None], sl, w.block, w.cap, meta, tau0=tau0[None], z=w.z,
                                scale=w.scale, rho=float(np.float32(rho)))
    else:
        Wn = None
        c, _ = oracle.calibrate(w.q_cal[:, b0:b0 + 1].cpu().numpy(), sl, w.block, w.cap, meta,
                                z=w.z, scale=w.scale, rho=float(np.float32(rho)))
    c = c.astype(np.float32)
    reps, t = 0, 0.0
    dens = 0.0
    while t < 10.0 and reps < 10000:
        a = time.perf_counter()
        r = oracle.step_batch(q, K, V, sl, w.block, meta, Wn, c, z=w.z, scale=w.scale)
        t += time.perf_counter() - a
        reps += 1
        dens = float(r["tokens"].sum()) / (H * int(sl.sum()))
    per = t / reps
    lib = oracle.load()
    cores = int(lib.eta_oracle_threads())
    # the same sample on one thread, for about 3 s
    lib.eta_oracle_set_threads(1)
    reps1, t1 = 0, 0.0
    while t1 < 3.0 and reps1 < 1000:
        a = time.perf_counter()
        oracle.step_batch(q, K, V, sl, w.block, meta, Wn, c, z=w.z, scale=w.scale)
        t1 += time.perf_counter() - a
        reps1 += 1
    lib.eta_oracle_set_threads(cores)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(int(sl.sum()) / per, 1), "unit": "tokens/s",
            "cores": cores, "kind": "oracle",
            "value_1thread": round(int(sl.sum()) / (t1 / reps1), 1),
            "host": {"nproc": os.cpu_count(), "model": model},
            "sample": f"sequence {b0} of the workload ({H} heads x {int(sl.sum())} keys), "
                      f"{reps} repetitions of threshold+screen+attention on {cores} threads "
                      f"({per * 1e3:.1f} ms each) and {reps1} on one thread "
                      f"({t1 / reps1 * 1e3:.1f} ms each), density {dens:.3f}"}


if __name__ == "__main__":
    main()
