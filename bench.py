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
`configs` section times the other decode workloads the same way (512K single
sequence, the ragged batch of 32 with frozen calibrated thresholds, 32K
single sequence), each with its dense decode, speedup, ideal speedup and
roofline.  A grouped-query section follows (32 sequences x 128K, 32 query heads on 4 KV
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
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_counters.json")
PREFILL_SRC = [os.path.join(CSRC, f) for f in ("kernels_prefill.hip", "eta_api.hip",
                                                "eta_internal.h")]
# Vector-ALU issue ceiling of the chip: the fp32 vector peak (157.3 TFLOP/s,
# 256 CUs x 4 SIMDs at 2.4 GHz) is 78.6e12 FMA lane-ops/s, i.e. 1.229e12
# wave64 instructions per second (one every 2 cycles per SIMD).  A
# transcendental (v_exp_f32, v_rcp_f32) is charged TRANS_SLOTS issue slots:
# in long independent chains on every SIMD, counted against GRBM_GUI_ACTIVE,
# an exp or a reciprocal took about 9.5 cycles per wave64 instruction where
# a multiply or FMA took about 2.6.
VALU_WAVE_INSTR_PER_S = 157.3e12 / 2 / 64
TRANS_SLOTS = 4


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
    ap.add_argument("--path", choices=("split", "fused", "auto"), default="split",
                    help="decode path of the --workload step (the configs section always "
                         "takes the Decoder's automatic choice)")
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
    ap.add_argument("--gqa-dim", type=int, default=64, choices=(64, 128),
                    help="head dim of the --gqa-only run (and of its counter summary)")
    ap.add_argument("--gqa-rho", default="0.38,0.25,0.10",
                    help="head densities of the grouped-query section")
    ap.add_argument("--configs", default="ctx512k,ragged,ctx32k",
                    help="other decode workloads timed after the headline one ('none': skip)")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--summarize-prefill-counters", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV",
                             "SQ_CSV"),
                    help="turn rocprofv3 counter csv files of a --prefill-only run (FETCH_SIZE, "
                         "WRITE_SIZE, the 1 GiB copy's FETCH_SIZE and WRITE_SIZE, and a pass "
                         "with SQ_INSTS_VALU, SQ_INSTS_VALU_TRANS_F32, SQ_INSTS_MFMA, "
                         "SQ_VALU_MFMA_BUSY_CYCLES) into profiles/prefill_counters.json")
    ap.add_argument("--summarize-counters", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and "
                         "WRITE_SIZE of a bench run, then of --copy-reference 1024) into the "
                         "per-launch HBM bytes of --workload's decode call, stored in "
                         "profiles/decode_counters.json (or gqa_decode_counters.json with "
                         "--gqa-only) with the hash of the kernel sources")
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


def graph_call_ms(torch, fn, steps, warmup, flush=None):
    """Mean duration of one call of `fn` (one or more kernel launches) on the
    current stream (the stream the library launches on).  Without `flush`:
    the call captured alone in a HIP graph and replayed `steps` times back to
    back between two HIP events, so no host launch gap enters the figure.
    With `flush` (a cache that could sit in the 256 MB last-level cache): the
    buffer is overwritten before every call and events bracket each call
    alone (the host has queued the call while the flush runs)."""
    if flush is not None:
        for _ in range(warmup):
            fn()
        pairs = []
        for _ in range(steps):
            flush.fill_(1.0)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            pairs.append((s, e))
        torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in pairs) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / steps


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
    on the same kernel sources (and this workload)."""
    if not os.path.exists(path):
        return None
    cj = json.load(open(path))
    if cj.get("kernel_hash") != kernel_hash(files):
        return None
    return cj.get("workloads", {}).get(workload, {}).get("hbm_bytes_per_launch")


def _counter_rows(path):
    """(kernel name, counter, value per dispatch) rows of a rocprofv3
    counter_collection.csv, summed per dispatch."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(k[1], k[2], v) for k, v in per.items()]


def summarize_prefill_counters(args):
    """Per-launch HBM bytes and vector/matrix instruction counts of the
    prefill kernel, stored with the hash of its sources."""
    fetch, write, cfetch, cwrite, sq = args.summarize_prefill_counters
    ref_bytes = 1 << 30

    def mean_of(rows, counter, pred):
        vals = [v for k, c, v in rows if c == counter and pred(k)]
        return sum(vals) / len(vals) if vals else 0.0

    is_copy = lambda k: "copyBuffer" in k or "copy" in k.lower()
    is_pf = lambda k: "prefill_kernel" in k
    f_factor = ref_bytes / (mean_of(_counter_rows(cfetch), "FETCH_SIZE", is_copy) * 1024.0)
    w_factor = ref_bytes / (mean_of(_counter_rows(cwrite), "WRITE_SIZE", is_copy) * 1024.0)
    f = mean_of(_counter_rows(fetch), "FETCH_SIZE", is_pf)
    w = mean_of(_counter_rows(write), "WRITE_SIZE", is_pf)
    sqrows = _counter_rows(sq)
    per = {c: mean_of(sqrows, c, is_pf) for c in
           ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU")}
    cj = {"kernel_hash": kernel_hash(PREFILL_SRC), "workload": "prefill",
          "fetch_factor": f_factor, "write_factor": w_factor,
          "fetch_kib": f, "write_kib": w,
          "hbm_bytes_per_launch": int(round(f * 1024.0 * f_factor + w * 1024.0 * w_factor)),
          "per_dispatch": {k: int(round(v)) for k, v in per.items()}}
    with open(PREFILL_COUNTERS, "w") as fh:
        json.dump(cj, fh, indent=1)
    print(json.dumps(cj, indent=1))


def summarize_counters(args):
    """Per-launch HBM bytes of the decode call of one workload from four
    counter runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of a bench run,
    each scaled by what the same counter reads for a plain 1 GiB device copy."""
    fetch, write, cfetch, cwrite = args.summarize_counters
    ref_bytes = 1 << 30

    def mean_of(rows, counter, pred):
        vals = [v for k, c, v in rows if c == counter and pred(k)]
        return sum(vals) / len(vals) if vals else 0.0, len(vals)

    is_copy = lambda k: "copyBuffer" in k or "copy" in k.lower()
    cf, _ = mean_of(_counter_rows(cfetch), "FETCH_SIZE", is_copy)
    cw, _ = mean_of(_counter_rows(cwrite), "WRITE_SIZE", is_copy)
    f_factor = ref_bytes / (cf * 1024.0)
    w_factor = ref_bytes / (cw * 1024.0)
    gqa = args.gqa_only
    frows, wrows = _counter_rows(fetch), _counter_rows(write)
    # The fused step's call is its fused kernel plus a combine whose partial
    # traffic (one (d+2)-float partial per chunk) is under 0.2% of it and is
    # shared by name with the dense baseline's combine, so it is left out.
    fused = any("screen_decode_kernel" in k for k, c, v in frows)
    parts = (("decode_gqa_flow_kernel", "combine_gqa_flow_kernel") if gqa else
             ("screen_decode_kernel",) if fused else
             ("decode_flow_kernel", "combine_flow_kernel"))
    table = []
    total = 0.0
    for kname in sorted({k for k, c, v in frows} | {k for k, c, v in wrows}):
        short = kname.split("(")[0].replace("void ", "")
        f, nf = mean_of(frows, "FETCH_SIZE", lambda k: k == kname)
        w, nw = mean_of(wrows, "WRITE_SIZE", lambda k: k == kname)
        rd, wr = f * 1024.0 * f_factor, w * 1024.0 * w_factor
        table.append((short, max(nf, nw), f, w, rd, wr))
        # the sparse decode call: balanced decode + combine, not the dense
        # baseline's decode (template arguments ending in `true`).  The grouped
        # dense baseline shares the combine kernel, so that row averages both.
        if any(short.startswith(f"eta::{p}<") for p in parts) and not short.endswith("true>"):
            total += rd + wr
    # the grouped workload is named by the head dim its decode kernel was built for
    gqa_d128 = gqa and any(k.startswith("void eta::decode_gqa_flow_kernel<128,")
                           for k, c, v in frows)
    workload = (("gqa128k_d128" if gqa_d128 else "gqa128k") if gqa
                else args.workload + ("_fused" if fused else ""))
    path = GQA_COUNTERS if gqa else COUNTERS
    cj = json.load(open(path)) if os.path.exists(path) else {}
    files = GQA_SRC if gqa else DECODE_SRC
    if cj.get("kernel_hash") != kernel_hash(files):
        cj = {}
    cj["kernel_hash"] = kernel_hash(files)
    cj["fetch_factor"], cj["write_factor"] = f_factor, w_factor
    cj.setdefault("workloads", {})[workload] = {
        "hbm_bytes_per_launch": int(round(total)),
        "note": f"{' + '.join(parts)} per "
                f"{'eta_decode_gqa' if gqa else 'eta_fused_step' if fused else 'eta_decode'} "
                "call; FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB device copy"}
    with open(path, "w") as f:
        json.dump(cj, f, indent=1)
    print(f"copy reference: FETCH_SIZE x {f_factor:.4f}, WRITE_SIZE x {w_factor:.4f}")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | "
          "scaled write MB |")
    print("|---|---|---|---|---|---|")
    for short, n, f, w, rd, wr in table:
        print(f"| `{short}` | {n} | {f:.1f} | {w:.1f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
    print(f"decode call ({workload}): {total / 1e9:.4f} GB of HBM traffic per call "
          f"(kernel hash {cj['kernel_hash']})")
class DecodeBench:
    """One decode workload resident on the GPU: cache, statistics, per-head
    constants from the library's calibration for each target density, and the
    step (threshold, screen, decode) timed eagerly per kernel and as a HIP
    graph, beside the in-house dense decode at the same shape."""

    def __init__(self, torch, np, eb, synth, name, seed, split=0, cap_extra_blocks=0,
                 path="split"):
        self.torch, self.np, self.eb, self.name = torch, np, eb, name
        dev = "cuda"
        t0 = time.time()
        blk = synth.CONFIGS[name]["block"]
        Tmax = synth.CONFIGS[name]["T"]
        Tmax = Tmax[1] if isinstance(Tmax, tuple) else Tmax
        w = synth.make(name, seed=seed, device=dev, cap=Tmax + cap_extra_blocks * blk)
        self.w = w
        B, H, D, bs = w.B, w.H, w.D, w.block
        self.cache = eb.KVCache(B, H, D, bs, w.cap, w.kv_dtype, device=dev, k=w.k, v=w.v)
        self.cache.seq_len.copy_(w.seq_len)
        eb.build_block_meta(self.cache)
        self.sl = w.seq_len.cpu().numpy().astype(np.int64)
        self.sumT = int(self.sl.sum())
        self.dec = eb.Decoder(self.cache, z=w.z, scale=w.scale, blocks_per_split=split or None,
                              path=path)
        self.split = self.dec.split
        self.fused = self.dec.path == "fused"
        self.frozen = w.W is None
        self.elt = 2 if w.kv_dtype == torch.bfloat16 else 4
        self.consts = {}
        kv_bytes = 2 * w.k.numel() * w.k.element_size()
        # a cache that could sit in the 256 MB last-level cache is flushed
        # (512 MiB written) before every step of the latency distribution
        self.flush = (torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
                      if kv_bytes < (2 << 30) else None)
        nbc = self.sl // bs
        # block index bytes the screen reads: mu, var (bf16) and maxnorm (fp32)
        self.meta_bytes = int(H * (nbc * (2 * D * 2 + 4)).sum())
        self.dense_bytes = self.sumT * H * D * 2 * self.elt
        print(f"[bench] workload {name}: B={B} H={H} D={D} b={bs} sumT={self.sumT} "
              f"path={self.dec.path} split={self.split} chunk={self.dec.fused_chunk} "
              f"dense split={self.dec.dense_split} "
              f"({time.time() - t0:.1f}s setup)", file=sys.stderr, flush=True)

    def calibrate(self, rhos):
        """Per-head constants for each target density (eta_calibrate_threshold;
        dynamic thresholds pool score - qbar W over the timed query, frozen
        ones pool the workload's calibration queries)."""
        torch, eb, w = self.torch, self.eb, self.w
        B, H = w.B, w.H
        if not self.frozen:
            tau0 = torch.zeros((B, H), device="cuda")
            tmp = torch.zeros_like(tau0)
            eb.predict_tau(w.q, w.W, torch.zeros(H, device="cuda"), 0.0, tau0, tmp)
            qs, t0s = w.q[None].contiguous(), tau0[None].contiguous()
        else:
            qs, t0s = w.q_cal.contiguous(), None
        cws = eb.workspace(eb.calibrate_workspace_bytes(qs.shape[0], B, H,
                                                        self.cache.cap_blocks))
        for rho in rhos:
            c = torch.zeros(H, device="cuda")
            eb.calibrate_threshold(self.cache, qs, t0s, w.z, w.scale, rho, cws, c)
            self.consts[rho] = c
        del cws
        torch.cuda.synchronize()

    def run(self, rho, steps, warmup):
        """Eager steps timed per kernel with HIP events, then the same step
        captured once in a HIP graph (checked bit for bit against the eager
        output) and timed over `steps` replays."""
        torch, np, w, dec = self.torch, self.np, self.w, self.dec
        c = self.consts[rho]
        W = w.W
        if self.frozen:  # no predictor in the timed step: tau is the constants
            dec.predict(w.q, None, c)

        # The timed call: eta_decode (balanced decode + combine) on the split
        # path, eta_fused_step (threshold, screen and decode, then the
        # combine) on the fused one, which is then the whole step.
        if self.fused:
            call = lambda: dec.step_fused(w.q, None if self.frozen else W, c)
        else:
            call = lambda: dec.attend(w.q)

        def step():
            if not self.fused:
                if not self.frozen:
                    dec.predict(w.q, W, c)
                dec.screen(w.q)
            call()

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ctr0 = int(dec.density_ctr.item())
        tdec, tscr = Timer(torch), Timer(torch)
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(steps):
            if not self.fused:
                if not self.frozen:
                    dec.predict(w.q, W, c)
                tscr.around(lambda: dec.screen(w.q))
            tdec.around(call)
        torch.cuda.synchronize()
        eager = time.perf_counter() - a
        toks = (int(dec.density_ctr.item()) - ctr0) // steps
        per_step = []
        for _ in range(steps):
            if self.flush is not None:
                self.flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            per_step.append((e0, e1))
        torch.cuda.synchronize()
        lat = sorted(s0.elapsed_time(s1) for s0, s1 in per_step)
        if self.fused:  # admitted blocks per stream from the chunk bits
            bits = dec.chunk_bits.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
            nbs = -(-self.sl // w.block)
            live = (np.arange(bits.shape[2])[None, :] * dec.fused_chunk) < nbs[:, None]
            bits = np.where(live[:, None, :], bits, 0)
            cnt = np.zeros(bits.shape[:2], np.int64)
            for i in range(dec.fused_chunk):
                cnt += ((bits >> i) & 1).sum(axis=2)
        else:
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
        # The decode call (balanced decode + combine kernels) and the screen
        # call (screen + compaction), each replayed alone as a graph.
        decode_ms = graph_call_ms(torch, call, steps, warmup, self.flush)
        screen_ms = (None if self.fused else
                     graph_call_ms(torch, lambda: dec.screen(w.q), steps, warmup, self.flush))
        pct = lambda f: lat[min(len(lat) - 1, int(f * (len(lat) - 1) + 0.5))]
        r = dict(ms=wall * 1e3 / steps, eager_ms=eager * 1e3 / steps,
                 step_ms_median=pct(0.5), step_ms_p10=pct(0.1), step_ms_p90=pct(0.9),
                 decode_ms=decode_ms, screen_ms=screen_ms,
                 eager_decode_ms=tdec.mean_ms(),
                 eager_screen_ms=None if self.fused else tscr.mean_ms(),
                 density=toks / (w.H * self.sumT), tokens=toks, cnt=cnt)
        r["decode_bytes"] = self.decode_bytes(r)
        r["step_bytes"] = self.step_bytes(r)
        scr = "fused" if screen_ms is None else f"{screen_ms:.4f}"
        print(f"[bench] {self.name} rho={rho:.2f} ({dec.path}): density {r['density']:.4f} step "
              f"{r['ms']:.4f} ms (eager {r['eager_ms']:.4f}; screen {scr}, "
              f"decode {r['decode_ms']:.4f}) {r['step_bytes'] / r['ms'] / 1e6:.0f} GB/s",
              file=sys.stderr, flush=True)
        return r

    def run_dense(self, steps, warmup):
        """The in-house dense decode at the same shape, captured in a HIP graph
        like the sparse step."""
        torch, dec, w = self.torch, self.dec, self.w
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
        ms = (time.perf_counter() - a) * 1e3 / steps
        print(f"[bench] {self.name} dense: {ms:.4f} ms ({self.dense_bytes / ms / 1e6:.0f} GB/s)",
              file=sys.stderr, flush=True)
        return ms

    def decode_bytes(self, r):
        """Algorithmic bytes of the timed call.  eta_decode: admitted K+V, q,
        the active lists, partials (m, l, acc) written and read for streams
        split over several ranges, output.  eta_fused_step: the predictor
        weights (dynamic thresholds), the block statistics, admitted K+V, q,
        the thresholds written, one partial per chunk of a stream with several
        chunks (written and read), the chunk bits, output."""
        np, w = self.np, self.w
        B, H, D = w.B, w.H, w.D
        if self.fused:
            nb = -(-self.sl // w.block)
            nch = -(-nb // self.dec.fused_chunk)  # chunks per stream of each sequence
            part = int(H * (np.where(nch > 1, nch, 0) * (D + 2) * 4 * 2).sum())
            weights = 0 if self.frozen else H * D * H * 4 + H * 4
            return (weights + self.meta_bytes + r["tokens"] * D * 2 * self.elt +
                    B * H * D * 4 * 2 + 2 * B * H * 4 + int(H * nch.sum()) * 4 + part)
        chunks = -(-r["cnt"] // self.split)
        part = int((np.where(chunks > 1, chunks, 0) * (D + 2) * 4 * 2).sum())
        return (r["tokens"] * D * 2 * self.elt + B * H * D * 4 * 2 + int(r["cnt"].sum()) * 4 +
                part)

    def step_bytes(self, r):
        w = self.w
        B, H, D = w.B, w.H, w.D
        if self.fused:  # the fused call is the whole step
            return r["decode_bytes"]
        pred = 0 if self.frozen else B * H * D * 4 + H * D * H * 4 + 2 * B * H * 4
        screen = self.meta_bytes + B * H * D * 4 + int(r["cnt"].sum()) * 4 + B * H * 4
        return pred + screen + r["decode_bytes"]

    def roofline(self, r, dense_ms):
        achieved = r["decode_bytes"] / (r["decode_ms"] * 1e-3) / 1e9
        stream_gbs = self.dense_bytes / dense_ms / 1e6
        kernel = ("eta_fused_step (fused threshold + screen + decode, combine kernels)" if self.fused
                  else "eta_decode (balanced decode + combine kernels)")
        return {"bound": "hbm", "kernel": kernel,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counters_traffic(COUNTERS, DECODE_SRC,
                                            self.name + ("_fused" if self.fused else "")),
                "algorithmic_bytes_per_launch": int(r["decode_bytes"]),
                "avg_launch_ms": round(r["decode_ms"], 5),
                "measured_stream_gbs": round(stream_gbs, 1),
                "frac_of_measured_stream": round(achieved / stream_gbs, 4)}

    def summary(self, r, dense_ms):
        return {"density": round(r["density"], 4), "ms": round(r["ms"], 5),
                "eager_ms": round(r["eager_ms"], 5),
                "tokens_per_s": round(self.sumT / (r["ms"] * 1e-3), 1),
                "step_gbs": round(r["step_bytes"] / r["ms"] / 1e6, 1),
                "decode_gbs": round(r["decode_bytes"] / r["decode_ms"] / 1e6, 1),
                "screen_ms": None if r["screen_ms"] is None else round(r["screen_ms"], 5),
                "path": self.dec.path,
                "decode_ms": round(r["decode_ms"], 5),
                "speedup_vs_dense": round(dense_ms / r["ms"], 3),
                "ideal_speedup": round(self.dense_bytes / r["step_bytes"], 3)}

    def describe(self, rho):
        w, sl = self.w, self.sl
        return (f"{self.name}: batch {w.B}, {w.H} heads, head dim {w.D}, context "
                f"{int(sl.min()) if sl.min() != sl.max() else int(sl.max())}"
                f"{'..' + str(int(sl.max())) if sl.min() != sl.max() else ''} "
                f"(sum {self.sumT}), block {w.block}, z {w.z}, "
                f"{'bf16' if self.elt == 2 else 'fp32'} KV, "
                f"{'frozen calibrated' if self.frozen else 'dynamic linear'} tau at "
                f"{rho:.0%} target density")

    def release(self):
        self.dec = self.cache = self.w = self.flush = None
        self.consts = {}
        self.torch.cuda.empty_cache()


def config_bench(torch, np, eb, synth, name, steps, warmup, seed):
    """One more decode workload at its target density: the step, the dense
    decode, speedup against the ideal (the ratio of algorithmic bytes) and the
    decode call's roofline."""
    target = synth.CONFIGS[name].get("rho", 0.38)
    rho = target if isinstance(target, float) else 0.38
    b = DecodeBench(torch, np, eb, synth, name, seed, path="auto")
    b.calibrate([rho])
    r = b.run(rho, steps, warmup)
    dense_ms = b.run_dense(steps, warmup)
    out = {"workload": b.describe(rho), **b.summary(r, dense_ms),
           "dense_ms": round(dense_ms, 5), "blocks_per_split": b.split,
           "blocks_per_chunk": b.dec.fused_chunk if b.fused else None,
           "dense_blocks_per_split": b.dec.dense_split,
           "step_ms_median": round(r["step_ms_median"], 5),
           "step_ms_p10": round(r["step_ms_p10"], 5), "step_ms_p90": round(r["step_ms_p90"], 5),
           "llc_flushed": b.flush is not None,
           "roofline": b.roofline(r, dense_ms)}
    if b.fused:  # the split path on the same cache and constants, for reference
        fused_dec = b.dec
        b.dec = eb.Decoder(b.cache, z=b.w.z, scale=b.w.scale, path="split")
        b.split, b.fused = b.dec.split, False
        rs = b.run(rho, steps, warmup)
        out["split_path"] = {"ms": round(rs["ms"], 5), "decode_ms": round(rs["decode_ms"], 5),
                             "screen_ms": round(rs["screen_ms"], 5),
                             "speedup_vs_dense": round(dense_ms / rs["ms"], 3),
                             "blocks_per_split": b.split}
        b.dec = fused_dec
    b.release()
    return out


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_prefill_counters:
        summarize_prefill_counters(args)
        return
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
    torch.cuda.set_device(0)
    gqa_rhos = [float(x) for x in args.gqa_rho.split(",")]
    if args.prefill_only:
        print(json.dumps(prefill_bench(torch, eb, synth, args.steps, args.warmup, args.seed)),
              flush=True)
        return
    if args.gqa_only:
        print(json.dumps(gqa_bench(torch, np, eb, synth, args.steps, args.warmup, args.seed,
                                   gqa_rhos, D=args.gqa_dim)), flush=True)
        return
    # room for the appends of the upkeep measurement (4 blocks per stream)
    hb = DecodeBench(torch, np, eb, synth, args.workload, args.seed, split=args.split,
                     cap_extra_blocks=4, path=args.path)
    w, dec, sumT = hb.w, hb.dec, hb.sumT
    B, H, D, bs = w.B, w.H, w.D, w.block
    rhos = sorted(set([args.rho] + ([] if args.no_sweep else [0.10, 0.38, 0.70, 1.0])))
    hb.calibrate(rhos)

    sweep = {rho: hb.run(rho, args.steps, args.warmup) for rho in rhos}
    dense_ms = hb.run_dense(args.steps, args.warmup)

    # Headline run: exactly `steps` timed steps at the headline density.
    r = hb.run(args.rho, args.steps, args.warmup)
    value = sumT / (r["ms"] * 1e-3)
    roofline = hb.roofline(r, dense_ms)

    offsets = None if args.no_sweep else offset_sweep(torch, np, eb, w, dec, hb.consts[args.rho],
                                                       hb.frozen, sumT, args.steps, args.warmup)
    upkeep = measure_upkeep(torch, eb, w, hb.cache, dec, hb.consts[args.rho], hb.frozen, sumT)
    print(f"[bench] upkeep: {json.dumps(upkeep)}", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_baseline(w, hb.consts[args.rho], args.rho)
    describe = hb.describe(args.rho)
    elt, sl, split, dense_split = hb.elt, hb.sl, hb.split, dec.dense_split
    llc_flushed = hb.flush is not None
    sweep_out = {f"{k:.2f}": hb.summary(v, dense_ms) for k, v in sweep.items()}
    hb.release()
    del w, dec

    configs = {}
    if args.configs != "none":
        for name in [x for x in args.configs.split(",") if x and x != args.workload]:
            configs[name] = config_bench(torch, np, eb, synth, name, args.steps, args.warmup,
                                         args.seed)
    gqa = gqa_d128 = None
    if not args.no_gqa:
        gqa = gqa_bench(torch, np, eb, synth, args.steps, args.warmup, args.seed, gqa_rhos)
        # the same grouped batch at head dim 128, at the 38% head density
        gqa_d128 = gqa_bench(torch, np, eb, synth, args.steps, args.warmup, args.seed, (0.38,),
                             D=128)
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
                          "llc_flushed": llc_flushed},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": describe,
            "global_batch": B, "seq_len": int(sl.max()), "parallelism": "single GPU",
            "kv_dtype": "bf16" if elt == 2 else "f32", "blocks_per_split": split,
            "dense_blocks_per_split": dense_split,
        },
        "density": round(r["density"], 4),
        "step_hbm_gbs": round(r["step_bytes"] / r["ms"] / 1e6, 1),
        "step_roofline_frac": round(r["step_bytes"] / r["ms"] / 1e6 / HBM_PEAK_GBS, 4),
        "dense_ms": round(dense_ms, 5),
        "speedup_vs_dense": round(dense_ms / r["ms"], 3),
        "ideal_speedup": round(hb.dense_bytes / r["step_bytes"], 3),
        "sweep": sweep_out,
        "roofline": roofline,
        "configs": configs,
        "offset_sweep": offsets,
        "upkeep": upkeep,
        "cpu_baseline": cpu,
        "gqa": gqa,
        "gqa_d128": gqa_d128,
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
    meta_bytes = sumT * H * D * elt + (sumT // bs) * H * (2 * D * 2 + 4)

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


def gqa_bench(torch, np, eb, synth, steps, warmup, seed, rhos=(0.38, 0.25, 0.10), D=None):
    """Grouped-query decode at the pages' benchmark shape (32 sequences x
    128K, 32 query heads on 4 KV heads, d 64, b 64, bf16; D overrides the
    head dim): dynamic Eq. 1 thresholds over the query heads with constants
    calibrated per query head (the library's calibration, one call per head
    position in the group) to 38%, 25% and 10% head density; step = predict +
    screen_gqa + decode_gqa, graph-captured; the grouped dense decode at the
    same shape alongside.  Decode bytes: union K+V rows, q, head masks and
    union lists, chunk partials, outputs."""
    dev = "cuda"
    w = synth.make("gqa128k", seed=seed, device=dev, D=D)
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
        decode_ms = graph_call_ms(torch, lambda: dec.attend(w.q), steps, warmup)
        screen_ms = graph_call_ms(torch, lambda: dec.screen(w.q), steps, warmup)
        union_tok = int(ctr[1])
        chunks = -(-ucnt // dec.split)
        part = int((np.where(chunks > 1, chunks, 0) * G * (D + 2) * 4 * 2).sum())
        dbytes = union_tok * D * 2 * 2 + 2 * B * Hq * D * 4 + int(ucnt.sum()) * 8 + part
        res[f"{rho:.2f}"] = {
            "decode_bytes": int(dbytes),
            "d_head": round(int(ctr[0]) / (sumT * Hq), 4),
            "d_union": round(union_tok / (sumT * Hkv), 4),
            "ms": round(ms, 5), "screen_ms": round(screen_ms, 5),
            "decode_ms": round(decode_ms, 5),
            "eager_screen_ms": round(tscr.mean_ms(), 5),
            "eager_decode_ms": round(tdec.mean_ms(), 5),
            "decode_gbs": round(dbytes / decode_ms / 1e6, 1),
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
                    "traffic": counters_traffic(GQA_COUNTERS, GQA_SRC,
                                                "gqa128k" if D in (None, 64) else f"gqa128k_d{D}"),
                    "algorithmic_bytes_per_launch": r["decode_bytes"],
                    "avg_launch_ms": r["decode_ms"],
                    "measured_stream_gbs": round(dense_bytes / dense_ms / 1e6, 1),
                    "frac_of_measured_stream": round(ach / (dense_bytes / dense_ms / 1e6), 4)}
    name = "gqa128k" if D == 64 else f"gqa128k_d{D}"
    out = {"workload": f"{name}: batch {B}, {Hq} query heads on {Hkv} KV heads, head dim {D}, "
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
    kms = ev.mean_ms()
    tfs = flops / (kms * 1e-3) / 1e12
    # Counter summary of the same kernel sources (instruction counts and HBM
    # bytes per launch), if present.
    cj = None
    if os.path.exists(PREFILL_COUNTERS):
        cj = json.load(open(PREFILL_COUNTERS))
        if cj.get("kernel_hash") != kernel_hash(PREFILL_SRC):
            cj = None
    alu = None
    if cj is not None:
        pd = cj["per_dispatch"]
        slots = pd["SQ_INSTS_VALU"] + (TRANS_SLOTS - 1) * pd["SQ_INSTS_VALU_TRANS_F32"]
        rate = slots / (kms * 1e-3)
        alu = {"bound": "alu", "achieved": float(f"{rate:.4g}"),
               "peak": float(f"{VALU_WAVE_INSTR_PER_S:.4g}"),
               "unit": f"wave64 VALU issue slots/s (a transcendental counts {TRANS_SLOTS})",
               "frac": round(rate / VALU_WAVE_INSTR_PER_S, 4),
               "valu_instructions_per_launch": pd["SQ_INSTS_VALU"],
               "transcendental_per_launch": pd["SQ_INSTS_VALU_TRANS_F32"],
               "mfma_instructions_per_launch": pd["SQ_INSTS_MFMA"],
               "mfma_busy_frac": round(pd["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 /
                                       (kms * 1e-3 * 2.4e9), 4)}
    res = {"workload": f"prefill: batch {w.B}, {w.Hq} query heads on {w.H} KV heads, head dim "
                       f"{w.D}, context {w.T}, bf16 q/k/v, beta 5",
           "ms": round(ms, 5), "kernel_ms": round(kms, 5),
           "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
           "mean_density": round(float(dens.mean()), 4),
           "roofline": {"bound": "mfma", "achieved": round(tfs, 1),
                        "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                        "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                        "traffic": None if cj is None else cj["hbm_bytes_per_launch"],
                        "algorithmic_flops_per_launch": int(flops),
                        "algorithmic_bytes_per_launch": int(
                            w.q.numel() * 2 + (w.k.numel() + w.v.numel()) * 2 +
                            w.tau.numel() * 4 + out.numel() * 4 + dens.numel() * 4),
                        "avg_launch_ms": round(kms, 5)},
           "alu_roofline": alu}
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
    meta = oracle.index_batch(K, sl, w.block)
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
