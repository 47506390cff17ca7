"""Seeded synthetic decode workloads (inputs only).

This module draws queries, keys, values and threshold-predictor weights with
the structure described for the decode benchmarks: keys are unit Gaussian
plus a per-block mean vector, a few "needle" blocks are shifted toward the
query, values are unit Gaussian.  It contains none of the method's arithmetic
(no statistics, scores, thresholds or attention): per-head threshold
constants that hit a target density are computed afterwards by a calibration
routine (the library's on the GPU, or the oracle's in tests), from the
``rho`` targets stored here.

Every draw comes from one ``torch.Generator`` seeded per workload, in a fixed
order, on the requested device (CPU draws for small test cases, GPU draws for
full-size ones).  The same tensors feed both the HIP path and the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# Shapes and generator settings of the decode workloads.
CONFIGS = {
    # correctness size; fp32 cache; frozen per-head tau ~ U(0.5, 1.5)
    "tiny": dict(B=1, H=4, D=64, T=2048, block=16, z=1.5, kv="f32", tau="frozen",
                 block_mean="normal", needles=dict(kind="query_mix", count=3, weight=0.8)),
    # 32K single sequence, dynamic tau at 38% density
    "ctx32k": dict(B=1, H=16, D=128, T=32768, block=64, z=1.0, kv="bf16", tau="dynamic",
                   rho=0.38, block_mean="t3", needles=dict(kind="uniform", frac=0.01)),
    # 128K, batch 8, density swept by the tau offset
    "ctx128k": dict(B=8, H=16, D=128, T=131072, block=32, z=1.0, kv="bf16", tau="dynamic",
                    rho=(0.10, 0.38, 0.70, 1.0), block_mean="t3",
                    needles=dict(kind="uniform", frac=(0.002, 0.02))),
    # 512K single sequence: needles in the first and last 1% plus 0.5% scattered
    "ctx512k": dict(B=1, H=16, D=128, T=524288, block=64, z=1.0, kv="bf16", tau="dynamic",
                    rho=0.38, block_mean="t3",
                    needles=dict(kind="ends", per_end=8, end_frac=0.01, frac=0.005)),
    # ragged batch 32, T ~ U{8192..65536}, frozen calibrated tau at 25%
    "ragged": dict(B=32, H=16, D=128, T=(8192, 65536), block=16, z=2.0, kv="bf16",
                   tau="frozen_calibrated", rho=0.25, n_cal_sets=2, block_mean="t3",
                   needles=dict(kind="uniform", frac=0.01)),
    # Grouped-query shapes (32 query heads on 4 KV heads, d=64, b=64).  The
    # queries of a group share a component (correlation q_corr) and a needle
    # block is lifted toward one head of its group, so heads admit different
    # blocks and the union exceeds each head's set.
    "gqa_tiny": dict(B=2, H=2, G=4, D=64, T=(1000, 3000), block=16, z=1.5, kv="bf16",
                     tau="frozen", block_mean="normal", q_corr=0.8,
                     needles=dict(kind="uniform", frac=0.03)),
    # q_corr 0.97 and a predictor at a quarter of the MHA weight scale give
    # union densities of about 54%, 38% and 16% at 38%, 25% and 10% per head.
    "gqa128k": dict(B=32, H=4, G=8, D=64, T=131072, block=64, z=1.0, kv="bf16", tau="dynamic",
                    rho=(0.38, 0.25, 0.10), block_mean="t3", q_corr=0.97, w_scale=0.25,
                    needles=dict(kind="uniform", frac=0.01)),
}

NEEDLE_DELTA = 4.0  # a needle block's mean is lifted by this many logits along q


@dataclass
class Workload:
    name: str
    B: int
    H: int                           # cache (KV) heads
    D: int
    block: int
    cap: int
    z: float
    kv_dtype: torch.dtype
    seq_len: torch.Tensor            # [B] int32
    q: torch.Tensor                  # [B][H*G][D] float32
    k: torch.Tensor                  # [B][H][cap][D]
    v: torch.Tensor                  # [B][H][cap][D]
    tau_kind: str                    # "frozen" | "dynamic" | "frozen_calibrated"
    W: torch.Tensor | None = None    # [H*D][H] block-diagonal predictor (dynamic)
    tau_const: torch.Tensor | None = None  # [H] frozen constants drawn directly (tiny)
    rho: tuple = ()                  # target densities for calibration
    q_cal: torch.Tensor | None = None      # [n][B][H][D] calibration queries
    needle_blocks: list = field(default_factory=list)  # per (b, h): LongTensor of blocks
    G: int = 1                       # query heads per KV head (q holds H*G heads)

    @property
    def cap_blocks(self) -> int:
        return -(-self.cap // self.block)

    @property
    def Hq(self) -> int:
        return self.H * self.G

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))


def _t3(g, shape, device):
    """Student-t with 3 degrees of freedom: N / sqrt(chi2_3 / 3)."""
    n = torch.randn(shape, generator=g, device=device)
    c = torch.randn((3,) + tuple(shape), generator=g, device=device).pow(2).sum(0)
    return n / torch.sqrt(c / 3.0)


def _uniform_int(g, lo, hi, n, device):
    """n integers uniform on [lo, hi] (inclusive)."""
    return torch.randint(lo, hi + 1, (n,), generator=g, device=device)


def _needles(g, spec, nb, device):
    """Block indices of the needle blocks of one (b, h) stream."""
    kind = spec["kind"]
    if kind == "uniform":
        frac = spec["frac"]
        if isinstance(frac, tuple):
            frac = float(frac[0] + (frac[1] - frac[0]) * torch.rand((), generator=g, device=device))
        n = max(1, int(round(frac * nb)))
        return torch.randperm(nb, generator=g, device=device)[:min(n, nb)]
    if kind == "ends":
        edge = max(1, int(round(spec["end_frac"] * nb)))
        per = min(spec["per_end"], edge)
        head = torch.randperm(edge, generator=g, device=device)[:per]
        tail = nb - edge + torch.randperm(edge, generator=g, device=device)[:per]
        n_mid = max(1, int(round(spec["frac"] * nb)))
        mid = torch.randperm(nb, generator=g, device=device)[:n_mid]
        return torch.unique(torch.cat([head, tail, mid]))
    if kind == "query_mix":
        return torch.randperm(nb, generator=g, device=device)[:min(spec["count"], nb)]
    raise ValueError(kind)


def make(name: str, *, seed: int = 1234, device="cpu", T=None, B=None, cap=None, pad="zero",
         block=None, H=None, kv=None, D=None, G=None) -> Workload:
    """Draw the workload `name` (a key of CONFIGS).  T, B, cap, block, H, kv, D
    and G (grouped-query configurations only) override the configuration's sizes for reduced test cases (T: one length,
    a (lo, hi) uniform range, or a list of per-sequence lengths); `pad` fills the
    unused cache slots beyond each T_b with zeros or NaN ("nan").  For a
    grouped-query configuration, H counts KV heads and q, W and the frozen
    constants cover the H*G query heads (query head h*G + g reads KV head h)."""
    cfg = dict(CONFIGS[name])
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    G = cfg.get("G", 1) if G is None else G
    assert G == 1 or "q_corr" in cfg, "G applies to grouped-query configurations"
    D = cfg["D"] if D is None else D
    bs = cfg["block"] if block is None else block
    kvname = cfg["kv"] if kv is None else kv
    kv_dtype = torch.float32 if kvname == "f32" else torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    Tspec = cfg["T"] if T is None else T
    if isinstance(Tspec, list):  # explicit per-sequence lengths
        assert len(Tspec) == B
        lens = torch.tensor(Tspec, dtype=torch.int32, device=device)
        Tmax = max(Tspec)
    elif isinstance(Tspec, tuple):
        lens = _uniform_int(g, Tspec[0], Tspec[1], B, device).to(torch.int32)
        Tmax = Tspec[1]
    else:
        lens = torch.full((B,), int(Tspec), dtype=torch.int32, device=device)
        Tmax = int(Tspec)
    cap = Tmax if cap is None else cap
    assert cap >= int(lens.max())
    nbcap = -(-cap // bs)

    if G == 1:
        q = torch.randn((B, H, D), generator=g, device=device)
    else:
        shared = torch.randn((B, H, 1, D), generator=g, device=device)
        own = torch.randn((B, H, G, D), generator=g, device=device)
        c = cfg["q_corr"]
        q = (math.sqrt(c) * shared + math.sqrt(1.0 - c) * own).reshape(B, H * G, D)
    spec = cfg["needles"]
    k = torch.empty((B, H, cap, D), dtype=kv_dtype, device=device)
    v = torch.empty((B, H, cap, D), dtype=kv_dtype, device=device)
    needle_blocks = []
    for b in range(B):
        Tb = int(lens[b])
        nb = -(-Tb // bs) if Tb > 0 else 0
        if cfg["block_mean"] == "normal":
            mu = 0.5 * torch.randn((H, nbcap, D), generator=g, device=device)
        else:
            mu = 0.5 * _t3(g, (H, nbcap, D), device)
        for h in range(H):
            idx = _needles(g, spec, nb, device) if nb > 0 else torch.zeros(0, dtype=torch.long,
                                                                            device=device)
            needle_blocks.append(idx)
            if spec["kind"] == "query_mix":
                if idx.numel():
                    q[b, h] += spec["weight"] * mu[h, idx].mean(0)
            elif idx.numel() and G == 1:
                qq = q[b, h]
                mu[h, idx] += NEEDLE_DELTA * math.sqrt(D) * qq / qq.dot(qq)
            elif idx.numel():
                # each needle block is lifted toward one query head of the group
                owner = torch.randint(0, G, (idx.numel(),), generator=g, device=device)
                qq = q[b, h * G + owner]                       # [n][D]
                lift = qq / (qq * qq).sum(1, keepdim=True)
                mu[h, idx] += NEEDLE_DELTA * math.sqrt(D) * lift
        kb = torch.randn((H, cap, D), generator=g, device=device)
        kb += mu.repeat_interleave(bs, dim=1)[:, :cap]
        vb = torch.randn((H, cap, D), generator=g, device=device)
        if Tb < cap:
            fill = float("nan") if pad == "nan" else 0.0
            kb[:, Tb:] = fill
            vb[:, Tb:] = fill
        k[b] = kb.to(kv_dtype)
        v[b] = vb.to(kv_dtype)
        del kb, vb, mu

    w = Workload(name=name, B=B, H=H, D=D, block=bs, cap=cap, z=cfg["z"], kv_dtype=kv_dtype,
                 seq_len=lens, q=q, k=k, v=v, tau_kind=cfg["tau"],
                 needle_blocks=needle_blocks, G=G)
    Hq = H * G
    if cfg["tau"] == "frozen":
        w.tau_const = 0.5 + torch.rand((Hq,), generator=g, device=device)
    if cfg["tau"] == "dynamic":
        wh = torch.randn((Hq, D), generator=g, device=device) / math.sqrt(D)
        if "w_scale" in cfg:
            wh *= cfg["w_scale"]
        W = torch.zeros((Hq * D, Hq), device=device)
        for h in range(Hq):
            W[h * D:(h + 1) * D, h] = wh[h]
        w.W = W
    if "rho" in cfg:
        w.rho = cfg["rho"] if isinstance(cfg["rho"], tuple) else (cfg["rho"],)
    if cfg["tau"] == "frozen_calibrated":
        w.q_cal = torch.randn((cfg["n_cal_sets"], B, H, D), generator=g, device=device)
    return w


# ---------------------------------------------------------------------------
# Prefill / training-forward workload: the pages' 1.45B training shape (32
# query heads on 4 KV heads, d 64, context 2048).  Keys are unit Gaussian plus
# a per-64-position mean (Student-t(3) x 0.5); the queries of a group share a
# component; per-position thresholds are drawn directly (tau ~ N(0.5, 0.25^2)
# in logit units), since the gate takes them as given.  All bf16 except tau.
PREFILL = dict(B=8, H=4, G=8, D=64, T=2048, q_corr=0.5, tau_mean=0.5, tau_std=0.25)


@dataclass
class PrefillWorkload:
    B: int
    H: int          # KV heads
    G: int
    D: int
    T: int
    q: torch.Tensor    # [B][H*G][T][D] bf16
    k: torch.Tensor    # [B][H][T][D] bf16
    v: torch.Tensor    # [B][H][T][D] bf16
    tau: torch.Tensor  # [B][H*G][T] float32

    @property
    def Hq(self) -> int:
        return self.H * self.G

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))


def make_prefill(*, seed: int = 1234, device="cpu", B=None, H=None, G=None, D=None,
                 T=None) -> PrefillWorkload:
    cfg = dict(PREFILL)
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    G = cfg["G"] if G is None else G
    D = cfg["D"] if D is None else D
    T = cfg["T"] if T is None else T
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    c = cfg["q_corr"]
    shared = torch.randn((B, H, 1, T, D), generator=g, device=device)
    own = torch.randn((B, H, G, T, D), generator=g, device=device)
    q = (math.sqrt(c) * shared + math.sqrt(1.0 - c) * own).reshape(B, H * G, T, D)
    nblk = -(-T // 64)
    mu = 0.5 * _t3(g, (B, H, nblk, D), device)
    k = torch.randn((B, H, T, D), generator=g, device=device)
    k += mu.repeat_interleave(64, dim=2)[:, :, :T]
    v = torch.randn((B, H, T, D), generator=g, device=device)
    tau = cfg["tau_mean"] + cfg["tau_std"] * torch.randn((B, H * G, T), generator=g,
                                                         device=device)
    return PrefillWorkload(B=B, H=H, G=G, D=D, T=T, q=q.to(torch.bfloat16),
                           k=k.to(torch.bfloat16), v=v.to(torch.bfloat16), tau=tau)


# ---------------------------------------------------------------------------
def kv_numpy(t: torch.Tensor) -> np.ndarray:
    """A cache tensor as the oracle reads it: float32 array, or the raw
    bfloat16 bit patterns as uint16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
