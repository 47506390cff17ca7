"""GPU parity of eta_gated_prefill (gated causal attention forward, Eqs. 2-3,
and the Eq. 4 per-row density) against the oracle's prefill.

Outputs: bf16 bar (2e-2 relative per (sequence, head) row block) and, in
addition, 1e-4 relative: the score product is exact in float32 from bf16
inputs and the softmax weights are split hi + lo, so the kernel's own
accuracy is float32-level.  Densities: 2e-6 absolute (a mean of gates in
[0, 1] summed in float32).  Cases: lengths around the 64-query and 32-key
tiles, d in {64, 128}, grouped and ungrouped heads, tau = +-inf, the full
training shape (8 x 2048, 32 query / 4 KV heads, d 64) on sampled heads, and
run-to-run determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_decode_eta_amd import binding as eb
from long_context_decode_eta_amd import synth
from parity import note

pytestmark = pytest.mark.gpu
OUT_BAR, OUT_TOL, DENS_TOL = 2e-2, 1e-4, 2e-6


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.name}")


def run_gpu(w, tau=None, beta=5.0):
    tau = w.tau if tau is None else tau
    out = torch.zeros((w.B, w.Hq, w.T, w.D), device="cuda")
    dens = torch.zeros((w.B, w.Hq, w.T), device="cuda")
    eb.gated_prefill(w.q.cuda(), w.k.cuda(), w.v.cuda(), tau.cuda(), w.G, beta, w.scale, out,
                     dens)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dens.cpu().numpy()


def compare(g_out, g_dens, o_out, o_dens):
    worst = 0.0
    B, H = g_out.shape[:2]
    for b in range(B):
        for h in range(H):
            den = np.abs(o_out[b, h]).max()
            err = np.abs(g_out[b, h] - o_out[b, h]).max() / den
            assert err <= OUT_BAR, (b, h, err)
            worst = max(worst, err)
    assert worst <= OUT_TOL, worst
    derr = np.abs(g_dens - o_dens).max()
    assert derr <= DENS_TOL, derr
    return worst, derr


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8, 16])
@pytest.mark.parametrize("T", [1, 31, 63, 64, 65, 127, 128, 129, 200])
def test_prefill_small(D, G, T):
    w = synth.make_prefill(seed=T + G + D, B=2, H=2, G=G, D=D, T=T)
    g_out, g_dens = run_gpu(w)
    o_out, o_dens = oracle.prefill(synth.kv_numpy(w.q), synth.kv_numpy(w.k),
                                   synth.kv_numpy(w.v), w.tau.numpy(), G, beta=5.0,
                                   scale=w.scale)
    worst, derr = compare(g_out, g_dens, o_out, o_dens)
    note(f"  out rel {worst:.2e}, dens abs {derr:.2e}, mean dens {o_dens.mean():.3f}")


@pytest.mark.parametrize("beta", [0.25, 50.0])
def test_prefill_gate_steepness(beta):
    w = synth.make_prefill(seed=31, B=2, H=2, G=4, D=64, T=150)
    g_out, g_dens = run_gpu(w, beta=beta)
    o_out, o_dens = oracle.prefill(synth.kv_numpy(w.q), synth.kv_numpy(w.k),
                                   synth.kv_numpy(w.v), w.tau.numpy(), 4, beta=beta,
                                   scale=w.scale)
    worst, derr = compare(g_out, g_dens, o_out, o_dens)
    note(f"  beta {beta}: out rel {worst:.2e}, dens abs {derr:.2e}, mean dens {o_dens.mean():.3f}")


@pytest.mark.parametrize("tau", [math.inf, -math.inf])
def test_prefill_threshold_extremes(tau):
    w = synth.make_prefill(seed=3, B=1, H=2, G=2, D=64, T=150)
    t = torch.full_like(w.tau, tau)
    g_out, g_dens = run_gpu(w, t)
    o_out, o_dens = oracle.prefill(synth.kv_numpy(w.q), synth.kv_numpy(w.k),
                                   synth.kv_numpy(w.v), t.numpy(), w.G, scale=w.scale)
    compare(g_out, g_dens, o_out, o_dens)
    assert np.all(g_dens == (1.0 if tau < 0 else 0.0))


def test_prefill_full_size_sampled_heads():
    # 8 x 2048, 32 query heads on 4 KV heads, d 64: every row of sampled
    # (sequence, query head) pairs against the oracle, the rest for finiteness.
    w = synth.make_prefill(seed=1234, device="cuda")
    out = torch.zeros((w.B, w.Hq, w.T, w.D), device="cuda")
    dens = torch.zeros((w.B, w.Hq, w.T), device="cuda")
    eb.gated_prefill(w.q, w.k, w.v, w.tau, w.G, 5.0, w.scale, out, dens)
    torch.cuda.synchronize()
    worst = 0.0
    for b, h in [(0, 0), (3, 13), (7, 31)]:
        kv = h // w.G
        o_out, o_dens = oracle.prefill(synth.kv_numpy(w.q[b:b + 1, h:h + 1]),
                                       synth.kv_numpy(w.k[b:b + 1, kv:kv + 1]),
                                       synth.kv_numpy(w.v[b:b + 1, kv:kv + 1]),
                                       w.tau[b:b + 1, h:h + 1].cpu().numpy(), 1, scale=w.scale)
        e, _ = compare(out[b:b + 1, h:h + 1].cpu().numpy(), dens[b:b + 1, h:h + 1].cpu().numpy(),
                       o_out, o_dens)
        worst = max(worst, e)
    assert torch.isfinite(out).all() and torch.isfinite(dens).all()
    note(f"  worst out rel {worst:.2e}, mean dens {float(dens.mean()):.3f}")


def test_prefill_deterministic():
    w = synth.make_prefill(seed=5, B=1, H=2, G=4, D=64, T=777)
    a, da = run_gpu(w)
    b, db = run_gpu(w)
    assert np.array_equal(a, b) and np.array_equal(da, db)
