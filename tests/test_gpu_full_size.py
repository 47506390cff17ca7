"""GPU parity at the benchmark sizes, in the launch configuration bench.py
times (the Decoder's automatic blocks_per_split), on sampled (sequence, head)
streams that the oracle recomputes one by one, plus whole-batch properties,
at every admitted density the benchmark reports.

Workloads (seeded, synthetic; shapes of the decode benchmarks):
  ctx32k   batch 1, 16 heads, d 128, T 32768, block 64, z 1, bf16, dynamic tau, 38%
  ctx128k  batch 8, 16 heads, d 128, T 131072, block 32, z 1, bf16, dynamic tau,
           10 / 38 / 70 / 100% (the benchmark's density sweep)
  ctx512k  batch 1, 16 heads, d 128, T 524288, block 64, z 1, bf16, dynamic tau, 38%
  ragged   batch 32, T ~ U{8192..65536}, 16 heads, block 16, z 2, bf16, frozen calibrated 25%
Per-head constants come from the oracle's calibration, pooled over every
sequence for the density sweep (as the benchmark's are) and over a subset of
sequences elsewhere; 100% is the constant -inf for every head.
"""
import math

import numpy as np
import pytest
import torch

from long_context_decode_eta_amd import binding as eb
from long_context_decode_eta_amd import synth
from parity import check_units, make_cache, note, oracle_constants, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.name}")


CASES = {
    # name: (sequences pooled for the constants, sampled streams, target densities)
    "ctx32k": ([0], [(0, 0), (0, 7), (0, 15)], [0.38]),
    "ctx128k": (list(range(8)), [(0, 0), (3, 5), (7, 15)], [0.10, 0.38, 0.70, 1.00]),
    "ctx512k": ([0], [(0, 2), (0, 11)], [0.38]),
    "ragged": ([0, 1, 2, 3], None, [0.25]),
}

_held = {}


def _workload(name):
    """The workload, its cache with statistics and the oracle's constants for
    every density of the case; one workload is held on the GPU at a time."""
    if name not in _held:
        _held.clear()
        torch.cuda.empty_cache()
        seqs, _, rhos = CASES[name]
        w = synth.make(name, seed=1234, device="cuda")
        cache = make_cache(w)
        eb.build_block_meta(cache)
        torch.cuda.synchronize()
        finite = [r for r in rhos if r < 1.0]
        consts = dict(zip(finite, [c for c, _ in oracle_constants(w, finite, seqs=seqs)]))
        if 1.0 in rhos:
            consts[1.0] = torch.full((w.H,), -math.inf)
        _held[name] = (w, cache, consts)
    return _held[name]


@pytest.mark.parametrize("name,rho", [(n, r) for n, (_, _, rs) in CASES.items() for r in rs])
def test_full_size_sampled_streams(name, rho):
    _, units, _ = CASES[name]
    w, cache, consts = _workload(name)
    c = consts[rho].cuda()
    if units is None:  # ragged: shortest, longest and two fixed streams
        sl = w.seq_len.cpu().numpy()
        units = [(int(sl.argmin()), 0), (int(sl.argmax()), 15), (5, 3), (17, 9)]
    g = run_gpu(cache, w.q, W=w.W, bias_or_c=c, z=w.z, scale=w.scale, build_meta=False)
    worst, flips, screened = check_units(w, g, units, W=w.W, bias_or_c=c, z=w.z,
                                         scale=w.scale)
    sl = w.seq_len.cpu().numpy()
    dens = g.density / (int(sl.sum()) * w.H)
    note(f"  target {rho:.2f}: density {dens:.4f}, worst out rel err {worst:.2e}, "
         f"flips {flips}/{screened}")
    if rho == 1.0:
        assert dens == 1.0
    elif name == "ctx128k":  # constants pooled over the whole batch
        assert abs(dens - rho) < 0.01
    else:
        assert abs(dens - rho) < 0.1
    assert not np.isnan(g.out).any()


def test_release_full_size_workloads():
    _held.clear()
    torch.cuda.empty_cache()
