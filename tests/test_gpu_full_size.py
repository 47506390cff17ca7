"""GPU parity at the benchmark sizes, in the launch configuration bench.py
times (the Decoder's automatic blocks_per_split), on sampled (sequence, head) streams
that the oracle recomputes one by one, plus whole-batch properties.

Workloads (seeded, synthetic; shapes of the decode benchmarks):
  ctx32k   batch 1, 16 heads, d 128, T 32768, block 64, z 1, bf16, dynamic tau, 38%
  ctx128k  batch 8, 16 heads, d 128, T 131072, block 32, z 1, bf16, dynamic tau, 38%
  ctx512k  batch 1, 16 heads, d 128, T 524288, block 64, z 1, bf16, dynamic tau, 38%
  ragged   batch 32, T ~ U{8192..65536}, 16 heads, block 16, z 2, bf16, frozen calibrated 25%
Per-head constants come from the oracle's calibration (pooled over a subset of
sequences where the full batch would take the oracle too long).
"""
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
    # name: (sequences pooled for the constants, sampled streams, target density)
    "ctx32k": ([0], [(0, 0), (0, 7), (0, 15)], 0.38),
    "ctx128k": ([0], [(0, 0), (3, 5), (7, 15)], 0.38),
    "ctx512k": ([0], [(0, 2), (0, 11)], 0.38),
    "ragged": ([0, 1, 2, 3], None, 0.25),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_sampled_streams(name):
    seqs, units, rho = CASES[name]
    w = synth.make(name, seed=1234, device="cuda")
    cache = make_cache(w)
    eb.build_block_meta(cache)
    torch.cuda.synchronize()
    c, _ = oracle_constants(w, rho, seqs=seqs)
    c = c.cuda()
    if units is None:  # ragged: shortest, longest and two fixed streams
        sl = w.seq_len.cpu().numpy()
        units = [(int(sl.argmin()), 0), (int(sl.argmax()), 15), (5, 3), (17, 9)]
    g = run_gpu(cache, w.q, W=w.W, bias_or_c=c, z=w.z, scale=w.scale, build_meta=False)
    worst, flips, screened = check_units(w, g, units, W=w.W, bias_or_c=c, z=w.z,
                                         scale=w.scale)
    sl = w.seq_len.cpu().numpy()
    dens = g.density / (int(sl.sum()) * w.H)
    note(f"  density {dens:.4f}, worst out rel err {worst:.2e}, flips {flips}/{screened}")
    assert 0.05 < dens < 0.9
    assert not np.isnan(g.out).any()
