"""GPU parity of the fused step (eta_fused_step: thresholds, screen and decode
in two launches) against the fp64 oracle, and against the separate
predict_tau -> screen -> decode path on the same inputs.

The fused step computes its thresholds in the threshold kernel's order and
scores blocks with the screen's own float32 arithmetic, so its thresholds and
admission mask must equal the separate path's bit for bit;
its output is held to the same bars as the separate decode (near-tie flips
against the oracle only, outputs within the cache dtype's bar and the 1e-5
internal bar).  Cases: the hand example, the tiny fp32 workload, ragged
lengths around block and chunk boundaries with an empty stream and NaN-filled
unused slots, every chunk size shape (1, 3, 8, 32 blocks), both logit modes,
threshold extremes and offsets, 40 heads, determinism, streams of over a
thousand blocks, and the single 32K sequence at its full size (all 16 heads
against the oracle) at 10%, 38% and 70% density.
"""
import math

import numpy as np
import pytest
import torch

from long_context_decode_eta_amd import binding as eb
from long_context_decode_eta_amd import synth
from parity import (check_against_oracle, check_units, make_cache, note, oracle_constants,
                    run_gpu, run_gpu_fused, to_gpu)
from test_gpu_parity_small import LENS, hand_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.name}")


def _same_as_separate(g_fused, g_sep):
    """Same thresholds, admission bits and token count as predict_tau and
    eta_screen."""
    np.testing.assert_array_equal(g_fused.tau_gate, g_sep.tau_gate)
    np.testing.assert_array_equal(g_fused.tau_screen, g_sep.tau_screen)
    np.testing.assert_array_equal(g_fused.mask, g_sep.mask)
    assert g_fused.density == g_sep.density


@pytest.mark.parametrize("mode", [eb.GATED, eb.RAW])
@pytest.mark.parametrize("z,tau", [(1.0, -math.inf), (1.0, 0.6), (2.0, 1.2), (math.inf, 1.2),
                                   (1.0, math.inf)])
def test_hand_example(z, tau, mode):
    w = to_gpu(hand_cache())
    cache = make_cache(w)
    c = torch.full((1,), tau, dtype=torch.float32, device="cuda")
    for chunk in (1, 3):
        g = run_gpu_fused(cache, w.q, bias_or_c=c, z=z, scale=0.5, mode=mode, chunk=chunk)
        st = check_against_oracle(w, g, cache, W=None, bias_or_c=c, z=z, scale=0.5, mode=mode)
        assert st["flips"] == 0
        assert g.out[0, 0, 1] == pytest.approx(1.0, abs=1e-6)


@pytest.mark.parametrize("mode", [eb.GATED, eb.RAW])
@pytest.mark.parametrize("chunk", [1, 3, 8, 32])
def test_tiny_workload(mode, chunk):
    w = to_gpu(synth.make("tiny", seed=1234))
    cache = make_cache(w)
    g = run_gpu_fused(cache, w.q, bias_or_c=w.tau_const, z=w.z, scale=w.scale, mode=mode,
                      chunk=chunk)
    st = check_against_oracle(w, g, cache, W=None, bias_or_c=w.tau_const, z=w.z, scale=w.scale,
                              mode=mode)
    s = run_gpu(cache, w.q, bias_or_c=w.tau_const, z=w.z, scale=w.scale, mode=mode,
                build_meta=False)
    _same_as_separate(g, s)
    note(f"  density {st['density']:.3f} out_rel {st['out_rel']:.2e} flips {st['flips']}")
    assert 0.0 < st["density"] < 1.0


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("block", [4, 16, 64])
def test_ragged_edges(kv, D, block):
    # Lengths around block and chunk boundaries, an empty stream, unused slots
    # NaN-filled, a dynamic threshold from the predictor.
    name = "tiny" if D == 64 else "ctx32k"
    w = synth.make(name, seed=7 + block, T=LENS, B=len(LENS), H=3, cap=1024, pad="nan",
                   block=block, kv=kv)
    to_gpu(w)
    cache = make_cache(w)
    rng = np.random.default_rng(block)
    W = torch.from_numpy((rng.standard_normal((3 * D, 3)) / math.sqrt(D)).astype(np.float32))
    W = W.cuda()
    c = torch.tensor([0.2, 0.6, 1.0], dtype=torch.float32, device="cuda")
    for mode in (eb.GATED, eb.RAW):
        s = run_gpu(cache, w.q, W=W, bias_or_c=c, z=1.0, scale=w.scale, mode=mode)
        for chunk in (1, 3, 8, 32):
            g = run_gpu_fused(cache, w.q, W=W, bias_or_c=c, z=1.0, scale=w.scale, mode=mode,
                              chunk=chunk, build_meta=False)
            _same_as_separate(g, s)
            st = check_against_oracle(w, g, cache, W=W, bias_or_c=c, z=1.0, scale=w.scale,
                                      mode=mode, check_meta=False)
            assert not np.isnan(g.out).any()
            assert np.all(g.out[0] == 0)  # the empty stream
    note(f"  density {st['density']:.3f} out_rel {st['out_rel']:.2e}")


@pytest.mark.parametrize("cap", [4096, 8196])
def test_long_block_lists(cap):
    # Block 4: 1024 and 2049 blocks per stream (128 and 257 chunks of 8),
    # ragged lengths up to the capacity and an empty stream.
    lens = [0, 5, 2049, cap - 3, cap]
    w = synth.make("tiny", seed=41, T=lens, B=len(lens), H=3, cap=cap, pad="nan", block=4)
    to_gpu(w)
    cache = make_cache(w)
    rng = np.random.default_rng(5)
    W = torch.from_numpy((rng.standard_normal((3 * 64, 3)) / 8.0).astype(np.float32)).cuda()
    c = torch.tensor([0.2, 0.6, 1.0], dtype=torch.float32, device="cuda")
    for mode in (eb.GATED, eb.RAW):
        s = run_gpu(cache, w.q, W=W, bias_or_c=c, z=1.0, scale=w.scale, mode=mode)
        for chunk in (8, 32):
            g = run_gpu_fused(cache, w.q, W=W, bias_or_c=c, z=1.0, scale=w.scale, mode=mode,
                              chunk=chunk, build_meta=False)
            _same_as_separate(g, s)
            st = check_against_oracle(w, g, cache, W=W, bias_or_c=c, z=1.0, scale=w.scale,
                                      mode=mode, check_meta=False)
            assert np.all(g.out[0] == 0)  # the empty stream
    note(f"  cap {cap}: density {st['density']:.3f} out_rel {st['out_rel']:.2e}")


@pytest.mark.parametrize("a", [-0.5, 0.7])
def test_threshold_offset_and_many_heads(a):
    # tau_screen = tau_gate - a, and a dynamic predictor over 40 heads
    # (H*D = 2560 terms per threshold, not a multiple of the 1024-term rounds).
    w = to_gpu(synth.make("tiny", seed=21, T=[300, 1000], B=2, H=40, cap=1024, block=16))
    cache = make_cache(w)
    rng = np.random.default_rng(3)
    W = torch.from_numpy((rng.standard_normal((40 * 64, 40)) / 8.0).astype(np.float32)).cuda()
    c = torch.from_numpy(rng.uniform(0.3, 1.2, 40).astype(np.float32)).cuda()
    s = run_gpu(cache, w.q, W=W, bias_or_c=c, z=1.5, scale=w.scale, a=a)
    g = run_gpu_fused(cache, w.q, W=W, bias_or_c=c, z=1.5, scale=w.scale, a=a, chunk=8,
                      build_meta=False)
    _same_as_separate(g, s)
    np.testing.assert_array_equal(g.tau_screen, g.tau_gate - np.float32(a))
    st = check_against_oracle(w, g, cache, W=W, bias_or_c=c, z=1.5, scale=w.scale, a=a,
                              mode=eb.GATED, check_meta=False)
    note(f"  a {a}: density {st['density']:.3f} out_rel {st['out_rel']:.2e}")


@pytest.mark.parametrize("tau", [math.inf, -math.inf])
def test_threshold_extremes(tau):
    w = to_gpu(synth.make("ctx128k", seed=3, T=(100, 3000), B=4, H=2, cap=3000, block=32))
    cache = make_cache(w)
    c = torch.full((2,), tau, dtype=torch.float32, device="cuda")
    g = run_gpu_fused(cache, w.q, bias_or_c=c, z=1.0, scale=w.scale, chunk=8)
    nb = -(-w.seq_len.cpu().numpy() // 32)
    assert np.all(g.cnt == (1 if tau == math.inf else nb[:, None]))
    check_against_oracle(w, g, cache, W=None, bias_or_c=c, z=1.0, scale=w.scale, mode=eb.GATED)


def test_chunk_invariance_and_determinism():
    w = to_gpu(synth.make("ctx128k", seed=11, T=(2000, 9000), B=3, H=4, cap=9000))
    cache = make_cache(w)
    eb.build_block_meta(cache)
    c = torch.full((4,), 1.2, dtype=torch.float32, device="cuda")
    ref = run_gpu(cache, w.q, bias_or_c=c, z=1.0, scale=w.scale, split=1, build_meta=False)
    for chunk in (1, 2, 5, 16, 32):
        first = None
        for _ in range(2):
            g = run_gpu_fused(cache, w.q, bias_or_c=c, z=1.0, scale=w.scale, chunk=chunk,
                              build_meta=False)
            if first is not None:
                assert np.array_equal(g.out, first), "run-to-run difference"
            first = g.out
        np.testing.assert_array_equal(g.mask, ref.mask)
        np.testing.assert_allclose(g.out, ref.out, rtol=2e-6, atol=2e-6)


def test_reused_workspace_and_changing_lengths():
    # One Decoder (one workspace) over many calls: repeated calls agree bit
    # for bit, and shorter and longer sequences on the same workspace match a
    # fresh one (no state carries over between calls).
    w = to_gpu(synth.make("ctx128k", seed=12, T=(3000, 9000), B=3, H=4, cap=9000, block=32))
    cache = make_cache(w)
    eb.build_block_meta(cache)
    c = torch.full((4,), 1.0, dtype=torch.float32, device="cuda")
    dec = eb.Decoder(cache, z=1.0, scale=w.scale, fused_blocks_per_chunk=8)
    first = dec.step_fused(w.q, None, c).clone()
    for _ in range(30):
        assert torch.equal(dec.step_fused(w.q, None, c), first)
    full = cache.seq_len.clone()
    for lens in ([1000, 9000, 4097], [0, 33, 8999], full.tolist()):
        cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
        got = dec.step_fused(w.q, None, c).clone()
        fresh = eb.Decoder(cache, z=1.0, scale=w.scale, fused_blocks_per_chunk=8)
        assert torch.equal(got, fresh.step_fused(w.q, None, c))
        if lens[0] == 0:
            assert torch.count_nonzero(got[0]).item() == 0  # the empty stream
    assert torch.equal(got, first)


_held = {}


def _ctx32k():
    if "w" not in _held:
        torch.cuda.empty_cache()
        w = synth.make("ctx32k", seed=1234, device="cuda")
        cache = make_cache(w)
        eb.build_block_meta(cache)
        torch.cuda.synchronize()
        rhos = [0.10, 0.38, 0.70]
        consts = dict(zip(rhos, [c for c, _ in oracle_constants(w, rhos, seqs=[0])]))
        _held.update(w=w, cache=cache, consts=consts)
    return _held["w"], _held["cache"], _held["consts"]


@pytest.mark.parametrize("rho", [0.10, 0.38, 0.70])
def test_ctx32k_full_size_every_head(rho):
    """The single 32K sequence, 16 heads, d 128, block 64, bf16, dynamic tau,
    in the chunking the Decoder picks by itself; every head against the
    oracle, and the admission bits against the separate screen."""
    w, cache, consts = _ctx32k()
    c = consts[rho].cuda()
    g = run_gpu_fused(cache, w.q, W=w.W, bias_or_c=c, z=w.z, scale=w.scale, build_meta=False)
    s = run_gpu(cache, w.q, W=w.W, bias_or_c=c, z=w.z, scale=w.scale, build_meta=False)
    _same_as_separate(g, s)
    worst, flips, screened = check_units(w, g, [(0, h) for h in range(w.H)], W=w.W,
                                         bias_or_c=c, z=w.z, scale=w.scale)
    dens = g.density / (int(w.seq_len.sum()) * w.H)
    note(f"  target {rho:.2f}: density {dens:.4f}, worst out rel err {worst:.2e}, "
         f"flips {flips}/{screened}")
    assert abs(dens - rho) < 0.1


def test_release_ctx32k():
    _held.clear()
    torch.cuda.empty_cache()
