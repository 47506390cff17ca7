"""Seeded synthetic workloads: determinism, shapes and stated structure."""
import math

import numpy as np
import torch

from long_context_decode_eta_amd import synth


def test_same_seed_same_tensors():
    a = synth.make("ragged", seed=5, T=(40, 200), B=3, H=2)
    b = synth.make("ragged", seed=5, T=(40, 200), B=3, H=2)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.seq_len, b.seq_len), (a.q_cal, b.q_cal)]:
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    c = synth.make("ragged", seed=6, T=(40, 200), B=3, H=2)
    assert not torch.equal(a.q, c.q)


def test_shapes_and_dtypes():
    w = synth.make("ctx128k", T=512, B=2, H=3)
    assert w.k.shape == (2, 3, 512, 128) and w.k.dtype == torch.bfloat16
    assert w.W.shape == (3 * 128, 3) and w.rho == (0.10, 0.38, 0.70, 1.0)
    t = synth.make("tiny")
    assert t.k.dtype == torch.float32 and t.tau_const.shape == (4,)
    assert torch.all((t.tau_const >= 0.5) & (t.tau_const <= 1.5))
    assert t.scale == np.float32(1 / 8)


def test_needles_lift_block_mean_along_query():
    # A needle block's mean is shifted by NEEDLE_DELTA * sqrt(D) * q / ||q||^2,
    # i.e. its mean logit <q, mean k> / sqrt(D) rises by NEEDLE_DELTA.
    w = synth.make("ctx32k", T=64 * 400, B=1, H=2, kv="f32")
    D, bs = w.D, w.block
    for h in range(2):
        idx = w.needle_blocks[h]
        assert len(idx) == round(0.01 * 400)
        q = w.q[0, h].double()
        blocks = w.k[0, h].double().reshape(-1, bs, D).mean(1)
        lift = (blocks @ q) / math.sqrt(D)
        others = np.setdiff1d(np.arange(400), idx.numpy())
        assert lift[idx].min() > lift[others].mean() + 1.5


def test_padding_beyond_length():
    w = synth.make("ragged", T=(33, 90), B=4, H=1, pad="nan", cap=96)
    for b in range(4):
        T = int(w.seq_len[b])
        assert torch.isnan(w.k[b, :, T:].float()).all() and not torch.isnan(w.k[b, :, :T].float()).any()


def test_bf16_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8], dtype=torch.float32)
    bits = synth.kv_numpy(x.to(torch.bfloat16))
    np.testing.assert_array_equal(synth.bf16_bits_to_float(bits), [1.0, 1.0 + 2**-6, -1.0])
