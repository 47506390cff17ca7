"""Randomised properties of the oracle (hypothesis): shapes, block sizes,
thresholds and value ranges drawn at random, each checked against a closed
form or a numpy routine rather than against the oracle itself.

Definitions: picx.dev summary page of "Elastic Threshold Attention":
Theoretical Foundation (dense and sparse attention, the latter normalised over
the admitted keys), Methodology 2 Eq. 3 (gated logits, the query's own key
ungated), Methodology 4 Eq. 5 (block statistics and the dual score, whose
geometric term is a Cauchy-Schwarz ceiling).
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None)


def stream(seed, T, d, b, spread, shift):
    rng = np.random.default_rng(seed)
    nb = -(-T // b)
    centre = np.repeat(rng.standard_normal((nb, d)) * shift, b, 0)[:T]
    K = (rng.standard_normal((T, d)) * spread + centre).astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    q = (rng.standard_normal(d) * spread).astype(np.float32)
    return q, K, V


def numpy_attend(q, K, V, scale, keep=None, logits=None):
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale if logits is None else logits
    if keep is not None:
        S, V = S[keep], V[keep]
    w = np.exp(S - S.max())
    return (w[:, None] * V.astype(np.float64)).sum(0) / w.sum()


shapes = st.tuples(st.integers(0, 2**31 - 1),      # seed
                   st.integers(1, 200),             # T
                   st.sampled_from([1, 2, 3, 8, 16, 64]),  # d
                   st.sampled_from([1, 2, 4, 5, 16]),      # b
                   st.floats(0.1, 4.0),             # spread of the keys
                   st.floats(0.0, 3.0))             # spread of the block centres


@SETTINGS
@given(shapes)
def test_statistics_are_mean_population_variance_and_max_norm(sh):
    seed, T, d, b, spread, shift = sh
    _, K, _ = stream(seed, T, d, b, spread, shift)
    mu, var, M = oracle.block_meta(K, b)
    assert len(M) == T // b  # complete blocks only
    for j in range(T // b):
        blk = K[j * b:(j + 1) * b].astype(np.float64)
        np.testing.assert_allclose(mu[j], blk.mean(0), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(var[j], blk.var(0), rtol=1e-10, atol=1e-12)
        assert M[j] == np.linalg.norm(blk, axis=1).max() or math.isclose(
            M[j], np.linalg.norm(blk, axis=1).max(), rel_tol=1e-12)


@SETTINGS
@given(shapes, st.floats(0.01, 2.0), st.floats(0.0, 8.0))
def test_geometric_term_bounds_every_score_and_the_dual_score(sh, scale, z):
    seed, T, d, b, spread, shift = sh
    q, K, _ = stream(seed, T, d, b, spread, shift)
    mu, var, M = oracle.block_meta(K, b)
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    for j in range(len(M)):
        ceiling = oracle.block_score(q, mu[j], var[j], M[j], math.inf, scale)
        assert math.isclose(ceiling, scale * np.linalg.norm(q.astype(np.float64)) * M[j],
                            rel_tol=1e-12, abs_tol=1e-300)
        assert S[j * b:(j + 1) * b].max() <= ceiling * (1 + 1e-12) + 1e-300
        assert oracle.block_score(q, mu[j], var[j], M[j], z, scale) <= ceiling


@SETTINGS
@given(shapes, st.floats(-3.0, 3.0), st.floats(0.0, 3.0))
def test_admitted_sets_shrink_as_tau_rises(sh, tau, step):
    seed, T, d, b, spread, shift = sh
    q, K, _ = stream(seed, T, d, b, spread, shift)
    mu, var, M = oracle.block_meta(K, b)
    sc = [oracle.block_score(q, mu[j], var[j], M[j], 1.0, 0.25) for j in range(len(M))]
    lo, _ = oracle.admit(T, b, sc, tau)
    hi, _ = oracle.admit(T, b, sc, tau + step)
    assert np.all(hi <= lo)
    assert lo[-1] == 1 and hi[-1] == 1  # the block holding the newest key
    # every complete block is admitted exactly when its score reaches tau
    for j, s in enumerate(sc):
        if j != len(lo) - 1:
            assert lo[j] == (s >= tau)


@SETTINGS
@given(st.tuples(st.integers(0, 2**31 - 1), st.integers(1, 150), st.sampled_from([2, 8, 64]),
                 st.sampled_from([1, 4, 16]), st.floats(0.1, 3.0), st.floats(0.0, 2.0)),
       st.floats(0.05, 1.0))
def test_everything_admitted_is_dense_softmax(sh, scale):
    seed, T, d, b, spread, shift = sh
    q, K, V = stream(seed, T, d, b, spread, shift)
    want = numpy_attend(q, K, V, scale)
    act = np.ones(-(-T // b), np.uint8)
    for mode in (oracle.GATED, oracle.RAW):
        got = oracle.attend(q, K, V, b, act, mode, 5.0, -math.inf, scale)
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


@SETTINGS
@given(st.tuples(st.integers(0, 2**31 - 1), st.integers(1, 150), st.sampled_from([2, 8, 64]),
                 st.sampled_from([1, 4, 16]), st.floats(0.1, 3.0), st.floats(0.0, 2.0)),
       st.floats(0.0, 1.0), st.floats(-2.0, 2.0), st.floats(0.5, 10.0))
def test_masked_gated_attention_matches_numpy(sh, density, tau, beta):
    seed, T, d, b, spread, shift = sh
    q, K, V = stream(seed, T, d, b, spread, shift)
    scale = 0.3
    rng = np.random.default_rng(seed ^ 0x5EED)
    act = (rng.random(-(-T // b)) < density).astype(np.uint8)
    act[-1] = 1
    keep = np.repeat(act.astype(bool), b)[:T]
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    gated = S / (1.0 + np.exp(-beta * (S - tau)))
    gated[-1] = S[-1]  # the query's own key is never gated
    np.testing.assert_allclose(oracle.attend(q, K, V, b, act, oracle.RAW, beta, tau, scale),
                               numpy_attend(q, K, V, scale, keep=keep), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(oracle.attend(q, K, V, b, act, oracle.GATED, beta, tau, scale),
                               numpy_attend(q, K, V, scale, keep=keep, logits=gated),
                               rtol=1e-10, atol=1e-12)
