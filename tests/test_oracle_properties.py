"""Oracle pinned on properties the paper's definitions fix.

Definitions: picx.dev summary page of "Elastic Threshold Attention":
Theoretical Foundation (dense / sparse attention), Methodology 1 Eq. 1
(threshold, zero-initialised weights with bias -8 admit every key),
Methodology 2 Eqs. 2-3 (gated logits), Methodology 4 Eq. 5 (dual score with a
Cauchy-Schwarz ceiling; blocks below the threshold are skipped).

Each test checks the oracle against something other than itself: numpy
library routines (mean, var, norms, softmax), closed forms, limits, exact
special cases and brute force on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng


def bf16_bits(x):
    """Round float32 -> bfloat16 (nearest even) and return the 16-bit patterns."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def np_softmax_attend(q, K, V, scale, logits=None):
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale if logits is None else logits
    w = np.exp(S - S.max())
    return (w[:, None] * V.astype(np.float64)).sum(0) / w.sum()


# --------------------------------------------------------------------------
# Block statistics
@pytest.mark.parametrize("b", [1, 4, 16, 64])
@pytest.mark.parametrize("bf16", [False, True])
def test_meta_matches_numpy(b, bf16):
    rng = RNG(b + 7 * bf16)
    T, d = 5 * b + (b // 2), 64
    Kf = (rng.standard_normal((T, d)) * 0.7 + rng.standard_normal(d)).astype(np.float32)
    K = bf16_bits(Kf) if bf16 else Kf
    Kv = widen(K) if bf16 else Kf
    mu, var, M = oracle.block_meta(K, b)
    nbc = T // b
    assert mu.shape[0] == nbc  # the partial last block gets no statistics
    blocks = Kv[: nbc * b].astype(np.float64).reshape(nbc, b, d)
    np.testing.assert_allclose(mu, blocks.mean(1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(var, blocks.var(1, ddof=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M, np.linalg.norm(blocks, axis=2).max(1), rtol=1e-14)


def test_meta_invariant_under_key_permutation_within_block():
    rng = RNG(3)
    b, d = 16, 64
    K = rng.standard_normal((4 * b, d)).astype(np.float32)
    P = K.copy()
    for j in range(4):
        P[j * b:(j + 1) * b] = K[j * b + rng.permutation(b)]
    a, c = oracle.block_meta(K, b), oracle.block_meta(P, b)
    for x, y in zip(a, c):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)  # 1, -1, 3.140625, tiny, max
    K = np.tile(bits, (1, 1))
    mu, _, _ = oracle.block_meta(np.repeat(K, 1, axis=0).reshape(1, 5), 1)
    np.testing.assert_array_equal(mu[0], widen(bits).astype(np.float64))


# --------------------------------------------------------------------------
# Threshold (Eq. 1)
def test_predictor_zero_init_gives_minus_eight():
    q = RNG(0).standard_normal((3, 4, 64)).astype(np.float32)
    W = np.zeros((4 * 64, 4), np.float32)
    tau, ts = oracle.predict_tau(q, W, np.full(4, -8.0, np.float32))
    assert np.all(tau == -8.0) and np.all(ts == -8.0)


def test_predictor_full_matrix_matches_numpy():
    rng = RNG(1)
    B, H, d = 3, 5, 64
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    W = (rng.standard_normal((H * d, H)) / 8).astype(np.float32)
    bias = rng.standard_normal(H).astype(np.float32)
    tau, ts = oracle.predict_tau(q, W, bias, a=0.25)
    want = q.reshape(B, H * d).astype(np.float64) @ W.astype(np.float64) + bias
    np.testing.assert_allclose(tau, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ts, want - 0.25, rtol=1e-12, atol=1e-12)


def test_predictor_block_diagonal_is_per_head_dot():
    rng = RNG(2)
    B, H, d = 2, 4, 64
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    w = rng.standard_normal((H, d)).astype(np.float32)
    W = np.zeros((H * d, H), np.float32)
    for h in range(H):
        W[h * d:(h + 1) * d, h] = w[h]
    c = rng.standard_normal(H).astype(np.float32)
    tau, _ = oracle.predict_tau(q, W, c)
    want = np.einsum("bhd,hd->bh", q.astype(np.float64), w.astype(np.float64)) + c
    np.testing.assert_allclose(tau, want, rtol=1e-12, atol=1e-12)


def test_predictor_frozen_broadcasts_constants():
    c = np.array([0.5, 1.25, -3.0], np.float32)
    tau, ts = oracle.predict_tau(np.zeros((4, 3, 64), np.float32), None, c, a=-0.5)
    np.testing.assert_array_equal(tau, np.tile(c.astype(np.float64), (4, 1)))
    np.testing.assert_array_equal(ts, tau + 0.5)


# --------------------------------------------------------------------------
# Screen (Eq. 5)
def _stream(seed, T, d, b, shift=0.5):
    rng = RNG(seed)
    nb = -(-T // b)
    mu = rng.standard_normal((nb, d)) * shift
    K = (rng.standard_normal((T, d)) + np.repeat(mu, b, 0)[:T]).astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    return q, K, V


@pytest.mark.parametrize("seed", range(5))
def test_geometric_ceiling_is_sound_for_every_block(seed):
    b, d = 16, 64
    q, K, _ = _stream(seed, 40 * b, d, b)
    scale = 1 / 8
    mu, var, M = oracle.block_meta(K, b)
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    for j in range(len(M)):
        ceil_ = oracle.block_score(q, mu[j], var[j], M[j], math.inf, scale)
        assert S[j * b:(j + 1) * b].max() <= ceil_ * (1 + 1e-12)
        # the dual score never exceeds the ceiling
        assert oracle.block_score(q, mu[j], var[j], M[j], 2.0, scale) <= ceil_


@pytest.mark.parametrize("z", [0.5, 1.0, 2.0])
def test_moment_term_is_exact_std_when_one_coordinate_varies(z):
    # If only coordinate i varies inside a block, S_s = scale (<q,base> + q_i r_s),
    # so sigma_S = sqrt(q_i^2 var_i) equals the population std of <q,k_s> exactly and
    # the dual score is mean(S) + z std(S) (the keys sit far from q, so the
    # geometric ceiling does not bind).
    rng = RNG(21)
    d, b, scale = 64, 16, 0.125
    q = (rng.standard_normal(d) * 1.7).astype(np.float32)
    for i in [0, 5, 63]:
        base = rng.standard_normal(d)
        base -= base @ q.astype(np.float64) / (q.astype(np.float64) @ q) * q  # orthogonal to q
        base *= 40 / np.linalg.norm(base)
        K = np.tile(base, (b, 1))
        K[:, i] += rng.standard_normal(b) * 3
        K = K.astype(np.float32)
        mu, var, M = oracle.block_meta(K, b)
        S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
        got = oracle.block_score(q, mu[0], var[0], M[0], z, scale)
        assert got == pytest.approx(S.mean() + z * S.std(), rel=1e-9, abs=1e-9)


def test_block_size_one_reduces_to_token_threshold():
    # b = 1: mu = k, var = 0, M = ||k|| >= <q,k>/||q||, so the score is S_s itself.
    d, T = 64, 300
    q, K, _ = _stream(11, T, d, 1)
    scale = 1 / 8
    mu, var, M = oracle.block_meta(K, 1)
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    sc = np.array([oracle.block_score(q, mu[j], var[j], M[j], 1.5, scale) for j in range(T)])
    np.testing.assert_allclose(sc, S, rtol=1e-12, atol=1e-13)
    tau = float(np.quantile(S, 0.6))
    act, _ = oracle.admit(T, 1, sc, tau)
    want = S >= tau
    want[-1] = True  # the query's own key (last position) is always admitted
    np.testing.assert_array_equal(act.astype(bool), want)


@pytest.mark.parametrize("seed", range(4))
def test_z_infinite_has_full_token_recall(seed):
    b, d, T = 8, 64, 8 * 50 + 3
    q, K, _ = _stream(seed, T, d, b)
    scale = 1 / 8
    mu, var, M = oracle.block_meta(K, b)
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    sc = [oracle.block_score(q, mu[j], var[j], M[j], math.inf, scale) for j in range(len(M))]
    for tau in np.quantile(S, [0.5, 0.9, 0.99]):
        act, _ = oracle.admit(T, b, sc, tau)
        for s in np.nonzero(S >= tau)[0]:
            assert act[s // b], (s, tau)


def test_admitted_sets_nested_in_tau_and_growing_in_z():
    b, d, T = 16, 64, 16 * 80
    q, K, _ = _stream(5, T, d, b)
    mu, var, M = oracle.block_meta(K, b)
    scale = 1 / 8
    prev = None
    for z in [0.0, 0.5, 1.0, 2.0, 4.0, math.inf]:
        sc = [oracle.block_score(q, mu[j], var[j], M[j], z, scale) for j in range(len(M))]
        sets = [oracle.admit(T, b, sc, t)[0].astype(bool) for t in np.linspace(-2, 4, 25)]
        for hi, lo in zip(sets[1:], sets[:-1]):
            assert np.all(hi <= lo)  # raising tau only removes blocks
        if prev is not None:
            for a_, b_ in zip(prev, sets):
                assert np.all(a_ <= b_)  # raising z only adds blocks
        prev = sets


def test_tie_is_admitted_and_tail_rules():
    sc = np.array([0.75, 0.25, 0.5])
    act, cnt = oracle.admit(3 * 4, 4, sc, 0.75)      # T = 12: block 2 is the last one
    assert list(act) == [1, 0, 1] and cnt == 2       # block 0 ties the threshold: kept
    act, cnt = oracle.admit(3 * 4 + 1, 4, sc, 5.0)   # T = 13: partial block 3 forced
    assert list(act) == [0, 0, 0, 1] and cnt == 1
    act, cnt = oracle.admit(3, 4, [], 5.0)           # T < b: only the partial block
    assert list(act) == [1] and cnt == 1
    act, cnt = oracle.admit(0, 4, [], -5.0)          # empty stream
    assert act.size == 0 and cnt == 0


# --------------------------------------------------------------------------
# Attention (Eq. 3 and the sparse / dense definitions)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T", [1, 5, 64, 203])
def test_all_admitted_equals_numpy_dense(T, bf16):
    b, d = 16, 64
    q, Kf, Vf = _stream(T, T, d, b)
    K, V = (bf16_bits(Kf), bf16_bits(Vf)) if bf16 else (Kf, Vf)
    Kw, Vw = (widen(K), widen(V)) if bf16 else (K, V)
    scale = 1 / 8
    act = np.ones(-(-T // b), np.uint8)
    want = np_softmax_attend(q, Kw, Vw, scale)
    for mode in (oracle.GATED, oracle.RAW):
        got = oracle.attend(q, K, V, b, act, mode, 5.0, -math.inf, scale)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.dense(q, K, V, scale), want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_raw_masked_matches_numpy_restricted_softmax(seed):
    b, d, T = 8, 64, 8 * 30 + 5
    q, K, V = _stream(seed, T, d, b)
    rng = RNG(100 + seed)
    act = (rng.random(-(-T // b)) < 0.4).astype(np.uint8)
    act[-1] = 1
    keep = np.repeat(act.astype(bool), b)[:T]
    want = np_softmax_attend(q, K[keep], V[keep], 1 / 8)
    got = oracle.attend(q, K, V, b, act, oracle.RAW, 5.0, 0.0, 1 / 8)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_gated_large_beta_limit_is_hard_contraction_to_zero():
    # beta -> inf: sigmoid(beta (S - tau)) -> 1[S > tau], so a key below tau
    # gets logit 0 (weight e^0) and a key above keeps S; the diagonal key keeps S.
    b, d, T = 8, 64, 8 * 20
    q, K, V = _stream(9, T, d, b)
    scale = 1 / 8
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    tau = float(np.median(S)) + 1e-3
    lim = np.where(S > tau, S, 0.0)
    lim[-1] = S[-1]
    want = np_softmax_attend(q, K, V, scale, logits=lim)
    act = np.ones(T // b, np.uint8)
    got = oracle.attend(q, K, V, b, act, oracle.GATED, 1e7, tau, scale)
    np.testing.assert_allclose(got, want, rtol=1e-9)


def test_gated_differs_from_raw_only_through_the_gate():
    # With the only admitted block holding just the diagonal key ungated and
    # the rest gated, GATED != RAW for a finite tau, and GATED(tau=+inf) puts
    # weight 1 on every non-diagonal key.
    b, d, T = 4, 64, 4 * 6 + 1
    q, K, V = _stream(4, T, d, b)
    act = np.ones(-(-T // b), np.uint8)
    scale = 1 / 8
    S = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    lg = np.zeros(T); lg[-1] = S[-1]
    want = np_softmax_attend(q, K, V, scale, logits=lg)
    got = oracle.attend(q, K, V, b, act, oracle.GATED, 5.0, math.inf, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12)


@pytest.mark.parametrize("mode", [oracle.GATED, oracle.RAW])
def test_constant_values_give_that_value(mode):
    b, d, T = 16, 64, 16 * 9 + 7
    q, K, _ = _stream(6, T, d, b)
    V = np.tile(np.linspace(-2, 3, d, dtype=np.float32), (T, 1))
    act = np.zeros(-(-T // b), np.uint8); act[[0, 3, -1]] = 1
    got = oracle.attend(q, K, V, b, act, mode, 5.0, 0.3, 1 / 8)
    np.testing.assert_allclose(got, V[0].astype(np.float64), rtol=1e-13, atol=1e-14)


def test_empty_stream_outputs_zero():
    d = 64
    q = np.ones(d, np.float32)
    K = np.zeros((4, d), np.float32)
    got = oracle.attend(q, K, K, 4, np.zeros(1, np.uint8), oracle.GATED, 5.0, 0.0, 1 / 8, T=0)
    assert np.all(got == 0)
    assert np.all(oracle.dense(q, K, K, 1 / 8, T=0) == 0)


# --------------------------------------------------------------------------
# Batch drivers and calibration
def _batch(seed, B, H, d, cap, lens, b, bf16=True):
    rng = RNG(seed)
    K = rng.standard_normal((B, H, cap, d)).astype(np.float32)
    V = rng.standard_normal((B, H, cap, d)).astype(np.float32)
    for bb, T in enumerate(lens):
        K[bb, :, T:] = np.nan  # slots past T_b must never be read
        V[bb, :, T:] = np.nan
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    if bf16:
        K, V = bf16_bits(K), bf16_bits(V)
    return q, K, V, np.array(lens, np.int32)


def test_step_batch_dense_limit_and_ragged_lengths():
    B, H, d, b, cap = 3, 2, 64, 8, 100
    lens = [100, 37, 8]
    q, K, V, sl = _batch(1, B, H, d, cap, lens, b)
    meta = oracle.meta_batch(K, sl, b)
    r = oracle.step_batch(q, K, V, sl, b, meta, None, np.full(H, -np.inf, np.float32),
                          z=1.0, scale=1 / 8)
    for bb in range(B):
        T = lens[bb]
        assert np.all(r["cnt"][bb] == -(-T // b))
        assert np.all(r["tokens"][bb] == T)
        for h in range(H):
            want = np_softmax_attend(q[bb, h], widen(K[bb, h, :T]), widen(V[bb, h, :T]), 1 / 8)
            np.testing.assert_allclose(r["out"][bb, h], want, rtol=1e-12, atol=1e-13)
    dn = oracle.dense_batch(q, K, V, sl, scale=1 / 8)
    np.testing.assert_allclose(dn, r["out"], rtol=1e-12, atol=1e-13)


def test_step_batch_counts_tokens_of_partial_tail():
    B, H, d, b, cap = 1, 1, 64, 8, 64
    q, K, V, sl = _batch(2, B, H, d, cap, [43], b)
    meta = oracle.meta_batch(K, sl, b)
    r = oracle.step_batch(q, K, V, sl, b, meta, None, np.full(H, np.inf, np.float32), z=1.0,
                          scale=1 / 8)
    assert r["cnt"][0, 0] == 1 and r["tokens"][0, 0] == 43 - 5 * 8
    assert list(np.nonzero(r["active"][0, 0])[0]) == [5]


@pytest.mark.parametrize("rho", [0.0, 0.1, 0.38, 0.7, 1.0])
def test_calibration_hits_target_density(rho):
    B, H, d, b, cap = 4, 3, 64, 8, 96
    lens = [96, 77, 50, 9]
    q, K, V, sl = _batch(3, B, H, d, cap, lens, b)
    meta = oracle.meta_batch(K, sl, b)
    qs = q[None]
    c, k = oracle.calibrate(qs, sl, b, cap, meta, z=1.0, scale=1 / 8, rho=rho)
    r = oracle.step_batch(q, K, V, sl, b, meta, None, c.astype(np.float32), z=1.0, scale=1 / 8)
    total = sum(lens)
    forced = sum(T - (-(-T // b) - 1) * b for T in lens)
    cand = sum(-(-T // b) - 1 for T in lens)
    for h in range(H):
        want_k = min(max(int(math.floor((rho * total - forced) / b + 0.5)), 0), cand)
        assert k[h] == want_k
        # float32 rounding of c can only matter at an exact tie; none here
        assert r["tokens"][:, h].sum() == forced + b * k[h]
    if rho == 1.0:
        assert np.all(np.isneginf(c))
    if rho == 0.0:
        assert np.all(np.isposinf(c))


# ---------------------------------------------------------------------------
# The stored form of the block index: mu and var rounded to bfloat16.
def _nearest_bf16_by_search(x: float) -> float:
    """The bfloat16 nearest to x (ties to the even significand), found by
    comparing x exactly (Fractions) with every bfloat16 of its binade and the
    next power of two: the 129 values 2^k (1 + i/128), i = 0..128."""
    from fractions import Fraction
    if x == 0.0:
        return 0.0
    s = -1.0 if x < 0 else 1.0
    ax = Fraction(abs(x))
    k = math.floor(math.log2(abs(x)))
    while Fraction(2) ** k > ax:
        k -= 1
    while Fraction(2) ** (k + 1) <= ax:
        k += 1
    best, best_i, best_d = None, None, None
    for i in range(129):
        v = Fraction(2) ** k * (1 + Fraction(i, 128))
        dist = abs(ax - v)
        # significand index i (i = 128 is the next binade's 1.0: even)
        even = (i % 2 == 0)
        if best is None or dist < best_d or (dist == best_d and even):
            best, best_i, best_d = v, i, dist
    return s * float(best)


def test_index_rounding_is_nearest_bf16_ties_to_even():
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400)))
    # exact ties between two bfloat16 values: odd and even lower neighbours
    for base in (1.0, 1.0078125, 3.0, 0.15625, 1000.0):
        for k in range(3):
            lo = base * (1 + k / 128.0)
            ulp = 2.0 ** (math.floor(math.log2(lo)) - 7)
            xs += [lo + ulp / 2, -(lo + ulp / 2), lo + ulp / 2 * (1 + 1e-15), lo + ulp * 0.4999]
    xs += [0.0, 1.0, -2.0, 255.5, 2.0 ** -100, 3.0 * 2.0 ** 100]
    got = oracle.round_bf16(np.array(xs))
    for x, g in zip(xs, got):
        assert g == _nearest_bf16_by_search(float(x)), (x, g)
    # every result is a bfloat16: its float32 bits have a zero low half
    bits = got.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_stored_meta_rounds_mu_and_var_only():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((2, 3, 64, 16)).astype(np.float32)
    sl = np.array([64, 40], np.int32)
    exact = oracle.meta_batch(K, sl, 8)
    mu, var, M = oracle.stored_meta(exact)
    np.testing.assert_array_equal(M, exact[2])
    np.testing.assert_array_equal(mu, oracle.round_bf16(exact[0]))
    np.testing.assert_array_equal(var, oracle.round_bf16(exact[1]))
    # within half a bfloat16 step (2^-8 relative) of the exact values
    nz = exact[1] != 0
    assert np.all(np.abs(var[nz] - exact[1][nz]) <= 2.0 ** -8 * np.abs(exact[1][nz]))
    assert np.any(mu != exact[0])
