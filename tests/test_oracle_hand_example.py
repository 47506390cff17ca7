"""Oracle pinned on a hand-checkable example (b=4, T=16, d=4).

Every expected value below is derived by hand from the definitions on the
picx.dev summary page of "Elastic Threshold Attention" (Methodology 4, Eq. 5:
population centroid, population variance, max norm and the dual score;
Methodology 2, Eq. 3: gated logits with the diagonal key exempt; Theoretical
Foundation: softmax attention over the admitted keys).  The inputs are in
tests/golden/hand_b4_t16.json; all statistics are exact in binary.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
EX = json.load(open(os.path.join(HERE, "golden", "hand_b4_t16.json")))
K = np.array(EX["K"], dtype=np.float32)
Q = np.array(EX["q"], dtype=np.float32)
V = np.array([[s, 1, s % 2, s // 4] for s in range(16)], dtype=np.float32)
B4, SCALE = EX["block"], EX["scale"]
R2 = math.sqrt(2.0)

# Hand derivation of the block statistics (population, divide by b = 4).
#   block 0: keys +-e1, +-e2          mu 0,          var (.5,.5,0,0),    M 1
#   block 1: 2e1, 2e1, 2e1+-2e3       mu (2,0,0,0),  var (0,0,2,0),      M 2 sqrt 2
#   block 2: (0,0,+-1,+-1)            mu 0,          var (0,0,1,1),      M sqrt 2
#   block 3: 0, 1, -1, 2e4            mu (0,0,0,.5), var (.5,.5,.5,1.25), M 2
MU = [[0, 0, 0, 0], [2, 0, 0, 0], [0, 0, 0, 0], [0, 0, 0, 0.5]]
VAR = [[.5, .5, 0, 0], [0, 0, 2, 0], [0, 0, 1, 1], [.5, .5, .5, 1.25]]
MAXN = [1.0, 2 * R2, R2, 2.0]
# Logits S_s = 0.5 * (sum of the key's coordinates), by hand:
S = [.5, -.5, .5, -.5, 1, 1, 2, 0, 1, 0, 0, -1, 0, 2, -2, 1]


def hand_score(j, z):
    """Eq. 5 by hand: q = (1,1,1,1), ||q|| = 2, so <q,mu> = sum mu,
    sigma_S = sqrt(sum var), geometric term = 2 M."""
    prob = sum(MU[j]) + (0.0 if math.isinf(z) else z * math.sqrt(sum(VAR[j])))
    geom = 2 * MAXN[j]
    return SCALE * (geom if math.isinf(z) else min(prob, geom))


def softmax_avg(logits, keys):
    """Closed-form evaluation of sum_s e^{l_s} v_s / sum_s e^{l_s} over a
    hand-listed set of (key index, logit) pairs."""
    w = [math.exp(l) for l in logits]
    return np.array([sum(wi * float(V[s][c]) for wi, s in zip(w, keys)) / sum(w)
                     for c in range(4)])


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_block_statistics_exact():
    mu, var, M = oracle.block_meta(K, B4)
    assert mu.shape == (4, 4)
    np.testing.assert_array_equal(mu, np.array(MU))
    np.testing.assert_array_equal(var, np.array(VAR))
    np.testing.assert_allclose(M, MAXN, rtol=0, atol=1e-15)


@pytest.mark.parametrize("z", [1.0, 2.0, math.inf])
def test_scores_match_hand_values(z):
    mu, var, M = oracle.block_meta(K, B4)
    for j in range(4):
        got = oracle.block_score(Q, mu[j], var[j], M[j], z, SCALE)
        assert got == pytest.approx(hand_score(j, z), rel=1e-15, abs=1e-15), (j, z)


def test_scores_numeric_spot_values():
    # The same hand values as decimals: z=1 -> (0.5, 1.707107, 0.707107, 1.079156)
    mu, var, M = oracle.block_meta(K, B4)
    got = [oracle.block_score(Q, mu[j], var[j], M[j], 1.0, SCALE) for j in range(4)]
    np.testing.assert_allclose(got, [0.5, 1 + R2 / 2, R2 / 2, 0.25 + 0.5 * math.sqrt(2.75)],
                               rtol=1e-15)


# (z, tau, admitted blocks derived by hand from hand_score)
CASES = [
    (1.0, -math.inf, [0, 1, 2, 3]),
    (1.0, 0.5, [0, 1, 2, 3]),   # block 0 scores exactly 0.5: a tie is kept
    (1.0, 0.6, [1, 2, 3]),
    (1.0, 0.8, [1, 3]),         # block 2 (score .7071) pruned though it holds S=1
    (1.0, 3.0, [3]),            # only the always-admitted last block
    (2.0, 0.8, [0, 1, 2, 3]),
    (2.0, 1.2, [1, 2, 3]),      # block 0 pruned by the geometric term (2*1*0.5 = 1 < 1.2)
]


@pytest.mark.parametrize("z,tau,blocks", CASES)
def test_admission_matches_hand_sets(z, tau, blocks):
    mu, var, M = oracle.block_meta(K, B4)
    sc = [oracle.block_score(Q, mu[j], var[j], M[j], z, SCALE) for j in range(4)]
    act, cnt = oracle.admit(16, B4, sc, tau)
    assert list(np.nonzero(act)[0]) == blocks
    assert cnt == len(blocks)


@pytest.mark.parametrize("z,tau,blocks", CASES)
def test_raw_output_matches_closed_form(z, tau, blocks):
    act = np.zeros(4, np.uint8); act[blocks] = 1
    got = oracle.attend(Q, K, V, B4, act, oracle.RAW, 5.0, tau, SCALE)
    keys = [s for s in range(16) if s // 4 in blocks]
    want = softmax_avg([S[s] for s in keys], keys)
    np.testing.assert_allclose(got, want, rtol=1e-14)
    assert got[1] == pytest.approx(1.0, abs=1e-15)  # the all-ones column


def test_raw_tau3_explicit():
    # Only block 3 (keys 12..15, logits 0, 2, -2, 1):
    e = math.e
    want0 = (12 + 13 * e**2 + 14 * e**-2 + 15 * e) / (1 + e**2 + e**-2 + e)
    act = np.array([0, 0, 0, 1], np.uint8)
    got = oracle.attend(Q, K, V, B4, act, oracle.RAW, 5.0, 3.0, SCALE)
    assert got[0] == pytest.approx(want0, rel=1e-14)
    assert got[3] == pytest.approx(3.0, rel=1e-15)


def test_gated_tau3_explicit():
    # Eq. 3 by hand for keys 12..15 at tau = 3, beta = 5: S * sigmoid(5 (S - 3)),
    # key 15 (the query's own key) ungated.
    logits = [0.0, 2 * sig(-5.0), -2 * sig(-25.0), 1.0]
    want = softmax_avg(logits, [12, 13, 14, 15])
    act = np.array([0, 0, 0, 1], np.uint8)
    got = oracle.attend(Q, K, V, B4, act, oracle.GATED, 5.0, 3.0, SCALE)
    np.testing.assert_allclose(got, want, rtol=1e-14)


def test_gated_tau_plus_inf_is_uniform_floor_plus_diagonal():
    # tau = +inf: every gate is 0, so every logit but the diagonal one is 0
    # (weight e^0 = 1); key 15 keeps S = 1.
    act = np.ones(4, np.uint8)
    got = oracle.attend(Q, K, V, B4, act, oracle.GATED, 5.0, math.inf, SCALE)
    want = softmax_avg([0.0] * 15 + [1.0], list(range(16)))
    np.testing.assert_allclose(got, want, rtol=1e-14)


@pytest.mark.parametrize("z,tau,blocks", CASES)
def test_gated_output_matches_hand_logits(z, tau, blocks):
    act = np.zeros(4, np.uint8); act[blocks] = 1
    got = oracle.attend(Q, K, V, B4, act, oracle.GATED, 5.0, tau, SCALE)
    keys = [s for s in range(16) if s // 4 in blocks]
    logits = [S[s] if s == 15 else S[s] * (1.0 if tau == -math.inf else sig(5 * (S[s] - tau)))
              for s in keys]
    np.testing.assert_allclose(got, softmax_avg(logits, keys), rtol=1e-14)


def test_gated_equals_raw_equals_dense_at_minus_inf():
    act = np.ones(4, np.uint8)
    g = oracle.attend(Q, K, V, B4, act, oracle.GATED, 5.0, -math.inf, SCALE)
    r = oracle.attend(Q, K, V, B4, act, oracle.RAW, 5.0, -math.inf, SCALE)
    d = oracle.dense(Q, K, V, SCALE)
    np.testing.assert_array_equal(g, r)
    np.testing.assert_allclose(r, d, rtol=1e-15)
    np.testing.assert_allclose(d, softmax_avg(S, list(range(16))), rtol=1e-14)
