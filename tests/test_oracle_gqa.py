"""Grouped-query oracle pinned on the pinned multi-head oracle and on
invariants of the grouping (v2 page of "Elastic Threshold Attention",
Table 5 shape H_Q = 32, H_KV = 4; summary page, Implications: a block is
loaded when any head of its group needs it, each head attends over its own
admitted blocks, D_union >= D_head).

- G = 1 reduces to the multi-head path exactly.
- Every query head equals the multi-head oracle run with that head's query
  against its KV head's stream (replicated KV).
- The union is the OR of the group's masks; union tokens >= every head's.
- tau = -inf gives numpy dense softmax attention per query head, and the
  dense grouped oracle agrees.
"""
import math

import numpy as np
import pytest

import oracle


def bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def setup(seed, B=2, Hkv=2, G=4, d=64, b=8, cap=200, lens=(200, 77)):
    rng = np.random.default_rng(seed)
    nb = -(-cap // b)
    mu_blk = rng.standard_normal((B, Hkv, nb, d)) * 0.6
    K = rng.standard_normal((B, Hkv, cap, d)) + np.repeat(mu_blk, b, axis=2)[:, :, :cap]
    V = rng.standard_normal((B, Hkv, cap, d))
    for bb, T in enumerate(lens):
        K[bb, :, T:] = np.nan
        V[bb, :, T:] = np.nan
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    return q, bf16(K), bf16(V), np.array(lens, np.int32)


@pytest.mark.parametrize("mode", [oracle.GATED, oracle.RAW])
def test_group_one_is_multi_head(mode):
    q, K, V, sl = setup(1, G=1)
    meta = oracle.meta_batch(K, sl, 8)
    tau = np.full((2, 2), 1.1)
    g = oracle.gqa_screen_attend_batch(q, K, V, sl, 8, meta, tau, tau, 1, z=1.0, scale=0.125,
                                       mode=mode)
    m = oracle.screen_attend_batch(q, K, V, sl, 8, meta, tau, tau, z=1.0, scale=0.125, mode=mode)
    np.testing.assert_array_equal(g["active"], m["active"])
    np.testing.assert_array_equal(g["out"], m["out"])
    np.testing.assert_array_equal(g["union"], m["active"])


@pytest.mark.parametrize("G", [2, 4, 8])
def test_each_query_head_is_multi_head_on_replicated_kv(G):
    q, K, V, sl = setup(2, G=G)
    b = 8
    meta = oracle.meta_batch(K, sl, b)
    rng = np.random.default_rng(3)
    tau = rng.uniform(0.6, 1.6, (2, 2 * G))
    g = oracle.gqa_screen_attend_batch(q, K, V, sl, b, meta, tau, tau - 0.1, G, z=1.5,
                                       scale=0.125)
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)  # KV head per query head
    metar = tuple(np.repeat(x, G, axis=1) for x in meta)
    m = oracle.screen_attend_batch(q, Kr, Vr, sl, b, metar, tau, tau - 0.1, z=1.5, scale=0.125)
    np.testing.assert_array_equal(g["active"], m["active"])
    np.testing.assert_array_equal(g["tokens"], m["tokens"])
    np.testing.assert_array_equal(g["out"], m["out"])
    # union = OR over the group; union tokens bound every head's tokens
    u = g["active"].reshape(2, 2, G, -1).max(axis=2)
    np.testing.assert_array_equal(g["union"], u)
    assert np.all(g["union_tokens"][:, :, None] >= g["tokens"].reshape(2, 2, G))
    assert np.all(g["union_cnt"] == u.sum(-1))


def test_minus_inf_is_dense_per_query_head():
    G = 4
    q, K, V, sl = setup(4, G=G)
    meta = oracle.meta_batch(K, sl, 8)
    tau = np.full((2, 2 * G), -math.inf)
    g = oracle.gqa_screen_attend_batch(q, K, V, sl, 8, meta, tau, tau, G, scale=0.125)
    d = oracle.gqa_dense_batch(q, K, V, sl, G, scale=0.125)
    Kf = (K.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Vf = (V.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for bb in range(2):
        T = sl[bb]
        for h in range(2 * G):
            kv = h // G
            S = Kf[bb, kv, :T] @ q[bb, h].astype(np.float64) * 0.125
            w = np.exp(S - S.max())
            want = (w[:, None] * Vf[bb, kv, :T]).sum(0) / w.sum()
            np.testing.assert_allclose(g["out"][bb, h], want, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(d[bb, h], want, rtol=1e-12, atol=1e-13)
