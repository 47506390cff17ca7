"""fp64 CPU oracle of ETA block-sparse decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding in ``long_context_decode_eta_amd``) never imports it, and the
two share no code: the arithmetic lives in ``eta_oracle.c`` (plain C, double
precision, one OpenMP iteration per (sequence, head) stream), and this module
only marshals numpy arrays into it.

Formulas follow the paper "Elastic Threshold Attention: Learned Contextual
Sparsity for Long-Context Decoding" (picx.dev summary page): Theoretical
Foundation (dense and sparse attention), Methodology 1 Eq. 1 (threshold),
Methodology 2 Eqs. 2-3 (gated logits), Methodology 4 Eq. 5 (block screen).

Array conventions: K/V are ``float32`` arrays (fp32 cache) or ``uint16``
arrays holding raw bfloat16 bit patterns (bf16 cache); q, W, bias are
``float32``; every result is ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16 = 0, 1
GATED, RAW = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eta_oracle.c")
_LIB = os.path.join(_HERE, "libeta_oracle.so")


def build(out: str = _LIB, src: str = _SRC, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (IEEE double arithmetic, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", *extra,
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_d = ctypes.c_double


def load(path: str | None = None):
    """Load (building first if absent) and type the oracle library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    # ETA_ORACLE_LIB lets the mutation test point the pins at a planted-mistake build.
    so = path or os.environ.get("ETA_ORACLE_LIB") or _LIB
    if not os.path.exists(so):
        build(so)
    lib = ctypes.CDLL(so)
    lib.eta_oracle_block_meta.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p]
    lib.eta_oracle_block_meta.restype = _i
    lib.eta_oracle_predict_tau.argtypes = [_i, _i, _i, _p, _p, _p, _d, _p, _p]
    lib.eta_oracle_predict_tau.restype = None
    lib.eta_oracle_block_score.argtypes = [_p, _p, _p, _d, _i, _d, _d]
    lib.eta_oracle_block_score.restype = _d
    lib.eta_oracle_admit.argtypes = [_i, _i, _p, _d, _p]
    lib.eta_oracle_admit.restype = _i
    lib.eta_oracle_attend.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p, _i, _d, _d, _d, _p]
    lib.eta_oracle_attend.restype = None
    lib.eta_oracle_dense.argtypes = [_p, _p, _p, _i, _i, _i, _d, _p]
    lib.eta_oracle_dense.restype = None
    lib.eta_oracle_meta_batch.argtypes = [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]
    lib.eta_oracle_meta_batch.restype = None
    lib.eta_oracle_step_batch.argtypes = (
        [_i] * 6 + [_p] * 7 + [_p, _p] + [_d, _d, _d, _i, _d] + [_p] * 6 + [_p])
    lib.eta_oracle_step_batch.restype = None
    lib.eta_oracle_screen_attend_batch.argtypes = (
        [_i] * 6 + [_p] * 7 + [_p, _p] + [_d, _d, _i, _d] + [_p] * 5)
    lib.eta_oracle_screen_attend_batch.restype = None
    lib.eta_oracle_attend_batch.argtypes = [_i] * 6 + [_p] * 5 + [_i, _d, _p, _d, _p]
    lib.eta_oracle_attend_batch.restype = None
    lib.eta_oracle_dense_batch.argtypes = [_i] * 5 + [_p] * 4 + [_d, _p]
    lib.eta_oracle_dense_batch.restype = None
    lib.eta_oracle_calibrate.argtypes = [_i] * 6 + [_p] * 6 + [_d, _d, _d, _p, _p]
    lib.eta_oracle_calibrate.restype = None
    lib.eta_oracle_gqa_screen_attend_batch.argtypes = (
        [_i] * 7 + [_p] * 7 + [_p, _p] + [_d, _d, _i, _d] + [_p] * 8)
    lib.eta_oracle_gqa_screen_attend_batch.restype = None
    lib.eta_oracle_gqa_dense_batch.argtypes = [_i] * 6 + [_p] * 4 + [_d, _p]
    lib.eta_oracle_gqa_dense_batch.restype = None
    lib.eta_oracle_prefill.argtypes = [_i] * 6 + [_p] * 4 + [_d, _d, _p, _p]
    lib.eta_oracle_prefill.restype = None
    lib.eta_oracle_round_bf16.argtypes = [_d]
    lib.eta_oracle_round_bf16.restype = _d
    lib.eta_oracle_round_bf16_array.argtypes = [_p, ctypes.c_size_t]
    lib.eta_oracle_round_bf16_array.restype = None
    lib.eta_oracle_threads.argtypes = []
    lib.eta_oracle_threads.restype = _i
    lib.eta_oracle_set_threads.argtypes = [_i]
    lib.eta_oracle_set_threads.restype = None
    if path is None:
        _lib = lib
    return lib


# ---------------------------------------------------------------------------
def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _kv(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"K/V must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def block_meta(K, b, lib=None):
    """Statistics of the complete blocks of one stream K [T][d]."""
    lib = lib or load()
    K, dt = _kv(K)
    T, d = K.shape
    nbc = T // b
    mu = np.zeros((nbc, d)); var = np.zeros((nbc, d)); M = np.zeros(nbc)
    lib.eta_oracle_block_meta(_ptr(K), dt, T, d, b, _ptr(mu), _ptr(var), _ptr(M))
    return mu, var, M


def predict_tau(q, W, bias_or_c, a=0.0, lib=None):
    """Eq. 1 for q [B][H][d]; W [H*d][H] or None (frozen constants)."""
    lib = lib or load()
    q = _f32(q); B, H, d = q.shape
    W = _f32(W); c = _f32(bias_or_c)
    tau = np.zeros((B, H)); ts = np.zeros((B, H))
    lib.eta_oracle_predict_tau(B, H, d, _ptr(q), _ptr(W), _ptr(c), float(a), _ptr(tau), _ptr(ts))
    return tau, ts


def block_score(q, mu, var, M, z, scale, lib=None):
    """Eq. 5 for one query vector against one block's statistics."""
    lib = lib or load()
    q = _f32(q)
    mu = np.ascontiguousarray(mu, dtype=np.float64)
    var = np.ascontiguousarray(var, dtype=np.float64)
    return lib.eta_oracle_block_score(_ptr(q), _ptr(mu), _ptr(var), float(M), q.shape[0],
                                      float(z), float(scale))


def admit(T, b, scores, tau_screen, lib=None):
    """Admission mask (uint8 [ceil(T/b)]) and admitted-block count."""
    lib = lib or load()
    nb = -(-T // b)
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    if sc.size < max(nb, 1):
        sc = np.concatenate([sc, np.full(max(nb, 1) - sc.size, np.nan)])
    act = np.zeros(max(nb, 1), dtype=np.uint8)
    cnt = lib.eta_oracle_admit(T, b, _ptr(sc), float(tau_screen), _ptr(act))
    return act[:nb], cnt


def attend(q, K, V, b, active, mode, beta, tau, scale, T=None, lib=None):
    """Attention of q [d] over the admitted keys of K, V [T][d]."""
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, dt2 = _kv(V)
    assert dt == dt2
    T = K.shape[0] if T is None else T
    act = np.ascontiguousarray(active, dtype=np.uint8)
    out = np.zeros(q.shape[0])
    lib.eta_oracle_attend(_ptr(q), _ptr(K), _ptr(V), dt, T, q.shape[0], b, _ptr(act), mode,
                          float(beta), float(tau), float(scale), _ptr(out))
    return out


def dense(q, K, V, scale, T=None, lib=None):
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, _ = _kv(V)
    T = K.shape[0] if T is None else T
    out = np.zeros(q.shape[0])
    lib.eta_oracle_dense(_ptr(q), _ptr(K), _ptr(V), dt, T, q.shape[0], float(scale), _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Batch forms over the cache layout [B][H][cap][d].
def meta_batch(K, seq_len, b, lib=None):
    lib = lib or load()
    K, dt = _kv(K)
    B, H, cap, d = K.shape
    nbcap = -(-cap // b)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    mu = np.zeros((B, H, nbcap, d)); var = np.zeros((B, H, nbcap, d)); M = np.zeros((B, H, nbcap))
    lib.eta_oracle_meta_batch(B, H, d, b, cap, dt, _ptr(sl), _ptr(K), _ptr(mu), _ptr(var), _ptr(M))
    return mu, var, M


def round_bf16(x, lib=None):
    """x (float64 array) rounded to the nearest bfloat16, ties to even."""
    lib = lib or load()
    out = np.array(x, dtype=np.float64, copy=True, order="C")
    lib.eta_oracle_round_bf16_array(_ptr(out), out.size)
    return out


def stored_meta(meta, lib=None):
    """The block index as the cache stores it: exact mu and var rounded to
    bfloat16, maxnorm exact."""
    mu, var, M = meta
    return round_bf16(mu, lib), round_bf16(var, lib), M


def index_batch(K, seq_len, b, lib=None):
    """meta_batch in the stored form (stored_meta): what the screen uses."""
    return stored_meta(meta_batch(K, seq_len, b, lib), lib)


def step_batch(q, K, V, seq_len, b, meta, W, bias_or_c, *, a=0.0, z=1.0, scale=None,
               mode=GATED, beta=5.0, lib=None):
    """One decode step (threshold, screen, attention) for every stream."""
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, dt2 = _kv(V)
    assert dt == dt2
    B, H, cap, d = K.shape
    nbcap = -(-cap // b)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    mu, var, M = (np.ascontiguousarray(x, dtype=np.float64) for x in meta)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    W = _f32(W); c = _f32(bias_or_c)
    r = dict(tau=np.zeros((B, H)), tau_screen=np.zeros((B, H)),
             score=np.zeros((B, H, nbcap)), active=np.zeros((B, H, nbcap), np.uint8),
             cnt=np.zeros((B, H), np.int32), tokens=np.zeros((B, H), np.int64),
             out=np.zeros((B, H, d)))
    lib.eta_oracle_step_batch(B, H, d, b, cap, dt, _ptr(sl), _ptr(q), _ptr(K), _ptr(V),
                              _ptr(mu), _ptr(var), _ptr(M), _ptr(W), _ptr(c), float(a),
                              float(z), float(scale), int(mode), float(beta),
                              _ptr(r["tau"]), _ptr(r["tau_screen"]), _ptr(r["score"]),
                              _ptr(r["active"]), _ptr(r["cnt"]), _ptr(r["tokens"]),
                              _ptr(r["out"]))
    return r


def screen_attend_batch(q, K, V, seq_len, b, meta, tau, tau_screen, *, z=1.0, scale=None,
                        mode=GATED, beta=5.0, lib=None):
    """Screen and attention for every stream given fp64 thresholds [B][H]."""
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, dt2 = _kv(V)
    assert dt == dt2
    B, H, cap, d = K.shape
    nbcap = -(-cap // b)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    mu, var, M = (np.ascontiguousarray(x, dtype=np.float64) for x in meta)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    tau = np.ascontiguousarray(tau, dtype=np.float64).reshape(B, H)
    ts = np.ascontiguousarray(tau_screen, dtype=np.float64).reshape(B, H)
    r = dict(tau=tau, tau_screen=ts, score=np.zeros((B, H, nbcap)),
             active=np.zeros((B, H, nbcap), np.uint8), cnt=np.zeros((B, H), np.int32),
             tokens=np.zeros((B, H), np.int64), out=np.zeros((B, H, d)))
    lib.eta_oracle_screen_attend_batch(B, H, d, b, cap, dt, _ptr(sl), _ptr(q), _ptr(K), _ptr(V),
                                       _ptr(mu), _ptr(var), _ptr(M), _ptr(tau), _ptr(ts),
                                       float(z), float(scale), int(mode), float(beta),
                                       _ptr(r["score"]), _ptr(r["active"]), _ptr(r["cnt"]),
                                       _ptr(r["tokens"]), _ptr(r["out"]))
    return r


def gqa_screen_attend_batch(q, K, V, seq_len, b, meta, tau, tau_screen, group, *, z=1.0,
                            scale=None, mode=GATED, beta=5.0, lib=None):
    """Grouped-query screen and attention: q [B][Hkv*G][d], K/V and statistics
    per KV head [B][Hkv][...], thresholds [B][Hkv*G] (fp64)."""
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, dt2 = _kv(V)
    assert dt == dt2
    B, Hkv, cap, d = K.shape
    G = int(group)
    Hq = Hkv * G
    assert q.shape == (B, Hq, d)
    nbcap = -(-cap // b)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    mu, var, M = (np.ascontiguousarray(x, dtype=np.float64) for x in meta)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    tau = np.ascontiguousarray(tau, dtype=np.float64).reshape(B, Hq)
    ts = np.ascontiguousarray(tau_screen, dtype=np.float64).reshape(B, Hq)
    r = dict(tau=tau, tau_screen=ts, score=np.zeros((B, Hq, nbcap)),
             active=np.zeros((B, Hq, nbcap), np.uint8), cnt=np.zeros((B, Hq), np.int32),
             tokens=np.zeros((B, Hq), np.int64), union=np.zeros((B, Hkv, nbcap), np.uint8),
             union_cnt=np.zeros((B, Hkv), np.int32), union_tokens=np.zeros((B, Hkv), np.int64),
             out=np.zeros((B, Hq, d)))
    lib.eta_oracle_gqa_screen_attend_batch(
        B, Hkv, G, d, b, cap, dt, _ptr(sl), _ptr(q), _ptr(K), _ptr(V), _ptr(mu), _ptr(var),
        _ptr(M), _ptr(tau), _ptr(ts), float(z), float(scale), int(mode), float(beta),
        _ptr(r["score"]), _ptr(r["active"]), _ptr(r["cnt"]), _ptr(r["tokens"]), _ptr(r["union"]),
        _ptr(r["union_cnt"]), _ptr(r["union_tokens"]), _ptr(r["out"]))
    return r


def gqa_dense_batch(q, K, V, seq_len, group, scale=None, lib=None):
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, _ = _kv(V)
    B, Hkv, cap, d = K.shape
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    out = np.zeros((B, Hkv * int(group), d))
    lib.eta_oracle_gqa_dense_batch(B, Hkv, int(group), d, cap, dt, _ptr(sl), _ptr(q), _ptr(K),
                                   _ptr(V), float(scale), _ptr(out))
    return out


def prefill(q, K, V, tau, group=1, *, beta=5.0, scale=None, lib=None):
    """Gated causal attention forward over whole sequences (Eqs. 2-3) and the
    per-row density term of Eq. 4.  q [B][H_kv*G][T][d], K/V [B][H_kv][T][d]
    (all float32, or all bf16 bits as uint16), tau [B][H_kv*G][T].  Returns
    (out [B][H_q][T][d], dens [B][H_q][T]) in float64."""
    lib = lib or load()
    q, dq = _kv(q); K, dt = _kv(K); V, dt2 = _kv(V)
    assert dq == dt == dt2
    B, Hkv, T, d = K.shape
    G = int(group)
    assert q.shape == (B, Hkv * G, T, d)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    tau = np.ascontiguousarray(np.broadcast_to(tau, (B, Hkv * G, T)), dtype=np.float64)
    out = np.zeros((B, Hkv * G, T, d))
    dens = np.zeros((B, Hkv * G, T))
    lib.eta_oracle_prefill(B, Hkv, G, T, d, dt, _ptr(q), _ptr(K), _ptr(V), _ptr(tau), float(beta),
                           float(scale), _ptr(out), _ptr(dens))
    return out, dens


def attend_batch(q, K, V, seq_len, b, active, tau, *, mode=GATED, beta=5.0, scale=None,
                 lib=None):
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, _ = _kv(V)
    B, H, cap, d = K.shape
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    act = np.ascontiguousarray(active, dtype=np.uint8)
    tau = np.ascontiguousarray(tau, dtype=np.float64)
    out = np.zeros((B, H, d))
    lib.eta_oracle_attend_batch(B, H, d, b, cap, dt, _ptr(sl), _ptr(q), _ptr(K), _ptr(V),
                                _ptr(act), int(mode), float(beta), _ptr(tau), float(scale),
                                _ptr(out))
    return out


def dense_batch(q, K, V, seq_len, scale=None, lib=None):
    lib = lib or load()
    q = _f32(q); K, dt = _kv(K); V, _ = _kv(V)
    B, H, cap, d = K.shape
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    out = np.zeros((B, H, d))
    lib.eta_oracle_dense_batch(B, H, d, cap, dt, _ptr(sl), _ptr(q), _ptr(K), _ptr(V),
                               float(scale), _ptr(out))
    return out


def calibrate(q_sets, seq_len, b, cap, meta, *, tau0=None, z=1.0, scale=None, rho=0.25,
              lib=None):
    """Per-head constants c [H] (and the admitted-block counts k [H]) that
    admit a pooled fraction rho of tokens; q_sets [n][B][H][d]."""
    lib = lib or load()
    q_sets = _f32(q_sets)
    n, B, H, d = q_sets.shape
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    mu, var, M = (np.ascontiguousarray(x, dtype=np.float64) for x in meta)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    t0 = None if tau0 is None else np.ascontiguousarray(tau0, dtype=np.float64)
    c = np.zeros(H); k = np.zeros(H, np.int64)
    lib.eta_oracle_calibrate(n, B, H, d, b, cap, _ptr(sl), _ptr(q_sets), _ptr(mu), _ptr(var),
                             _ptr(M), _ptr(t0), float(z), float(scale), float(rho), _ptr(c),
                             _ptr(k))
    return c, k
