"""C ABI of libeta.so without a GPU: the library loads, exports every function
include/eta.h declares, and rejects bad arguments on the host before any HIP
call (so these run on a machine with no GPU).  Pointers below are dummies that
the library never dereferences on an error path."""
import ctypes
import os
import re

import pytest

from long_context_decode_eta_amd import binding as eb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eta.h")
FAKE = 0x1000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(eb.LIB_PATH):
        from long_context_decode_eta_amd import build
        build.build()
    return eb.lib()


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(eta_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/eta.h but not exported"


def test_version_and_strings(lib):
    assert lib.eta_abi_version() == 4
    for s, name in [(0, b"ETA_OK"), (1, b"ETA_ERR_NULL_PTR"), (5, b"ETA_ERR_WORKSPACE"),
                    (6, b"ETA_ERR_HIP")]:
        assert lib.eta_status_string(s) == name


def cache(**kw):
    c = dict(batch=2, heads=4, head_dim=128, block=32, cap_tokens=1000, kv_dtype=eb.DT_BF16)
    c.update(kw)
    ptrs = {n: kw.pop(n, FAKE) for n in ("k", "v", "mu", "var", "maxnorm", "seq_len")}
    s = eb.EtaCacheStruct(c["batch"], c["heads"], c["head_dim"], c["block"], c["cap_tokens"],
                          c["kv_dtype"], ptrs["k"], ptrs["v"], ptrs["mu"], ptrs["var"],
                          ptrs["maxnorm"], ptrs["seq_len"])
    return ctypes.byref(s)


def err(lib):
    return lib.eta_last_error().decode()


def test_cache_validation(lib):
    L = lib
    assert L.eta_build_block_meta(None, 0, -1, None) == eb.ETA_ERR_NULL_PTR
    assert L.eta_build_block_meta(cache(head_dim=96), 0, -1, None) == eb.ETA_ERR_BAD_SHAPE
    assert "head_dim" in err(L)
    assert L.eta_build_block_meta(cache(block=24), 0, -1, None) == eb.ETA_ERR_BAD_SHAPE
    assert L.eta_build_block_meta(cache(block=256), 0, -1, None) == eb.ETA_ERR_BAD_SHAPE
    assert L.eta_build_block_meta(cache(cap_tokens=0), 0, -1, None) == eb.ETA_ERR_BAD_SHAPE
    assert L.eta_build_block_meta(cache(batch=-1), 0, -1, None) == eb.ETA_ERR_BAD_SHAPE
    assert L.eta_build_block_meta(cache(kv_dtype=7), 0, -1, None) == eb.ETA_ERR_BAD_ARG
    assert L.eta_build_block_meta(cache(k=None), 0, -1, None) == eb.ETA_ERR_NULL_PTR
    assert L.eta_build_block_meta(cache(seq_len=None), 0, -1, None) == eb.ETA_ERR_NULL_PTR
    assert L.eta_build_block_meta(cache(), 0, 33, None) == eb.ETA_ERR_CAPACITY  # 32 blocks
    assert L.eta_build_block_meta(cache(), -1, 1, None) == eb.ETA_ERR_BAD_ARG
    assert L.eta_cache_blocks(cache()) == 32


def test_empty_problem_is_ok_without_launch(lib):
    L = lib
    # batch 0 with NULL data pointers: nothing is launched, so no GPU is touched.
    c = cache(batch=0, k=None, v=None, mu=None, var=None, maxnorm=None, seq_len=None)
    assert L.eta_build_block_meta(c, 0, -1, None) == eb.ETA_OK
    assert L.eta_append_kv(c, None, None, None, None) == eb.ETA_OK
    assert L.eta_screen(c, None, None, 1.0, 0.1, None, None, None, None, 0, None) == eb.ETA_OK
    assert L.eta_decode(c, None, None, None, None, 0, 5.0, 0.1, 16, None, 0, None, None) == eb.ETA_OK
    assert L.eta_predict_tau(0, 4, 128, None, None, None, 0.0, None, None, None) == eb.ETA_OK


def test_screen_validation(lib):
    L = lib
    ws = L.eta_screen_workspace_bytes(2, 4, 32)
    assert ws >= 2 * 4 * 1 * 8
    args = lambda **o: [o.get("c", cache()), o.get("q", FAKE), o.get("t", FAKE),
                        o.get("z", 1.0), o.get("scale", 0.088), o.get("idx", FAKE),
                        o.get("cnt", FAKE), None, o.get("ws", FAKE), o.get("wsb", ws), None]
    assert L.eta_screen(*args(z=-1.0)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_screen(*args(z=float("nan"))) == eb.ETA_ERR_BAD_ARG
    assert L.eta_screen(*args(scale=0.0)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_screen(*args(scale=float("inf"))) == eb.ETA_ERR_BAD_ARG
    assert L.eta_screen(*args(q=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_screen(*args(idx=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_screen(*args(wsb=ws - 1)) == eb.ETA_ERR_WORKSPACE
    assert L.eta_screen(*args(ws=None)) == eb.ETA_ERR_WORKSPACE


def test_decode_validation(lib):
    L = lib
    ws = L.eta_decode_workspace_bytes(2, 4, 128, 32, 16)
    assert ws >= 2 * 4 * 2 * (128 + 2) * 4
    args = lambda **o: [o.get("c", cache()), FAKE, o.get("tau", FAKE), o.get("idx", FAKE),
                        FAKE, o.get("mode", 0), o.get("beta", 5.0), o.get("scale", 0.088),
                        o.get("split", 16), FAKE, o.get("wsb", ws), o.get("out", FAKE), None]
    assert L.eta_decode(*args(mode=2)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode(*args(beta=0.0)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode(*args(beta=float("nan"))) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode(*args(split=0)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode(*args(split=4097)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode(*args(tau=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_decode(*args(idx=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_decode(*args(out=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_decode(*args(wsb=ws - 4)) == eb.ETA_ERR_WORKSPACE
    # RAW mode needs no tau
    assert L.eta_decode(*args(mode=1, tau=None, wsb=ws - 4)) == eb.ETA_ERR_WORKSPACE
    assert L.eta_dense_decode(cache(), FAKE, 0.088, 16, FAKE, ws - 4, FAKE, None) == eb.ETA_ERR_WORKSPACE
    assert L.eta_dense_decode(cache(), FAKE, -1.0, 16, FAKE, ws, FAKE, None) == eb.ETA_ERR_BAD_ARG
    # block positions of all streams together must fit int32: 2^14 streams x 2^17 blocks
    huge = cache(batch=1024, heads=16, head_dim=64, block=4, cap_tokens=1 << 19)
    assert L.eta_decode(*args(c=huge, wsb=1 << 62)) == eb.ETA_ERR_BAD_SHAPE
    assert "2^31" in err(L)


def test_decode_noalloc_validation(lib):
    L = lib
    args = lambda **o: [o.get("c", cache()), FAKE, o.get("tau", FAKE), FAKE, FAKE,
                        o.get("mode", 0), 5.0, 0.088, o.get("split", 16), o.get("out", FAKE),
                        None]
    assert L.eta_decode_noalloc(*args(split=0)) == eb.ETA_ERR_BAD_ARG
    assert L.eta_decode_noalloc(*args(tau=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_decode_noalloc(*args(out=None)) == eb.ETA_ERR_NULL_PTR
    assert L.eta_decode_noalloc(*args(c=cache(batch=0, k=None, v=None, mu=None, var=None,
                                                maxnorm=None, seq_len=None))) == eb.ETA_OK
    # 16384 streams: one partial slot per stream beyond the waves' (520 bytes
    # each at d 128) is over 8 MiB, beyond the static scratch; refused on the
    # host, before any HIP call.
    big = cache(batch=16384, heads=1, head_dim=128, block=4, cap_tokens=64)
    assert L.eta_decode_noalloc(*args(c=big, split=1)) == eb.ETA_ERR_CAPACITY
    assert "scratch" in err(L)


def test_fused_step_validation(lib):
    L = lib
    ws = L.eta_fused_step_workspace_bytes(2, 4, 128, 32, 8)
    # the size covers one partial (max, sum, 128 floats) per possible chunk
    assert ws >= 2 * 4 * 4 * (128 + 2) * 4

    def call(**o):
        return L.eta_fused_step(o.get("c", cache()), o.get("q", FAKE), o.get("W", FAKE),
                                o.get("bias", FAKE), o.get("a", 0.0), o.get("z", 1.0),
                                o.get("mode", 0), o.get("beta", 5.0), o.get("scale", 0.088),
                                o.get("cb", 8), None, None, None, None, o.get("ws", FAKE),
                                o.get("wsb", ws), o.get("out", FAKE), None)

    assert call(cb=0) == eb.ETA_ERR_BAD_ARG
    assert call(cb=33) == eb.ETA_ERR_BAD_ARG
    assert call(z=-1.0) == eb.ETA_ERR_BAD_ARG
    assert call(z=float("nan")) == eb.ETA_ERR_BAD_ARG
    assert call(a=float("nan")) == eb.ETA_ERR_BAD_ARG
    assert call(beta=0.0) == eb.ETA_ERR_BAD_ARG
    assert call(scale=float("inf")) == eb.ETA_ERR_BAD_ARG
    assert call(mode=7) == eb.ETA_ERR_BAD_ARG
    assert call(q=None) == eb.ETA_ERR_NULL_PTR
    assert call(bias=None) == eb.ETA_ERR_NULL_PTR
    assert call(out=None) == eb.ETA_ERR_NULL_PTR
    assert call(wsb=ws - 1) == eb.ETA_ERR_WORKSPACE
    assert call(ws=None) == eb.ETA_ERR_WORKSPACE
    assert call(c=cache(heads=300)) == eb.ETA_ERR_BAD_SHAPE
    assert call(c=cache(batch=0, k=None, v=None, mu=None, var=None, maxnorm=None,
                        seq_len=None)) == eb.ETA_OK


def test_predict_and_calibrate_validation(lib):
    L = lib
    assert L.eta_predict_tau(2, 300, 128, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE, None) == eb.ETA_ERR_BAD_SHAPE
    assert L.eta_predict_tau(2, 4, 128, FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, None) == eb.ETA_ERR_BAD_ARG
    assert L.eta_predict_tau(2, 4, 128, None, FAKE, FAKE, 0.0, FAKE, FAKE, None) == eb.ETA_ERR_NULL_PTR
    assert L.eta_predict_tau(2, 4, 128, FAKE, FAKE, None, 0.0, FAKE, FAKE, None) == eb.ETA_ERR_NULL_PTR
    ws = L.eta_calibrate_workspace_bytes(2, 2, 4, 32)
    call = lambda **o: L.eta_calibrate_threshold(cache(), o.get("n", 2), FAKE, None, o.get("z", 1.0),
                                                 0.088, o.get("rho", 0.25), FAKE, o.get("wsb", ws),
                                                 FAKE, None)
    assert call(n=0) == eb.ETA_ERR_BAD_SHAPE
    assert call(rho=1.5) == eb.ETA_ERR_BAD_ARG
    assert call(z=-2.0) == eb.ETA_ERR_BAD_ARG
    assert call(wsb=ws - 1) == eb.ETA_ERR_WORKSPACE


def test_append_validation(lib):
    L = lib
    assert L.eta_append_kv(cache(), None, FAKE, None, None) == eb.ETA_ERR_NULL_PTR
    assert L.eta_append_kv(cache(head_dim=32), FAKE, FAKE, None, None) == eb.ETA_ERR_BAD_SHAPE
    # the capacity flag is required: without it an append to a full sequence
    # could drop its token unseen
    assert L.eta_append_kv(cache(), FAKE, FAKE, None, None) == eb.ETA_ERR_NULL_PTR
    assert "overflow" in err(L)


def test_gqa_validation(lib):
    L = lib
    ws_s = L.eta_screen_gqa_workspace_bytes(2, 4, 32)
    assert ws_s >= 2 * 4 * 8
    scr = lambda **o: L.eta_screen_gqa(o.get("c", cache()), o.get("g", 8), o.get("q", FAKE),
                                       FAKE, o.get("z", 1.0), 0.088, FAKE, o.get("mask", FAKE),
                                       FAKE, None, FAKE, o.get("wsb", ws_s), None)
    assert scr(g=0) == eb.ETA_ERR_BAD_SHAPE
    assert scr(g=17) == eb.ETA_ERR_BAD_SHAPE
    assert "group" in err(L)
    assert scr(z=-1.0) == eb.ETA_ERR_BAD_ARG
    assert scr(q=None) == eb.ETA_ERR_NULL_PTR
    assert scr(mask=None) == eb.ETA_ERR_NULL_PTR
    assert scr(wsb=ws_s - 1) == eb.ETA_ERR_WORKSPACE
    assert scr(c=cache(batch=0, k=None, v=None, mu=None, var=None, maxnorm=None,
                       seq_len=None), q=None) == eb.ETA_OK
    # partials of every query head: 2 * 4 * 8 heads, 2 chunks, 128 + 2 floats
    ws = L.eta_decode_gqa_workspace_bytes(2, 4, 8, 128, 32, 16)
    assert ws >= 2 * 4 * 8 * 2 * (128 + 2) * 4
    dec = lambda **o: L.eta_decode_gqa(o.get("c", cache()), o.get("g", 8), FAKE,
                                       o.get("tau", FAKE), o.get("idx", FAKE), o.get("mask", FAKE),
                                       FAKE, o.get("mode", 0), o.get("beta", 5.0), 0.088,
                                       o.get("split", 16), FAKE, o.get("wsb", ws), FAKE, None)
    assert dec(c=cache(kv_dtype=eb.DT_F32)) == eb.ETA_ERR_BAD_ARG
    assert "bf16" in err(L)
    assert dec(g=17) == eb.ETA_ERR_BAD_SHAPE
    assert dec(mode=3) == eb.ETA_ERR_BAD_ARG
    assert dec(beta=-1.0) == eb.ETA_ERR_BAD_ARG
    assert dec(split=2049) == eb.ETA_ERR_BAD_ARG
    assert dec(tau=None) == eb.ETA_ERR_NULL_PTR
    assert dec(mask=None) == eb.ETA_ERR_NULL_PTR
    assert dec(wsb=ws - 4) == eb.ETA_ERR_WORKSPACE
    assert dec(mode=1, tau=None, wsb=ws - 4) == eb.ETA_ERR_WORKSPACE
    assert L.eta_dense_decode_gqa(cache(), 8, FAKE, 0.088, 16, FAKE, ws - 4, FAKE,
                                  None) == eb.ETA_ERR_WORKSPACE
    assert L.eta_dense_decode_gqa(cache(kv_dtype=eb.DT_F32), 8, FAKE, 0.088, 16, FAKE, ws, FAKE,
                                  None) == eb.ETA_ERR_BAD_ARG
    huge = cache(batch=4096, heads=4, head_dim=64, block=4, cap_tokens=1 << 19)
    assert dec(c=huge, wsb=1 << 62) == eb.ETA_ERR_BAD_SHAPE
    assert "2^31" in err(L)


def test_prefill_validation(lib):
    L = lib
    call = lambda **o: L.eta_gated_prefill(o.get("B", 2), o.get("Hkv", 4), o.get("G", 8),
                                           o.get("T", 100), o.get("d", 64), o.get("q", FAKE),
                                           FAKE, FAKE, o.get("tau", FAKE), o.get("beta", 5.0),
                                           o.get("scale", 0.125), o.get("out", FAKE), None, None)
    assert call(d=96) == eb.ETA_ERR_BAD_SHAPE
    assert call(G=0) == eb.ETA_ERR_BAD_SHAPE
    assert call(T=-1) == eb.ETA_ERR_BAD_SHAPE
    assert call(beta=0.0) == eb.ETA_ERR_BAD_ARG
    assert call(scale=float("nan")) == eb.ETA_ERR_BAD_ARG
    assert call(q=None) == eb.ETA_ERR_NULL_PTR
    assert call(tau=None) == eb.ETA_ERR_NULL_PTR
    assert call(out=None) == eb.ETA_ERR_NULL_PTR
    assert call(T=0, q=None, out=None) == eb.ETA_OK  # empty: nothing launched
    # rows of one K/V stream are addressed with 32-bit byte offsets
    assert call(B=1, Hkv=1, G=1, T=1 << 24, d=128) == eb.ETA_ERR_BAD_SHAPE
    assert "2^32" in err(L)
    assert call(B=1, Hkv=1, G=1, T=1 << 25, d=64) == eb.ETA_ERR_BAD_SHAPE


def test_binding_refuses_cpu_tensors(lib):
    import torch
    c = eb.KVCache.__new__(eb.KVCache)
    with pytest.raises(ValueError):
        eb._dev(torch.zeros(4), torch.float32, "x")
