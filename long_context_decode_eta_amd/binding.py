"""Thin ctypes binding of libeta.so (C ABI in include/eta.h).

The functions here only marshal arguments: they check that torch tensors sit
on the GPU with the expected dtype and contiguity, pass ``data_ptr()`` values
and the current HIP stream, and turn status codes into exceptions.  Every step
of the decode path runs in the library's HIP kernels; torch provides device
memory and streams and nothing else.  There is no CPU fallback: if
``libeta.so`` is missing the import of :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_size_t, c_void_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeta.so")

ETA_OK, ETA_ERR_NULL_PTR, ETA_ERR_BAD_SHAPE, ETA_ERR_BAD_ARG = 0, 1, 2, 3
ETA_ERR_CAPACITY, ETA_ERR_WORKSPACE, ETA_ERR_HIP = 4, 5, 6
DT_F32, DT_BF16 = 0, 1
GATED, RAW = 0, 1


class EtaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status} ({detail})")
        self.status = status


class EtaCacheStruct(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("block", c_int32), ("cap_tokens", c_int32), ("kv_dtype", c_int32),
                ("k", c_void_p), ("v", c_void_p), ("mu", c_void_p), ("var", c_void_p),
                ("maxnorm", c_void_p), ("seq_len", c_void_p)]


_P = ctypes.POINTER(EtaCacheStruct)
_SIGS = {
    "eta_abi_version": ([], c_int32),
    "eta_status_string": ([c_int32], ctypes.c_char_p),
    "eta_last_error": ([], ctypes.c_char_p),
    "eta_cache_blocks": ([_P], c_int32),
    "eta_append_kv": ([_P, c_void_p, c_void_p, c_void_p, c_void_p], c_int32),
    "eta_build_block_meta": ([_P, c_int32, c_int32, c_void_p], c_int32),
    "eta_predict_tau": ([c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_float,
                         c_void_p, c_void_p, c_void_p], c_int32),
    "eta_screen_workspace_bytes": ([c_int32, c_int32, c_int32], c_size_t),
    "eta_screen": ([_P, c_void_p, c_void_p, c_float, c_float, c_void_p, c_void_p, c_void_p,
                    c_void_p, c_size_t, c_void_p], c_int32),
    "eta_decode_workspace_bytes": ([c_int32, c_int32, c_int32, c_int32, c_int32], c_size_t),
    "eta_decode": ([_P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_float,
                    c_int32, c_void_p, c_size_t, c_void_p, c_void_p], c_int32),
    "eta_decode_noalloc": ([_P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                            c_float, c_int32, c_void_p, c_void_p], c_int32),
    "eta_dense_decode": ([_P, c_void_p, c_float, c_int32, c_void_p, c_size_t, c_void_p,
                          c_void_p], c_int32),
    "eta_fused_step_workspace_bytes": ([c_int32, c_int32, c_int32, c_int32, c_int32],
                                       c_size_t),
    "eta_fused_step": ([_P, c_void_p, c_void_p, c_void_p, c_float, c_float, c_int32, c_float,
                        c_float, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                        c_size_t, c_void_p, c_void_p], c_int32),
    "eta_calibrate_workspace_bytes": ([c_int32, c_int32, c_int32, c_int32], c_size_t),
    "eta_calibrate_threshold": ([_P, c_int32, c_void_p, c_void_p, c_float, c_float, c_float,
                                 c_void_p, c_size_t, c_void_p, c_void_p], c_int32),
    "eta_screen_gqa_workspace_bytes": ([c_int32, c_int32, c_int32], c_size_t),
    "eta_screen_gqa": ([_P, c_int32, c_void_p, c_void_p, c_float, c_float, c_void_p, c_void_p,
                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p], c_int32),
    "eta_decode_gqa_workspace_bytes": ([c_int32, c_int32, c_int32, c_int32, c_int32, c_int32],
                                       c_size_t),
    "eta_decode_gqa": ([_P, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                        c_float, c_float, c_int32, c_void_p, c_size_t, c_void_p, c_void_p],
                       c_int32),
    "eta_dense_decode_gqa": ([_P, c_int32, c_void_p, c_float, c_int32, c_void_p, c_size_t,
                              c_void_p, c_void_p], c_int32),
    "eta_gated_prefill": ([c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                           c_void_p, c_void_p, c_float, c_float, c_void_p, c_void_p, c_void_p],
                          c_int32),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libeta.so (built in-tree by ``long_context_decode_eta_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with "
                              "`python -m long_context_decode_eta_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def _check(status: int, fn: str) -> None:
    if status != ETA_OK:
        raise EtaError(status, fn, lib().eta_last_error().decode())


def _stream(stream) -> c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor | None, dtype=None, name: str = "tensor") -> c_void_p:
    if t is None:
        return c_void_p(None)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
class KVCache:
    """Device buffers of one layer's cache (layout as in include/eta.h)."""

    def __init__(self, batch, heads, head_dim, block, cap_tokens, kv_dtype=torch.bfloat16,
                 device="cuda", k=None, v=None):
        self.batch, self.heads, self.head_dim = batch, heads, head_dim
        self.block, self.cap_tokens = block, cap_tokens
        self.cap_blocks = -(-cap_tokens // block)
        self.kv_dtype = kv_dtype
        shape = (batch, heads, cap_tokens, head_dim)
        self.k = k if k is not None else torch.zeros(shape, dtype=kv_dtype, device=device)
        self.v = v if v is not None else torch.zeros(shape, dtype=kv_dtype, device=device)
        assert tuple(self.k.shape) == shape and tuple(self.v.shape) == shape
        assert self.k.dtype == kv_dtype and self.v.dtype == kv_dtype
        # block statistics: mu and var as bfloat16, maxnorm as float32
        self.mu = torch.zeros((batch, heads, self.cap_blocks, head_dim), dtype=torch.bfloat16,
                              device=device)
        self.var = torch.zeros_like(self.mu)
        self.maxnorm = torch.zeros((batch, heads, self.cap_blocks), dtype=torch.float32,
                                   device=device)
        self.seq_len = torch.zeros((batch,), dtype=torch.int32, device=device)
        # set to 1 by an append to a full sequence (never cleared by the library)
        self.overflow = torch.zeros((1,), dtype=torch.int32, device=device)

    def struct(self) -> EtaCacheStruct:
        dt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[self.kv_dtype]
        return EtaCacheStruct(
            self.batch, self.heads, self.head_dim, self.block, self.cap_tokens, dt,
            _dev(self.k, self.kv_dtype, "k"), _dev(self.v, self.kv_dtype, "v"),
            _dev(self.mu, torch.bfloat16, "mu"), _dev(self.var, torch.bfloat16, "var"),
            _dev(self.maxnorm, torch.float32, "maxnorm"),
            _dev(self.seq_len, torch.int32, "seq_len"))


def _ref(cache: KVCache):
    return ctypes.byref(cache.struct())


# ---------------------------------------------------------------------------
def append_kv(cache: KVCache, k_new, v_new, overflow=None, stream=None):
    """Append one token per sequence.  The capacity flag is required by the C
    call; without an explicit one the cache's own ``cache.overflow`` is used.
    A flagged sequence keeps its length, so its step must not be decoded."""
    if overflow is None:
        overflow = cache.overflow
    _check(lib().eta_append_kv(_ref(cache), _dev(k_new, cache.kv_dtype, "k_new"),
                               _dev(v_new, cache.kv_dtype, "v_new"),
                               _dev(overflow, torch.int32, "overflow"), _stream(stream)),
           "eta_append_kv")


def build_block_meta(cache: KVCache, first_block=0, n_blocks=-1, stream=None):
    _check(lib().eta_build_block_meta(_ref(cache), first_block, n_blocks, _stream(stream)),
           "eta_build_block_meta")


def predict_tau(q, W, bias_or_c, a, tau_gate, tau_screen, stream=None):
    B, H, D = q.shape
    _check(lib().eta_predict_tau(B, H, D, _dev(q, torch.float32, "q"),
                                 _dev(W, torch.float32, "W"),
                                 _dev(bias_or_c, torch.float32, "bias_or_c"), float(a),
                                 _dev(tau_gate, torch.float32, "tau_gate"),
                                 _dev(tau_screen, torch.float32, "tau_screen"), _stream(stream)),
           "eta_predict_tau")


def screen_workspace_bytes(batch, heads, cap_blocks) -> int:
    return int(lib().eta_screen_workspace_bytes(batch, heads, cap_blocks))


def screen(cache: KVCache, q, tau_screen, z, scale, active_idx, active_cnt, density_ctr,
           workspace, stream=None):
    _check(lib().eta_screen(_ref(cache), _dev(q, torch.float32, "q"),
                            _dev(tau_screen, torch.float32, "tau_screen"), float(z), float(scale),
                            _dev(active_idx, torch.int32, "active_idx"),
                            _dev(active_cnt, torch.int32, "active_cnt"),
                            _dev(density_ctr, None, "density_ctr"),
                            _dev(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream)),
           "eta_screen")


def decode_workspace_bytes(batch, heads, head_dim, cap_blocks, blocks_per_split) -> int:
    return int(lib().eta_decode_workspace_bytes(batch, heads, head_dim, cap_blocks,
                                                blocks_per_split))


def decode(cache: KVCache, q, tau_gate, active_idx, active_cnt, logit_mode, beta, scale,
           blocks_per_split, workspace, out, stream=None):
    _check(lib().eta_decode(_ref(cache), _dev(q, torch.float32, "q"),
                            _dev(tau_gate, torch.float32, "tau_gate"),
                            _dev(active_idx, torch.int32, "active_idx"),
                            _dev(active_cnt, torch.int32, "active_cnt"), int(logit_mode),
                            float(beta), float(scale), int(blocks_per_split),
                            _dev(workspace, None, "workspace"),
                            workspace.numel() * workspace.element_size(),
                            _dev(out, torch.float32, "out"), _stream(stream)),
           "eta_decode")


def decode_noalloc(cache: KVCache, q, tau_gate, active_idx, active_cnt, logit_mode, beta, scale,
                   blocks_per_split, out, stream=None):
    """eta_decode on the library's static device scratch (no workspace)."""
    _check(lib().eta_decode_noalloc(_ref(cache), _dev(q, torch.float32, "q"),
                                    _dev(tau_gate, torch.float32, "tau_gate"),
                                    _dev(active_idx, torch.int32, "active_idx"),
                                    _dev(active_cnt, torch.int32, "active_cnt"),
                                    int(logit_mode), float(beta), float(scale),
                                    int(blocks_per_split), _dev(out, torch.float32, "out"),
                                    _stream(stream)),
           "eta_decode_noalloc")


def dense_decode(cache: KVCache, q, scale, blocks_per_split, workspace, out, stream=None):
    _check(lib().eta_dense_decode(_ref(cache), _dev(q, torch.float32, "q"), float(scale),
                                  int(blocks_per_split), _dev(workspace, None, "workspace"),
                                  workspace.numel() * workspace.element_size(),
                                  _dev(out, torch.float32, "out"), _stream(stream)),
           "eta_dense_decode")


def calibrate_workspace_bytes(n_sets, batch, heads, cap_blocks) -> int:
    return int(lib().eta_calibrate_workspace_bytes(n_sets, batch, heads, cap_blocks))


def calibrate_threshold(cache: KVCache, q_sets, tau0, z, scale, target_density, workspace,
                        c_out, stream=None):
    _check(lib().eta_calibrate_threshold(_ref(cache), int(q_sets.shape[0]),
                                         _dev(q_sets, torch.float32, "q_sets"),
                                         _dev(tau0, torch.float32, "tau0"), float(z),
                                         float(scale), float(target_density),
                                         _dev(workspace, None, "workspace"),
                                         workspace.numel() * workspace.element_size(),
                                         _dev(c_out, torch.float32, "c_out"), _stream(stream)),
           "eta_calibrate_threshold")


# Grouped-query attention: the cache holds the KV heads, q and the thresholds
# hold kv_heads * group query heads (query head kv * group + g reads KV head kv).
def screen_gqa_workspace_bytes(batch, kv_heads, cap_blocks) -> int:
    return int(lib().eta_screen_gqa_workspace_bytes(batch, kv_heads, cap_blocks))


def screen_gqa(cache: KVCache, group, q, tau_screen, z, scale, union_idx, head_mask, union_cnt,
               density_ctr, workspace, stream=None):
    _check(lib().eta_screen_gqa(_ref(cache), int(group), _dev(q, torch.float32, "q"),
                                _dev(tau_screen, torch.float32, "tau_screen"), float(z),
                                float(scale), _dev(union_idx, torch.int32, "union_idx"),
                                _dev(head_mask, torch.int32, "head_mask"),
                                _dev(union_cnt, torch.int32, "union_cnt"),
                                _dev(density_ctr, None, "density_ctr"),
                                _dev(workspace, None, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "eta_screen_gqa")


def decode_gqa_workspace_bytes(batch, kv_heads, group, head_dim, cap_blocks,
                               blocks_per_split) -> int:
    return int(lib().eta_decode_gqa_workspace_bytes(batch, kv_heads, group, head_dim, cap_blocks,
                                                    blocks_per_split))


def decode_gqa(cache: KVCache, group, q, tau_gate, union_idx, head_mask, union_cnt, logit_mode,
               beta, scale, blocks_per_split, workspace, out, stream=None):
    _check(lib().eta_decode_gqa(_ref(cache), int(group), _dev(q, torch.float32, "q"),
                                _dev(tau_gate, torch.float32, "tau_gate"),
                                _dev(union_idx, torch.int32, "union_idx"),
                                _dev(head_mask, torch.int32, "head_mask"),
                                _dev(union_cnt, torch.int32, "union_cnt"), int(logit_mode),
                                float(beta), float(scale), int(blocks_per_split),
                                _dev(workspace, None, "workspace"),
                                workspace.numel() * workspace.element_size(),
                                _dev(out, torch.float32, "out"), _stream(stream)),
           "eta_decode_gqa")


def dense_decode_gqa(cache: KVCache, group, q, scale, blocks_per_split, workspace, out,
                     stream=None):
    _check(lib().eta_dense_decode_gqa(_ref(cache), int(group), _dev(q, torch.float32, "q"),
                                      float(scale), int(blocks_per_split),
                                      _dev(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _dev(out, torch.float32, "out"), _stream(stream)),
           "eta_dense_decode_gqa")


def gated_prefill(q, k, v, tau, group, beta, scale, out, dens=None, stream=None):
    """Gated causal attention forward over whole sequences: q [B][H_kv*G][T][d]
    bf16, k/v [B][H_kv][T][d] bf16, tau [B][H_kv*G][T] float32 -> out
    [B][H_kv*G][T][d] float32 and, if given, dens [B][H_kv*G][T] float32."""
    B, Hkv, T, D = k.shape
    _check(lib().eta_gated_prefill(B, Hkv, int(group), T, D, _dev(q, torch.bfloat16, "q"),
                                   _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                                   _dev(tau, torch.float32, "tau"), float(beta), float(scale),
                                   _dev(out, torch.float32, "out"),
                                   _dev(dens, torch.float32, "dens"), _stream(stream)),
           "eta_gated_prefill")


def fused_step_workspace_bytes(batch, heads, head_dim, cap_blocks, blocks_per_chunk) -> int:
    return int(lib().eta_fused_step_workspace_bytes(batch, heads, head_dim, cap_blocks,
                                                    blocks_per_chunk))


def fused_step(cache: KVCache, q, W, bias_or_c, a, z, logit_mode, beta, scale, blocks_per_chunk,
               tau_gate, tau_screen, chunk_bits, density_ctr, workspace, out, stream=None):
    _check(lib().eta_fused_step(_ref(cache), _dev(q, torch.float32, "q"),
                                _dev(W, torch.float32, "W"),
                                _dev(bias_or_c, torch.float32, "bias_or_c"), float(a), float(z),
                                int(logit_mode), float(beta), float(scale),
                                int(blocks_per_chunk), _dev(tau_gate, torch.float32, "tau_gate"),
                                _dev(tau_screen, torch.float32, "tau_screen"),
                                _dev(chunk_bits, torch.int32, "chunk_bits"),
                                _dev(density_ctr, None, "density_ctr"),
                                _dev(workspace, None, "workspace"),
                                workspace.numel() * workspace.element_size(),
                                _dev(out, torch.float32, "out"), _stream(stream)),
           "eta_fused_step")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A caller-owned byte workspace (torch allocation; 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def auto_split(units: int, cap_blocks: int, block: int, dense: bool = False) -> int:
    """blocks_per_split.  Sparse decode: the balanced kernel uses
    min(waves, ceil(N / split)) waves for N admitted blocks, so up to 512 keys
    per wave share keeps big jobs on every wave, and a small cache gets a
    smaller value (units*cap_blocks/4096) so that it still spreads over enough
    waves (32K x 16 heads, b=64: 2 blocks).  Dense baseline: chunks of up to
    2048 keys (units*cap_blocks/2048 for a small cache).  Chosen from sweeps
    on MI355X over the 32K..512K workloads."""
    if dense:
        return max(1, min(2048 // block, (units * cap_blocks) // 2048))
    return max(1, min(512 // block, (units * cap_blocks) // 4096))


def auto_fused_chunk(units: int, cap_blocks: int) -> int:
    """Blocks per chunk of the fused step: the largest of 32, 16, ..., 1 that
    still gives at least 256 work-groups (one per compute unit).  Swept on
    MI355X at 32K x 16 heads, b=64 (8192 blocks), 8 waves per chunk: 32
    blocks per chunk (256 work-groups) took 0.021 / 0.035 / 0.047 ms at 10 /
    38 / 70% density, 16 blocks 0.027 / 0.039 / 0.052 ms, 8 blocks 0.035 /
    0.049 / 0.060 ms (one work-group fits a compute unit at a time, so
    smaller chunks queue behind each other)."""
    for cb in (32, 16, 8, 4, 2):
        if units * (-(-cap_blocks // cb)) >= 256:
            return cb
    return 1


# Caches up to this many bytes of K+V take the fused screen + decode under
# path="auto": a step that small is dominated by its launches.  Measured on
# MI355X: at 32K x 16 heads (268 MB) the fused step takes 0.026 / 0.040 /
# 0.051 ms against 0.036 / 0.043 / 0.059 ms for screen -> decode at 10 / 38 /
# 70% density, while at 512K x 16 heads (4.3 GB) it loses (0.122 vs 0.118 ms
# at 10%, 0.323 vs 0.313 ms at 38%), as at 8 x 128K and on the ragged batch.
FUSED_MAX_KV_BYTES = 1 << 30


class Decoder:
    """One decode step over a cache with every buffer preallocated:
    predict_tau (skipped in frozen mode when tau is precomputed) -> screen ->
    decode (path "split"), or predict_tau -> the fused screen + decode (path
    "fused"); path "auto" takes the fused one for caches of at most
    FUSED_MAX_KV_BYTES of K+V.  Pure orchestration of the C entry points."""

    def __init__(self, cache: KVCache, *, z, scale=None, beta=5.0, a=0.0,
                 logit_mode=GATED, blocks_per_split=None, dense_blocks_per_split=None,
                 fused_blocks_per_chunk=None, path="split"):
        self.cache, self.z, self.beta, self.a = cache, float(z), float(beta), float(a)
        self.scale = float(scale) if scale is not None else float(
            torch.tensor(1.0 / cache.head_dim ** 0.5, dtype=torch.float32).item())
        B, H, D, nbc = cache.batch, cache.heads, cache.head_dim, cache.cap_blocks
        self.mode = logit_mode
        self.split = int(blocks_per_split or auto_split(B * H, nbc, cache.block))
        self.dense_split = int(dense_blocks_per_split or
                               auto_split(B * H, nbc, cache.block, dense=True))
        dev = cache.k.device
        self.tau_gate = torch.zeros((B, H), dtype=torch.float32, device=dev)
        self.tau_screen = torch.zeros_like(self.tau_gate)
        self.active_idx = torch.zeros((B, H, nbc), dtype=torch.int32, device=dev)
        self.active_cnt = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.density_ctr = torch.zeros((1,), dtype=torch.int64, device=dev)
        self.screen_ws = workspace(screen_workspace_bytes(B, H, nbc), dev)
        self.decode_ws = workspace(decode_workspace_bytes(
            B, H, D, nbc, min(self.split, self.dense_split)), dev)
        self.out = torch.zeros((B, H, D), dtype=torch.float32, device=dev)
        if path not in ("split", "fused", "auto"):
            raise ValueError(f"path must be 'split', 'fused' or 'auto', got {path!r}")
        if path == "auto":
            kv_bytes = 2 * B * H * cache.cap_tokens * D * cache.k.element_size()
            path = "fused" if kv_bytes <= FUSED_MAX_KV_BYTES else "split"
        self.path = path
        self.fused_chunk = int(fused_blocks_per_chunk or auto_fused_chunk(B * H, nbc))
        self.chunk_bits = torch.zeros((B, H, -(-nbc // self.fused_chunk)), dtype=torch.int32,
                                      device=dev)
        self.fused_ws = workspace(fused_step_workspace_bytes(B, H, D, nbc, self.fused_chunk),
                                  dev)

    def predict(self, q, W, bias_or_c, stream=None):
        predict_tau(q, W, bias_or_c, self.a, self.tau_gate, self.tau_screen, stream)

    def screen(self, q, stream=None):
        screen(self.cache, q, self.tau_screen, self.z, self.scale, self.active_idx,
               self.active_cnt, self.density_ctr, self.screen_ws, stream)

    def attend(self, q, stream=None):
        decode(self.cache, q, self.tau_gate, self.active_idx, self.active_cnt, self.mode,
               self.beta, self.scale, self.split, self.decode_ws, self.out, stream)

    def step(self, q, W=None, bias_or_c=None, stream=None):
        """One step on this Decoder's path.  Path "split" leaves the admitted
        lists in active_idx / active_cnt, path "fused" the admission bits of
        each chunk in chunk_bits."""
        if self.path == "fused":
            return self.step_fused(q, W, bias_or_c, stream)
        if bias_or_c is not None:
            self.predict(q, W, bias_or_c, stream)
        self.screen(q, stream)
        self.attend(q, stream)
        return self.out

    def step_fused(self, q, W=None, bias_or_c=None, stream=None):
        """eta_fused_step: thresholds (into tau_gate / tau_screen), screen
        and decode in two launches.  bias_or_c is required (the fused step
        always computes its thresholds)."""
        if bias_or_c is None:
            raise ValueError("the fused step needs bias_or_c (and W in dynamic mode)")
        fused_step(self.cache, q, W, bias_or_c, self.a, self.z, self.mode, self.beta, self.scale,
                   self.fused_chunk, self.tau_gate, self.tau_screen, self.chunk_bits,
                   self.density_ctr, self.fused_ws, self.out, stream)
        return self.out

    def dense(self, q, stream=None):
        dense_decode(self.cache, q, self.scale, self.dense_split, self.decode_ws, self.out, stream)
        return self.out


def auto_split_gqa(units: int, cap_blocks: int, block: int, dense: bool = False) -> int:
    """blocks_per_split of the grouped-query decode: the least union blocks
    of a wave's range, about 1024 keys (4096 dense), fewer for a small cache
    so the ranges still spread over the chip.  From sweeps on MI355X at 32 x
    128K, 4 KV heads, b = 64: 16 blocks at 57% and 19% union (vs 8 or 32), 64
    blocks dense."""
    if dense:
        return max(1, min(4096 // block, (units * cap_blocks) // 2048))
    return max(1, min(1024 // block, (units * cap_blocks) // 1024))


class GqaDecoder:
    """Grouped-query decode step with preallocated buffers: predict_tau over
    the query heads -> screen_gqa (per-head masks, union lists) ->
    decode_gqa.  ``density_ctr[0]`` accumulates admitted tokens over query
    heads, ``density_ctr[1]`` union tokens over KV heads."""

    def __init__(self, cache: KVCache, group: int, *, z, scale=None, beta=5.0, a=0.0,
                 logit_mode=GATED, blocks_per_split=None, dense_blocks_per_split=None):
        self.cache, self.group = cache, int(group)
        self.z, self.beta, self.a = float(z), float(beta), float(a)
        self.scale = float(scale) if scale is not None else float(
            torch.tensor(1.0 / cache.head_dim ** 0.5, dtype=torch.float32).item())
        B, Hkv, D, nbc = cache.batch, cache.heads, cache.head_dim, cache.cap_blocks
        Hq = Hkv * self.group
        self.mode = logit_mode
        self.split = int(blocks_per_split or auto_split_gqa(B * Hkv, nbc, cache.block))
        self.dense_split = int(dense_blocks_per_split or
                               auto_split_gqa(B * Hkv, nbc, cache.block, dense=True))
        dev = cache.k.device
        self.tau_gate = torch.zeros((B, Hq), dtype=torch.float32, device=dev)
        self.tau_screen = torch.zeros_like(self.tau_gate)
        self.union_idx = torch.zeros((B, Hkv, nbc), dtype=torch.int32, device=dev)
        self.head_mask = torch.zeros((B, Hkv, nbc), dtype=torch.int32, device=dev)
        self.union_cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        self.density_ctr = torch.zeros((2,), dtype=torch.int64, device=dev)
        self.screen_ws = workspace(screen_gqa_workspace_bytes(B, Hkv, nbc), dev)
        self.decode_ws = workspace(decode_gqa_workspace_bytes(
            B, Hkv, self.group, D, nbc, min(self.split, self.dense_split)), dev)
        self.out = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)

    def predict(self, q, W, bias_or_c, stream=None):
        predict_tau(q, W, bias_or_c, self.a, self.tau_gate, self.tau_screen, stream)

    def screen(self, q, stream=None):
        screen_gqa(self.cache, self.group, q, self.tau_screen, self.z, self.scale,
                   self.union_idx, self.head_mask, self.union_cnt, self.density_ctr,
                   self.screen_ws, stream)

    def attend(self, q, stream=None):
        decode_gqa(self.cache, self.group, q, self.tau_gate, self.union_idx, self.head_mask,
                   self.union_cnt, self.mode, self.beta, self.scale, self.split, self.decode_ws,
                   self.out, stream)

    def step(self, q, W=None, bias_or_c=None, stream=None):
        if bias_or_c is not None:
            self.predict(q, W, bias_or_c, stream)
        self.screen(q, stream)
        self.attend(q, stream)
        return self.out

    def dense(self, q, stream=None):
        dense_decode_gqa(self.cache, self.group, q, self.scale, self.dense_split,
                         self.decode_ws, self.out, stream)
        return self.out
