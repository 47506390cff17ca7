"""eta_decode_noalloc (the decode on the library's static device scratch,
for callers that cannot allocate) against eta_decode through the C ABI: the
same kernels on the same inputs, so the outputs must be bit-identical.  Two
calls in a row, the second on a smaller problem (the scratch keeps the first
call's contents), then a repeat of the first.  (The host-side refusal of a problem beyond
the scratch is in the C-ABI tests.)"""
import pytest
import torch

from long_context_decode_eta_amd import binding as eb
from long_context_decode_eta_amd import synth
from parity import make_cache, note, to_gpu

pytestmark = pytest.mark.gpu


def _case(seed, B, H, T, block, mode):
    w = to_gpu(synth.make("ragged", seed=seed, T=T, B=B, H=H, cap=max(T) if isinstance(T, list)
                          else T[1], block=block, pad="nan"))
    cache = make_cache(w)
    eb.build_block_meta(cache)
    dec = eb.Decoder(cache, z=w.z, scale=w.scale, logit_mode=mode)
    c = torch.linspace(0.2, 1.0, H, device="cuda")
    dec.predict(w.q, None, c)
    dec.screen(w.q)
    dec.attend(w.q)  # eta_decode with a workspace
    torch.cuda.synchronize()
    return w, cache, dec, dec.out.clone()


def _noalloc(w, cache, dec):
    out = torch.full_like(dec.out, float("nan"))
    eb.decode_noalloc(cache, w.q, dec.tau_gate, dec.active_idx, dec.active_cnt, dec.mode,
                      dec.beta, dec.scale, dec.split, out)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_decode_on_two_calls():
    note("[gpu] noalloc: 12 x 16 streams, 1..20000 keys, b 32, gated")
    big = _case(5, 12, 16, (1, 20000), 32, eb.GATED)
    note("[gpu] noalloc: 3 x 4 streams, 1..3000 keys, b 16, raw")
    small = _case(6, 3, 4, (1, 3000), 16, eb.RAW)
    for name, (w, cache, dec, ref) in (("first", big), ("second, smaller", small),
                                       ("first again", big)):
        got = _noalloc(w, cache, dec)
        assert not torch.isnan(got).any(), name
        assert torch.equal(got, ref), f"{name}: differs from eta_decode"
        dens = float(dec.active_cnt.sum()) / max(1, int(cache.cap_blocks) * w.B * w.H)
        note(f"  {name}: {w.B} x {w.H} streams, bit-identical to eta_decode "
             f"(block share {dens:.3f})")
