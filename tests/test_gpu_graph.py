"""A decode step captured in a HIP graph reproduces the eager step exactly.

The step (threshold, screen, decode and combine kernels) records no memset:
every buffer a kernel reads was written earlier in the same step (the density
counter only accumulates), and the decode keeps no state between calls.
The graph is replayed several times with eager work and synchronisations in
between, and every replay is compared bit for bit with the eager result.
"""
import pytest
import torch

from long_context_decode_eta_amd import binding as eb
from long_context_decode_eta_amd import synth
from parity import make_cache, note, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,split", [("ctx128k", 16), ("ragged", 32)])
def test_graph_replay_matches_eager(name, split):
    note(f"[gpu] graph replay {name}")
    T = (2000, 20000) if name == "ragged" else 20000
    w = to_gpu(synth.make(name, seed=77, T=T, B=4, cap=20000))
    cache = make_cache(w)
    eb.build_block_meta(cache)
    H = w.H
    c = torch.linspace(0.5, 1.5, H, device="cuda")
    dec = eb.Decoder(cache, z=w.z, scale=w.scale, blocks_per_split=split)

    def step():
        dec.predict(w.q, w.W, c)
        dec.screen(w.q)
        dec.attend(w.q)

    step()
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_cnt = dec.out.clone(), dec.active_idx.clone(), dec.active_cnt.clone()
    ctr0 = int(dec.density_ctr.item())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ctr1 = int(dec.density_ctr.item())
    ws2 = eb.workspace(eb.decode_workspace_bytes(w.B, H, w.D, cache.cap_blocks, 8))
    other = torch.empty_like(dec.out)
    for rep in range(4):
        dec.out.fill_(float("nan"))
        dec.active_cnt.zero_()
        eb.dense_decode(cache, w.q, w.scale, 8, ws2, other)  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out, ref_out), f"replay {rep}"
        assert torch.equal(dec.active_cnt, ref_cnt)
        for b in range(w.B):
            for h in range(H):
                n = int(ref_cnt[b, h])
                assert torch.equal(dec.active_idx[b, h, :n], ref_idx[b, h, :n])
    # capture does not execute; each replay adds one step's admitted tokens
    assert ctr1 == ctr0
    assert int(dec.density_ctr.item()) - ctr1 == 4 * ctr0, "density counter per replay"
