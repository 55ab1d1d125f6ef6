"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph around the
binding, which launches on torch's current stream and allocates nothing
when out= is given).  A graph of several steps, replayed several times with
eager work and synchronisations between the replays, must give every replay
bit for bit what the same steps give eagerly from the same state."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_graph_replays_equal_eager_steps():
    import gated_delta_rule_108_amd as kda
    spec = wl.DECODE["longctx_decode"]
    N, H, steps = 2, spec.H, 8
    mask = wl.mixture_low_channels(H, spec.dk, spec.seed)
    st = wl.make_decode_steps(spec, DEV, N=N, steps=steps, alpha_mask=mask)
    S = (0.1 * torch.randn(N, H, spec.dk, spec.dv, device=DEV)).contiguous()
    o = torch.empty(N, H, spec.dv, dtype=spec.dtype, device=DEV)
    outs = torch.empty(steps, N, H, spec.dv, dtype=spec.dtype, device=DEV)

    def run_steps(state, out_all):
        for i in range(steps):
            kda.decode_step(st["q"][i], st["k"][i], st["v"][i], st["alpha"][i], st["beta"][i],
                            state, out=o)
            out_all[i].copy_(o)

    run_steps(S.clone(), outs.clone())          # warm the library and the allocator
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_steps(S, outs)
    torch.cuda.synchronize()
    for rep in range(3):
        ref_S = S.clone()
        ref_o = torch.empty_like(outs)
        run_steps(ref_S, ref_o)                 # eager, from the same state
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device=DEV) * 2).sum()   # unrelated eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}: state max diff {float((S - ref_S).abs().max()):.3e}", flush=True)
        assert torch.equal(outs, ref_o), rep
        assert torch.equal(S, ref_S), rep
