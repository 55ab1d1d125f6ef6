"""kda_prefill_chunked_noalloc on the GPU, through the C ABI: its outputs
against kda_prefill_chunked's on the same inputs, on calls in a row (the
second smaller than the first, so the shared scratch array holds the first
call's records when the second starts), and against the float64 oracle on a
head."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import kda_recurrence
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def kda():
    import gated_delta_rule_108_amd as m
    return m


def noalloc(g, C, o, S_T):
    """One kda_prefill_chunked_noalloc call through ctypes on preallocated
    outputs; returns the status."""
    lib = kda().lib()
    B, T, H, dk = g["q"].shape
    dv = g["v"].shape[-1]
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.kda_prefill_chunked_noalloc(p(g["q"]), p(g["k"]), p(g["v"]), p(g["alpha"]),
                                           p(g["beta"]), p(g["S0"]), p(o), p(S_T), B, T, H, dk,
                                           dv, C, 1, stream)


def reference(g, C):
    o, S = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"],
                                 chunk=C)
    torch.cuda.synchronize()
    return o, S


def one(label, spec, C, **shape):
    print(f"[noalloc] {label}: {shape} C={C}", flush=True)
    g = {k: (None if t is None else t.to(DEV))
         for k, t in wl.make_prefill_inputs(spec, **shape).items()}
    B, T, H, dk = g["q"].shape
    dv = g["v"].shape[-1]
    o = torch.full((B, T, H, dv), float("nan"), dtype=g["q"].dtype, device=DEV)
    S_T = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=DEV)
    st = noalloc(g, C, o, S_T)
    assert st == 0, kda().lib().kda_status_string(st)
    torch.cuda.synchronize()
    o_ref, S_ref = reference(g, C)
    assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref), label
    h = H - 1
    sl = {k: g[k][:, :, h:h + 1].contiguous().cpu() for k in ("q", "k", "v", "alpha", "beta")}
    sl["S0"] = None if g["S0"] is None else g["S0"][:, h:h + 1].contiguous().cpu()
    o64, S64 = kda_recurrence(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"], sl["S0"])
    parity.report(f"noalloc {label}, head {h}", 2e-2,
                  o[:, :, h:h + 1].double().cpu().numpy(), o64,
                  S_T[:, h:h + 1].double().cpu().numpy(), S64)
    return g


def test_noalloc_equals_the_workspace_call_on_calls_in_a_row():
    spec = wl.PREFILL["prefill_h16_t4k"]
    lib = kda().lib()
    # the first call needs more records than the scratch holds in one
    # segment (16 heads x 64 chunks x 74,240 B = 76 MB): more segments than
    # the workspace call, bit-identical results
    assert lib.kda_prefill_workspace_bytes(1, 4096, 16, 128, 128, 64, 1) > 64 << 20
    one("H=16 T=4096", spec, 64)
    # a smaller call right after it, on the scratch the first one filled
    one("H=4 T=1000", spec, 64, T=1000, H=4)
    # more chains than the record path takes: the fused kernel, no scratch
    one("B=3 H=48 T=130 (fused)", wl.PREFILL["prefill_b8_h32_t8k"], 64, T=130, B=3, H=48)
    # T = 0 copies the initial state
    g = {k: (None if t is None else t.to(DEV))
         for k, t in wl.make_prefill_inputs(wl.PREFILL["prefill_b8_h32_t8k"], T=0, B=1,
                                            H=2).items()}
    S_T = torch.empty(1, 2, 128, 128, device=DEV)
    o = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device=DEV)
    assert noalloc(g, 64, o, S_T) == 0
    torch.cuda.synchronize()
    assert torch.equal(S_T, g["S0"])


def test_noalloc_binding_and_chunk_sizes():
    """The binding's prefill_chunked_noalloc, the C = 16 and 32 record paths
    and C = 128, each against the workspace call."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    for C in (16, 32, 128):
        print(f"[noalloc] binding C={C}", flush=True)
        g = {k: (None if t is None else t.to(DEV))
             for k, t in wl.make_prefill_inputs(spec, T=700, H=5).items()}
        o, S = kda().prefill_chunked_noalloc(g["q"], g["k"], g["v"], g["alpha"], g["beta"],
                                             g["S0"], chunk=C)
        torch.cuda.synchronize()
        o_ref, S_ref = reference(g, C)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), C
    assert np.isfinite(o.float().cpu().numpy()).all()
