"""The prologue's forward and adjoint kernels (kda_prologue_forward,
kda_prologue_backward) and the backward from raw projections (prologue
forward, prefill backward, prologue adjoint) on the GPU, against the float64
oracle (oracle.kda_prologue, oracle.kda_prologue_backward,
oracle.kda_prefill_backward_logits; pinned by finite differences in
tests/test_prologue_backward_pins.py).  Same inputs on both sides; relative
Frobenius error per output; 1e-4 for fp32 I/O and 2e-2 for bf16 (the mapped
q and k are written in the I/O type, and SiLU output is rounded to it before
the norm, as in the fused forward)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import kda_prologue
from oracle.kda_backward import kda_prefill_backward_logits, kda_prologue_backward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
MAPS = {"as_given": 0, "l2": 1, "silu_l2": 2}


def kda():
    import gated_delta_rule_108_amd as m
    return m


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def f64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


def spec_of(dk, dv, dtype):
    base = wl.PREFILL["prefill_h16_t4k"]
    return dataclasses.replace(base, name=f"pro_{dk}_{dv}", dk=dk, dv=dv, dtype=dtype, s0_std=0.1)


def raw(spec, T, H, zero_row=False):
    x = wl.make_prefill_logit_inputs(spec, "cpu", T=T, B=1, H=H)
    if zero_row:                     # a zero query and key row: the norm floor
        x["q"][0, 0, 0].zero_()
        x["k"][0, 0, 0].zero_()
    return x


@pytest.mark.parametrize("qk_map", sorted(MAPS))
@pytest.mark.parametrize("dk,dtype", [(16, torch.float32), (64, torch.float32),
                                      (128, torch.float32), (128, torch.bfloat16),
                                      (32, torch.bfloat16)])
def test_prologue_forward(qk_map, dk, dtype):
    print(f"prologue forward {qk_map} dk={dk} {dtype}", flush=True)
    x = raw(spec_of(dk, 16, dtype), T=37, H=3, zero_row=True)    # 111 rows: a ragged block
    g = {n: t.to(DEV) for n, t in x.items() if t is not None}
    out = kda().prologue_forward(g["q"], g["k"], g["g"], g["b"], qk_map)
    torch.cuda.synchronize()
    ref = kda_prologue(f64(x["q"]), f64(x["k"]), f64(x["g"]), f64(x["b"]), MAPS[qk_map])
    for name, a, r in zip(("q_hat", "k_hat", "alpha", "beta"), out, ref):
        tol = TOL[dtype] if name in ("q_hat", "k_hat") else 1e-5
        assert rel(f64(a), r) < tol, (name, rel(f64(a), r))
    assert torch.equal(out[0][0, 0, 0], torch.zeros_like(out[0][0, 0, 0]))


@pytest.mark.parametrize("qk_map", sorted(MAPS))
@pytest.mark.parametrize("dk,dtype", [(16, torch.float32), (128, torch.float32),
                                      (128, torch.bfloat16), (64, torch.bfloat16)])
def test_prologue_backward(qk_map, dk, dtype):
    print(f"prologue backward {qk_map} dk={dk} {dtype}", flush=True)
    x = raw(spec_of(dk, 16, dtype), T=37, H=3)
    gen = torch.Generator().manual_seed(dk + 7)
    dqh = torch.randn(x["q"].shape, generator=gen)
    dkh = torch.randn(x["q"].shape, generator=gen)
    da = torch.randn(x["q"].shape, generator=gen)
    dbe = torch.randn(x["b"].shape, generator=gen)
    g = {n: t.to(DEV) for n, t in x.items() if t is not None}
    out = kda().prologue_backward(g["q"], g["k"], g["g"], g["b"], dqh.to(DEV), dkh.to(DEV),
                                  da.to(DEV), dbe.to(DEV), qk_map)
    torch.cuda.synchronize()
    ref = kda_prologue_backward(f64(x["q"]), f64(x["k"]), f64(x["g"]), f64(x["b"]), f64(dqh),
                                f64(dkh), f64(da), f64(dbe), MAPS[qk_map])
    for name, a, r in zip(("dq", "dk", "dg", "db"), out, ref):
        assert rel(f64(a), r) < TOL[dtype], (name, rel(f64(a), r))


@pytest.mark.parametrize("qk_map,dk,dv,dtype,T", [("l2", 32, 32, torch.float32, 40),
                                                 ("silu_l2", 64, 32, torch.float32, 33),
                                                 ("as_given", 16, 16, torch.float32, 17),
                                                 ("l2", 128, 128, torch.bfloat16, 70),
                                                 ("silu_l2", 128, 128, torch.bfloat16, 50)])
def test_backward_from_raw_projections(qk_map, dk, dv, dtype, T):
    print(f"backward from raw projections {qk_map} dk={dk} dv={dv} {dtype} T={T}", flush=True)
    spec = spec_of(dk, dv, dtype)
    x = raw(spec, T=T, H=2)
    gr = wl.make_prefill_backward_grads(spec, "cpu", T=T, B=1, H=2)
    g = {n: (None if t is None else t.to(DEV)) for n, t in {**x, **gr}.items()}
    out = kda().prefill_backward_logits(g["q"], g["k"], g["v"], g["g"], g["b"], g["dO"],
                                        S0=g["S0"], dS_T=g["dS_T"], qk_map=qk_map)
    torch.cuda.synchronize()
    ref = kda_prefill_backward_logits(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]),
                                      f64(x["b"]), f64(x["S0"]), f64(gr["dO"]), f64(gr["dS_T"]),
                                      MAPS[qk_map])
    errs = {n: rel(f64(a), r) for n, a, r in zip(("dq", "dk", "dv", "dg", "db", "dS0"), out, ref)}
    print("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    assert all(e < TOL[dtype] for e in errs.values()), errs
