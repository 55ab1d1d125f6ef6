"""The step adjoint on the GPU (kda_decode_step_backward) against the float64
oracle (oracle.kda_decode_step_backward, pinned by finite differences in
tests/test_backward_pins.py).  Same inputs on both sides; relative Frobenius
error per gradient; 1e-4 for fp32 inputs and 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

from oracle import kda_decode_step, kda_decode_step_backward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS")


def kda():
    import gated_delta_rule_108_amd as m
    return m


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def f64(t):
    return t.detach().to("cpu").double().numpy()


def make(seed, N, H, dk, dv, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(N, H, dk, generator=g)
    k = torch.randn(N, H, dk, generator=g)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    return dict(q=q, k=k, v=torch.randn(N, H, dv, generator=g).to(dtype),
                alpha=0.8 + 0.2 * torch.rand(N, H, dk, generator=g),
                beta=torch.rand(N, H, generator=g),
                S=0.1 * torch.randn(N, H, dk, dv, generator=g),
                dO=torch.randn(N, H, dv, generator=g).to(dtype),
                dS_new=torch.randn(N, H, dk, dv, generator=g))


def run(x, in_place=False):
    d = {k: t.to(DEV) for k, t in x.items()}
    out = kda().decode_step_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S"],
                                     d["dO"], d["dS_new"], in_place=in_place)
    torch.cuda.synchronize()
    return out


def oracle(x):
    return kda_decode_step_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S"],
                                    x["dO"], x["dS_new"])


@pytest.mark.parametrize("dk,dv,N,H,dtype", [
    (16, 16, 3, 2, torch.float32), (32, 128, 2, 5, torch.float32), (128, 16, 1, 3, torch.float32),
    (64, 32, 2, 2, torch.float32), (16, 128, 3, 1, torch.bfloat16), (64, 64, 4, 4, torch.bfloat16),
    (128, 128, 2, 3, torch.bfloat16), (128, 128, 64, 32, torch.bfloat16),
])
def test_step_adjoint(dk, dv, N, H, dtype):
    x = make(dk + 3 * dv + N, N, H, dk, dv, dtype)
    got = run(x)
    ref = oracle(x)
    errs = {n: rel(f64(g), r) for n, g, r in zip(NAMES, got, ref)}
    print(f"[step adjoint dk={dk} dv={dv} {dtype}] " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert max(errs.values()) < TOL[dtype], errs


def test_in_place_equals_out_of_place():
    x = make(5, 4, 3, 128, 128, torch.bfloat16)
    a = run(x)
    b = run(x, in_place=True)
    for g1, g2 in zip(a, b):
        assert torch.equal(g1, g2)


def test_chained_steps_give_the_sequence_gradient():
    """Twelve decode steps forward (states kept), then the adjoint applied
    backwards: every per-token gradient and the initial state's gradient
    match the oracle's chain."""
    T, N, H, dk, dv = 12, 2, 4, 128, 64
    g = torch.Generator().manual_seed(9)
    xs = [make(100 + t, N, H, dk, dv, torch.float32) for t in range(T)]
    S0 = 0.1 * torch.randn(N, H, dk, dv, generator=g)
    dST = torch.randn(N, H, dk, dv, generator=g)
    states = [S0]
    for t in range(T):
        _, S = kda_decode_step(xs[t]["q"], xs[t]["k"], xs[t]["v"], xs[t]["alpha"], xs[t]["beta"],
                               states[-1])
        states.append(torch.from_numpy(S).float())
    dS_g = dST.to(DEV)
    dS_r = dST.double().numpy()
    worst = 0.0
    for t in reversed(range(T)):
        x = dict(xs[t], S=states[t])
        d = {k: v.to(DEV) for k, v in x.items()}
        got = kda().decode_step_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S"],
                                         d["dO"], dS_g)
        ref = kda_decode_step_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S"],
                                       x["dO"], dS_r)
        torch.cuda.synchronize()
        worst = max(worst, *(rel(f64(a), b) for a, b in zip(got[:5], ref[:5])))
        dS_g, dS_r = got[5], ref[5]
    es = rel(f64(dS_g), dS_r)
    print(f"[chained adjoint T={T}] worst per-token rel={worst:.2e} dS0 rel={es:.2e}", flush=True)
    assert worst < 1e-4 and es < 1e-4


@pytest.mark.parametrize("gated,dk,dv,N,H,dtype", [
    (True, 16, 16, 3, 2, torch.float32), (True, 128, 32, 2, 3, torch.float32),
    (False, 64, 128, 2, 2, torch.float32), (True, 128, 128, 4, 8, torch.bfloat16),
    (False, 32, 64, 3, 3, torch.bfloat16),
])
def test_gdn_step_adjoint(gated, dk, dv, N, H, dtype):
    """Gated DeltaNet (one gate per head) and DeltaNet (none) against
    oracle.gdn_decode_step_backward; the gate's gradient sums every row of
    the head."""
    from oracle import gdn_decode_step_backward
    x = make(dk + dv + N + 7, N, H, dk, dv, dtype)
    a = (0.8 + 0.2 * torch.rand(N, H, generator=torch.Generator().manual_seed(N))) if gated \
        else None
    d = {k: t.to(DEV) for k, t in x.items()}
    got = kda().gdn_decode_step_backward(d["q"], d["k"], d["v"], None if a is None else a.to(DEV),
                                         d["beta"], d["S"], d["dO"], d["dS_new"])
    torch.cuda.synchronize()
    ref = gdn_decode_step_backward(x["q"], x["k"], x["v"], a, x["beta"], x["S"], x["dO"],
                                   x["dS_new"])
    assert (got[3] is None) == (ref[3] is None) == (not gated)
    errs = {n: rel(f64(g), r) for n, g, r in zip(NAMES, got, ref) if r is not None}
    print(f"[gdn step adjoint gated={gated} dk={dk} dv={dv} {dtype}] " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert max(errs.values()) < TOL[dtype], errs
