"""The prefill backward on the GPU (kda_prefill_backward) against the
float64 oracle (oracle.kda_prefill_backward, pinned by finite differences of
the prefill recurrence in tests/test_backward_pins.py).  Same inputs on both
sides (bf16 values upcast exactly); relative Frobenius error per gradient,
1e-4 for fp32 inputs and 2e-2 for bf16 inputs.  Sizes span several 16-token
pieces with a ragged last piece, every key/value width, both optional
states, T = 0 and T = 1, and the full B = 1, H = 16, T = 4096, d = 128 bf16
workload checked on sampled heads (heads are independent chains)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import kda_prefill_backward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def kda():
    import gated_delta_rule_108_amd as m
    return m


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def f64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


def spec_of(dk, dv, dtype, alpha_kind="softplus", s0_std=0.1):
    base = wl.PREFILL["prefill_h16_t4k"]
    return dataclasses.replace(base, name=f"bwd_{dk}_{dv}", dk=dk, dv=dv, dtype=dtype,
                               alpha_kind=alpha_kind, s0_std=s0_std)


def run_case(spec, B, T, H, with_dST=True, heads=None):
    print(f"case {spec.name} {spec.dtype} B={B} T={T} H={H} dST={with_dST}", flush=True)
    x = wl.make_prefill_inputs(spec, "cpu", T=T, B=B, H=H)
    gr = wl.make_prefill_backward_grads(spec, "cpu", T=T, B=B, H=H, with_dST=with_dST)
    g = {n: (None if t is None else t.to(DEV)) for n, t in {**x, **gr}.items()}
    out = kda().prefill_backward(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["dO"],
                                 S0=g["S0"], dS_T=g["dS_T"])
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else heads
    sl = lambda t, st=False: None if t is None else (t[:, hs] if st else t[:, :, hs])  # noqa: E731
    ref = kda_prefill_backward(*(f64(sl(x[n])) for n in ("q", "k", "v", "alpha", "beta")),
                               f64(sl(x["S0"], True)), f64(sl(gr["dO"])),
                               f64(sl(gr["dS_T"], True)))
    got = [sl(t) for t in out[:5]] + [sl(out[5], True)]
    errs = {n: rel(f64(a), b) for n, a, b in zip(NAMES, got, ref)}
    for n, a in zip(NAMES, got):
        assert torch.isfinite(a).all(), n
    print("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    tol = TOL[spec.dtype]
    assert all(e < tol for e in errs.values()), errs
    return errs


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16),
                                   (16, 128)])
def test_fp32_widths(dk, dv):
    run_case(spec_of(dk, dv, torch.float32), B=2, T=37, H=2)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 48, 100])
def test_fp32_lengths(T):
    run_case(spec_of(64, 64, torch.float32), B=1, T=T, H=3)


def test_fp32_optional_states():
    run_case(spec_of(32, 32, torch.float32, s0_std=0.0), B=2, T=40, H=2, with_dST=False)
    run_case(spec_of(32, 32, torch.float32, s0_std=0.0), B=1, T=40, H=2, with_dST=True)
    run_case(spec_of(32, 32, torch.float32), B=1, T=40, H=2, with_dST=False)


def test_fp32_mixture_gates():
    # channels that forget fast next to slow ones (the long-context gate mix)
    run_case(spec_of(128, 128, torch.float32, alpha_kind="mixture"), B=1, T=70, H=2)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_bf16(dk, dv):
    errs = run_case(spec_of(dk, dv, torch.bfloat16), B=2, T=90, H=2)
    # arithmetic is fp32 on exact bf16 inputs: far inside the bf16 bar
    assert max(errs.values()) < 1e-4, errs


def test_no_tokens_passes_the_state_gradient_through():
    m = kda()
    B, H, d = 2, 3, 32
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device=DEV)  # noqa: E731
    dST = torch.randn(B, H, d, d, device=DEV)
    out = m.prefill_backward(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d),
                             z(B, 0, H), z(B, 0, H, d), S0=None, dS_T=dST)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dST)
    out = m.prefill_backward(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d),
                             z(B, 0, H), z(B, 0, H, d))
    torch.cuda.synchronize()
    assert torch.equal(out[5], torch.zeros_like(dST))


def test_repeat_calls_agree():
    # the float atomics may change the last bits only
    spec = spec_of(128, 128, torch.bfloat16)
    x = wl.make_prefill_inputs(spec, DEV, T=64, B=1, H=4)
    gr = wl.make_prefill_backward_grads(spec, DEV, T=64, B=1, H=4)
    a = kda().prefill_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                               S0=x["S0"], dS_T=gr["dS_T"])
    b = kda().prefill_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                               S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    for n, s, t in zip(NAMES, a, b):
        assert rel(f64(s), f64(t)) < 1e-6, n
    assert torch.equal(a[2], b[2]) and torch.equal(a[5], b[5])   # no atomics in dv, dS0


def test_full_workload_sampled_heads():
    """B = 1, H = 16, T = 4096, d = 128, bf16: the whole launch on the GPU,
    the oracle on heads 0 and 11."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    run_case(spec, B=1, T=spec.T, H=spec.H, heads=[0, 11])


def test_state_gradient_in_place_through_the_abi():
    """dS0 written over dS_T (the one overlap the call accepts) equals the
    out-of-place result bit for bit (dS0 takes no atomics)."""
    import ctypes
    from gated_delta_rule_108_amd import _lib
    m = kda()
    spec = spec_of(64, 64, torch.float32)
    x = wl.make_prefill_inputs(spec, DEV, T=40, B=1, H=2)
    gr = wl.make_prefill_backward_grads(spec, DEV, T=40, B=1, H=2)
    ref = m.prefill_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                             S0=x["S0"], dS_T=gr["dS_T"])
    L = m.lib()
    outs = [torch.empty_like(t) for t in ref[:5]]
    dS = gr["dS_T"].clone()
    nws = m.prefill_backward_workspace_bytes(1, 40, 2, 64, 64)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.kda_prefill_backward(p(x["q"]), p(x["k"]), p(x["v"]), p(x["alpha"]), p(x["beta"]),
                                p(x["S0"]), p(gr["dO"]), p(dS), *[p(o) for o in outs], p(dS),
                                1, 40, 2, 64, 64, _lib.KDA_F32, p(ws), nws,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == _lib.KDA_OK
    assert torch.equal(dS, ref[5])
    assert torch.equal(outs[2], ref[2])


@pytest.mark.parametrize("gated,dk,dv,dtype,T", [(True, 64, 32, torch.float32, 37),
                                                (True, 16, 16, torch.float32, 16),
                                                (False, 32, 32, torch.float32, 41),
                                                (True, 128, 128, torch.bfloat16, 70),
                                                (False, 128, 128, torch.bfloat16, 33)])
def test_gdn_backward(gated, dk, dv, dtype, T):
    """Gated DeltaNet (one gate per token and head) and DeltaNet (no gate)
    against oracle.gdn_prefill_backward."""
    from oracle import gdn_prefill_backward
    print(f"gdn backward gated={gated} dk={dk} dv={dv} {dtype} T={T}", flush=True)
    spec = spec_of(dk, dv, dtype)
    x = wl.make_gdn_inputs(spec, "cpu", T=T, B=2, H=2, gated=gated)
    gr = wl.make_prefill_backward_grads(spec, "cpu", T=T, B=2, H=2)
    g = {n: (None if t is None else t.to(DEV)) for n, t in {**x, **gr}.items()}
    out = kda().gdn_prefill_backward(g["q"], g["k"], g["v"], g["a"], g["beta"], g["dO"],
                                     S0=g["S0"], dS_T=g["dS_T"])
    torch.cuda.synchronize()
    ref = gdn_prefill_backward(*(f64(x[n]) for n in ("q", "k", "v", "a", "beta", "S0")),
                               f64(gr["dO"]), f64(gr["dS_T"]))
    names = ("dq", "dk", "dv", "da", "dbeta", "dS0")
    assert (out[3] is None) == (ref[3] is None) == (not gated)
    errs = {n: rel(f64(a), r) for n, a, r in zip(names, out, ref) if r is not None}
    print("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    assert all(e < TOL[dtype] for e in errs.values()), errs


def test_largest_workload_sampled_chains():
    """B = 8, H = 32, T = 8192, d = 128, bf16 (4096 workgroups in 16 rounds):
    the whole launch on the GPU, the oracle on two chains (b, h) = (3, 17)
    and (7, 0), each its own independent slice of the inputs."""
    spec = wl.PREFILL["prefill_b8_h32_t8k"]
    print(f"case {spec.name} full size", flush=True)
    x = wl.make_prefill_inputs(spec, DEV)
    gr = wl.make_prefill_backward_grads(spec, DEV)
    out = kda().prefill_backward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                                 S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    for b, h in ((3, 17), (7, 0)):
        tok = lambda t: f64(t[b:b + 1, :, h:h + 1])   # noqa: E731
        st = lambda t: None if t is None else f64(t[b:b + 1, h:h + 1])   # noqa: E731
        ref = kda_prefill_backward(tok(x["q"]), tok(x["k"]), tok(x["v"]), tok(x["alpha"]),
                                   tok(x["beta"]), st(x["S0"]), tok(gr["dO"]), st(gr["dS_T"]))
        got = [tok(t) for t in out[:5]] + [st(out[5])]
        errs = {n: rel(a, r) for n, a, r in zip(NAMES, got, ref)}
        print(f"  chain ({b},{h}): " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()),
              flush=True)
        assert all(e < TOL[spec.dtype] for e in errs.values()), errs
