"""Gated DeltaNet (one gate per token and head) and DeltaNet (no gate) on the
GPU (kda_gdn_prefill_chunked, kda_gdn_decode_step) against the float64
oracle (oracle.gdn_recurrence: the KDA recurrence with the gate repeated on
every key channel, pinned in tests/test_gdn_pins.py).

Each case draws its inputs once (seeded), hands the same tensors to the HIP
path through the C ABI binding and, upcast to float64, to the oracle.  Error:
relative Frobenius norm, separately for o and the state; bar 1e-4 for fp32
inputs and 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity
from oracle import gdn_decode_step, gdn_recurrence

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def kda():
    import gated_delta_rule_108_amd as m
    return m


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def f64(t):
    return t.detach().to("cpu").double().numpy()


def run(inp, C):
    d = {k: (None if t is None else t.to(DEV)) for k, t in inp.items()}
    o, S = kda().gdn_prefill_chunked(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], chunk=C)
    torch.cuda.synchronize()
    return o, S


def oracle(inp):
    return gdn_recurrence(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["S0"])


def check(inp, C, label=""):
    tol = TOL[inp["q"].dtype]
    o, S = run(inp, C)
    o_ref, S_ref = oracle(inp)
    parity.report(f"{label} C={C} gate={'scalar' if inp['a'] is not None else 'none'}", tol,
                  f64(o), o_ref, f64(S), S_ref)


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("C", [16, 32])
def test_tiny_fp32(gated, C):
    check(wl.make_gdn_inputs(wl.PREFILL["tiny_fp32"], gated=gated), C, label="tiny fp32")


@pytest.mark.parametrize("gated,C", [(True, 64), (False, 64), (True, 128)])
def test_prefill_h16_t4k(gated, C):
    """The H=16, T=4096 workload's shape in full (split path)."""
    check(wl.make_gdn_inputs(wl.PREFILL["prefill_h16_t4k"], gated=gated), C, label="h16 t4k")


@pytest.mark.parametrize("gated", [True, False])
def test_fused_and_split_paths(gated):
    spec = wl.PREFILL["prefill_b8_h32_t8k"]
    big = wl.make_gdn_inputs(spec, T=160, B=33, H=4, gated=gated)
    assert kda().prefill_workspace_bytes(33, 160, 4, 128, 128, 64) == 0
    o_big, S_big = run(big, 64)
    few = {k: (v[3:4].contiguous() if v is not None else v) for k, v in big.items()}
    o_few, S_few = run(few, 64)
    o_ref, S_ref = oracle(few)
    for o, S in ((o_big[3:4], S_big[3:4]), (o_few, S_few)):
        parity.report("gdn paths", 2e-2, f64(o), o_ref, f64(S), S_ref)


@pytest.mark.parametrize("dk,dv,dtype,C,T", [
    (16, 16, torch.float32, 16, 77), (32, 64, torch.float32, 32, 45),
    (64, 128, torch.float32, 16, 100), (16, 32, torch.bfloat16, 16, 200),
    (64, 32, torch.bfloat16, 64, 77), (128, 64, torch.bfloat16, 32, 1),
    (128, 128, torch.bfloat16, 64, 131),
])
def test_head_dims_and_ragged_lengths(dk, dv, dtype, C, T):
    spec = wl.PrefillSpec("case", 2, 3, T, dk, dv, dtype, (C,), 60 + dk + dv, "softplus",
                          0.05, "sigmoid")
    check(wl.make_gdn_inputs(spec), C, label=f"dk={dk} dv={dv} T={T}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_zero_and_tiny_gates(dtype):
    """a = 0 clears the memory; gates small enough that a 16-row block's decay
    falls below 2^-100 take the exact per-channel fallback."""
    spec = wl.PrefillSpec("case", 1, 2, 160, 32 if dtype == torch.float32 else 128,
                          32 if dtype == torch.float32 else 128, dtype, (32,), 71, "softplus",
                          0.5, "sigmoid")
    inp = wl.make_gdn_inputs(spec)
    a = inp["a"].clone()
    a[:, 5] = 0.0
    a[:, 40:56, 0] = 0.0
    a[:, 70:90, 1] = 1e-7
    a[:, 100] = 0.0
    inp["a"] = a
    check(inp, 32, label="zero gates")


@pytest.mark.parametrize("dk,dv,N,H,dtype,gated", [
    (16, 16, 3, 2, torch.float32, True), (32, 128, 2, 5, torch.float32, False),
    (128, 16, 1, 3, torch.float32, True), (64, 64, 4, 4, torch.bfloat16, True),
    (128, 128, 2, 3, torch.bfloat16, False), (128, 128, 64, 32, torch.bfloat16, True),
])
def test_decode_steps(dk, dv, N, H, dtype, gated):
    spec = wl.DecodeSpec("case", N, H, dk, dv, dtype, 5, dk + dv + N + 1, 0.1, 0.9, 1.0)
    S = wl.make_decode_state(spec)
    st = wl.make_decode_steps(spec)
    a = st["alpha"][..., 0].contiguous() if gated else None      # one gate per head
    Sg, Sr = S.to(DEV), S.double().numpy()
    tol = TOL[dtype]
    for s in range(5):
        x = {k: st[k][s].contiguous() for k in ("q", "k", "v", "beta")}
        xs = None if a is None else a[s].contiguous()
        og, Sg = kda().gdn_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                                       None if xs is None else xs.to(DEV), x["beta"].to(DEV), Sg)
        orf, Sr = gdn_decode_step(x["q"], x["k"], x["v"], xs, x["beta"], Sr)
        torch.cuda.synchronize()
        assert rel(f64(og), orf) < tol
    es = rel(f64(Sg), Sr)
    print(f"[gdn decode dk={dk} dv={dv} gated={gated}] rel_S={es:.3e}", flush=True)
    assert es < tol


@pytest.mark.parametrize("gated", [True, False])
def test_prefill_then_decode_equals_longer_prefill(gated):
    inp = wl.make_gdn_inputs(wl.PREFILL["prefill_h16_t4k"], T=105, H=4, gated=gated)
    T0 = 100
    head = {k: (v[:, :T0].contiguous() if v is not None and k != "S0" else v)
            for k, v in inp.items()}
    o_long, S_long = run(inp, 64)
    _, S = run(head, 64)
    outs = []
    for t in range(T0, 105):
        a_t = None if inp["a"] is None else inp["a"][:, t].contiguous().to(DEV)
        og, S = kda().gdn_decode_step(inp["q"][:, t].contiguous().to(DEV),
                                      inp["k"][:, t].contiguous().to(DEV),
                                      inp["v"][:, t].contiguous().to(DEV), a_t,
                                      inp["beta"][:, t].contiguous().to(DEV), S)
        outs.append(og)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1)
    o_ref, S_ref = oracle(inp)
    assert rel(f64(o_dec), o_ref[:, T0:]) < 2e-2 and rel(f64(S), S_ref) < 2e-2
    assert rel(f64(o_dec), f64(o_long[:, T0:])) < 2e-2 and rel(f64(S), f64(S_long)) < 1e-2


@pytest.mark.parametrize("gated,C", [(True, 16), (False, 32)])
def test_fp32_dk128(gated, C):
    spec = wl.PrefillSpec("case", 1, 3, 90, 128, 64, torch.float32, (C,), 91, "softplus",
                          0.05, "sigmoid")
    check(wl.make_gdn_inputs(spec, gated=gated), C, label="fp32 dk=128")


def test_empty_sequence_and_null_state_out():
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_gdn_inputs(spec, T=0, H=2)
    S0 = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(6))
    d = {k: (None if t is None else t.to(DEV)) for k, t in inp.items()}
    o, S = kda().gdn_prefill_chunked(d["q"], d["k"], d["v"], d["a"], d["beta"], S0.to(DEV))
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 128) and torch.equal(S.cpu(), S0)
    inp = wl.make_gdn_inputs(spec, T=70, H=2, gated=False)
    d = {k: (None if t is None else t.to(DEV)) for k, t in inp.items()}
    o, S = kda().gdn_prefill_chunked(d["q"], d["k"], d["v"], None, d["beta"], None,
                                     return_state=False)
    torch.cuda.synchronize()
    o_ref, _ = oracle(inp)
    assert S is None and rel(f64(o), o_ref) < 2e-2


@pytest.mark.parametrize("gated", [True, False])
def test_split_segments(gated):
    """16 chains x 438 chunks (T = 28000): three segments of the split path
    with the state carried between them; two chains match the oracle."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    T, H = 28000, 16
    inp = wl.make_gdn_inputs(spec, T=T, H=H, gated=gated)
    inp["S0"] = 0.05 * torch.randn(1, H, 128, 128, generator=torch.Generator().manual_seed(9))
    o, S = run(inp, 64)
    for h in (2, 15):
        sl = {k: (None if v is None else (v[:, :, h:h + 1].contiguous() if k != "S0"
                                          else v[:, h:h + 1].contiguous()))
              for k, v in inp.items()}
        o_ref, S_ref = oracle(sl)
        eo, es = rel(f64(o[:, :, h:h + 1]), o_ref), rel(f64(S[:, h:h + 1]), S_ref)
        print(f"[gdn segments T={T} head {h} gated={gated}] rel_o={eo:.3e} rel_S={es:.3e}", flush=True)
        assert eo < 2e-2 and es < 2e-2
