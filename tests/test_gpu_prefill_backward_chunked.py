"""The chunked prefill backward on the GPU (kda_prefill_backward_chunked, bf16,
dk = dv = 128) against the float64 oracle (oracle.kda_prefill_backward,
pinned by finite differences in tests/test_backward_pins.py; the chunk form
itself is checked against it on the CPU in tests/test_chunk_backward_model.py).

Same inputs on both sides (bf16 values upcast exactly).  Bar: the bf16 bar of
2e-2 on the relative Frobenius error of every gradient, also over every head
and every 64-token chunk of a head (tests/parity.py); matrix-core operands
are bf16, so the measured errors sit near 3e-3.  Lengths span one token, a
16-token sub-chunk, ragged sub-chunks and chunks, and several chunks; closed
gates (alpha = 0) are included; repeated calls must agree bit for bit (no
atomics); the full B = 1, H = 16, T = 4096 workload is checked on sampled
heads and B = 8, H = 32, T = 8192 on sampled chains."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import kda_prefill_backward
from tests.parity import rel, worst_state, worst_token_major

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def kda():
    import gated_delta_rule_108_amd as m
    return m


def f64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


def spec(alpha_kind="softplus", s0_std=0.1):
    base = wl.PREFILL["prefill_h16_t4k"]
    return dataclasses.replace(base, name="cbwd", dk=128, dv=128, dtype=torch.bfloat16,
                               alpha_kind=alpha_kind, s0_std=s0_std)


def check(label, got, ref):
    """Every gradient: whole, worst head, worst 64-token chunk (token-major
    ones), worst head (states)."""
    m = {}
    for n, g, r in zip(NAMES, got, ref):
        g = f64(g)
        assert np.isfinite(g).all(), (label, n)
        m[n] = rel(g, r)
        if n == "dS0":
            m[n + "_head"] = worst_state(g, r)
        else:
            if g.ndim == 3:                      # dbeta [B, T, H]
                g, r = g[..., None], r[..., None]
            m[n + "_head"], m[n + "_chunk"] = worst_token_major(g, r)
    print(f"[{label}] " + " ".join(f"{k}={v:.2e}" for k, v in m.items()), flush=True)
    bad = {k: v for k, v in m.items() if not v < TOL}
    assert not bad, (label, bad)
    return m


def run(sp, B, T, H, with_dST=True, heads=None, zero_gates=False):
    print(f"case {sp.name} B={B} T={T} H={H} dST={with_dST} zero_gates={zero_gates}", flush=True)
    x = wl.make_prefill_inputs(sp, "cpu", T=T, B=B, H=H)
    if zero_gates:
        a = x["alpha"].clone()
        a[:, min(5, T - 1), :, :40] = 0.0
        a[:, T // 2] = 0.0
        x["alpha"] = a
    gr = wl.make_prefill_backward_grads(sp, "cpu", T=T, B=B, H=H, with_dST=with_dST)
    g = {n: (None if t is None else t.to(DEV)) for n, t in {**x, **gr}.items()}
    out = kda().prefill_backward_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["dO"],
                                         S0=g["S0"], dS_T=g["dS_T"])
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else heads
    sl = lambda t, st=False: None if t is None else (t[:, hs] if st else t[:, :, hs])  # noqa: E731
    ref = kda_prefill_backward(*(f64(sl(x[n])) for n in ("q", "k", "v", "alpha", "beta")),
                               f64(sl(x["S0"], True)), f64(sl(gr["dO"])),
                               f64(sl(gr["dS_T"], True)))
    got = [sl(t) for t in out[:5]] + [sl(out[5], True)]
    return check(f"chunked bwd B={B} T={T} H={H}", got, ref), out


@pytest.mark.parametrize("T", [1, 16, 37, 64, 100, 130])
def test_lengths(T):
    run(spec(), B=2, T=T, H=2)


def test_many_chains():
    """64 chains: the state-gradient walk takes two column tiles per wave."""
    run(spec(), B=4, T=100, H=16)


def test_more_chains_than_the_split_path_takes():
    """144 chains: the forward pass runs the fused chunk kernel, which stores
    the chunk states and writes no output (ragged last chunk)."""
    run(spec(), B=2, T=150, H=72, heads=[0, 35, 71])


def test_optional_states():
    run(spec(s0_std=0.0), B=1, T=70, H=2, with_dST=False)


def test_initial_state_without_final_gradient():
    """S0 given, dS_T absent: the state gradient starts at zero at the end."""
    run(spec(), B=1, T=70, H=2, with_dST=False)


def test_odd_chain_count_and_ragged_chunks():
    """Nine chains (one state-gradient tile per workgroup, a grid that is no
    multiple of the CU count) over 11 chunks, the last of 60 rows."""
    run(spec(), B=3, T=700, H=3)


def test_closed_gates_and_mixture():
    run(spec(), B=1, T=90, H=2, zero_gates=True)
    run(spec(alpha_kind="mixture"), B=1, T=128, H=2)


def test_repeat_calls_are_bit_identical():
    sp = spec()
    x = wl.make_prefill_inputs(sp, DEV, T=200, B=1, H=4)
    gr = wl.make_prefill_backward_grads(sp, DEV, T=200, B=1, H=4)
    a = kda().prefill_backward_chunked(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                                       S0=x["S0"], dS_T=gr["dS_T"])
    b = kda().prefill_backward_chunked(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                                       S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    for n, s, t in zip(NAMES, a, b):
        assert torch.equal(s, t), n


def test_graph_capture_replays_match_the_eager_call():
    """Captured into a graph the call runs in order on the captured stream
    (eagerly, with few chains, part of it runs on the library's second
    stream); every replay, with eager work and synchronisations between,
    equals the eager call bit for bit."""
    sp = spec()
    x = wl.make_prefill_inputs(sp, DEV, T=200, B=1, H=4)
    gr = wl.make_prefill_backward_grads(sp, DEV, T=200, B=1, H=4)
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"])
    ref = kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"])
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(NAMES, out, ref):
            assert torch.equal(a, b), (i, n)
        (x["q"].float() * 2.0).sum().item()
        torch.cuda.synchronize()


def test_concurrent_calls_from_two_threads():
    """Two host threads call the backward at once, each on a stream of its
    own, five times: they share the library's second stream and its events,
    and every result equals the single-threaded call bit for bit."""
    import threading
    sp = spec()
    x = wl.make_prefill_inputs(sp, DEV, T=300, B=1, H=4)
    gr = wl.make_prefill_backward_grads(sp, DEV, T=300, B=1, H=4)
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"])
    ref = kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    outs, errs = [[], []], []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(5):
                    outs[i].append(kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"]))
            st.synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errs.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errs, errs
    for i in range(2):
        assert len(outs[i]) == 5
        for o in outs[i]:
            for n, a, b in zip(NAMES, o, ref):
                assert torch.equal(a, b), (i, n)


def test_no_tokens_passes_the_state_gradient_through():
    m = kda()
    B, H, d = 2, 3, 128
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=DEV)  # noqa: E731
    f = lambda *s: torch.zeros(*s, dtype=torch.float32, device=DEV)  # noqa: E731
    dST = torch.randn(B, H, d, d, device=DEV)
    out = m.prefill_backward_chunked(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), f(B, 0, H, d),
                                     f(B, 0, H), z(B, 0, H, d), S0=None, dS_T=dST)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dST)


def test_full_workload_sampled_heads():
    """B = 1, H = 16, T = 4096, d = 128, bf16: the whole launch on the GPU,
    the oracle on heads 0 and 11."""
    sp = wl.PREFILL["prefill_h16_t4k"]
    run(sp, B=1, T=sp.T, H=sp.H, heads=[0, 11])


def test_largest_workload_sampled_chains():
    """B = 8, H = 32, T = 8192, d = 128, bf16: the whole launch on the GPU,
    the oracle on chains (b, h) = (3, 17) and (7, 0)."""
    sp = wl.PREFILL["prefill_b8_h32_t8k"]
    print(f"case {sp.name} full size", flush=True)
    x = wl.make_prefill_inputs(sp, DEV)
    gr = wl.make_prefill_backward_grads(sp, DEV)
    out = kda().prefill_backward_chunked(x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"],
                                         S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    for b, h in ((3, 17), (7, 0)):
        tok = lambda t: t[b:b + 1, :, h:h + 1]   # noqa: E731
        st = lambda t: None if t is None else t[b:b + 1, h:h + 1]   # noqa: E731
        ref = kda_prefill_backward(*(f64(tok(x[n])) for n in ("q", "k", "v", "alpha", "beta")),
                                   f64(st(x["S0"])), f64(tok(gr["dO"])), f64(st(gr["dS_T"])))
        got = [tok(t) for t in out[:5]] + [st(out[5])]
        check(f"cfg3 chain ({b},{h})", got, ref)


def test_agrees_with_the_fp32_backward():
    """The token-walk backward (fp32 arithmetic) and the chunked one on the
    same inputs: the same gradients up to the bf16 bar."""
    sp = spec()
    x = wl.make_prefill_inputs(sp, DEV, T=300, B=2, H=3)
    gr = wl.make_prefill_backward_grads(sp, DEV, T=300, B=2, H=3)
    args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], gr["dO"])
    a = kda().prefill_backward_chunked(*args, S0=x["S0"], dS_T=gr["dS_T"])
    b = kda().prefill_backward(*args, S0=x["S0"], dS_T=gr["dS_T"])
    torch.cuda.synchronize()
    for n, s, t in zip(NAMES, a, b):
        e = rel(f64(s), f64(t))
        print(f"  {n}: {e:.2e}", flush=True)
        assert e < TOL, n
