"""Chunked prefill on the GPU against the float64 oracle.

Every case draws its inputs once (seeded, workloads.py), hands the same
tensors to the HIP path (through the C ABI binding) and, upcast to float64,
to the oracle.  The error measure is the relative Frobenius norm over the
compared slice, separately for o and S_T, and its worst value over every head
and every 64-token chunk of every head (tests/parity.py); the bar is 1e-4 for
fp32 inputs and 2e-2 for bf16 inputs, for each of them.  Large workloads run in full on the GPU, in the launch
configuration the benchmark times, and the oracle checks a slice of chains
(prefixes by causality).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import kda_recurrence, kda_decode_step
from tests import parity

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


def to_dev(inp):
    return {k: (None if t is None else t.to(DEV)) for k, t in inp.items()}


def run(inp, C, **kw):
    g = to_dev(inp)
    o, S = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"],
                                 chunk=C, **kw)
    torch.cuda.synchronize()
    return o, S


def oracle(inp):
    return kda_recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"])


def check(inp, C, tol=None, label=""):
    tol = tol or TOL[inp["q"].dtype]
    o, S = run(inp, C)
    o_ref, S_ref = oracle(inp)
    parity.report(f"{label} C={C}", tol, f64(o), o_ref, f64(S), S_ref)
    return o, S


@pytest.mark.parametrize("C", [16, 32, 128])
def test_tiny_fp32_full(C):
    spec = wl.PREFILL["tiny_fp32"]
    check(wl.make_prefill_inputs(spec), C, label="tiny_fp32")


def test_tiny_fp32_null_state_equals_explicit_zeros():
    spec = wl.PREFILL["tiny_fp32"]
    inp = wl.make_prefill_inputs(spec)
    o1, S1 = run(inp, 16)
    inp2 = dict(inp, S0=torch.zeros(1, 1, 16, 16))
    o2, S2 = run(inp2, 16)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_prefill_h16_t4k_chunks(C):
    """The bf16 H=16, T=4096, d=128 workload in full; every chunk size (128
    runs as two 64-token chunks)."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    check(wl.make_prefill_inputs(spec), C, label="h16_t4k")


def test_chunk_128_runs_as_64():
    """C = 128 is accepted and computed with 64-token chunks: bit-identical."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=300, H=4)
    o1, S1 = run(inp, 64)
    o2, S2 = run(inp, 128)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("T,C", [(1, 64), (15, 64), (17, 64), (63, 64), (65, 64), (200, 64),
                                 (127, 128), (200, 128)])
def test_ragged_lengths(T, C):
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=T, H=3)
    inp["S0"] = 0.1 * torch.randn(1, 3, 128, 128, generator=torch.Generator().manual_seed(T))
    check(inp, C, label=f"ragged T={T}")


def test_empty_sequence_copies_state():
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=0, H=2)
    S0 = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(5))
    g = to_dev(dict(inp, S0=S0))
    o, S = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], chunk=64)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S.cpu(), S0)
    g0 = to_dev(inp)
    _, Sz = kda().prefill_chunked(g0["q"], g0["k"], g0["v"], g0["alpha"], g0["beta"], None,
                                  chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Sz).item() == 0


@pytest.mark.parametrize("dk,dv,dtype,C", [
    (16, 16, torch.float32, 16), (32, 64, torch.float32, 32), (64, 16, torch.float32, 32),
    (128, 32, torch.float32, 32), (16, 128, torch.bfloat16, 16), (32, 32, torch.bfloat16, 64),
    (64, 128, torch.bfloat16, 64), (128, 64, torch.bfloat16, 32), (128, 16, torch.bfloat16, 64),
    (16, 64, torch.bfloat16, 64), (16, 16, torch.float32, 64),
])
def test_head_dims(dk, dv, dtype, C):
    g = torch.Generator().manual_seed(dk * 1000 + dv)
    B, T, H = 2, 150, 3
    q = torch.randn(B, T, H, dk, generator=g)
    k = torch.randn(B, T, H, dk, generator=g)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn(B, T, H, dv, generator=g).to(dtype)
    alpha = 0.8 + 0.2 * torch.rand(B, T, H, dk, generator=g)
    beta = torch.rand(B, T, H, generator=g)
    S0 = 0.1 * torch.randn(B, H, dk, dv, generator=g)
    check(dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0), C, label=f"dk={dk} dv={dv}")


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("alpha_one", [True, False])
def test_inter_chunk_read_alone(dk, C, alpha_one):
    """beta = 0 never writes, so o_t = q_t Diag(alpha_1..alpha_t) S0 (pure
    decayed read of the initial state): isolates the (Q E) S product,
    including its first rows, from the intra-chunk terms."""
    g = torch.Generator().manual_seed(dk + C)
    B, T, H, dv = 1, 48, 2, 128
    q = torch.randn(B, T, H, dk, generator=g)
    q = (q / q.norm(dim=-1, keepdim=True)).bfloat16()
    k = torch.randn(B, T, H, dk, generator=g)
    k = (k / k.norm(dim=-1, keepdim=True)).bfloat16()
    v = torch.randn(B, T, H, dv, generator=g).bfloat16()
    alpha = torch.ones(B, T, H, dk) if alpha_one else 0.9 + 0.1 * torch.rand(B, T, H, dk, generator=g)
    beta = torch.zeros(B, T, H)
    S0 = torch.randn(B, H, dk, dv, generator=g)
    inp = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)
    o, S = run(inp, C)
    o_ref, S_ref = oracle(inp)
    rows = np.linalg.norm(f64(o) - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)
    print(f"[read alone dk={dk} C={C}] worst row rel={rows.max():.3e}", flush=True)
    assert rows.max() < 1e-2
    assert rel(f64(S), S_ref) < 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_zero_and_extreme_gates(dtype):
    """Exact zero gates (memory cleared) and gates so small that a 16-row
    block's decay falls below 2^-100: the exact per-channel fallback."""
    g = torch.Generator().manual_seed(11)
    B, T, H, d = 1, 160, 2, 32 if dtype == torch.float32 else 128
    C = 32
    q = torch.randn(B, T, H, d, generator=g)
    k = torch.randn(B, T, H, d, generator=g)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn(B, T, H, d, generator=g).to(dtype)
    alpha = 0.9 + 0.1 * torch.rand(B, T, H, d, generator=g)
    alpha[:, 5, :, 3] = 0.0                      # one exact zero
    alpha[:, 40:56, 0, 7] = 0.0                  # a whole block of zeros
    alpha[:, 70:90, 1, :8] = 1e-4                # strong decay on 8 channels
    alpha[:, 100, :, :] = 0.0                    # every channel cleared at t=100
    alpha[:, 130:134, :, 20] = 1e-12
    beta = torch.rand(B, T, H, generator=g)
    S0 = torch.randn(B, H, d, d, generator=g)
    check(dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0), C, label="zero gates")


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_split_and_fused_paths_agree(C):
    """Few chains take the split path (chunk-parallel prep + scan, with a
    workspace); more than 128 take the fused kernel.  The same 4 chains, run
    alone and inside a batch of 132 chains, both match the oracle."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    big = wl.make_prefill_inputs(spec, T=160, B=33, H=4)
    big["S0"] = 0.05 * torch.randn(33, 4, 128, 128, generator=torch.Generator().manual_seed(C))
    ws_few = kda().prefill_workspace_bytes(1, 160, 4, 128, 128, C)
    ws_many = kda().prefill_workspace_bytes(33, 160, 4, 128, 128, C)
    assert ws_few > 0 and ws_many == 0
    o_big, S_big = run(big, C)
    few = {k: (v[3:4].contiguous() if v is not None else v) for k, v in big.items()}
    o_few, S_few = run(few, C)
    o_ref, S_ref = oracle(few)
    for o, S in ((o_big[3:4], S_big[3:4]), (o_few, S_few)):
        assert rel(f64(o), o_ref) < 2e-2 and rel(f64(S), S_ref) < 2e-2
    assert rel(f64(o_big[3:4]), f64(o_few)) < 1e-2


def test_prep_chunk_runs_ragged():
    """Split path with several chunks per prep workgroup: 8 chains x 101
    chunks gives runs of 4 chunks, the last run of each chain holds one chunk,
    and the last chunk holds 23 of its 64 rows."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    T = 64 * 100 + 23
    inp = wl.make_prefill_inputs(spec, T=T, H=8)
    assert kda().prefill_workspace_bytes(1, T, 8, 128, 128, 64) > 0   # split path
    check(inp, 64, label="prep runs, ragged")


def test_split_segments():
    """A sequence whose records exceed one segment: 16 chains x 438 chunks
    (T = 28000, the last chunk 32 rows) run as three segments of 160, 160 and
    118 chunks with the state carried between them (inputs loaded
    non-temporally).  Two chains match the oracle; resuming at a chunk
    boundary (tokens 6400.., itself three segments with other boundaries)
    reproduces the full run bit for bit."""
    spec = wl.PREFILL["prefill_h16_t4k"]
    T, H, cut = 28000, 16, 100 * 64
    ws = kda().prefill_workspace_bytes(1, T, H, 128, 128, 64)
    assert ws == 16 * 160 * 74240 + 16 * 128 * 128 * 4            # three segments
    inp = wl.make_prefill_inputs(spec, T=T, H=H)
    inp["S0"] = 0.05 * torch.randn(1, H, 128, 128, generator=torch.Generator().manual_seed(7))
    g = to_dev(inp)
    o, S = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], chunk=64)
    torch.cuda.synchronize()
    for h in (0, 11):
        sl = {k: (inp[k][:, :, h:h + 1].contiguous() if k != "S0" else inp[k][:, h:h + 1].contiguous())
              for k in inp}
        o_ref, S_ref = oracle(sl)
        eo, es = rel(f64(o[:, :, h:h + 1]), o_ref), rel(f64(S[:, h:h + 1]), S_ref)
        print(f"[segments T={T} head {h}] rel_o={eo:.3e} rel_S={es:.3e}", flush=True)
        assert eo < 2e-2 and es < 2e-2
    first = {k: (g[k][:, :cut].contiguous() if k != "S0" else g[k]) for k in g}
    rest = {k: g[k][:, cut:].contiguous() for k in g if k != "S0"}
    o1, S1 = kda().prefill_chunked(first["q"], first["k"], first["v"], first["alpha"], first["beta"],
                                   first["S0"], chunk=64)
    o2, S2 = kda().prefill_chunked(rest["q"], rest["k"], rest["v"], rest["alpha"], rest["beta"], S1,
                                   chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o[:, :cut]) and torch.equal(o2, o[:, cut:]) and torch.equal(S2, S)
    # no final state requested: the carried state still links the segments
    o3, _ = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], chunk=64,
                                  return_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o3, o)


def test_split_resume_and_in_place_state():
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=300, H=2)
    o_full, S_full = run(inp, 64)
    first = {k: (v[:, :137].contiguous() if k not in ("S0",) and v is not None else v)
             for k, v in inp.items()}
    second = {k: (v[:, 137:].contiguous() if k not in ("S0",) and v is not None else v)
              for k, v in inp.items()}
    o1, S1 = run(first, 64)
    g2 = to_dev(second)
    S_buf = S1.clone()
    o2, S2 = kda().prefill_chunked(g2["q"], g2["k"], g2["v"], g2["alpha"], g2["beta"], S_buf,
                                   chunk=64, state_out=S_buf)      # in place
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_buf.data_ptr()
    o_cat = torch.cat([o1, o2], 1)
    assert rel(f64(o_cat), f64(o_full)) < 1e-2
    assert rel(f64(S2), f64(S_full)) < 1e-2
    o_ref, S_ref = oracle(inp)
    assert rel(f64(o_cat), o_ref) < 2e-2 and rel(f64(S2), S_ref) < 2e-2


def test_deterministic():
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=700, H=4)
    o1, S1 = run(inp, 64)
    o2, S2 = run(inp, 64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_prefill_then_decode_equals_longer_prefill():
    spec = wl.PREFILL["prefill_h16_t4k"]
    inp = wl.make_prefill_inputs(spec, T=140, H=2)
    n_pre = 128
    pre = {k: (v[:, :n_pre].contiguous() if k != "S0" and v is not None else v)
           for k, v in inp.items()}
    _, S = run(pre, 64)
    outs = []
    for t in range(n_pre, 140):
        a = {k: inp[k][:, t].contiguous().to(DEV) for k in ("q", "k", "v", "alpha", "beta")}
        o_t, S = kda().decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], S)
        outs.append(o_t)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle(inp)
    assert rel(f64(torch.stack(outs, 1)), o_ref[:, n_pre:]) < 2e-2
    assert rel(f64(S), S_ref) < 2e-2


# ---------------------------------------------------------------------------
# Full-size workloads: the GPU runs them whole; the oracle checks slices.
# ---------------------------------------------------------------------------
CHAINS_B8 = [(0, 0), (3, 7), (5, 20), (7, 31)]


@pytest.mark.parametrize("C", [64])
def test_prefill_b8_h32_t8k_slices(C):
    spec = wl.PREFILL["prefill_b8_h32_t8k"]
    torch.cuda.empty_cache()
    g = wl.make_prefill_inputs(spec, DEV)
    o, S = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], chunk=C)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    for (b, h) in CHAINS_B8:
        sl = {k: g[k][b:b + 1, :, h:h + 1].contiguous().cpu() for k in
              ("q", "k", "v", "alpha", "beta")}
        sl["S0"] = g["S0"][b:b + 1, h:h + 1].contiguous().cpu()
        o_ref, S_ref = oracle(sl)
        parity.report(f"b8_h32_t8k C={C} chain ({b},{h})", 2e-2, f64(o[b:b + 1, :, h:h + 1]),
                      o_ref, f64(S[b:b + 1, h:h + 1]), S_ref)
    del g, o, S
    torch.cuda.empty_cache()


def test_longctx_h32_t1m_prefix_then_decode():
    """T = 1,048,576 tokens, 32 heads, channel-mixture gates with exact
    zeros; the oracle checks head 0 over the first 65,536 tokens (o from the
    full run, S from a prefix-only run), then 256 decode steps from S_T."""
    spec = wl.PREFILL["longctx_h32_t1m"]
    torch.cuda.empty_cache()
    g = wl.make_prefill_inputs(spec, DEV)
    n_zero = int((g["alpha"] == 0).sum().item())
    o, S_T = kda().prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, chunk=64)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S_T).all()
    P = 65536
    pre = {k: g[k][:, :P].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
    _, S_P = kda().prefill_chunked(pre["q"], pre["k"], pre["v"], pre["alpha"], pre["beta"], None,
                                   chunk=64)
    torch.cuda.synchronize()
    sl = {k: pre[k][:, :, 0:1].contiguous().cpu() for k in pre}
    sl["S0"] = None
    o_ref, S_ref = oracle(sl)
    parity.report(f"longctx head 0, t<{P}, {n_zero} exact zero gates", 2e-2,
                  f64(o[:, :P, 0:1]), o_ref, f64(S_P[:, 0:1]), S_ref)
    del pre, g
    torch.cuda.empty_cache()

    dspec = wl.DECODE["longctx_decode"]
    mask = wl.mixture_low_channels(32, 128, spec.seed)
    steps = wl.make_decode_steps(dspec, DEV, N=1, alpha_mask=mask)
    Sg = S_T.clone()
    Sr = f64(S_T)
    outs_g, outs_r = [], []
    for s in range(dspec.steps):
        a = {k: t[s].contiguous() for k, t in steps.items()}
        og, Sg = kda().decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], Sg)
        outs_g.append(og)
        ac = {k: t.cpu() for k, t in a.items()}
        orf, Sr = kda_decode_step(ac["q"], ac["k"], ac["v"], ac["alpha"], ac["beta"], Sr)
        outs_r.append(orf)
    torch.cuda.synchronize()
    parity.report("longctx decode 256 steps, 32 heads", 2e-2, f64(torch.stack(outs_g)),
                  np.stack(outs_r), f64(Sg), Sr, steps_major=True)
