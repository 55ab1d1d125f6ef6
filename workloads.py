"""Seeded synthetic KDA workloads shared by the tests, the smoke check and the
benchmark.

This module only draws random inputs of the right shapes and distributions;
it holds none of the attention arithmetic.  The same tensors (after rounding
to the stated dtype) go to the HIP path and, upcast to float64, to the oracle.

Workloads (token-major layouts: q,k [B,T,H,dk], v [B,T,H,dv], alpha
[B,T,H,dk], beta [B,T,H], S0 [B,H,dk,dv]):

  tiny_fp32         B=1  H=1  T=256      dk=dv=16  fp32  C=16
                    q,k ~ N(0,1) then L2-normalised per token, v ~ N(0,1),
                    alpha ~ U(0.9,1.0), beta ~ U(0,1), S0 = 0
  prefill_h16_t4k   B=1  H=16 T=4096     d=128     bf16  C=64
                    q,k L2-normalised N(0,1), v ~ N(0,1),
                    alpha = exp(-softplus(g)), g ~ N(0,1), beta = sigmoid(N(0,1)),
                    S0 = 0
  prefill_b8_h32_t8k B=8 H=32 T=8192     d=128     bf16  C=64 and C=128
                    as above, S0 ~ N(0, sd 0.01)
  decode_n256_h32   N=256 sequences x H=32, d=128, state ~ N(0, sd 0.01) fp32,
                    every step: fresh q,k (L2-normalised, bf16), v bf16,
                    alpha ~ U(0.95,1.0), beta ~ U(0,1); 1000 steps
  longctx_h32_t1m   B=1  H=32 T=1048576  d=128     bf16  C=64, S0 = 0;
                    per head 13 of the 128 channels (a seeded choice, fixed
                    over t) draw alpha ~ U(0,0.5), the rest ~ U(0.99,1.0);
                    q,k,v,beta as prefill_h16_t4k; then 256 decode steps.

Raw-projection inputs for the fused prologue (make_prefill_logit_inputs,
make_decode_logit_steps) use the same shapes and draw the pre-activation
values the recipes above name: q, k ~ N(0,1) NOT normalised, gate logits
g ~ N(0,1) in the I/O dtype (the recurrence then uses alpha = exp(-softplus(g))),
write-strength logits b ~ N(0,1) fp32 (beta = sigmoid(b)).

Random numbers come from torch.Generator(device).manual_seed(seed).  The
streams differ between CPU and GPU generators, so a test that compares the
two paths always generates once and hands the same tensors to both.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["PrefillSpec", "DecodeSpec", "PREFILL", "DECODE",
           "make_prefill_inputs", "make_decode_state", "make_decode_step_inputs",
           "make_decode_steps", "make_prefill_logit_inputs", "make_decode_logit_steps",
           "make_gdn_inputs"]


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: torch.dtype
    chunks: tuple
    seed: int
    alpha_kind: str          # "uniform_0.9_1" | "softplus" | "mixture"
    s0_std: float            # 0 => S0 = zeros
    beta_kind: str           # "uniform" | "sigmoid"


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    steps: int
    seed: int
    s_std: float
    alpha_lo: float
    alpha_hi: float


PREFILL = {
    "tiny_fp32": PrefillSpec("tiny_fp32", 1, 1, 256, 16, 16, torch.float32, (16,), 1,
                             "uniform_0.9_1", 0.0, "uniform"),
    "prefill_h16_t4k": PrefillSpec("prefill_h16_t4k", 1, 16, 4096, 128, 128, torch.bfloat16,
                                   (64,), 2, "softplus", 0.0, "sigmoid"),
    "prefill_b8_h32_t8k": PrefillSpec("prefill_b8_h32_t8k", 8, 32, 8192, 128, 128,
                                      torch.bfloat16, (64, 128), 3, "softplus", 0.01, "sigmoid"),
    "longctx_h32_t1m": PrefillSpec("longctx_h32_t1m", 1, 32, 1 << 20, 128, 128, torch.bfloat16,
                                   (64,), 5, "mixture", 0.0, "sigmoid"),
}

DECODE = {
    "decode_n256_h32": DecodeSpec("decode_n256_h32", 256, 32, 128, 128, torch.bfloat16, 1000, 4,
                                  0.01, 0.95, 1.0),
    # decode after the long-context prefill: N=1, H=32, fresh inputs drawn like
    # the prefill's (alpha from the same per-head channel mixture)
    "longctx_decode": DecodeSpec("longctx_decode", 1, 32, 128, 128, torch.bfloat16, 256, 55,
                                 0.0, 0.0, 0.0),
}

# number of "fast-forgetting" channels per head in the long-context mixture:
# 10% of 128 channels, rounded to the nearest integer
MIXTURE_LOW_FRACTION = 0.10


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(x):
    """L2-normalise the last axis (input recipe: the caller's feature map)."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def mixture_low_channels(H, dk, seed, device="cpu"):
    """Boolean mask [H, dk]: the channels of each head that forget fast."""
    n_low = int(round(MIXTURE_LOW_FRACTION * dk))
    g = _gen("cpu", seed + 7919)
    mask = torch.zeros(H, dk, dtype=torch.bool)
    for h in range(H):
        perm = torch.randperm(dk, generator=g)
        mask[h, perm[:n_low]] = True
    return mask.to(device)


def _alpha(kind, shape, g, device, H=None, dk=None, seed=None):
    if kind == "uniform_0.9_1":
        return 0.9 + 0.1 * torch.rand(shape, generator=g, device=device)
    if kind == "softplus":
        x = torch.randn(shape, generator=g, device=device)
        return torch.exp(-torch.nn.functional.softplus(x))
    if kind == "mixture":
        low = mixture_low_channels(H, dk, seed, device)            # [H, dk]
        u = torch.rand(shape, generator=g, device=device)
        a_low = 0.5 * u
        a_high = 0.99 + 0.01 * u
        return torch.where(low, a_low, a_high)
    raise ValueError(kind)


def make_prefill_inputs(spec: PrefillSpec, device="cpu", T=None, B=None, H=None):
    """Draw one prefill batch.  T/B/H may be overridden to make a smaller case
    with the same distributions.  Returns a dict of contiguous tensors."""
    B = spec.B if B is None else B
    H = spec.H if H is None else H
    T = spec.T if T is None else T
    dk, dv = spec.dk, spec.dv
    g = _gen(device, spec.seed)
    q = _unit_rows(torch.randn(B, T, H, dk, generator=g, device=device)).to(spec.dtype)
    k = _unit_rows(torch.randn(B, T, H, dk, generator=g, device=device)).to(spec.dtype)
    v = torch.randn(B, T, H, dv, generator=g, device=device).to(spec.dtype)
    alpha = _alpha(spec.alpha_kind, (B, T, H, dk), g, device, H=H, dk=dk, seed=spec.seed)
    if spec.beta_kind == "sigmoid":
        beta = torch.sigmoid(torch.randn(B, T, H, generator=g, device=device))
    else:
        beta = torch.rand(B, T, H, generator=g, device=device)
    if spec.s0_std > 0:
        S0 = spec.s0_std * torch.randn(B, H, dk, dv, generator=g, device=device)
    else:
        S0 = None
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                alpha=alpha.float().contiguous(), beta=beta.float().contiguous(),
                S0=None if S0 is None else S0.float().contiguous())


def make_prefill_logit_inputs(spec: PrefillSpec, device="cpu", T=None, B=None, H=None):
    """Raw projections for the fused prologue: q, k, v and g in spec.dtype,
    b fp32, S0 as make_prefill_inputs.  Returns a dict of contiguous tensors
    (keys q, k, v, g, b, S0)."""
    B = spec.B if B is None else B
    H = spec.H if H is None else H
    T = spec.T if T is None else T
    dk, dv = spec.dk, spec.dv
    g = _gen(device, spec.seed + 1000)
    q = torch.randn(B, T, H, dk, generator=g, device=device).to(spec.dtype)
    k = torch.randn(B, T, H, dk, generator=g, device=device).to(spec.dtype)
    v = torch.randn(B, T, H, dv, generator=g, device=device).to(spec.dtype)
    gl = torch.randn(B, T, H, dk, generator=g, device=device).to(spec.dtype)
    b = torch.randn(B, T, H, generator=g, device=device)
    S0 = None
    if spec.s0_std > 0:
        S0 = (spec.s0_std * torch.randn(B, H, dk, dv, generator=g, device=device)).float()
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=gl.contiguous(),
                b=b.float().contiguous(), S0=None if S0 is None else S0.contiguous())


def make_decode_logit_steps(spec: DecodeSpec, device="cpu", N=None, steps=None):
    """Every step's raw projections at once: q, k, g [S,N,H,dk] and v
    [S,N,H,dv] in spec.dtype, b [S,N,H] fp32, all N(0,1)."""
    N = spec.N if N is None else N
    steps = spec.steps if steps is None else steps
    H, dk, dv = spec.H, spec.dk, spec.dv
    g = _gen(device, spec.seed + 1001)
    q = torch.randn(steps, N, H, dk, generator=g, device=device).to(spec.dtype)
    k = torch.randn(steps, N, H, dk, generator=g, device=device).to(spec.dtype)
    v = torch.randn(steps, N, H, dv, generator=g, device=device).to(spec.dtype)
    gl = torch.randn(steps, N, H, dk, generator=g, device=device).to(spec.dtype)
    b = torch.randn(steps, N, H, generator=g, device=device)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=gl.contiguous(),
                b=b.float().contiguous())


def make_gdn_inputs(spec: PrefillSpec, device="cpu", T=None, B=None, H=None, gated=True):
    """A Gated DeltaNet batch: make_prefill_inputs with the per-channel alpha
    replaced by one gate per token and head, a [B,T,H] fp32 drawn like the
    spec's alpha (exp(-softplus(N(0,1))) or U(0.9, 1)); gated=False gives
    a=None (DeltaNet).  Returns a dict with keys q, k, v, a, beta, S0."""
    d = make_prefill_inputs(spec, device, T=T, B=B, H=H)
    Bv, Tv, Hv = d["beta"].shape
    a = None
    if gated:
        kind = "uniform_0.9_1" if spec.alpha_kind == "uniform_0.9_1" else "softplus"
        a = _alpha(kind, (Bv, Tv, Hv), _gen(device, spec.seed + 2000), device).float().contiguous()
    return dict(q=d["q"], k=d["k"], v=d["v"], a=a, beta=d["beta"], S0=d["S0"])


def make_prefill_backward_grads(spec: PrefillSpec, device="cpu", T=None, B=None, H=None,
                                with_dST=True):
    """Incoming gradients for a prefill backward: dO [B,T,H,dv] in spec.dtype
    and dS_T [B,H,dk,dv] fp32 (None if with_dST is False), standard normal."""
    B = spec.B if B is None else B
    H = spec.H if H is None else H
    T = spec.T if T is None else T
    g = _gen(device, spec.seed + 2000)
    dO = torch.randn(B, T, H, spec.dv, generator=g, device=device).to(spec.dtype)
    dST = torch.randn(B, H, spec.dk, spec.dv, generator=g, device=device) if with_dST else None
    return dict(dO=dO.contiguous(), dS_T=None if dST is None else dST.float().contiguous())


def make_decode_state(spec: DecodeSpec, device="cpu", N=None):
    N = spec.N if N is None else N
    g = _gen(device, spec.seed)
    return (spec.s_std * torch.randn(N, spec.H, spec.dk, spec.dv, generator=g,
                                     device=device)).float().contiguous()


def make_decode_steps(spec: DecodeSpec, device="cpu", N=None, steps=None, alpha_mask=None):
    """Draw every step's inputs at once: q,k [S,N,H,dk], v [S,N,H,dv],
    alpha [S,N,H,dk], beta [S,N,H].  With alpha_mask (bool [H,dk]) alpha
    follows the long-context channel mixture instead of U(lo, hi)."""
    N = spec.N if N is None else N
    steps = spec.steps if steps is None else steps
    H, dk, dv = spec.H, spec.dk, spec.dv
    g = _gen(device, spec.seed + 1)
    q = _unit_rows(torch.randn(steps, N, H, dk, generator=g, device=device)).to(spec.dtype)
    k = _unit_rows(torch.randn(steps, N, H, dk, generator=g, device=device)).to(spec.dtype)
    v = torch.randn(steps, N, H, dv, generator=g, device=device).to(spec.dtype)
    u = torch.rand(steps, N, H, dk, generator=g, device=device)
    if alpha_mask is None:
        alpha = spec.alpha_lo + (spec.alpha_hi - spec.alpha_lo) * u
    else:
        alpha = torch.where(alpha_mask.to(device), 0.5 * u, 0.99 + 0.01 * u)
    beta = torch.rand(steps, N, H, generator=g, device=device)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                alpha=alpha.float().contiguous(), beta=beta.float().contiguous())


def make_decode_step_inputs(spec: DecodeSpec, device="cpu", N=None):
    """One step's inputs (the first step of make_decode_steps)."""
    d = make_decode_steps(spec, device, N=N, steps=1)
    return {k_: t[0].contiguous() for k_, t in d.items()}


def prefill_token_heads(B, T, H):
    return B * T * H


def chunk_count(T, C):
    return math.ceil(T / C)
