"""Parity measures shared by the GPU tests: the relative Frobenius error over
a whole compared slice, and its worst value over every head and over every
64-token chunk of every head, so that an error confined to one chunk of one
head cannot hide under the norm of the rest.

All arrays are float64 numpy arrays (the GPU output upcast, the oracle's
result as it is).  Token-major outputs are [B, T, H, dv]; states are
[B, H, dk, dv]; decode outputs stacked over steps are [steps, N, H, dv].
"""
from __future__ import annotations

import numpy as np


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _rel_rows(d, r):
    """rel over the trailing axes of [n, ...] stacks -> [n]."""
    n = d.shape[0]
    num = np.linalg.norm(d.reshape(n, -1), axis=1)
    den = np.maximum(np.linalg.norm(r.reshape(n, -1), axis=1), 1e-300)
    return num / den


def worst_token_major(x, ref, chunk=64):
    """(worst per head, worst per chunk of a head) for [B, T, H, dv] outputs.

    A head or chunk whose reference is all zeros (identity padding, zero
    input) is left out of the maxima; the whole-slice error still covers it."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    B, T, H, dv = ref.shape
    d = x - ref
    dh = d.transpose(0, 2, 1, 3).reshape(B * H, T * dv)
    rh = ref.transpose(0, 2, 1, 3).reshape(B * H, T * dv)
    lh = np.linalg.norm(rh, axis=1) > 0
    heads = _rel_rows(dh[lh], rh[lh]) if lh.any() else np.zeros(0)
    nc = -(-T // chunk)
    pad = nc * chunk - T
    dp = np.pad(d, ((0, 0), (0, pad), (0, 0), (0, 0)))
    rp = np.pad(ref, ((0, 0), (0, pad), (0, 0), (0, 0)))
    dc = dp.reshape(B, nc, chunk, H, dv).transpose(0, 3, 1, 2, 4).reshape(B * H * nc, chunk * dv)
    rc = rp.reshape(B, nc, chunk, H, dv).transpose(0, 3, 1, 2, 4).reshape(B * H * nc, chunk * dv)
    live = np.linalg.norm(rc, axis=1) > 0
    chunks = _rel_rows(dc[live], rc[live]) if live.any() else np.zeros(1)
    return float(heads.max()) if heads.size else 0.0, float(chunks.max())


def worst_state(S, S_ref):
    """Worst per-head relative error of [B, H, dk, dv] states (heads whose
    reference state is all zeros are left to the whole-slice error)."""
    S = np.asarray(S, dtype=np.float64)
    S_ref = np.asarray(S_ref, dtype=np.float64)
    B, H = S_ref.shape[:2]
    d = (S - S_ref).reshape(B * H, -1)
    r = S_ref.reshape(B * H, -1)
    live = np.linalg.norm(r, axis=1) > 0
    return float(_rel_rows(d[live], r[live]).max()) if live.any() else 0.0


def report(label, tol, o=None, o_ref=None, S=None, S_ref=None, chunk=64, steps_major=False):
    """Print and assert every measure against `tol`.

    o is token-major [B, T, H, dv], or [steps, N, H, dv] for decode runs when
    steps_major (steps play the role of tokens).  Returns the measures."""
    m = {}
    if o is not None:
        if steps_major:
            o = np.asarray(o).transpose(1, 0, 2, 3)
            o_ref = np.asarray(o_ref).transpose(1, 0, 2, 3)
        m["o"] = rel(o, o_ref)
        m["o_head_max"], m["o_chunk_max"] = worst_token_major(o, o_ref, chunk)
    if S is not None:
        m["S"] = rel(S, S_ref)
        m["S_head_max"] = worst_state(S, S_ref)
    print(f"[{label}] " + " ".join(f"{k}={v:.3e}" for k, v in m.items()), flush=True)
    if o is not None:
        assert np.isfinite(np.asarray(o, dtype=np.float64)).all(), label
    if S is not None:
        assert np.isfinite(np.asarray(S, dtype=np.float64)).all(), label
    bad = {k: v for k, v in m.items() if not v < tol}
    assert not bad, f"{label}: {bad} (bar {tol})"
    return m
