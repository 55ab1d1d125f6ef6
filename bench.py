"""KDA benchmark on one MI355X: chunked prefill tokens/s (plus decode state
GB/s) with roofline fractions and the CPU oracle as a reported baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one kda_prefill_chunked call over the long-context workload, the
largest that fits one GPU: B=1, H=32, T=1,048,576, dk=dv=128, bf16 q/k/v/o,
fp32 gates, strengths and state, C=64, inputs already resident in HBM.  Prints
ONE JSON line.  Alongside the headline it measures, on the same GPU:
  * the H=16, T=4096 prefill and the B=8, H=32, T=8192 prefill (tokens/s and
    roofline);
  * 256 single-sequence decode steps from the long-context final state;
  * decode: 256 sequences x 32 heads, 64 KiB fp32 state per head, in-place
    kda_decode_step calls (state GB/s against the HBM peak);
  * the H=16 prefill and the 256 x 32-head decode from raw projections
    (gate logits, write-strength logits, q/k L2-normalised in the kernels);
  * the same two with one gate per token and head (Gated DeltaNet);
  * the adjoint of one decode step for 256 sequences x 32 heads, the prefill
    backward and the prologue kernels on the H=16 workload;
  * the float64 oracle on the host cores over bounded samples of the
    long-context prefill and of the decode workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def prefill_alg_bytes(B, T, H, dk, dv, esize, with_s0):
    """Inputs and outputs only: q, k, v, o in the I/O dtype, fp32 alpha and
    beta, the final state (and the initial state when one is given)."""
    tok = B * T * H
    per_tok = esize * (2 * dk + dv) + 4 * dk + 4 + esize * dv
    state = B * H * dk * dv * 4
    return tok * per_tok + state * (2 if with_s0 else 1)


def prefill_logit_alg_bytes(B, T, H, dk, dv, esize, with_s0):
    """As prefill_alg_bytes, with the gate read as logits of the I/O type
    instead of fp32 alpha, and beta read as fp32 logits."""
    tok = B * T * H
    per_tok = esize * (2 * dk + dv) + esize * dk + 4 + esize * dv
    state = B * H * dk * dv * 4
    return tok * per_tok + state * (2 if with_s0 else 1)


def gdn_alg_bytes(B, T, H, dk, dv, esize, with_s0):
    """As prefill_alg_bytes, with one fp32 gate per token and head."""
    tok = B * T * H
    per_tok = esize * (2 * dk + dv) + 4 + 4 + esize * dv
    state = B * H * dk * dv * 4
    return tok * per_tok + state * (2 if with_s0 else 1)


def prefill_flops(B, T, H, dk, dv, C):
    """Useful flops: 6 dk dv per token-head for the state work (W S, Q S,
    K^T U) plus 2 C (3 dk + 2 dv) for the chunk-local products (gated K K^T,
    gated Q K^T, W, U~, P U)."""
    return B * T * H * (6 * dk * dv + 2 * C * (3 * dk + 2 * dv))


def decode_alg_bytes(N, H, dk, dv, esize, gate_bytes=4):
    """State read and write plus one token's inputs and output per head; the
    gate is fp32 alpha (4 bytes) or a logit of the I/O type."""
    per_head = 2 * dk * dv * 4 + esize * (2 * dk + dv) + gate_bytes * dk + 4 + esize * dv
    return N * H * per_head


def decode_bwd_alg_bytes(N, H, dk, dv, esize):
    """Step adjoint: state and incoming state gradient read, outgoing state
    gradient written (fp32), the step's vectors read and their gradients
    written."""
    per_head = (3 * dk * dv * 4 + esize * (2 * dk + dv) + 4 * dk + 4 + esize * dv
                + esize * (2 * dk + dv) + 4 * dk + 4)
    return N * H * per_head


def prefill_bwd_alg_bytes(B, T, H, dk, dv, esize):
    """Prefill backward: the forward inputs (q, k, v, alpha, beta) and dO read
    once, the gradients (dq, dk, dv, dalpha fp32, dbeta) written once, and
    dS_T read and dS0 written per head; the stored states (dk dv / 16 floats
    per token-head, written and read back) are the method's own traffic."""
    per_tok = esize * (2 * dk + dv) + 4 * dk + 4 + esize * dv + 4 * (3 * dk + dv) + 4
    return B * T * H * per_tok + 2 * B * H * dk * dv * 4


def prologue_alg_bytes(rows, dk, esize):
    """The prologue alone, per row: forward reads q, k, g (I/O type) and b,
    writes q_hat, k_hat (I/O type), alpha and beta (fp32); the adjoint reads
    q, k, g, b and the fp32 gradients of q_hat, k_hat, alpha, beta and writes
    the fp32 gradients of q, k, g, b.  Returns (forward, adjoint) bytes."""
    fwd = rows * (3 * esize * dk + 4 + 2 * esize * dk + 4 * dk + 4)
    bwd = rows * (3 * esize * dk + 4 + 3 * 4 * dk + 4 + 3 * 4 * dk + 4)
    return fwd, bwd


def _code_only(text):
    """C++ source without comments and with whitespace runs collapsed, so that
    editing a comment does not count as changing a kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                   # string or char literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """sha256 over the library's kernel sources (file names and code, comments
    and whitespace excluded)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_108_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def profiled_traffic(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (profiles/<name>.txt), or None when the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"{name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def prefill_kernels(kda, B, T, H, dk, dv, C):
    """Names of the kernels one prefill call launches (the path the library
    picks: a workspace means the split path, prep kernel + scan kernel)."""
    if kda.prefill_workspace_bytes(B, T, H, dk, dv, C) > 0:
        return f"kda_prefill_kernel<bf16,{dk},{C},{dv},prep> + kda_scan_kernel<bf16,{dk},{C}>"
    return f"kda_prefill_kernel<bf16,{dk},{C},dv-slab>"


def time_launches(fn, steps, warmup, torch):
    """Warm up, then time `steps` calls bracketed by synchronisations, with
    HIP events on the current stream (the stream the kernels run on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall * 1e3 / steps


def _oracle_chain(args):
    import numpy as np  # noqa: F401
    from oracle import kda_recurrence
    q, k, v, a, b = args
    t = time.perf_counter()
    kda_recurrence(q, k, v, a, b, None)
    return time.perf_counter() - t


def _oracle_decode_run(args):
    """One sequence's decode steps through the oracle: (seconds, steps)."""
    from oracle import kda_decode_step
    S, q, k, v, a, b = args
    t = time.perf_counter()
    for i in range(q.shape[0]):
        _, S = kda_decode_step(q[i], k[i], v[i], a[i], b[i], S)
    return time.perf_counter() - t


# Bounded samples the oracle is timed on (seconds of work, not the full jobs).
CPU_PREFILL_SAMPLE_T = 4096        # tokens of every head of the long-context workload
CPU_DECODE_SAMPLE_N = 8            # sequences x 32 heads of the decode workload
CPU_DECODE_SAMPLE_STEPS = 1000          # all steps of the decode workload


def cpu_baseline(wl):
    """The float64 oracle as it stands, one process per host core (at most 16),
    each running whole chains with single-threaded BLAS, on bounded samples:
    the long-context prefill's first CPU_PREFILL_SAMPLE_T tokens of all 32
    heads (the same distributions and channel-mixture gates), repeated to
    about 10 core-s, and 8 sequences x 32 heads of the decode workload over
    all of its 1000 steps."""
    import concurrent.futures as cf
    import multiprocessing as mp
    spec = wl.PREFILL["longctx_h32_t1m"]
    inp = wl.make_prefill_inputs(spec, "cpu", T=CPU_PREFILL_SAMPLE_T)
    B, T, H, _ = inp["q"].shape
    f = lambda t: t.float().numpy()  # noqa: E731  (bf16 -> fp32 is exact)
    chains = [(f(inp["q"][b:b + 1, :, h:h + 1]), f(inp["k"][b:b + 1, :, h:h + 1]),
               f(inp["v"][b:b + 1, :, h:h + 1]), f(inp["alpha"][b:b + 1, :, h:h + 1]),
               f(inp["beta"][b:b + 1, :, h:h + 1]))
              for b in range(B) for h in range(H)]
    dspec = wl.DECODE["decode_n256_h32"]
    S = wl.make_decode_state(dspec, "cpu", N=CPU_DECODE_SAMPLE_N)
    st = wl.make_decode_steps(dspec, "cpu", N=CPU_DECODE_SAMPLE_N, steps=CPU_DECODE_SAMPLE_STEPS)
    runs = [(S[n:n + 1].double().numpy(),) + tuple(f(st[x][:, n:n + 1])
                                                   for x in ("q", "k", "v", "alpha", "beta"))
            for n in range(CPU_DECODE_SAMPLE_N)]
    cores = min(len(os.sched_getaffinity(0)), 16, len(chains))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx,
                                initializer=_single_thread_blas) as ex:
        # one untimed pass starts the processes and sizes the sample: the
        # timed sample repeats the prefill slice to about 10 core-s of work
        first = sum(ex.map(_oracle_chain, chains))
        reps = max(1, min(40, math.ceil(10.0 / max(first, 1e-3))))
        t0 = time.perf_counter()
        busy = sum(ex.map(_oracle_chain, chains * reps))
        wall = time.perf_counter() - t0
        t1 = time.perf_counter()
        dbusy = sum(ex.map(_oracle_decode_run, runs))
        dwall = time.perf_counter() - t1
    head_steps = CPU_DECODE_SAMPLE_N * dspec.H * CPU_DECODE_SAMPLE_STEPS
    dcores = min(cores, CPU_DECODE_SAMPLE_N)
    return dict(
        value=reps * B * T / wall, unit="tokens/s", cores=cores, kind="oracle",
        sample=f"the long-context workload's first {T} tokens of all {H} heads "
               f"({B * T * H} token-heads, {len(chains)} chains, same distributions and "
               f"gates) run {reps} times over {cores} processes; {busy:.1f} core-s of oracle "
               f"work, {wall:.1f} s wall",
        tok_heads_per_s=reps * B * T * H / wall,
        decode={"head_steps_per_s": head_steps / dwall, "unit": "head-steps/s",
                "state_GBps": head_steps * 2 * dspec.dk * dspec.dv * 4 / dwall / 1e9,
                "cores": dcores, "kind": "oracle",
                "sample": f"{CPU_DECODE_SAMPLE_N} sequences x {dspec.H} heads of the decode "
                          f"workload (state sd 0.01, alpha U(0.95, 1), bf16 q/k/v), "
                          f"{CPU_DECODE_SAMPLE_STEPS} steps each, one process per sequence; "
                          f"{dbusy:.1f} core-s, {dwall:.1f} s wall"})


def _single_thread_blas():
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline prefill only (no decode / large prefill lines)")
    ap.add_argument("--only", choices=["longctx", "prefill", "decode", "large", "logits",
                                       "decode_logits", "gdn", "decode_gdn", "longctx_decode",
                                       "decode_bwd", "prefill_bwd", "prefill_bwd_large",
                                       "prologue", "copy"],
                    default=None,
                    help="run one leg only (for profiler runs); 'copy' times a plain "
                         "1 GiB device-to-device copy used to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(chains are independent, so N GPUs would each run their own share).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_108_amd as kda
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out = {}
    if args.only == "copy":
        n = 1 << 28                                     # 2^28 floats = 1 GiB
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        ms, _ = time_launches(lambda: y.copy_(x), args.steps, args.warmup, torch)
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "ms_per_copy": ms, "GBps": 8 * n / (ms * 1e-3) / 1e9}), flush=True)
        return
    legs = ({"longctx", "prefill", "decode", "large", "logits", "decode_logits", "gdn",
             "decode_gdn", "longctx_decode", "decode_bwd", "prefill_bwd", "prefill_bwd_large",
             "prologue"}
            if args.only is None else {args.only})
    if args.no_extra:
        legs = {"longctx"}

    # ---------------- headline: long-context prefill, H=32, T=2^20, d=128, bf16, C=64
    if "longctx" in legs:
        headline(args, out, torch, kda, wl, dev)
    extras(args, legs, out, torch, kda, wl, dev)
    if not args.no_cpu and args.only is None:
        out["cpu_baseline"] = cpu_baseline(wl)
        print(f"# cpu_baseline: {out['cpu_baseline']['value']:.1f} tokens/s; decode "
              f"{out['cpu_baseline']['decode']['head_steps_per_s']:.0f} head-steps/s",
              file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def measure_prefill(args, spec, C, torch, kda, dev, steps, warmup, name):
    """Time kda_prefill_chunked on one workload (inputs drawn on the device);
    returns the figures of one call against the HBM and bf16 MFMA peaks."""
    import workloads as wl
    g = wl.make_prefill_inputs(spec, dev)
    o = torch.empty(spec.B, spec.T, spec.H, spec.dv, dtype=spec.dtype, device=dev)
    S_T = torch.empty(spec.B, spec.H, spec.dk, spec.dv, dtype=torch.float32, device=dev)
    B, T, H, dk, dv = spec.B, spec.T, spec.H, spec.dk, spec.dv
    ws_bytes = kda.prefill_workspace_bytes(B, T, H, dk, dv, C)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        kda.prefill_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"], chunk=C,
                            out=o, state_out=S_T, workspace=ws)

    ms_ev, ms_wall = time_launches(step, steps, warmup, torch)
    nbytes = prefill_alg_bytes(B, T, H, dk, dv, 2, g["S0"] is not None)
    flops = prefill_flops(B, T, H, dk, dv, C)
    gbs = nbytes / (ms_ev * 1e-3) / 1e9
    tfl = flops / (ms_ev * 1e-3) / 1e12
    del g, o, S_T, ws
    torch.cuda.empty_cache()
    return dict(C=C, kernel=prefill_kernels(kda, B, T, H, dk, dv, C), ms_per_launch=ms_ev,
                ms_wall=ms_wall, tokens_per_s=B * T / (ms_wall * 1e-3),
                tok_heads_per_s=B * T * H / (ms_wall * 1e-3), GBps=gbs,
                frac_hbm=gbs / HBM_PEAK_GBS, traffic=profiled_traffic(name),
                alg_bytes_per_launch=nbytes, tflops=tfl,
                frac_mfma=tfl / MFMA_BF16_PEAK_TFLOPS, flops_per_launch=flops)


def headline(args, out, torch, kda, wl, dev):
    """The long-context prefill: B=1, H=32, T=1,048,576, d=128, bf16, C=64."""
    spec = wl.PREFILL["longctx_h32_t1m"]
    C = 64
    r = measure_prefill(args, spec, C, torch, kda, dev, args.steps, args.warmup,
                        "longctx_h32_t1m")
    B, T, H, dk, dv = spec.B, spec.T, spec.H, spec.dk, spec.dv
    out.update({
        "metric": "KDA prefill tokens/s + % bf16 MFMA peak; decode state GB/s + % HBM peak",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_wall"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "longctx_h32_t1m", "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
                   "C": C, "io_dtype": "bf16", "state_dtype": "fp32",
                   "gates": "13 of 128 channels per head U(0, 0.5), the rest U(0.99, 1)"},
        "roofline": {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r["frac_hbm"], "traffic": r["traffic"],
                     "kernel": r["kernel"], "kernel_ms": r["ms_per_launch"],
                     "alg_bytes_per_launch": r["alg_bytes_per_launch"]},
        "mfma": {"achieved_tflops": r["tflops"], "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": r["frac_mfma"], "flops_per_launch": r["flops_per_launch"]},
        "tok_heads_per_s": r["tok_heads_per_s"],
    })
    print(f"# longctx_h32_t1m: {r['ms_per_launch']:.2f} ms/launch (events), "
          f"{r['GBps']:.0f} GB/s, {r['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)



def extras(args, legs, out, torch, kda, wl, dev):
    if "decode" in legs:
        # ---------------- decode: 256 x 32 heads, d = 128, in place
        dspec = wl.DECODE["decode_n256_h32"]
        S = wl.make_decode_state(dspec, dev)
        nst = 8
        st = wl.make_decode_steps(dspec, dev, steps=nst)
        od = torch.empty(dspec.N, dspec.H, dspec.dv, dtype=dspec.dtype, device=dev)
        it = [0]

        def dstep():
            i = it[0] % nst
            it[0] += 1
            kda.decode_step(st["q"][i], st["k"][i], st["v"][i], st["alpha"][i], st["beta"][i],
                            S, out=od)

        dsteps = max(args.steps, 20)
        ms_d, ms_dw = time_launches(dstep, dsteps, args.warmup, torch)
        state_bytes = 2 * dspec.N * dspec.H * dspec.dk * dspec.dv * 4
        dbytes = decode_alg_bytes(dspec.N, dspec.H, dspec.dk, dspec.dv, 2)
        out["decode"] = {
            "workload": "decode_n256_h32", "N": dspec.N, "H": dspec.H, "dk": dspec.dk,
            "dv": dspec.dv, "us_per_step": ms_d * 1e3,
            "state_GBps": state_bytes / (ms_d * 1e-3) / 1e9,
            "alg_GBps": dbytes / (ms_d * 1e-3) / 1e9,
            "frac_hbm": dbytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("decode_n256_h32"), "alg_bytes_per_step": dbytes,
            "head_steps_per_s": dspec.N * dspec.H / (ms_dw * 1e-3),
        }
        print(f"# decode_n256_h32: {ms_d * 1e3:.1f} us/step, "
              f"{out['decode']['alg_GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        del S, st, od
        torch.cuda.empty_cache()

    if "prefill" in legs:
        # ---------------- the H=16, T=4096 prefill (split path, launch-latency regime)
        spec = wl.PREFILL["prefill_h16_t4k"]
        r = measure_prefill(args, spec, 64, torch, kda, dev, args.steps, args.warmup,
                            "prefill_h16_t4k")
        out["prefill_h16_t4k"] = {k_: v_ for k_, v_ in r.items() if k_ != "ms_wall"}
        print(f"# prefill_h16_t4k: {r['ms_per_launch'] * 1e3:.1f} us/launch, "
              f"{r['GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    if "large" in legs:
        # ---------------- large prefill: B=8, H=32, T=8192 (fused path)
        lspec = wl.PREFILL["prefill_b8_h32_t8k"]
        lsteps = max(3, args.steps // 5)
        r = measure_prefill(args, lspec, 64, torch, kda, dev, lsteps, 2, "prefill_b8_h32_t8k")
        out["prefill_b8_h32_t8k"] = {k_: v_ for k_, v_ in r.items() if k_ != "ms_wall"}
        # the chunk-size comparison on the same workload: C = 16 and 32 are
        # their own kernels; C = 128 runs as two 64-token chunks (its tiles do
        # not fit one CU's LDS), so its row is the C = 64 kernel
        sweep = {}
        for C in (16, 32):
            rc = measure_prefill(args, lspec, C, torch, kda, dev, lsteps, 1, None)
            sweep[f"C{C}_ms_per_launch"] = rc["ms_per_launch"]
        sweep["C64_ms_per_launch"] = r["ms_per_launch"]
        sweep["C128_ms_per_launch"] = r["ms_per_launch"]
        sweep["C128_note"] = "runs as two 64-token chunks (same kernel as C = 64)"
        out["prefill_b8_h32_t8k"]["chunk_sweep"] = sweep
        print(f"# prefill_b8_h32_t8k: {r['ms_per_launch']:.3f} ms/launch; C=16 "
              f"{sweep['C16_ms_per_launch']:.3f}, C=32 {sweep['C32_ms_per_launch']:.3f}",
              file=sys.stderr, flush=True)

    if "logits" in legs:
        # ---------------- H=16 prefill from raw projections (fused prologue)
        spec = wl.PREFILL["prefill_h16_t4k"]
        rg = wl.make_prefill_logit_inputs(spec, dev)
        ro = torch.empty(spec.B, spec.T, spec.H, spec.dv, dtype=spec.dtype, device=dev)
        rS = torch.empty(spec.B, spec.H, spec.dk, spec.dv, dtype=torch.float32, device=dev)

        def rstep():
            kda.prefill_chunked_logits(rg["q"], rg["k"], rg["v"], rg["g"], rg["b"], rg["S0"],
                                       chunk=64, qk_map="l2", out=ro, state_out=rS)

        ms_r, ms_rw = time_launches(rstep, args.steps, args.warmup, torch)
        B, T, H, dk, dv = spec.B, spec.T, spec.H, spec.dk, spec.dv
        rb = prefill_logit_alg_bytes(B, T, H, dk, dv, 2, False)
        rf = prefill_flops(B, T, H, dk, dv, 64)
        out["prefill_h16_t4k_logits"] = {
            "C": 64, "qk_map": "l2", "us_per_launch": ms_r * 1e3,
            "tokens_per_s": B * T / (ms_rw * 1e-3),
            "GBps": rb / (ms_r * 1e-3) / 1e9, "frac_hbm": rb / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("prefill_h16_t4k_logits"), "alg_bytes_per_launch": rb,
            "tflops": rf / (ms_r * 1e-3) / 1e12,
            "frac_mfma": rf / (ms_r * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        }
        print(f"# prefill_h16_t4k_logits: {ms_r * 1e3:.1f} us/launch", file=sys.stderr,
              flush=True)
        del rg, ro, rS
        torch.cuda.empty_cache()

    if "decode_logits" in legs:
        # ---------------- decode from raw projections: 256 x 32 heads, in place
        dspec = wl.DECODE["decode_n256_h32"]
        S = wl.make_decode_state(dspec, dev)
        nst = 8
        st = wl.make_decode_logit_steps(dspec, dev, steps=nst)
        od = torch.empty(dspec.N, dspec.H, dspec.dv, dtype=dspec.dtype, device=dev)
        it = [0]

        def lstep():
            i = it[0] % nst
            it[0] += 1
            kda.decode_step_logits(st["q"][i], st["k"][i], st["v"][i], st["g"][i], st["b"][i],
                                   S, qk_map="l2", out=od)

        ms_d, _ = time_launches(lstep, max(args.steps, 20), args.warmup, torch)
        dbytes = decode_alg_bytes(dspec.N, dspec.H, dspec.dk, dspec.dv, 2, gate_bytes=2)
        out["decode_n256_h32_logits"] = {
            "qk_map": "l2", "us_per_step": ms_d * 1e3,
            "alg_GBps": dbytes / (ms_d * 1e-3) / 1e9,
            "frac_hbm": dbytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("decode_n256_h32_logits"), "alg_bytes_per_step": dbytes,
        }
        print(f"# decode_n256_h32_logits: {ms_d * 1e3:.1f} us/step", file=sys.stderr,
              flush=True)
        del S, st, od
        torch.cuda.empty_cache()

    if "gdn" in legs:
        # ---------------- H=16 prefill with one gate per token and head (GDN)
        spec = wl.PREFILL["prefill_h16_t4k"]
        gi = wl.make_gdn_inputs(spec, dev)
        go = torch.empty(spec.B, spec.T, spec.H, spec.dv, dtype=spec.dtype, device=dev)
        gS = torch.empty(spec.B, spec.H, spec.dk, spec.dv, dtype=torch.float32, device=dev)

        def gstep():
            kda.gdn_prefill_chunked(gi["q"], gi["k"], gi["v"], gi["a"], gi["beta"], gi["S0"],
                                    chunk=64, out=go, state_out=gS)

        ms_g, ms_gw = time_launches(gstep, args.steps, args.warmup, torch)
        B, T, H, dk, dv = spec.B, spec.T, spec.H, spec.dk, spec.dv
        gb = gdn_alg_bytes(B, T, H, dk, dv, 2, False)
        gf = prefill_flops(B, T, H, dk, dv, 64)
        out["prefill_h16_t4k_gdn"] = {
            "C": 64, "us_per_launch": ms_g * 1e3, "tokens_per_s": B * T / (ms_gw * 1e-3),
            "GBps": gb / (ms_g * 1e-3) / 1e9, "frac_hbm": gb / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("prefill_h16_t4k_gdn"), "alg_bytes_per_launch": gb,
            "tflops": gf / (ms_g * 1e-3) / 1e12,
            "frac_mfma": gf / (ms_g * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        }
        print(f"# prefill_h16_t4k_gdn: {ms_g * 1e3:.1f} us/launch", file=sys.stderr, flush=True)
        del gi, go, gS
        torch.cuda.empty_cache()

    if "decode_gdn" in legs:
        # ---------------- GDN decode: 256 x 32 heads, one gate per head, in place
        dspec = wl.DECODE["decode_n256_h32"]
        S = wl.make_decode_state(dspec, dev)
        nst = 8
        st = wl.make_decode_steps(dspec, dev, steps=nst)
        ga = st["alpha"][..., 0].contiguous()
        od = torch.empty(dspec.N, dspec.H, dspec.dv, dtype=dspec.dtype, device=dev)
        it = [0]

        def gdstep():
            i = it[0] % nst
            it[0] += 1
            kda.gdn_decode_step(st["q"][i], st["k"][i], st["v"][i], ga[i], st["beta"][i], S,
                                out=od)

        ms_d, _ = time_launches(gdstep, max(args.steps, 20), args.warmup, torch)
        dbytes = decode_alg_bytes(dspec.N, dspec.H, dspec.dk, dspec.dv, 2, gate_bytes=0) \
            + dspec.N * dspec.H * 4
        out["decode_n256_h32_gdn"] = {
            "us_per_step": ms_d * 1e3, "alg_GBps": dbytes / (ms_d * 1e-3) / 1e9,
            "frac_hbm": dbytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("decode_n256_h32_gdn"), "alg_bytes_per_step": dbytes,
        }
        print(f"# decode_n256_h32_gdn: {ms_d * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        del S, st, od, ga
        torch.cuda.empty_cache()

    if "decode_bwd" in legs:
        # ---------------- step adjoint: 256 x 32 heads, dS in place over dS_new
        dspec = wl.DECODE["decode_n256_h32"]
        S = wl.make_decode_state(dspec, dev)
        gS = wl.make_decode_state(dspec, dev, N=dspec.N)
        st = wl.make_decode_step_inputs(dspec, dev)
        dO = st["v"].clone()

        def bstep():
            kda.decode_step_backward(st["q"], st["k"], st["v"], st["alpha"], st["beta"], S, dO,
                                     gS, in_place=True)

        ms_b, _ = time_launches(bstep, max(args.steps, 20), args.warmup, torch)
        bbytes = decode_bwd_alg_bytes(dspec.N, dspec.H, dspec.dk, dspec.dv, 2)
        ga = st["alpha"][..., 0].contiguous()            # one gate per head

        def gstep():
            kda.gdn_decode_step_backward(st["q"], st["k"], st["v"], ga, st["beta"], S, dO, gS,
                                         in_place=True)

        ms_gb, _ = time_launches(gstep, max(args.steps, 20), args.warmup, torch)
        out["decode_bwd_n256_h32"] = {
            "us_per_step": ms_b * 1e3, "alg_GBps": bbytes / (ms_b * 1e-3) / 1e9,
            "frac_hbm": bbytes / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": profiled_traffic("decode_bwd_n256_h32"), "alg_bytes_per_step": bbytes,
            "gdn_us_per_step": ms_gb * 1e3,
        }
        print(f"# decode_bwd_n256_h32: {ms_b * 1e3:.1f} us/step, "
              f"{out['decode_bwd_n256_h32']['alg_GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        del S, gS, st, dO, ga
        torch.cuda.empty_cache()

    if "prefill_bwd" in legs:
        # ---------------- prefill backward on the headline workload
        pspec = wl.PREFILL["prefill_h16_t4k"]
        px = wl.make_prefill_inputs(pspec, dev)
        pg = wl.make_prefill_backward_grads(pspec, dev)

        def pbstep():
            kda.prefill_backward(px["q"], px["k"], px["v"], px["alpha"], px["beta"], pg["dO"],
                                 S0=px["S0"], dS_T=pg["dS_T"])

        ms_p, _ = time_launches(pbstep, 5, 1, torch)
        B, T, H, dk, dv = pspec.B, pspec.T, pspec.H, pspec.dk, pspec.dv
        pbytes = prefill_bwd_alg_bytes(B, T, H, dk, dv, 2)
        cws = torch.empty(kda.prefill_backward_chunked_workspace_bytes(B, T, H, dk, dv),
                          dtype=torch.uint8, device=dev)

        def cbstep():
            kda.prefill_backward_chunked(px["q"], px["k"], px["v"], px["alpha"], px["beta"],
                                         pg["dO"], S0=px["S0"], dS_T=pg["dS_T"], workspace=cws)

        ms_c, _ = time_launches(cbstep, 20, 3, torch)
        gx = wl.make_gdn_inputs(pspec, dev)

        def gbstep():
            kda.gdn_prefill_backward(gx["q"], gx["k"], gx["v"], gx["a"], gx["beta"], pg["dO"],
                                     S0=gx["S0"], dS_T=pg["dS_T"])

        ms_g, _ = time_launches(gbstep, 5, 1, torch)
        out["prefill_bwd_h16_t4k"] = {
            "kernel": "kda_prefill_backward_chunked (forward split path with chunk states, "
                      "sub-chunk records, state-gradient scan, gradient kernel)",
            "ms_per_call": ms_c, "tokens_per_s": B * T / (ms_c * 1e-3),
            "alg_GBps": pbytes / (ms_c * 1e-3) / 1e9,
            "frac_hbm": pbytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": pbytes, "traffic": profiled_traffic("prefill_bwd_h16_t4k"),
            "deterministic": True,
            "token_walk_ms_per_call": ms_p,
            "gdn_token_walk_ms_per_call": ms_g,
        }
        print(f"# prefill_bwd_h16_t4k: chunked {ms_c:.3f} ms/call, token walk {ms_p:.3f} ms "
              f"(Gated DeltaNet {ms_g:.3f} ms)", file=sys.stderr, flush=True)
        del px, pg, gx, cws
        torch.cuda.empty_cache()

    if "prefill_bwd_large" in legs:
        # ---------------- the chunked backward on the largest batch
        lspec = wl.PREFILL["prefill_b8_h32_t8k"]
        lx = wl.make_prefill_inputs(lspec, dev)
        lg = wl.make_prefill_backward_grads(lspec, dev)
        B, T, H, dk, dv = lspec.B, lspec.T, lspec.H, lspec.dk, lspec.dv
        lws = torch.empty(kda.prefill_backward_chunked_workspace_bytes(B, T, H, dk, dv),
                          dtype=torch.uint8, device=dev)

        def lbstep():
            kda.prefill_backward_chunked(lx["q"], lx["k"], lx["v"], lx["alpha"], lx["beta"],
                                         lg["dO"], S0=lx["S0"], dS_T=lg["dS_T"], workspace=lws)

        ms_l, _ = time_launches(lbstep, 5, 1, torch)
        lbytes = prefill_bwd_alg_bytes(B, T, H, dk, dv, 2)
        out["prefill_bwd_b8_h32_t8k"] = {
            "ms_per_call": ms_l, "tokens_per_s": B * T / (ms_l * 1e-3),
            "alg_GBps": lbytes / (ms_l * 1e-3) / 1e9,
            "frac_hbm": lbytes / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": lbytes, "traffic": profiled_traffic("prefill_bwd_b8_h32_t8k"),
        }
        print(f"# prefill_bwd_b8_h32_t8k: chunked {ms_l:.3f} ms/call", file=sys.stderr, flush=True)
        del lx, lg, lws
        torch.cuda.empty_cache()

    if "prologue" in legs:
        # ---------------- the prologue alone, forward and adjoint, on the H=16 T=4096 rows
        lspec = wl.PREFILL["prefill_h16_t4k"]
        lx = wl.make_prefill_logit_inputs(lspec, dev)
        rows, dk = lspec.B * lspec.T * lspec.H, lspec.dk
        grad = [torch.randn(lx["q"].shape, device=dev) for _ in range(3)]
        gb = torch.randn(lx["b"].shape, device=dev)

        def pf():
            kda.prologue_forward(lx["q"], lx["k"], lx["g"], lx["b"], "silu_l2")

        def pbk():
            kda.prologue_backward(lx["q"], lx["k"], lx["g"], lx["b"], *grad, gb, "silu_l2")

        ms_f, _ = time_launches(pf, max(args.steps, 20), args.warmup, torch)
        ms_b, _ = time_launches(pbk, max(args.steps, 20), args.warmup, torch)
        fb, bb = prologue_alg_bytes(rows, dk, 2)
        out["prologue_h16_t4k"] = {
            "forward_us": ms_f * 1e3, "forward_GBps": fb / (ms_f * 1e-3) / 1e9,
            "adjoint_us": ms_b * 1e3, "adjoint_GBps": bb / (ms_b * 1e-3) / 1e9,
            "frac_hbm_forward": fb / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "frac_hbm_adjoint": bb / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes": [fb, bb], "traffic": profiled_traffic("prologue_h16_t4k"),
            "note": "65,536 rows of 128 channels, bf16, SiLU + L2 map; events bracket "
                    "back-to-back calls from Python (per-call host time included)",
        }
        print(f"# prologue_h16_t4k: forward {ms_f * 1e3:.1f} us, adjoint {ms_b * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        del lx, grad, gb
        torch.cuda.empty_cache()

    if "longctx_decode" in legs:
        # ---------------- 256 single-sequence decode steps after the long-context prefill
        cspec = wl.PREFILL["longctx_h32_t1m"]
        cg = wl.make_prefill_inputs(cspec, dev)
        _, cS = kda.prefill_chunked(cg["q"], cg["k"], cg["v"], cg["alpha"], cg["beta"], None,
                                    chunk=64)
        del cg
        torch.cuda.empty_cache()
        dspec = wl.DECODE["longctx_decode"]
        mask = wl.mixture_low_channels(32, 128, cspec.seed)
        st = wl.make_decode_steps(dspec, dev, N=1, alpha_mask=mask)
        od = torch.empty(1, 32, 128, dtype=dspec.dtype, device=dev)
        it = [0]

        def dstep():
            i = it[0] % dspec.steps
            it[0] += 1
            kda.decode_step(st["q"][i], st["k"][i], st["v"][i], st["alpha"][i], st["beta"][i],
                            cS, out=od)

        ms_d, _ = time_launches(dstep, dspec.steps, 8, torch)
        # the same steady loop captured once as a HIP graph (no memset nodes:
        # the steps write o and the state in place) and replayed
        graph = torch.cuda.CUDAGraph()
        it[0] = 0
        with torch.cuda.graph(graph):
            for _ in range(dspec.steps):
                dstep()
        ms_g, _ = time_launches(graph.replay, 4, 1, torch)
        out["longctx_decode"] = {
            "N": 1, "H": 32, "steps": dspec.steps, "decode_us_per_step": ms_d * 1e3,
            "graph_us_per_step": ms_g * 1e3 / dspec.steps,
            "decode_note": "one sequence x 32 heads: 4 MiB of state per step; "
                           "decode_us_per_step: events around back-to-back calls from "
                           "Python (the binding's per-call host time included); "
                           "graph_us_per_step: the 256 steps captured as one HIP graph "
                           "and replayed (kernel time: profiles/)",
        }
        print(f"# longctx_decode: {ms_d * 1e3:.1f} us/step eager, "
              f"{ms_g * 1e3 / dspec.steps:.1f} us/step graph", file=sys.stderr, flush=True)
        del graph
        del st, od, cS
        torch.cuda.empty_cache()

if __name__ == "__main__":
    main()
