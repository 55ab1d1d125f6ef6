"""Build libkda.so in-tree for gfx950 with hipcc.

Every HIP translation unit under csrc/ is compiled in parallel, then linked
into gated_delta_rule_108_amd/libkda.so.  Run directly
(`python -m gated_delta_rule_108_amd.build`) or through
`__graft_entry__.build()`; a build always recompiles every source.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
ARCH = "gfx950"

# Packed-fp32 instructions are switched off on purpose: ordinary float code
# only, no v_pk_* fp32 forms generated behind our back.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file extra flags.  The state-gradient scan of the chunked backward
# otherwise keeps its matrix-core results in accumulation registers and copies
# each out before use (40 copies per 16-token step of a wave that is bound by
# instruction issue); this backend option makes the products write ordinary
# vector registers.
EXTRA = {
    "chunk_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the KDA library needs ROCm to build")
    return h


def _compile(args):
    cmd, src = args
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    return src


def build(jobs: int | None = None, verbose: bool = True) -> str:
    hipcc = _hipcc()
    jobs = jobs or min(16, os.cpu_count() or 4)
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        objs, work = [], []
        for s in srcs:
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            objs.append(o)
            extra = EXTRA.get(os.path.basename(s), [])
            work.append(([hipcc, *HIPFLAGS, *extra, "-c", s, "-o", o], s))
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            for s in ex.map(_compile, work):
                if verbose:
                    print(f"  compiled {os.path.basename(s)}", flush=True)
        tmp_lib = os.path.join(tmp, "libkda.so")
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        shutil.move(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(int(sys.argv[1]) if len(sys.argv) > 1 else None)
