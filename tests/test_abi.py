"""The C ABI on the CPU: the library loads, exports every entry point that
include/kda.h declares, and rejects bad arguments on the host before any GPU
call (no pointer is dereferenced, so fake aligned addresses are enough).

Cases whose arguments pass validation would, on a machine with a GPU, launch
kernels on those fake addresses.  They run only where no GPU is visible (the
GPU-less build container): every such call goes through `may_launch`, which
skips the test when a GPU is visible, and the tests holding them carry the
same skip.  Real-buffer versions of those cases are in test_gpu_abi.py.
"""
import ctypes
import os
import re

import pytest


def gpu_visible():
    """True when a GPU could run a kernel launched from this process.

    KDA_TEST_ASSUME_GPU=1 forces True (to check, on a GPU-less machine, that
    every launching case is skipped)."""
    if os.environ.get("KDA_TEST_ASSUME_GPU") == "1":
        return True
    try:
        import torch
        if torch.cuda.device_count() > 0:   # counts devices without initialising them
            return True
    except Exception:
        pass
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_int(0)
        if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
            return True
    except OSError:
        pass
    return False


HOST_ONLY_REASON = ("fake device addresses pass validation here: with a GPU visible the call "
                    "would launch kernels on them (real-buffer cases: test_gpu_abi.py)")
host_only = pytest.mark.skipif(gpu_visible(), reason=HOST_ONLY_REASON)


def may_launch(call, **kw):
    """A call whose arguments are valid: it reaches the device check and, on a
    GPU, a launch.  Never made where a GPU is visible."""
    if gpu_visible():
        pytest.skip(HOST_ONLY_REASON)
    return call(**kw)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _lib():
    from gated_delta_rule_108_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_eighteen_calls():
    assert declared_functions() == ["kda_decode_step", "kda_decode_step_backward",
                                    "kda_decode_step_logits",
                                    "kda_gdn_decode_step", "kda_gdn_decode_step_backward",
                                    "kda_gdn_prefill_backward",
                                    "kda_gdn_prefill_chunked",
                                    "kda_prefill_backward", "kda_prefill_backward_chunked",
                                    "kda_prefill_backward_chunked_workspace_bytes",
                                    "kda_prefill_backward_workspace_bytes",
                                    "kda_prefill_chunked", "kda_prefill_chunked_logits",
                                    "kda_prefill_chunked_noalloc",
                                    "kda_prefill_workspace_bytes", "kda_prologue_backward",
                                    "kda_prologue_forward", "kda_status_string"]


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(L.SIGNATURES) == set(declared_functions())


def test_status_strings():
    L = _lib()
    for code in range(-9, 1):
        s = L.status_string(code)
        assert s and s != "unknown status"
    assert L.status_string(5) == "unknown status"


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
BASE = 1 << 40
SPAN = 1 << 36


def addr(i):
    return BASE + i * SPAN


def prefill(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), S0=addr(5),
             o=addr(6), S_T=addr(7), B=1, T=64, H=2, dk=128, dv=128, C=64, dt=1,
             ws=addr(8), wsb=1 << 34, stream=None)
    a.update(kw)
    return lib.kda_prefill_chunked(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"],
                                   a["o"], a["S_T"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                   a["C"], a["dt"], a["ws"], a["wsb"], a["stream"])


def decode(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), S=addr(5),
             o=addr(6), S_out=addr(5), N=4, H=2, dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"], a["o"],
                               a["S_out"], a["N"], a["H"], a["dk"], a["dv"], a["dt"], a["stream"])


def test_prefill_validation_errors():
    L = _lib()
    lib = L.load()
    assert prefill(lib, q=None) == L.KDA_ERR_NULL
    assert prefill(lib, o=None) == L.KDA_ERR_NULL
    assert prefill(lib, B=0) == L.KDA_ERR_SHAPE
    assert prefill(lib, H=0) == L.KDA_ERR_SHAPE
    assert prefill(lib, T=-1) == L.KDA_ERR_SHAPE
    assert prefill(lib, dk=48) == L.KDA_ERR_UNSUPPORTED
    assert prefill(lib, dv=256) == L.KDA_ERR_UNSUPPORTED
    assert prefill(lib, C=8) == L.KDA_ERR_UNSUPPORTED
    assert prefill(lib, dt=7) == L.KDA_ERR_UNSUPPORTED
    assert prefill(lib, dt=0) == L.KDA_ERR_UNSUPPORTED          # fp32, dk=128, C=64: no fit
    assert prefill(lib, alpha=addr(3) + 4) == L.KDA_ERR_ALIGN
    assert prefill(lib, o=addr(0)) == L.KDA_ERR_ALIAS            # o on top of q
    assert prefill(lib, S_T=addr(5) + 256) == L.KDA_ERR_ALIAS    # partial overlap with S0
    assert prefill(lib, S_T=addr(1)) == L.KDA_ERR_ALIAS          # S_T on top of k


@host_only
def test_prefill_valid_arguments_reach_the_device_check():
    L = _lib()
    lib = L.load()
    # In-place state (S_T == S0) and T = 0 with NULL token arrays are valid; on
    # a machine without a GPU the call then fails at the device query.
    for kw in (dict(), dict(S_T=addr(5)), dict(S0=None),
               dict(T=0, q=None, k=None, v=None, alpha=None, beta=None, o=None)):
        st = may_launch(prefill, lib=lib, **kw)
        assert st in (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE), (kw, st)


def prefill_noalloc(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), S0=addr(5),
             o=addr(6), S_T=addr(7), B=1, T=64, H=2, dk=128, dv=128, C=64, dt=1, stream=None)
    a.update(kw)
    return lib.kda_prefill_chunked_noalloc(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                           a["S0"], a["o"], a["S_T"], a["B"], a["T"], a["H"],
                                           a["dk"], a["dv"], a["C"], a["dt"], a["stream"])


def test_prefill_noalloc_validation_errors():
    """The same host checks as kda_prefill_chunked, before any device call
    (the scratch address is looked up only after them)."""
    L = _lib()
    lib = L.load()
    pn = lambda **kw: prefill_noalloc(lib, **kw)
    assert pn(q=None) == L.KDA_ERR_NULL and pn(o=None) == L.KDA_ERR_NULL
    assert pn(B=0) == L.KDA_ERR_SHAPE and pn(T=-1) == L.KDA_ERR_SHAPE
    assert pn(dk=48) == L.KDA_ERR_UNSUPPORTED and pn(C=8) == L.KDA_ERR_UNSUPPORTED
    assert pn(dt=0) == L.KDA_ERR_UNSUPPORTED                     # fp32, dk=128, C=64: no fit
    assert pn(alpha=addr(3) + 4) == L.KDA_ERR_ALIGN
    assert pn(o=addr(0)) == L.KDA_ERR_ALIAS and pn(S_T=addr(5) + 256) == L.KDA_ERR_ALIAS


@host_only
def test_prefill_noalloc_valid_arguments_reach_the_device_check():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    for kw in (dict(), dict(S_T=addr(5)), dict(S0=None), dict(B=8, H=32, T=8192),
               dict(T=1 << 20, H=32), dict(T=0, q=None, k=None, v=None, alpha=None,
                                           beta=None, o=None)):
        assert may_launch(prefill_noalloc, lib=lib, **kw) in ok, kw


def test_decode_validation_errors():
    L = _lib()
    lib = L.load()
    assert decode(lib, S=None) == L.KDA_ERR_NULL
    assert decode(lib, N=0) == L.KDA_ERR_SHAPE
    assert decode(lib, dk=8) == L.KDA_ERR_UNSUPPORTED
    assert decode(lib, beta=addr(4) + 8) == L.KDA_ERR_ALIGN
    assert decode(lib, o=addr(2)) == L.KDA_ERR_ALIAS
    assert decode(lib, S_out=addr(5) + 64) == L.KDA_ERR_ALIAS
    assert decode(lib, S_out=addr(3)) == L.KDA_ERR_ALIAS


@host_only
def test_decode_valid_arguments_reach_the_device_check():
    L = _lib()
    lib = L.load()
    assert may_launch(decode, lib=lib, S_out=addr(7)) in (L.KDA_OK, L.KDA_ERR_HIP,
                                                          L.KDA_ERR_DEVICE)


def test_prefill_workspace_errors():
    L = _lib()
    lib = L.load()
    # few chains take the split path, which needs the workspace
    assert prefill(lib, ws=None) == L.KDA_ERR_WORKSPACE
    need = lib.kda_prefill_workspace_bytes(1, 64, 2, 128, 128, 64, 1)
    assert need > 0
    assert prefill(lib, wsb=need - 1) == L.KDA_ERR_WORKSPACE
    assert prefill(lib, ws=addr(8) + 8) == L.KDA_ERR_ALIGN
    assert prefill(lib, ws=addr(2)) == L.KDA_ERR_ALIAS              # workspace on top of v


@host_only
def test_prefill_exact_workspace_reaches_the_device_check():
    L = _lib()
    lib = L.load()
    need = lib.kda_prefill_workspace_bytes(1, 64, 2, 128, 128, 64, 1)
    assert may_launch(prefill, lib=lib, wsb=need) in (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)


def test_workspace_query():
    L = _lib()
    lib = L.load()
    bad = (1 << 64) - 1
    # one record per chunk: W, Q.E, (K.E')^T [C x dk each], P [C x C] in the
    # operand type, decay [dk] fp32, U~ [C x dv] in the operand type
    def rec(C, dk, dv, eb):
        return ((3 * C * dk + C * C + C * dv) * eb + 4 * dk + 255) // 256 * 256

    def split(B, T, H, dk, dv, C, eb):
        # records of one segment of chunks (segments keep them within 192 MiB),
        # plus the carried fp32 state when there are several segments
        r, nc = rec(C, dk, dv, eb), -(-T // C)
        if nc == 0:
            return 0
        segmax = max(1, (192 << 20) // (B * H * r))
        runs = 256 // (B * H) if B * H < 256 else 1
        if segmax > runs:
            segmax -= segmax % runs
        nseg = -(-nc // segmax)
        segch = -(-nc // nseg)
        if nseg > 1:
            segch = min(segmax, -(-segch // runs) * runs)
        return B * H * segch * r + (B * H * dk * dv * 4 if nseg > 1 else 0)
    assert lib.kda_prefill_workspace_bytes(1, 4096, 16, 128, 128, 64, 1) == 16 * 64 * rec(64, 128, 128, 2)
    assert lib.kda_prefill_workspace_bytes(1, 4096, 16, 128, 64, 64, 1) == 16 * 64 * rec(64, 128, 64, 2)
    assert lib.kda_prefill_workspace_bytes(8, 8192, 32, 128, 128, 64, 1) == 0   # fused path
    # one segment up to 192 MiB of records, in a multiple of the prep's 16
    # runs per chain: 16 heads x 160 chunks of 74240 bytes
    assert rec(64, 128, 128, 2) == 74240
    assert lib.kda_prefill_workspace_bytes(1, 160 * 64, 16, 128, 128, 64, 1) == 16 * 160 * 74240
    # one chunk more: two segments of 96 and 65 chunks, plus the carried state
    assert (lib.kda_prefill_workspace_bytes(1, 160 * 64 + 1, 16, 128, 128, 64, 1)
            == 16 * 96 * 74240 + 16 * 128 * 128 * 4)
    for args in ((1, 20000, 16, 128, 128, 64, 2), (1, 1 << 20, 32, 128, 128, 64, 2),
                 (4, 100000, 8, 64, 32, 32, 2), (1, 5000, 3, 16, 16, 16, 4)):
        B, T, H, dk, dv, C, eb = args
        dt = 1 if eb == 2 else 0
        assert lib.kda_prefill_workspace_bytes(B, T, H, dk, dv, C, dt) == split(*args), args
    # the workspace no longer grows with T
    assert lib.kda_prefill_workspace_bytes(1, 1 << 20, 32, 128, 128, 64, 1) < 200 << 20
    # C = 128 runs as 64-token chunks: same workspace as C = 64
    for args in ((1, 4096, 16, 128, 128), (1, 100, 3, 64, 32), (8, 8192, 32, 128, 128)):
        assert (lib.kda_prefill_workspace_bytes(*args, 128, 1)
                == lib.kda_prefill_workspace_bytes(*args, 64, 1))
    assert lib.kda_prefill_workspace_bytes(1, 256, 1, 16, 16, 16, 0) == 16 * rec(16, 16, 16, 4)
    assert lib.kda_prefill_workspace_bytes(1, 256, 1, 16, 16, 12, 0) == bad
    assert lib.kda_prefill_workspace_bytes(0, 256, 1, 16, 16, 16, 0) == bad


def prefill_logits(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), b=addr(4), S0=addr(5),
             o=addr(6), S_T=addr(7), B=1, T=64, H=2, dk=128, dv=128, C=64, dt=1, qk=1,
             ws=addr(8), wsb=1 << 34, stream=None)
    a.update(kw)
    return lib.kda_prefill_chunked_logits(a["q"], a["k"], a["v"], a["g"], a["b"], a["S0"],
                                          a["o"], a["S_T"], a["B"], a["T"], a["H"], a["dk"],
                                          a["dv"], a["C"], a["dt"], a["qk"], a["ws"], a["wsb"],
                                          a["stream"])


def decode_logits(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), b=addr(4), S=addr(5),
             o=addr(6), S_out=addr(5), N=4, H=2, dk=128, dv=128, dt=1, qk=2, stream=None)
    a.update(kw)
    return lib.kda_decode_step_logits(a["q"], a["k"], a["v"], a["g"], a["b"], a["S"], a["o"],
                                      a["S_out"], a["N"], a["H"], a["dk"], a["dv"], a["dt"],
                                      a["qk"], a["stream"])


def test_logits_entry_points_validate_like_the_plain_ones():
    L = _lib()
    lib = L.load()
    for qk in (3, -1):
        assert prefill_logits(lib, qk=qk) == L.KDA_ERR_UNSUPPORTED
        assert decode_logits(lib, qk=qk) == L.KDA_ERR_UNSUPPORTED
    assert prefill_logits(lib, g=None) == L.KDA_ERR_NULL
    assert prefill_logits(lib, b=addr(4) + 4) == L.KDA_ERR_ALIGN
    assert prefill_logits(lib, ws=None) == L.KDA_ERR_WORKSPACE
    assert decode_logits(lib, g=None) == L.KDA_ERR_NULL
    assert decode_logits(lib, N=0) == L.KDA_ERR_SHAPE
    # the gate logits have the I/O type's width: with bf16 the gate array of
    # B*T*H*dk elements spans 2 bytes each, so an output just past it is fine
    # and one inside it overlaps
    ntok = 1 * 64 * 2
    g_end = addr(3) + ntok * 128 * 2
    assert prefill_logits(lib, o=g_end - 16) == L.KDA_ERR_ALIAS
    assert prefill_logits(lib, o=g_end, dt=0, C=32) == L.KDA_ERR_ALIAS   # fp32: 4 bytes each


@host_only
def test_logits_entry_points_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    g_end = addr(3) + 1 * 64 * 2 * 128 * 2   # just past the bf16 gate logits
    assert may_launch(prefill_logits, lib=lib, o=g_end) in ok
    for qk in (0, 1, 2):
        assert may_launch(prefill_logits, lib=lib, qk=qk) in ok
        assert may_launch(decode_logits, lib=lib, qk=qk) in ok


def gdn_prefill(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), a=addr(3), beta=addr(4), S0=addr(5),
             o=addr(6), S_T=addr(7), B=1, T=64, H=2, dk=128, dv=128, C=64, dt=1,
             ws=addr(8), wsb=1 << 34, stream=None)
    a.update(kw)
    return lib.kda_gdn_prefill_chunked(a["q"], a["k"], a["v"], a["a"], a["beta"], a["S0"],
                                       a["o"], a["S_T"], a["B"], a["T"], a["H"], a["dk"],
                                       a["dv"], a["C"], a["dt"], a["ws"], a["wsb"], a["stream"])


def gdn_decode(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), a=addr(3), beta=addr(4), S=addr(5),
             o=addr(6), S_out=addr(5), N=4, H=2, dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    return lib.kda_gdn_decode_step(a["q"], a["k"], a["v"], a["a"], a["beta"], a["S"],
                                   a["o"], a["S_out"], a["N"], a["H"], a["dk"], a["dv"],
                                   a["dt"], a["stream"])


def test_gdn_entry_points_validate():
    L = _lib()
    lib = L.load()
    gp = lambda **kw: gdn_prefill(lib, **kw)
    gd = lambda **kw: gdn_decode(lib, **kw)
    assert gp(beta=None) == L.KDA_ERR_NULL and gd(beta=None) == L.KDA_ERR_NULL
    assert gp(a=addr(3) + 4) == L.KDA_ERR_ALIGN and gd(a=addr(3) + 8) == L.KDA_ERR_ALIGN
    assert gp(ws=None) == L.KDA_ERR_WORKSPACE
    # the gate array is B*T*H fp32 values: an output inside it overlaps
    g_end = addr(3) + 1 * 64 * 2 * 4
    assert gp(o=g_end - 16) == L.KDA_ERR_ALIAS
    assert gd(o=addr(3)) == L.KDA_ERR_ALIAS


@host_only
def test_gdn_entry_points_take_a_null_gate():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    assert may_launch(gdn_prefill, lib=lib, a=None) in ok     # DeltaNet: no gate
    assert may_launch(gdn_decode, lib=lib, a=None) in ok
    assert may_launch(gdn_prefill, lib=lib) in ok and may_launch(gdn_decode, lib=lib) in ok
    # an output just past the B*T*H fp32 gates is fine
    assert may_launch(gdn_prefill, lib=lib, o=addr(3) + 1 * 64 * 2 * 4) in ok
    assert may_launch(gdn_decode, lib=lib, o=addr(3) + 4 * 2 * 4) in ok


def step_backward(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), S=addr(5),
             dO=addr(6), dSn=addr(7), dq=addr(8), dk=addr(9), dv=addr(10), da=addr(11),
             db=addr(12), dS=addr(13), N=4, H=2, dk_=128, dv_=128, dt=1, stream=None)
    a.update(kw)
    return lib.kda_decode_step_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                        a["S"], a["dO"], a["dSn"], a["dq"], a["dk"],
                                        a["dv"], a["da"], a["db"], a["dS"], a["N"], a["H"],
                                        a["dk_"], a["dv_"], a["dt"], a["stream"])


def test_step_backward_validation():
    L = _lib()
    lib = L.load()
    bw = lambda **kw: step_backward(lib, **kw)
    assert bw(dS=addr(5)) == L.KDA_ERR_ALIAS                     # over the state
    assert bw(dS=addr(7) + 64) == L.KDA_ERR_ALIAS                # partial overlap with dS_new
    assert bw(dq=addr(9)) == L.KDA_ERR_ALIAS                     # two outputs together
    assert bw(dv=addr(6)) == L.KDA_ERR_ALIAS                     # output over dO
    assert bw(db=None) == L.KDA_ERR_NULL
    assert bw(da=addr(11) + 4) == L.KDA_ERR_ALIGN
    assert bw(N=0) == L.KDA_ERR_SHAPE
    assert bw(dk_=24) == L.KDA_ERR_UNSUPPORTED


@host_only
def test_step_backward_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    assert may_launch(step_backward, lib=lib) in ok
    assert may_launch(step_backward, lib=lib, dS=addr(7)) in ok   # in place over dS_new


def test_prefill_backward_workspace_bytes():
    L = _lib()
    lib = L.load()
    # states every 16 tokens, then the write and read of every token and column
    assert lib.kda_prefill_backward_workspace_bytes(1, 4096, 16, 128, 128) == 320 << 20
    assert lib.kda_prefill_backward_workspace_bytes(2, 17, 3, 64, 32) == \
        2 * 3 * 2 * 64 * 32 * 4 + 2 * 2 * 17 * 3 * 32 * 4
    assert lib.kda_prefill_backward_workspace_bytes(1, 0, 1, 16, 16) == 0
    bad = ctypes.c_size_t(-1).value
    assert lib.kda_prefill_backward_workspace_bytes(1, 16, 1, 24, 16) == bad
    assert lib.kda_prefill_backward_workspace_bytes(0, 16, 1, 16, 16) == bad


PB_B, PB_T, PB_H, PB_D = 1, 64, 2, 128


def prefill_backward(lib, fn="kda_prefill_backward", **kw):
    ws_need = lib.kda_prefill_backward_workspace_bytes(PB_B, PB_T, PB_H, PB_D, PB_D)
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), S0=addr(5),
             dO=addr(6), dST=addr(7), dq=addr(8), dk=addr(9), dv=addr(10), da=addr(11),
             db=addr(12), dS0=addr(13), B=PB_B, T=PB_T, H=PB_H, dk_=PB_D, dv_=PB_D, dt=1,
             ws=addr(14), wsb=ws_need, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"],
                            a["dO"], a["dST"], a["dq"], a["dk"], a["dv"], a["da"],
                            a["db"], a["dS0"], a["B"], a["T"], a["H"], a["dk_"],
                            a["dv_"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_prefill_backward_validation():
    L = _lib()
    lib = L.load()
    pb = lambda **kw: prefill_backward(lib, **kw)
    ws_need = lib.kda_prefill_backward_workspace_bytes(PB_B, PB_T, PB_H, PB_D, PB_D)
    assert pb(dS0=addr(7) + 64) == L.KDA_ERR_ALIAS               # partial overlap with dS_T
    assert pb(dS0=addr(5)) == L.KDA_ERR_ALIAS                    # over S0
    assert pb(dq=addr(9)) == L.KDA_ERR_ALIAS                     # two outputs together
    assert pb(ws=addr(6)) == L.KDA_ERR_ALIAS                     # workspace over dO
    # dq is B*T*H*dk fp32: an output inside it overlaps
    dq_end = addr(8) + PB_B * PB_T * PB_H * PB_D * 4
    assert pb(dk=dq_end - 16) == L.KDA_ERR_ALIAS
    assert pb(dO=None) == L.KDA_ERR_NULL and pb(db=None) == L.KDA_ERR_NULL
    assert pb(da=addr(11) + 4) == L.KDA_ERR_ALIGN
    assert pb(ws=None) == L.KDA_ERR_WORKSPACE and pb(wsb=ws_need - 1) == L.KDA_ERR_WORKSPACE
    assert pb(T=-1) == L.KDA_ERR_SHAPE and pb(H=0) == L.KDA_ERR_SHAPE
    assert pb(dk_=24) == L.KDA_ERR_UNSUPPORTED and pb(dt=7) == L.KDA_ERR_UNSUPPORTED


@host_only
def test_prefill_backward_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    pb = lambda **kw: may_launch(prefill_backward, lib=lib, **kw)
    assert pb() in ok
    assert pb(S0=None, dST=None, dS0=None) in ok                 # optional states
    assert pb(dS0=addr(7)) in ok                                 # in place over dS_T
    dq_end = addr(8) + PB_B * PB_T * PB_H * PB_D * 4
    assert pb(dk=dq_end) in ok                                   # just past dq
    # no tokens: only the state gradient is passed through, the rest may be NULL
    assert pb(T=0, q=None, k=None, v=None, alpha=None, beta=None, dO=None, dq=None, dk=None,
              dv=None, da=None, db=None, ws=None, wsb=0) in ok



def test_prefill_backward_chunked_workspace_bytes():
    """The forward's split-path records (C = 64, split path), the state
    and the state gradient every 64 tokens (fp32), one
    15 KiB record per 16 tokens, and per 64 tokens the four 16-token states
    and their writes (bf16)."""
    L = _lib()
    lib = L.load()

    def expect(B, T, H):
        chains, nc, ns = B * H, -(-T // 64), -(-T // 16)
        fwd_rec = ((3 * 64 * 128 + 64 * 64 + 64 * 128) * 2 + 4 * 128 + 255) // 256 * 256
        segmax = max(1, (192 << 20) // (chains * fwd_rec))
        runs = 256 // chains if chains < 256 else 1
        if segmax > runs:
            segmax -= segmax % runs
        nseg = -(-nc // segmax)
        segch = -(-nc // nseg)
        if nseg > 1:
            segch = min(segmax, -(-segch // runs) * runs)
        fwd = chains * segch * fwd_rec + (chains * 128 * 128 * 4 if nseg > 1 else 0)
        return (fwd + 2 * chains * nc * 128 * 128 * 4 + chains * ns * 15360
                + chains * nc * 4 * 128 * 128 * 2 + chains * nc * 4 * 16 * 128 * 2)

    for B, T, H in ((1, 4096, 16), (2, 100, 3), (8, 8192, 32), (1, 1, 1)):
        assert lib.kda_prefill_backward_chunked_workspace_bytes(B, T, H, 128, 128) == expect(B, T, H)
    assert lib.kda_prefill_backward_chunked_workspace_bytes(1, 4096, 16, 128, 128) >> 20 == 404
    bad = ctypes.c_size_t(-1).value
    assert lib.kda_prefill_backward_chunked_workspace_bytes(1, 64, 2, 64, 128) == bad   # dk
    assert lib.kda_prefill_backward_chunked_workspace_bytes(1, 64, 2, 128, 64) == bad   # dv
    assert lib.kda_prefill_backward_chunked_workspace_bytes(0, 64, 2, 128, 128) == bad


def prefill_backward_chunked(lib, **kw):
    kw.setdefault("wsb", lib.kda_prefill_backward_chunked_workspace_bytes(
        kw.get("B", PB_B), kw.get("T", PB_T), kw.get("H", PB_H), PB_D, PB_D))
    return prefill_backward(lib, fn="kda_prefill_backward_chunked", **kw)


def test_prefill_backward_chunked_validation():
    """The host checks of the token-walk backward, plus its own sizes: bf16 at
    dk = dv = 128 only."""
    L = _lib()
    lib = L.load()
    pb = lambda **kw: prefill_backward_chunked(lib, **kw)
    ws_need = lib.kda_prefill_backward_chunked_workspace_bytes(PB_B, PB_T, PB_H, PB_D, PB_D)
    assert pb(dS0=addr(7) + 64) == L.KDA_ERR_ALIAS               # partial overlap with dS_T
    assert pb(dq=addr(9)) == L.KDA_ERR_ALIAS                     # two outputs together
    assert pb(ws=addr(6)) == L.KDA_ERR_ALIAS                     # workspace over dO
    assert pb(dO=None) == L.KDA_ERR_NULL and pb(db=None) == L.KDA_ERR_NULL
    assert pb(da=addr(11) + 4) == L.KDA_ERR_ALIGN
    assert pb(ws=None) == L.KDA_ERR_WORKSPACE and pb(wsb=ws_need - 1) == L.KDA_ERR_WORKSPACE
    assert pb(T=-1) == L.KDA_ERR_SHAPE and pb(H=0) == L.KDA_ERR_SHAPE
    assert pb(dt=0) == L.KDA_ERR_UNSUPPORTED                     # fp32 I/O: the token walk's
    assert pb(dk_=64, dv_=64) == L.KDA_ERR_UNSUPPORTED
    assert pb(dt=7) == L.KDA_ERR_UNSUPPORTED


@host_only
def test_prefill_backward_chunked_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    pb = lambda **kw: may_launch(prefill_backward_chunked, lib=lib, **kw)
    assert pb() in ok
    assert pb(S0=None, dST=None, dS0=None) in ok                 # optional states
    assert pb(dS0=addr(7)) in ok                                 # in place over dS_T
    assert pb(T=0, q=None, k=None, v=None, alpha=None, beta=None, dO=None, dq=None, dk=None,
              dv=None, da=None, db=None, ws=None, wsb=0) in ok

PRO_ROWS, PRO_D = 64, 128


def prologue_fwd(lib, **kw):
    a = dict(q=addr(0), k=addr(1), g=addr(2), b=addr(3), qh=addr(4), kh=addr(5), al=addr(6),
             be=addr(7), rows=PRO_ROWS, dk=PRO_D, dt=1, m=1, stream=None)
    a.update(kw)
    return lib.kda_prologue_forward(a["q"], a["k"], a["g"], a["b"], a["qh"], a["kh"],
                                    a["al"], a["be"], a["rows"], a["dk"], a["dt"], a["m"],
                                    a["stream"])


def prologue_bwd(lib, **kw):
    a = dict(q=addr(0), k=addr(1), g=addr(2), b=addr(3), dqh=addr(4), dkh=addr(5),
             da=addr(6), dbe=addr(7), dq=addr(8), dk=addr(9), dg=addr(10), db=addr(11),
             rows=PRO_ROWS, dk_=PRO_D, dt=1, m=2, stream=None)
    a.update(kw)
    return lib.kda_prologue_backward(a["q"], a["k"], a["g"], a["b"], a["dqh"], a["dkh"],
                                     a["da"], a["dbe"], a["dq"], a["dk"], a["dg"], a["db"],
                                     a["rows"], a["dk_"], a["dt"], a["m"], a["stream"])


def test_prologue_validation():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    pf = lambda **kw: prologue_fwd(lib, **kw)
    pb = lambda **kw: prologue_bwd(lib, **kw)
    for f in (pf, pb):
        # rows = 0 returns before the device check and launches nothing
        assert f(rows=0, q=None, k=None) == L.KDA_OK              # nothing to do
        assert f(rows=-1) == L.KDA_ERR_SHAPE
        assert f(m=3) == L.KDA_ERR_UNSUPPORTED and f(dt=5) == L.KDA_ERR_UNSUPPORTED
        assert f(q=None) == L.KDA_ERR_NULL and f(b=addr(3) + 4) == L.KDA_ERR_ALIGN
    assert pf(dk=24) == L.KDA_ERR_UNSUPPORTED and pb(dk_=24) == L.KDA_ERR_UNSUPPORTED
    # q_hat over the raw keys, alpha over beta, dg over dalpha: rejected
    assert pf(qh=addr(1)) == L.KDA_ERR_ALIAS and pf(al=addr(7)) == L.KDA_ERR_ALIAS
    assert pb(dg=addr(6)) == L.KDA_ERR_ALIAS and pb(db=addr(8)) == L.KDA_ERR_ALIAS
    # an output inside an input's last bytes overlaps (bf16 q is rows*dk*2 bytes)
    assert pf(qh=addr(0) + PRO_ROWS * PRO_D * 2 - 16) == L.KDA_ERR_ALIAS


@host_only
def test_prologue_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    assert may_launch(prologue_fwd, lib=lib) in ok
    assert may_launch(prologue_bwd, lib=lib) in ok
    # an output right after an input's last byte is fine
    assert may_launch(prologue_fwd, lib=lib, qh=addr(0) + PRO_ROWS * PRO_D * 2) in ok


def test_gdn_prefill_backward_validation():
    L = _lib()
    lib = L.load()
    gb = lambda **kw: prefill_backward(lib, fn="kda_gdn_prefill_backward", **kw)
    # the gate and its gradient are B*T*H floats: an output inside them overlaps
    a_end = addr(3) + PB_B * PB_T * PB_H * 4
    assert gb(dq=a_end - 16) == L.KDA_ERR_ALIAS
    assert gb(da=addr(12)) == L.KDA_ERR_ALIAS and gb(beta=None) == L.KDA_ERR_NULL
    assert gb(ws=None) == L.KDA_ERR_WORKSPACE and gb(dk_=24) == L.KDA_ERR_UNSUPPORTED


@host_only
def test_gdn_prefill_backward_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    gb = lambda **kw: may_launch(prefill_backward, lib=lib, fn="kda_gdn_prefill_backward", **kw)
    assert gb() in ok
    assert gb(alpha=None, da=None) in ok                  # DeltaNet: no gate
    assert gb(alpha=None) in ok                           # da ignored without a gate
    assert gb(dq=addr(3) + PB_B * PB_T * PB_H * 4) in ok  # just past the gates


def test_gdn_step_backward_validation():
    L = _lib()
    lib = L.load()
    gs = lambda **kw: gdn_step_backward(lib, **kw)
    a_end = addr(3) + 4 * 2 * 4                            # one gate per head
    assert gs(dq=a_end - 16) == L.KDA_ERR_ALIAS
    assert gs(beta=None) == L.KDA_ERR_NULL and gs(da=addr(11) + 4) == L.KDA_ERR_ALIGN


def gdn_step_backward(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), a=addr(3), beta=addr(4), S=addr(5),
             dO=addr(6), dSn=addr(7), dq=addr(8), dk=addr(9), dv=addr(10), da=addr(11),
             db=addr(12), dS=addr(13), N=4, H=2, dk_=128, dv_=128, dt=1, stream=None)
    a.update(kw)
    return lib.kda_gdn_decode_step_backward(a["q"], a["k"], a["v"], a["a"], a["beta"],
                                            a["S"], a["dO"], a["dSn"], a["dq"], a["dk"],
                                            a["dv"], a["da"], a["db"], a["dS"], a["N"],
                                            a["H"], a["dk_"], a["dv_"], a["dt"], a["stream"])


@host_only
def test_gdn_step_backward_valid_arguments():
    L = _lib()
    lib = L.load()
    ok = (L.KDA_OK, L.KDA_ERR_HIP, L.KDA_ERR_DEVICE)
    gs = lambda **kw: may_launch(gdn_step_backward, lib=lib, **kw)
    assert gs() in ok and gs(a=None, da=None) in ok and gs(dS=addr(7)) in ok
    assert gs(dq=addr(3) + 4 * 2 * 4) in ok


def test_every_launching_case_is_host_only():
    """Every test here that calls with arguments passing validation is marked
    host_only and goes through may_launch (checked on the source)."""
    import inspect
    import sys
    mod = sys.modules[__name__]
    for name, fn in inspect.getmembers(mod, inspect.isfunction):
        if not name.startswith("test_") or name == "test_every_launching_case_is_host_only":
            continue
        body = inspect.getsource(fn)
        launches = "may_launch(" in body
        marked = any(m.name == "skipif" for m in getattr(fn, "pytestmark", []))
        if launches:
            assert marked, f"{name} may launch kernels but is not host_only"
        if marked:
            assert launches, f"{name} is host_only but makes no may_launch call"
