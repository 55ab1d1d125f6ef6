"""bench.py's host logic on the CPU: the algorithmic byte and flop counts per
unit that the roofline figures divide by, the kernel-source hash that decides
whether a profile's traffic still applies, the profile reader, and the
refusal of more than one GPU.  Each per-unit figure is written out here from
the list of arrays the call reads and writes once (d = 128, bf16 I/O)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

D = 128


def test_prefill_bytes_per_token_head():
    # q, k, v, o bf16 (2 B x 4 x 128) + fp32 alpha (4 x 128) + fp32 beta
    assert bench.prefill_alg_bytes(1, 1, 1, D, D, 2, False) - D * D * 4 == 1540
    # the final state once, and the initial state too when given
    assert bench.prefill_alg_bytes(1, 10, 1, D, D, 2, True) == 10 * 1540 + 2 * D * D * 4


def test_prologue_and_gdn_bytes_per_token_head():
    # gate logits in bf16 (2 B per channel) instead of fp32 alpha
    assert bench.prefill_logit_alg_bytes(1, 1, 1, D, D, 2, False) - D * D * 4 == 1284
    # one fp32 gate per token and head
    assert bench.gdn_alg_bytes(1, 1, 1, D, D, 2, False) - D * D * 4 == 1032


def test_decode_bytes_per_head_step():
    # state read and written (fp32), q, k, v, o bf16, alpha fp32, beta
    assert bench.decode_alg_bytes(1, 1, D, D, 2) == 2 * D * D * 4 + 2 * 4 * D + 4 * D + 4
    assert bench.decode_alg_bytes(1, 1, D, D, 2) == 132612
    assert bench.decode_alg_bytes(1, 1, D, D, 2, gate_bytes=2) == 132356
    assert bench.decode_alg_bytes(256, 32, D, D, 2) == 256 * 32 * 132612


def test_backward_bytes():
    # step adjoint: S and dS_new read, dS written; q, k, v, alpha, beta, dO read,
    # dq, dk, dv (bf16), dalpha, dbeta (fp32) written
    reads = 2 * (2 * D + D) + 4 * D + 4 + 2 * D       # q, k, v, alpha, beta, dO: 1540
    writes = 2 * (2 * D + D) + 4 * D + 4               # dq, dk, dv, dalpha, dbeta: 1284
    assert bench.decode_bwd_alg_bytes(1, 1, D, D, 2) == 3 * D * D * 4 + reads + writes == 199432
    # prefill backward per token-head: q, k, v, alpha, beta, dO read; dq, dk, dv,
    # dalpha, dbeta written in fp32; per head dS_T read and dS0 written
    per_tok = 2 * (2 * D + D) + 4 * D + 4 + 2 * D + 4 * (3 * D + D) + 4
    assert per_tok == 3592
    assert bench.prefill_bwd_alg_bytes(1, 4096, 16, D, D, 2) == \
        4096 * 16 * 3592 + 2 * 16 * D * D * 4


def test_prefill_flops_per_token_head():
    # 6 dk dv of state work + 2 C (3 dk + 2 dv) of chunk-local products, C = 64
    assert bench.prefill_flops(1, 1, 1, D, D, 64) == 180224


def test_source_hash_ignores_comments_but_not_code():
    a = "int f() { return 1; } // one\n/* block */ const char* s = \"// kept\";"
    b = "int f() {   return 1; }\n const char* s = \"// kept\";  // other"
    c = "int f() { return 2; }\n const char* s = \"// kept\";"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert "// kept" in bench._code_only(a)


def test_profiled_traffic_needs_the_current_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    (prof / "w.txt").write_text("# title\n  command: x\ntraffic_bytes_per_launch: 1234\n"
                                "source_sha256: abc\n")
    (prof / "old.txt").write_text("traffic_bytes_per_launch: 99\nsource_sha256: zzz\n")
    assert bench.profiled_traffic("w") == 1234
    assert bench.profiled_traffic("old") is None          # kernels changed since
    assert bench.profiled_traffic("missing") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prologue_bytes_per_row():
    # forward: q, k, g bf16 read + b; q_hat, k_hat bf16 + alpha fp32 + beta written
    fwd = 3 * 2 * D + 4 + 2 * 2 * D + 4 * D + 4
    # adjoint: q, k, g bf16 + b read, three fp32 row gradients + dbeta read,
    # three fp32 row gradients + db written
    bwd = 3 * 2 * D + 4 + 3 * 4 * D + 4 + 3 * 4 * D + 4
    assert bench.prologue_alg_bytes(1, D, 2) == (fwd, bwd) == (1800, 3852)
