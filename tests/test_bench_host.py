"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte
counts the roofline divides by, and the source hash that keys a stored
counter profile."""
import os
import subprocess
import sys

import bench
from gated_delta_rule_decay_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
W = synth.WORKLOADS


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_chunk_bytes_of_the_full_workload():
    # per token-head: q, k, v bf16 (3 x 128 x 2), three per-channel fp32 gates
    # (3 x 128 x 4), o fp32 (128 x 4) = 2816 B; plus S0 read and S_T written
    w = W[2]
    tokens = w.B * w.T * w.H
    state = w.B * w.H * w.dk * w.dv * 4
    assert bench.chunk_bytes(w) == tokens * 2816 + 2 * state == 1_493_172_224


def test_chunk_bytes_of_scalar_gates_and_zero_state():
    # Gated DeltaNet mode: one fp32 decay and one (tied) gate per token-head,
    # no initial state to read
    w = W[1]
    tokens = w.B * w.T * w.H
    per_tok = 3 * 128 * 2 + 2 * 4 + 128 * 4
    assert bench.chunk_bytes(w) == tokens * per_tok + w.B * w.H * w.dk * w.dv * 4


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "gated_delta_rule_decay_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    f.write_text("int f(int x) {\n    return x + 1;\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash(["k.hip"])
    f.write_text("// a comment\nint f(int x) {  /* inline */\n\n    return x + 1;  // trailing\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    f.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.source_hash(["k.hip"]) != h0


def test_stored_traffic_is_used_only_for_its_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "traffic_k_w.txt").write_text("# header\nsource_hash: abc\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k", "w", "abc") == 1234.0
    assert bench.read_traffic("k", "w", "abd") is None
    assert bench.read_traffic("k", "other", "abc") is None
