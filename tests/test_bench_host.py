"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte
counts the roofline divides by, and the source hash that keys a stored
counter profile."""
import os
import subprocess
import sys

import pytest

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


# ---- bench.py --summarize: the profiler's dispatches attributed to lines ----

PREP = "void gdn2::(anonymous namespace)::chunk_prep_kernel<false, 1, false, false>(gdn2::ChunkArgs, " \
       "gdn2::(anonymous namespace)::SplitWs, int)"
SCAN = "void gdn2::(anonymous namespace)::chunk_scan_kernel<false, 1, false, 0>(gdn2::ChunkArgs, int)"
STEP = "void gdn2::(anonymous namespace)::step128_kernel(gdn2::StepArgs)"
COPY = "__amd_rocclr_copyBuffer"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int, float)"


def test_short_names():
    assert bench.short_name(PREP) == "chunk_prep_kernel<false, 1, false, false>"
    assert bench.short_name(STEP) == "step128_kernel"
    assert bench.short_name(COPY) == COPY


def _write_run(d, names, counters=None, durs=None):
    """A rocprofv3-style run directory: a kernel trace, or a counter
    collection with one row per (dispatch, counter)."""
    import csv
    d.mkdir(parents=True)
    if counters is None:
        with open(d / "run_kernel_trace.csv", "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(["Kind", "Agent_Id", "Queue_Id", "Kernel_Id", "Kernel_Name", "Correlation_Id",
                         "Start_Timestamp", "End_Timestamp", "Dispatch_Id"])
            t = 1000
            for i, (n, dur) in enumerate(zip(names, durs)):
                wr.writerow(["KERNEL_DISPATCH", 1, 1, 7, n, i, t, t + dur, i + 1])
                t += dur + 10
    else:
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            for i, n in enumerate(names):
                for cname, val in counters[i].items():
                    wr.writerow([i, i + 1, n, cname, val])


def test_attribution_and_summaries(tmp_path, monkeypatch):
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    plan = {"plan": [{"label": "fwd", "calls": 3, "timed": 2, "profile": "chunk_fwd_w"},
                     {"label": "dec", "calls": 4, "timed": 3, "profile": None}],
            "source_hash": {"chunk_fwd": "h1", "recurrent_step": "h2", "chunk_bwd": "h3"}}
    # three calibration copies first, foreign kernels in between
    names = [COPY] * 3 + [FILL, PREP, SCAN, PREP, FILL, SCAN, PREP, SCAN, STEP, STEP, FILL, STEP, STEP]
    durs = [5] * 3 + [1, 100, 50, 110, 1, 52, 120, 54, 9, 10, 1, 11, 12]
    _write_run(tmp_path / "prof" / "trace", names, durs=durs)
    fetch = [{"FETCH_SIZE": 131072.0}] * 3 + [{"FETCH_SIZE": 1.0}] + \
        [{"FETCH_SIZE": v} for v in (1000, 500, 1000, 1, 500, 1000, 500, 7, 7, 1, 7, 7)]
    write = [{"WRITE_SIZE": 262144.0}] * 3 + [{"WRITE_SIZE": 1.0}] + \
        [{"WRITE_SIZE": v} for v in (800, 300, 800, 1, 300, 800, 300, 5, 5, 1, 5, 5)]
    _write_run(tmp_path / "prof" / "fetch", names, counters=fetch)
    _write_run(tmp_path / "prof" / "write", names, counters=write)
    for sub in ("trace", "fetch", "write"):
        (tmp_path / "prof" / sub / "plan.json").write_text(json.dumps(plan))
        (tmp_path / "prof" / sub / "command.txt").write_text(f"rocprofv3 ({sub}) -- python3 bench.py")
    bench.summarize(str(tmp_path / "prof"))
    stats = (tmp_path / "profiles" / "kernel_stats_all_lines.txt").read_text().splitlines()
    rows = [r.split(" | ") for r in stats if not r.startswith("#") and " | " in r][1:]
    # fwd: the last two calls timed; dec: the last three
    assert rows[0][:4] == ["fwd", "chunk_prep_kernel<false, 1, false, false>", "2", "115"]
    assert rows[1][:4] == ["fwd", "chunk_scan_kernel<false, 1, false, 0>", "2", "53"]
    assert rows[2][:6] == ["dec", "step128_kernel", "3", "11", "10", "12"]
    traffic = (tmp_path / "profiles" / "traffic_chunk_fwd_w.txt").read_text()
    # calibration: fetch counts half the bytes (scale 2), write all (scale 1)
    assert "fetch_scale: 2.0000" in traffic and "write_scale: 1.0000" in traffic
    assert f"hbm_bytes_per_launch: {(1500 * 2 + 1100) * 1024}" in traffic
    assert "source_hash: h1" in traffic
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    assert bench.read_traffic("chunk_fwd", "w", "h1") == (1500 * 2 + 1100) * 1024


def test_attribution_rejects_a_plan_that_does_not_fit():
    disp = [{"name": n, "counters": {}, "dur_ns": 1} for n in (PREP, SCAN, PREP, SCAN, STEP, STEP)]
    with pytest.raises(ValueError):  # one call too many of the forward
        bench.attribute(disp, {"plan": [{"label": "fwd", "calls": 3, "timed": 1}]})
    with pytest.raises(ValueError):  # dispatches left over
        bench.attribute([dict(x) for x in disp], {"plan": [{"label": "fwd", "calls": 2, "timed": 1}]})
