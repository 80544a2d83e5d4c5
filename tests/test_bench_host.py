"""bench.py's host-side accounting without a GPU: the algorithmic bytes and
flops its roofline divides by (worked out here by hand at the chat-wave
shape), the counter scaling of its profile summary (on a synthetic rocprofv3
CSV set), the source key of the traffic record, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

import bench as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def chat_shape(chunk=64):
    """The chat wave's sizes: 32 prompts x 1,024 tokens, 16 qk heads, 32
    value heads, d = 128, bf16 io, no initial state."""
    return types.SimpleNamespace(dtype="bf16", Hqk=16, Hv=32, dk=128, dv=128, n_tokens=32 * 1024,
                                 n_seqs=32, chunk=chunk, init=None)


def test_algorithmic_bytes_at_chat_shape():
    p = chat_shape()
    # per token: q and k (16 heads x 128, bf16) + v (32 x 128, bf16) in,
    # g and beta (32 fp32 each) in, out (32 x 128, bf16)
    per_token = 16 * 128 * 2 * 2 + 32 * 128 * 2 + 32 * 4 * 2 + 32 * 128 * 2
    assert per_token == 24832
    state = 32 * 128 * 128 * 4          # one prompt's fp32 state: 2 MiB
    expect = 32768 * per_token + 32 * state + 96 * state
    assert expect == 1082130432
    assert B.prefill_alg_bytes(p, 96, False) == expect
    # an initial state is read as well as the final one written
    assert B.prefill_alg_bytes(p, 96, True) == expect + 32 * state


def test_algorithmic_flops_at_the_executed_chunk():
    p = chat_shape(chunk=64)
    assert B.kernel_chunk(p) == 32 and B.kernel_chunk(chat_shape(chunk=16)) == 16
    C, d = 32, 128
    # per token and value head: X, QS, U, P.U, update and the Gram / K Q^T
    # tiles at C = 32 (2C(3dk + 2dv)), the state's own terms (6 dk dv), the
    # triangular solve (C^2 / 3)
    per = 2 * C * (3 * d + 2 * d) + 6 * d * d + C * C / 3
    assert abs(per - 139605.333) < 1e-2
    assert B.prefill_alg_flops(p) == pytest.approx(32768 * 32 * per)


def test_step_min_bytes_adds_only_the_conv_weights_states_and_windows():
    p = chat_shape()
    conv_dim = 2 * 16 * 128 + 32 * 128
    # fp32 weights [conv_dim, 4]; bf16 conv states [32, 3, conv_dim] and windows [96, 3, conv_dim]
    assert B.step_min_bytes(p, 96) == (B.prefill_alg_bytes(p, 96, False) + conv_dim * 16 +
                                       (32 + 96) * 3 * conv_dim * 2)
    assert B.step_min_bytes(p, 96) == 1082130432 + 131072 + 6291456


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summarize_profiles_scales_counters_by_the_copy(tmp_path, monkeypatch):
    d = str(tmp_path)
    scan = "void gdn::chunked::pipelined_prefill_kernel<128, 128, false>(gdn::ScanArgs)"
    copy = "gdn::snapshot_copy_kernel(gdn::CopyArgs)"
    grid = 786432   # the chat wave: 1,024 workgroups x 768
    trace = [{"Kernel_Name": scan, "Grid_Size_X": 1024 * 768, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
              "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + 400} for i in range(3)]
    _write_csv(os.path.join(d, "trace", "run_kernel_trace.csv"), trace)
    _write_csv(os.path.join(d, "trace", "run_kernel_stats.csv"),
               [{"Name": scan, "Calls": 3, "TotalDurationNs": 1200, "AverageNs": 400, "MinNs": 400,
                 "MaxNs": 400, "Percentage": 100.0}])
    # the copy of 96 x 2 MiB: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    true_kib = 96 * 2 * 1024
    for c, copy_kib, scan_kib in (("FETCH_SIZE", true_kib / 2, 1000.0), ("WRITE_SIZE", true_kib, 500.0)):
        _write_csv(os.path.join(d, c, "run_counter_collection.csv"),
                   [{"Kernel_Name": copy, "Grid_Size": 96 * 256, "Counter_Value": copy_kib},
                    {"Kernel_Name": scan, "Grid_Size": grid, "Counter_Value": scan_kib},
                    {"Kernel_Name": scan, "Grid_Size": grid, "Counter_Value": scan_kib}])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(B, "TRAFFIC_FILE", str(out))
    res = B.summarize_profiles(d)
    rec = json.loads(out.read_text())
    assert rec == res["traffic"]
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    chat = rec["workloads"]["chat"]
    assert chat["dispatches"] == 2 and chat["trace_dispatches"] == 3
    assert chat["hbm_bytes_per_launch"] == pytest.approx((1000.0 * 2 + 500.0) * 1024)
    assert chat["trace_avg_us"] == pytest.approx(0.4)
    assert rec["csrc_sha256"] == B.csrc_digest()


def test_traffic_record_is_keyed_to_the_device_sources(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(B, "TRAFFIC_FILE", str(out))
    rec = {"csrc_sha256": B.csrc_digest(), "workloads": {"chat": {"hbm_bytes_per_launch": 123.0}}}
    out.write_text(json.dumps(rec))
    assert B.measured_traffic("chat") == 123.0
    assert B.measured_traffic("long") is None
    rec["csrc_sha256"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert B.measured_traffic("chat") is None
    # the host-only validation file is outside the key; a kernel source is inside it
    assert "gdn_api.hip" in B.HOST_ONLY_SOURCES
    assert "scan_pipe_kernel.h" in os.listdir(B.CSRC) and "scan_pipe_kernel.h" not in B.HOST_ONLY_SOURCES


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
