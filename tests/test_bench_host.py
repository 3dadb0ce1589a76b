"""Host logic of bench.py (CPU only): the algorithmic byte and flop counts the rooflines
divide by, the refusal of more than one GPU, and the rule that a committed traffic record
is reported only when it was taken on the current kernel sources and plan."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_forward_bytes_and_flops_per_token_head():
    # q, k, v in bf16 (768 B at d = 128), x (4 B), o in fp32 (512 B)
    assert bench.algorithmic_bytes_per_token_head(128, 128, 2) == 1284
    assert bench.algorithmic_bytes_per_token_head(64, 64, 4) == 3 * 64 * 4 + 4 + 4 * 64
    # q.S and the state update (2 dk dv each) + q k^T and A v over 40 keys on average
    assert bench.algorithmic_flops_per_token_head(128, 128) == 4 * 128 * 128 + 80 * 256


def test_backward_and_per_channel_bytes_per_token_head():
    # q, k, v, dO in bf16 + x in; dq, dk, dv in fp32 + dx out
    assert bench.backward_bytes_per_token_head(128, 128, 2) == 4 * 256 + 4 + 3 * 512 + 4 == 2568
    # the per-channel gate input is fp32 per key channel: 512 B instead of 4
    assert bench.per_channel_bytes_per_token_head(128, 128, 2) == 1792


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_output_kernel_name():
    assert bench.output_kernel_name(2, 128, 128) == "chunk_output_ws_kernel"
    assert bench.output_kernel_name(4, 64, 64) == "chunk_output_kernel"


def test_traffic_record_needs_current_sources_and_plan(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()  # of the sources in this tree
    rec = {"kernel_source_sha": sha, "plan": [8, 1], "path": "unified", "bytes_per_launch": 123.0}
    (tmp_path / "profiles").mkdir()
    fn = tmp_path / "profiles" / "k_w_traffic.json"
    fn.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("k", "w", (8, 1), "unified") == 123.0
    assert bench.load_traffic("k", "w", (4, 1), "unified") is None
    assert bench.load_traffic("k", "w", (8, 1), "diag_branch") is None
    rec["kernel_source_sha"] = "0" * 16
    fn.write_text(json.dumps(rec))
    assert bench.load_traffic("k", "w", (8, 1), "unified") is None
    assert bench.load_traffic("k", "missing", (8, 1), "unified") is None

