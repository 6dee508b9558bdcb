"""bench.py's contract pieces that need no GPU: one GPU only, the algorithmic byte counts, and the
counter table's staleness rule."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr + r.stdout


def test_algorithmic_bytes_per_token_head():
    # bf16 r, w, k, v, a, b read (6 x 64 x 2 bytes), fp32 y written (64 x 4): 1,024 bytes per token*head,
    # plus the fp32 state read and written once per head
    B, T, H, N = 8, 4096, 12, 64
    assert bench.algo_bytes(B, T, H) == B * T * H * 1024 + 2 * B * H * N * N * 4
    assert bench.algo_bytes(1, 1, 1, in_bytes=4) == 6 * 64 * 4 + 64 * 4 + 2 * 64 * 64 * 4


def test_counter_entries_follow_their_sources(tmp_path, monkeypatch):
    src = ["linear_rnn_amd/csrc/wkv7_fused.hip"]
    key = "k:w"
    tab = {key: {"bytes_per_launch": 123.0, "src_sha": bench.source_hash(src)}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(tab))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(key, src) == 123.0
    # another source set (as after an edit of the kernel) makes the entry stale
    assert bench.measured_traffic(key, src + ["linear_rnn_amd/csrc/wkv7_fused.hpp"]) is None
    assert bench.measured_traffic("absent:w", src) is None


@pytest.mark.parametrize("name", ["D4096-long-prefill", "L12-D768-prefill", "L24-D1024-prefill-resume"])
def test_committed_counter_entries_name_their_workload(name):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        tab = json.load(fh)
    keys = [k for k in tab if k.endswith(":" + name)]
    assert keys, name
    for k in keys:
        assert tab[k]["bytes_per_launch"] > 0 and len(tab[k]["src_sha"]) == 16
