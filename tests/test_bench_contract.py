"""The benchmark's contract on the host (no GPU): the algorithmic work per
token that every roofline figure divides by, and the refusal of more than one
GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_work_per_token_at_the_full_shape():
    """H = 5,120, hc = 4 (N = 25,600), per token and layer: gather + decode
    reads 24 rows of 256 code bytes and 8 scale bytes plus 24 four-byte
    indices and writes 6,144 BF16 values; the projection is 2 x 25,600 x
    6,144 FLOP and moves mem and k/v per token plus wkv once per call; the
    gate reads the hidden state, 4 keys and the value and writes the hidden
    state."""
    w = bench.stage_work(1, 5120, 4)
    assert w["gather_bytes"] == 24 * 256 + 24 * 8 + 24 * 4 + 6144 * 2 == 18_720
    assert w["project_flops"] == 2 * 25_600 * 6_144 == 314_572_800
    assert w["gate_bytes"] == 4 * 5120 * 2 * 2 + 4 * 5120 * 2 + 5120 * 2 == 133_120
    assert w["hash_bytes"] == 4 + 24 * 4
    # the projection's bytes: mem and k/v scale with T, wkv does not
    w2 = bench.stage_work(2, 5120, 4)
    assert w2["project_bytes"] - w["project_bytes"] == 2 * (6144 + 25_600)
    assert w["project_bytes"] - 2 * (6144 + 25_600) == 2 * 25_600 * 6144
    # and every per-token figure scales linearly with T
    w50 = bench.stage_work(50_032, 5120, 4)
    for k in ("gather_bytes", "gate_bytes", "hash_bytes", "project_flops"):
        assert w50[k] == 50_032 * w[k]


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
