"""Host-side checks of bench.py's contract (no GPU): the one-GPU guard, the
algorithmic byte counts the roofline is priced on, and the committed HBM
counter summary those counts are compared with."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fp4_kv_cache_02_amd import synth  # noqa: E402

# one attention row-layer: 512 FP4 entries of 256 B codes + 32 B scales, the
# 128-entry window's K and V (bf16, 512 channels), 16 query heads (bf16),
# the fp32 output of 16 heads and the 512 int32 indices
PER_ATTN = 512 * (256 + 32) + 2 * 128 * 512 * 2 + 16 * 512 * 2 + 16 * 512 * 4 + 512 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_decode_128k():
    w = synth.workload("decode_128k")
    total, scan, layers = bench.algorithmic_bytes(w)
    assert PER_ATTN == 460800
    # one Full layer: 8 rows x (131072 bf16 keys of 64 channels + the 4x64
    # bf16 indexer query + the 512 int32 Top-512 positions)
    assert scan == 8 * (131072 * 128 + 512 + 2048)
    assert layers == 4
    assert total == scan + 4 * 8 * PER_ATTN


def test_algorithmic_bytes_fp8_keys():
    w = synth.workload("decode_128k")
    _, scan, _ = bench.algorithmic_bytes(w, key_bytes=68)   # 64 E4M3 codes + a float32 scale
    assert scan == 8 * (131072 * 68 + 512 + 2048)


def test_algorithmic_bytes_decode_1m():
    w = synth.workload("decode_1m")
    total, scan, layers = bench.algorithmic_bytes(w)
    # the Full layer only builds the candidate set (keys, query, and the
    # 2048 int32 candidate block ids written) and attends nothing; the
    # Reindex layer reads those ids and scores the 2048 blocks of 8 positions
    full = 1048576 * 128 + 512 + 2048 + 8192
    reindex = 2048 * 8 * 128 + 8192 + 512 + 2048
    assert scan == full + reindex
    assert layers == 4                      # Reindex + 3 Reuse
    assert total == scan + 4 * PER_ATTN


def test_committed_scan_traffic_is_close_to_algorithmic():
    path = os.path.join(ROOT, "profiles", "index_scan_decode_F3R_b8_L131072_traffic.json")
    d = json.load(open(path))
    w = synth.workload("decode_128k")
    algo = sum(128 * L + 512 for L in w.seq_lens)
    assert d["algorithmic_bytes_per_launch"] == algo
    fetch = d["fetch_kib_per_dispatch"] * 1024 * d["copy_calibration"]["fetch_scale"]
    write = d["write_kib_per_dispatch"] * 1024 * d["copy_calibration"]["write_scale"]
    assert d["bytes_per_launch"] == pytest.approx(fetch + write, rel=1e-4)
    # the scan reads every key once: measured HBM bytes within 5 % above
    assert algo <= d["bytes_per_launch"] <= 1.05 * algo
