"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic byte count behind the
W4A16 roofline figures, and that the committed search traffic counters belong to the current
search source."""
import json
import os
import subprocess
import sys

import bench

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(HERE, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus_requested"] == 2 and "one GPU" in line["error"]


def test_gemv_bytes_of_the_70b_block():
    # codes K N / 2, float32 steps and uint8 zeros (5 K N / g), x and s (6 K), y (2 N), per linear
    layers = [(8192, 8192), (8192, 1024), (8192, 1024), (8192, 8192), (8192, 28672), (8192, 28672), (28672, 8192)]
    total = sum(bench._gemv_bytes(K, N) for K, N in layers)
    assert total == sum(K * N // 2 + 5 * K * N // 128 + 6 * K + 2 * N for K, N in layers) == 461877248
    fused = [(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)]
    assert sum(bench._gemv_bytes(K, N) for K, N in fused) == 461729792


def test_search_traffic_counters_match_the_current_source():
    # the bench reports roofline.traffic only while the search code is the one the counters were
    # taken on; the committed profile must describe the committed kernel
    t = bench.search_traffic()
    assert t is not None, "profiles/search_c2_hbm_traffic.md was taken on a different search source"
    algorithmic = 2 * 8192 * 4096 + 2 * 4096 * 4096    # X and W read once (bf16)
    assert algorithmic < t < 40 * algorithmic
