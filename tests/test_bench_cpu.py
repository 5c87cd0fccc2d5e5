"""bench.py's contract pieces that need no GPU: the one-GPU guard, the algorithmic-byte
count behind the roofline figure, and the CPU-baseline record."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_of_the_resident_step():
    import bench
    # 8 rows, every one of the 2048 selected rows valid: each selected 576-wide bf16 row
    # once, the query (128 x 576) and output (128 x 512) rows once, the index row once
    rows, K, H = 8, 2048, 128
    expect = rows * K * 576 * 2 + rows * (H * 576 * 2 + H * 512 * 2 + K * 4)
    assert bench.attn_alg_bytes([K] * rows, H, 576, 512, K) == expect == 21168128
    # padded entries carry no KV bytes; the index row is still read whole
    assert bench.attn_alg_bytes([K, 0], H, 576, 512, K) == \
        K * 1152 + 2 * (H * 576 * 2 + H * 512 * 2 + K * 4)


def test_cpu_baseline_record():
    """The oracle leg on a small mixed + finalize workload: every stage of the step is timed
    and the record carries the fields the benchmark line needs."""
    import bench
    from workloads import generate, spec
    s = spec("mixed_finalize", num_reqs=6, vocab=64, topk=128, capacity=512,
             seq_rule=("uniform", 300, 900))
    w = generate(s)
    pool_before = w.kv_pool.clone()
    r = bench.cpu_baseline(s, w, sample_reqs=4, reps=2)
    assert r["kind"] == "oracle" and r["unit"] == "rows/s"
    assert r["value"] > 0 and r["cores"] >= 1 and "first 4 of 6 requests (12 rows" in r["sample"]
    assert set(r["stage_ms"]) == {"resolve", "swap_in", "attention", "accept", "finalize"}
    assert r["one_thread"]["value"] > 0
    assert __import__("torch").equal(w.kv_pool, pool_before)   # finalize's host rows put back
