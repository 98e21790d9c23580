"""Host-side checks of bench.py: the one-GPU contract and the algorithmic work
it divides by (no GPU needed)."""
import os
import subprocess
import sys

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_work_of_the_gpt2_workload():
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    work = bench.work_per_kind(wl)
    n = 84_934_656
    assert wl.params == n
    # momentum: G fp32 read, M bf16 read and written, for 8 workers
    assert work["momentum"] == ("hbm", 8 * n * (4 + 2 * 2))
    # Newton-Schulz: r^2 c per worker for the symmetric Gram, 2 r^2 c for the product
    r2c = 12 * (768 * 768 * 2304 + 768 * 768 * 768 + 768 * 768 * 3072 + 768 * 768 * 3072)
    assert work["ns_gram"] == ("mfma", 8 * r2c)
    assert work["ns_product"] == ("mfma", 2 * 8 * r2c)
    # every shape has C % 64 == 0: the sign is packed in the product, no standalone pass
    assert work["sign_pack"][1] == 0
    # vote + update: the 8 workers' packed bits, W read and written
    assert work["vote_update"] == ("hbm", n * (8 / 8 + 8))


def test_traffic_is_reported_only_for_the_profiled_sources():
    wl = synthetic.WORKLOADS["gpt2s_mw8_k1"]
    t = bench.counter_traffic(wl, "ns_product")
    # either the profile matches the current sources (a byte count) or it does not (None)
    assert t is None or t > 0
    assert bench.counter_traffic(wl, "no_such_kernel") is None
