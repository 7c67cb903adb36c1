"""Host-side pieces of bench.py that need no GPU: the one-GPU refusal and the
CPU baseline record."""
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
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in rec["error"]


def test_cpu_baseline_record():
    import bench
    from few_row_quantized_amd import accounting, synth
    s = synth.WORKLOADS["tiny_k256_n512_4b_g64"]
    p = synth.make_problem(s)
    W = accounting.weight_bytes(s.N, s.K, s.bits, s.group_size)
    rec = bench.cpu_baseline(p, list(s.m_values), W, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["cpu_count"] == os.cpu_count()
    assert set(rec["median_ms_per_call"]) == {str(M) for M in s.m_values}
    one = rec["one_thread"]
    assert one["steps"] >= 3 and one["GBps"] > 0
