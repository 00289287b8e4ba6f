"""Host-side checks of bench.py: one GPU only, and the oracle baseline's shape."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_reports_a_bounded_oracle_sample():
    sys.path.insert(0, ROOT)
    import bench
    from mla_inputs import make_inputs
    inp = make_inputs("single_b1_l128", seed=0)
    cb = bench.cpu_baseline(inp, 0.5)
    assert cb["kind"] == "oracle" and cb["unit"] == "cache-tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "passes over the batch" in cb["sample"]      # the one 128-row sequence is repeated
