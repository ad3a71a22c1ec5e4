"""bench.py's host side: the one-GPU guard and the CPU oracle baselines
(the oracle timed on the host; no GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
    assert "--gpus 1" in r.stderr


def test_cpu_baseline_fields_on_the_tiny_batch():
    sys.path.insert(0, ROOT)
    import bench
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import tiny_batch
    hb = tiny_batch(seed=0)
    r = bench.cpu_baseline(hb, "tiny", 2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1 and len(r["run_seconds"]) == 2
    # the median of the runs sets the rate (run_seconds are rounded to 1 ms)
    t_med = sorted(r["run_seconds"])[1]
    M = hb.x.shape[0]
    assert M / (t_med + 0.0006) <= r["value"] <= M / max(t_med - 0.0006, 1e-6)
    one = r["one_thread"]
    assert one["cores"] == 1 and one["value"] > 0


def test_cpu_table_writes_the_rows(tmp_path, capsys):
    sys.path.insert(0, ROOT)
    import bench
    out = tmp_path / "cpu.md"
    bench.cpu_table(1, str(out), keys=["tiny"], prompt_chunks=())
    text = out.read_text()
    assert "| tiny layer (H=256): Lp=64 (64 cached) + Bd=4 | 68 | median of 1 |" in text
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["rows"][0]["rows"] == 68 and line["rows"][0]["tokens_per_s"] > 0
