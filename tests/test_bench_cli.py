"""bench.py's command line on the CPU: it measures one GPU and refuses more, before touching any GPU."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), *argv, "--steps", "1", "--warmup", "0"],
                       cwd=ROOT, env=e, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_timed_step_average_reads_the_last_dispatches_of_the_kernel(tmp_path):
    """The profile summaries quote a kernel's time as the mean over the run's timed steps: the last --steps
    dispatches of that kernel in the per-dispatch trace (after the settle phase and warm-up), other kernels and
    the order of the rows in the file not counting."""
    sys.path.insert(0, str(ROOT))
    import bench
    d = tmp_path / "trace"
    d.mkdir()
    rows = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    # 6 dispatches of kernel A (durations 10, 20, 30, 40, 50, 60 ns) interleaved with kernel B, rows shuffled
    disp = [("A", 100 * i, 100 * i + 10 * (i + 1)) for i in range(6)] + [("B", 100 * i + 50, 100 * i + 99)
                                                                           for i in range(6)]
    for name, s, e in reversed(disp):
        rows.append(f'"KERNEL_DISPATCH","{name}",{s},{e}')
    (d / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    assert bench._timed_avg_us(str(d), "A", "python bench.py --steps 2") == pytest.approx((50 + 60) / 2 / 1e3)
    assert bench._timed_avg_us(str(d), "A", "python bench.py --steps 100") == pytest.approx(35 / 1e3)
    assert bench._timed_avg_us(str(d), "C", "python bench.py --steps 2") is None
    assert bench._timed_avg_us(str(d), "A", "python bench.py") is None  # no --steps in the command
    assert bench._timed_avg_us(str(tmp_path / "missing"), "A", "python bench.py --steps 2") is None


def test_headline_line_keeps_the_json_contract():
    """The headline line from synthetic timings: every key the driver reads, with the throughput, the per-step time
    and the roofline fraction computed from the timed region (not from the per-call events), all JSON-serialisable."""
    import json
    import math

    sys.path.insert(0, str(ROOT))
    import bench
    import attn_inputs as ai

    w = ai.WORKLOADS[bench.HEADLINE]
    steps, warmup = 40, 5
    k_ms = 0.25                                      # average launch duration over the timed region
    wall = steps * 0.26e-3                           # seconds for the K timed steps, host clock
    durs = [0.27] * (steps - 1) + [0.40]             # per-call events of the pass before the region
    line = bench.headline_line(w, steps, warmup, 0.3, wall, k_ms * steps, durs, 2 * wall, [0.5] * warmup)
    json.dumps(line)
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(line[key], typ), key
    assert line["vs_baseline"] is None
    assert (line["n_gpus"], line["steps"], line["warmup"], line["higher_is_better"]) == (1, steps, warmup, True)
    assert line["config"]["workload"] == w.name and "model" not in line["config"]
    assert line["dtype"] == "bf16" and line["unit"] == "TFLOP/s"
    assert line["ms_per_step"] == pytest.approx(0.26, abs=1e-4)
    assert line["value"] == pytest.approx(w.flops / 0.26e-3 / 1e12, abs=0.01)
    r = line["roofline"]
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= set(r)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_BF16_TFLOPS
    assert r["achieved"] == pytest.approx(w.flops / (k_ms * 1e-3) / 1e12, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["traffic"] is None or (math.isfinite(r["traffic"]) and r["traffic"] >= w.algorithmic_bytes)
    assert line["kernel_ms"]["mean"] == pytest.approx(k_ms) and line["kernel_ms"]["per_call_mean"] > k_ms
    assert r["hbm_gbs"] == pytest.approx(w.algorithmic_bytes / (k_ms * 1e-3) / 1e9, abs=0.1)
    assert r["hbm_frac"] == pytest.approx(r["hbm_gbs"] / bench.PEAK_HBM_GBS, abs=1e-4) and r["hbm_frac"] < 1
    assert line["cold_start"]["ms_per_step"] == pytest.approx(0.52, abs=1e-4)


def test_kernel_hash_ignores_comments_and_layout_only(tmp_path):
    """A profile's source hash covers the code: editing a comment or re-indenting keeps it, changing a token or a
    literal does not."""
    sys.path.insert(0, str(ROOT))
    import bench
    f = tmp_path / "k.hip"
    base = "// header\nint f(int x) {  /* a\n block */ return x + 1; }  // tail\n"
    f.write_text(base)
    h0 = bench.kernel_src_hash([f])
    f.write_text("// another header, two lines\n// of it\nint f(int x) {\n    return x + 1;\n}\n")
    assert bench.kernel_src_hash([f]) == h0
    f.write_text(base.replace("x + 1", "x + 2"))
    assert bench.kernel_src_hash([f]) != h0
    f.write_text(base.replace("return", "return -"))
    assert bench.kernel_src_hash([f]) != h0
