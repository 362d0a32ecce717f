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
