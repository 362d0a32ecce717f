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
