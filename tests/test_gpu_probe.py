"""The matrix-core probe (libfa_probe.so) that bench.py quotes the kernels against: it runs, every workgroup
records a positive cycle and real-time count, and the derived clock and rate are physically possible."""
import ctypes
import math
from pathlib import Path

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

LIB = Path(__file__).resolve().parent.parent / "exact_attention_13_amd" / "libfa_probe.so"


def test_probe_runs_and_reads_a_plausible_clock():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(str(LIB))
    f = lib.fa_probe_mfma_bf16
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_flop_per_wg_iter.restype = ctypes.c_double
    n_wg, iters = 1024, 256
    sink = torch.full((n_wg * lib.fa_probe_threads(),), float("nan"), dtype=torch.float32, device="cuda")
    clk = torch.zeros((2 * n_wg,), dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    print(f"[probe] n_wg={n_wg} iters={iters}", flush=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    assert f(sink.data_ptr(), clk.data_ptr(), n_wg, iters, st.cuda_stream) == 0  # warm-up
    a.record(st)
    assert f(sink.data_ptr(), clk.data_ptr(), n_wg, iters, st.cuda_stream) == 0
    b.record(st)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    c = clk.view(n_wg, 2)
    assert (c > 0).all()
    ghz = c[:, 0].sum().item() / c[:, 1].sum().item() * 0.1
    assert 0.3 < ghz < 3.0, ghz
    tflops = n_wg * iters * lib.fa_probe_flop_per_wg_iter() / (a.elapsed_time(b) * 1e-3) / 1e12
    assert math.isfinite(tflops) and 0 < tflops < 2516.6 * 3.0 / 2.4, tflops
