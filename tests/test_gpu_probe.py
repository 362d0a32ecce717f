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


def test_issue_mix_probe_runs_every_mode():
    """The issue-mix probe (matrix cores against exponentials and FMAs, in the same wave or in the two waves of a
    SIMD): every mode runs, every wave records a positive cycle count, and the results are finite."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(str(LIB))
    g = lib.fa_probe_issue_mix
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_wg, iters = 256, 64
    sink = torch.full((n_wg * lib.fa_probe_issue_mix_threads(),), float("nan"), dtype=torch.float32, device="cuda")
    cyc = torch.zeros((8 * n_wg,), dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    for mode in range(5):
        print(f"[probe] issue mix mode={mode} n_wg={n_wg} iters={iters}", flush=True)
        sink.fill_(float("nan"))
        cyc.zero_()
        assert g(mode, sink.data_ptr(), cyc.data_ptr(), n_wg, iters, st.cuda_stream) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all()
        assert (cyc > 0).all()


def test_atomic_add_probe_sums_exactly_in_every_mode():
    """The atomic-add probe: in each atomic placement every add lands (the buffer sums to the adds issued, exact in
    fp32 at these counts), and the store mode writes every float of the tiles it reaches."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(str(LIB))
    h = lib.fa_probe_atomic_add
    h.restype = ctypes.c_int
    h.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    tf = lib.fa_probe_atomic_tile_floats()
    tiles, n_wg, rounds = 64, 96, 3
    buf = torch.zeros((tiles * tf,), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    for mode in range(4):
        print(f"[probe] atomic add mode={mode} tiles={tiles} n_wg={n_wg} rounds={rounds}", flush=True)
        buf.fill_(-1.0 if mode == 3 else 0.0)
        assert h(mode, buf.data_ptr(), tiles, n_wg, rounds, st.cuda_stream) == 0
        torch.cuda.synchronize()
        per_tile = buf.view(tiles, tf)
        if mode == 3:
            # tiles (7 wg + r) mod 64 for wg < 96, r < 3 cover every residue: all set to 1
            assert (per_tile == 1.0).all()
        else:
            assert float(buf.double().sum()) == n_wg * rounds * tf
            # within a tile every float received the same number of adds
            assert (per_tile == per_tile[:, :1]).all()
