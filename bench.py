"""Benchmark of the exact attention forward (and its gradients) on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload c3_bf16_b2h16n4096d128]

One step = one fa_fwd call (the whole hot path: Q/K/V read, S = QK^T, online softmax, PV, 1/l, o and lse
written) over the workload's synthetic inputs, already resident in device memory. Prints ONE JSON line:
value = attention-forward TFLOP/s (4*B*H*N^2*d, halved when causal) over the timed steps; roofline = the
kernel's MFMA roofline from HIP-event launch durations; cpu_baseline = the fp64 oracle timed on every query
row of the same workload on this host's cores (about 4 s of CPU work on 16 threads for the headline workload).

The line also carries `backward`: the gradient call fa_bwd (dq, then dk and dv) on the headline workload and on
the long causal one, timed the same way, in the usual FLOP convention 2.5 x the forward's (five matrix products:
the recomputed QK^T, dO V^T, dV, dQ, dK); `fp8`: fa_fwd_fp8 on the same two shapes with the inputs quantized
per tensor to float8_e4m3fn, against the fp8 peak; `varlen` and `varlen_backward`: fa_fwd_varlen and fa_bwd_varlen
on the packed workloads; `mfma_probe`: the dense bf16 rate this GPU's matrix cores sustain on back-to-back MFMAs
with random register operands, and the shader clock meanwhile (libfa_probe.so), with roofline.frac_of_probe =
the headline kernel's rate over it (boxes differ by up to ~15 % in the clock their power limit allows).

    --bwd-only          time only the gradient call of --workload (one JSON line; for profiling)
    --no-mfma-probe     leave out the matrix-core probe (mfma_probe, roofline.frac_of_probe)

Other modes (used to produce the rocprofv3 summaries under profiles/):
    --pmc-pass          run a copy kernel of known size, then the workload kernel, a few times each
    --summarize DIR     print a summary of the rocprofv3 output found under DIR
    --write-profiles    turn the outputs of PROFILE_COMMANDS (under gpurun_out/) into profiles/ summaries
    --bwd-pmc-pass      like --pmc-pass for the gradient call (copy kernel, then fa_bwd a few times)
    --write-profiles-bwd  the same for BWD_PROFILE_COMMANDS: profiles/bwd_<workload>_rocprof.md
    --fp8-only          time only fa_fwd_fp8 on --workload's shape (one JSON line; for profiling)
    --fp8-pmc-pass      like --pmc-pass for the fp8 forward
    --write-profiles-fp8  the same for FP8_PROFILE_COMMANDS: profiles/fp8_<workload>_rocprof.md and _hbm_traffic.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk (AMD's published 2.5 PF)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (AMD's published 5.0 PF; twice the bf16 rate)
PEAK_HBM_GBS = 8000.0
HEADLINE = "c3_bf16_b2h16n4096d128"
KERNEL_SRC = ROOT / "exact_attention_13_amd" / "csrc" / "fa_fwd_kernel.hip"
KERNEL_SRCS = (KERNEL_SRC, ROOT / "exact_attention_13_amd" / "csrc" / "fa_gfx950.h")
BWD_SRCS = (ROOT / "exact_attention_13_amd" / "csrc" / "fa_bwd_kernel.hip",
            ROOT / "exact_attention_13_amd" / "csrc" / "fa_gfx950.h")
BWD_WORKLOADS = ("c3_bf16_b2h16n4096d128", "c4_bf16_b1h32n16384d128_causal", "kpad_bf16_b8h16n4096d128",
                 "mqa_bf16_b1h32kv1n16384d128_causal")
FP8_WORKLOADS = ("c3_bf16_b2h16n4096d128", "c4_bf16_b1h32n16384d128_causal")  # the same shapes, fp8 inputs
FP8_SRCS = (ROOT / "exact_attention_13_amd" / "csrc" / "fa_fwd_fp8_kernel.hip",
            ROOT / "exact_attention_13_amd" / "csrc" / "fa_gfx950.h")
PROFILES = ROOT / "profiles"


# The rocprofv3 runs whose outputs --write-profiles summarises ({w} = workload name). Counter runs hold one
# counter group each; the copy kernel of --pmc-pass calibrates FETCH_SIZE / WRITE_SIZE against known bytes.
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_{w}_trace -o run -- "
             "python bench.py --workload {w} --no-cpu-baseline --no-other-workloads --no-backward --steps 50 "
             "--warmup 10",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_{w}_fetch -o run -- "
             "python bench.py --workload {w} --pmc-pass",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_{w}_write -o run -- "
             "python bench.py --workload {w} --pmc-pass",
    "sq": "rocprofv3 --kernel-trace --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU "
          "SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE "
          "--output-format csv -d gpurun_out/prof_{w}_sq -o run -- python bench.py --workload {w} --pmc-pass",
    # where the wave-cycles go: waiting, issuing, co-issue of vector instructions with busy matrix cores
    "stall": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
             "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE --output-format csv "
             "-d gpurun_out/prof_{w}_stall -o run -- python bench.py --workload {w} --pmc-pass",
    # L2 hit rate, dual-issued vector cycles, transcendental instructions, LDS data-queue pressure
    "l2": "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum SQ_ACTIVE_INST_VALU2 SQ_INSTS_VALU_TRANS_F32 SQ_LDS_DATA_FIFO_FULL "
          "SQ_INSTS_LDS SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
          "-d gpurun_out/prof_{w}_l2 -o run -- python bench.py --workload {w} --pmc-pass",
}


# The same four runs for the gradient call (two kernels per call).
BWD_PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_bwd_{w}_trace -o run -- "
             "python bench.py --workload {w} --bwd-only --steps 20 --warmup 3",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_bwd_{w}_fetch -o run -- "
             "python bench.py --workload {w} --bwd-pmc-pass",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_bwd_{w}_write -o run -- "
             "python bench.py --workload {w} --bwd-pmc-pass",
    "sq": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_MFMA "
          "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv "
          "-d gpurun_out/prof_bwd_{w}_sq -o run -- python bench.py --workload {w} --bwd-pmc-pass",
}


# The same four runs for the fp8 forward (fa_fwd_fp8 on a bf16 workload's shape, inputs quantized to e4m3).
FP8_PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_fp8_{w}_trace -o run -- "
             "python bench.py --workload {w} --fp8-only --steps 50 --warmup 10",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fp8_{w}_fetch -o run -- "
             "python bench.py --workload {w} --fp8-pmc-pass",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_fp8_{w}_write -o run -- "
             "python bench.py --workload {w} --fp8-pmc-pass",
    "sq": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT "
          "SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv "
          "-d gpurun_out/prof_fp8_{w}_sq -o run -- python bench.py --workload {w} --fp8-pmc-pass",
}


# Kernel trace of the packed variable-length forward ({w} = packed workload name).
VARLEN_PROFILE_COMMAND = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_{w}_trace -o run -- "
                          "python bench.py --varlen-only {w} --steps 50 --warmup 10")


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_src_hash(srcs=KERNEL_SRCS) -> str:
    """sha256[:16] of the kernel sources' code: comments removed and whitespace collapsed, so that a profile taken
    on the code stays valid across edits of its comments or layout, and only across those."""
    h = hashlib.sha256()
    for f in srcs:
        h.update(" ".join(_COMMENTS.sub(" ", f.read_text()).split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def kernel_name(w) -> str:
    """The kernel instance the library launches for workload w, as the library itself reports it (fa_fwd_instance;
    the fp32 forward has one instance per head dim and causal flag)."""
    import exact_attention_13_amd as fa

    if w.dtype != "bf16":
        return f"fa_fwd_f32_kernel<{w.d}, {'true' if w.causal else 'false'}>"
    return fa.fa_fwd_instance(w.B, w.H, w.N, w.d, int(w.causal), 0)


def _device_inputs(w):
    import torch
    import attn_inputs as ai

    q, k, v = ai.make_workload(w)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    lens = torch.tensor(w.kv_len, dtype=torch.int32, device="cuda") if w.kv_len else None
    return q, k, v, o, lse, lens


def _caller(w, q, k, v, o, lse, lens, stream_handle):
    """One raw C-ABI call for workload w: fa_fwd, fa_fwd_gqa (fewer key/value heads), fa_fwd_kpad (key
    padding) or fa_fwd_f32."""
    import exact_attention_13_amd as fa

    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    tail = (w.N, w.d, int(w.causal), w.scale, stream_handle)
    if lens is not None:
        fn, args = fa.fa_fwd_kpad, ptrs + (lens.data_ptr(), w.B, w.H, w.Hk) + tail
    elif w.Hk != w.H:
        fn, args = fa.fa_fwd_gqa, ptrs + (w.B, w.H, w.Hk) + tail
    else:
        fn, args = (fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32), ptrs + (w.B, w.H) + tail

    def call():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"fa_fwd failed: {fa.fa_strerror(rc)}")
    return call


SETTLE_S = 0.3  # seconds of untimed back-to-back calls before a leg's warm-up


def _settle(call, settle_s: float):
    """Run `call` back to back, untimed, for settle_s seconds. After an idle spell (the seconds the host spends
    making a workload's inputs) the GPU's clock needs about a hundred launches of the headline kernel (≈ 30 ms of
    load) to reach the level it then holds; the launches in between run up to 30 % slower, and a few warm-up steps
    end inside that transient."""
    import torch

    if settle_s <= 0:
        return
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    batch = 1
    while time.perf_counter() < t_end:
        for _ in range(batch):
            call()
        torch.cuda.synchronize()
        batch = min(2 * batch, 64)


def _time_calls(call, stream, steps: int, warmup: int, settle_s: float = 0.0):
    """The settle phase (settle_s seconds of untimed calls), `warmup` untimed calls, then `steps` calls each bracketed
    by HIP events on `stream`, with a device synchronisation before and after the timed ones. Returns (wall_s for
    the `steps` calls, per-call durations in ms)."""
    import torch

    _settle(call, settle_s)
    for _ in range(warmup):
        call()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in zip(starts, ends)]


def _time_region_calls(call, stream, steps: int, warmup: int, settle_s: float):
    """The settle phase, `steps` calls timed one by one with HIP events (their spread), `warmup` untimed calls, then
    the timed region: `steps` calls back to back with one HIP event pair around them on `stream` and a device
    synchronisation on both sides. Returns (wall_s of the region, its event time / steps in ms, the per-call
    durations of the first pass)."""
    import torch

    _, per_call = _time_calls(call, stream, steps, 0, settle_s)
    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, a.elapsed_time(b) / steps, per_call


def time_region(w, steps: int, warmup: int, settle_s: float):
    """The headline leg. After the settle phase, `steps` calls timed one by one with HIP events (their spread:
    median, min, p90), then `warmup` untimed calls, then the timed region: `steps` calls back to back with one HIP
    event pair around them on the launch stream and a device synchronisation on both sides. Events between the
    launches cost the region ≈ 5 µs of wall time per call on C3 (0.2487 against 0.2424 ms per step), so the region
    has none. Returns (wall_s of the region, its event time in ms, the per-call durations of the first pass)."""
    import torch

    q, k, v, o, lse, lens = _device_inputs(w)
    stream = torch.cuda.current_stream()
    call = _caller(w, q, k, v, o, lse, lens, stream.cuda_stream)
    wall, mean_ms, per_call = _time_region_calls(call, stream, steps, warmup, settle_s)
    del q, k, v, o, lse, lens
    return wall, mean_ms * steps, per_call


def clock_settle(w, launches: int = 300, idle_s: float = 2.0, trials: int = 2):
    """Per-launch kernel times of workload w after `idle_s` seconds with the GPU idle: the means of each 20 launches
    in order and the first 10 launches, per trial. Shows how long the clock takes to settle under load."""
    import torch

    q, k, v, o, lse, lens = _device_inputs(w)
    stream = torch.cuda.current_stream()
    call = _caller(w, q, k, v, o, lse, lens, stream.cuda_stream)
    out = []
    for trial in range(trials):
        torch.cuda.synchronize()
        time.sleep(idle_s)
        _, durs = _time_calls(call, stream, launches, 0)
        out.append({"trial": trial, "idle_s": idle_s,
                    "mean_ms_per_20": [round(statistics.fmean(durs[i:i + 20]), 4) for i in range(0, launches, 20)],
                    "first10_ms": [round(d, 4) for d in durs[:10]]})
    return out


def time_workload(w, steps: int, warmup: int, settle_s: float = 0.0, region: bool = True):
    """Returns (wall_s for `steps` calls, mean launch duration in ms, per-launch durations in ms), from HIP events on
    the launch stream: with `region`, the mean over a timed region of back-to-back calls (_time_region_calls),
    otherwise the mean of calls timed one by one."""
    import torch

    q, k, v, o, lse, lens = _device_inputs(w)
    stream = torch.cuda.current_stream()
    call = _caller(w, q, k, v, o, lse, lens, stream.cuda_stream)
    if region:
        wall, mean, durs = _time_region_calls(call, stream, steps, warmup, settle_s)
    else:
        wall, durs = _time_calls(call, stream, steps, warmup, settle_s)
        mean = statistics.fmean(durs)
    del q, k, v, o, lse, lens
    return wall, mean, durs


def time_backward(w, steps: int, warmup: int, settle_s: float = 0.0, region: bool = True):
    """Gradient call of workload w (bf16): (wall_s for `steps` calls, mean call duration in ms, per-call durations in
    ms), from HIP events as time_workload. The forward runs once first to provide o and lse; dout is seeded N(0, 1)."""
    import torch

    import exact_attention_13_amd as fa

    q, k, v, o, lse, lens = _device_inputs(w)
    g = torch.Generator("cpu").manual_seed(w.seed + 500)
    dout = torch.randn(tuple(q.shape), generator=g).to(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()
    fwd = _caller(w, q, k, v, o, lse, lens, stream.cuda_stream)
    fwd()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((fa.fa_bwd_workspace_bytes(w.B, w.H, w.Hk, w.N, w.d),), dtype=torch.uint8, device="cuda")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), ws.data_ptr())
    tail = (w.B, w.H, w.Hk, w.N, w.d, int(w.causal), w.scale, stream.cuda_stream)
    entry, args = (fa.fa_bwd, ptrs + tail) if lens is None else (fa.fa_bwd_kpad, ptrs + (lens.data_ptr(),) + tail)

    def call():
        rc = entry(*args)
        if rc != 0:
            raise RuntimeError(f"fa_bwd failed: {fa.fa_strerror(rc)}")
    if region:
        wall, mean, durs = _time_region_calls(call, stream, steps, warmup, settle_s)
    else:
        wall, durs = _time_calls(call, stream, steps, warmup, settle_s)
        mean = statistics.fmean(durs)
    del q, k, v, o, lse, dout, dq, dk, dv, ws
    return wall, mean, durs


def backward_record(w, steps: int, warmup: int, settle_s: float = 0.0):
    wall, mean, durs = time_backward(w, steps, warmup, settle_s)
    flops = 2.5 * w.flops
    return {"workload": w.name, "tflops": round(flops * steps / wall / 1e12, 2),
            "pct_of_peak": round(100 * flops * steps / wall / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernel_ms": {"mean": round(mean, 4), "median": round(statistics.median(durs), 4),
                          "min": round(min(durs), 4)},
            "roofline": {"bound": "mfma", "achieved": round(flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "flops_per_call": flops, "kernels": ["fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"],
            "kernel_src_sha256_16": kernel_src_hash(BWD_SRCS)}


def fp8_record(w, steps: int, warmup: int, settle_s: float = 0.0):
    """fa_fwd_fp8 on workload w's shape with the seeded inputs quantized per tensor to float8_e4m3fn."""
    import torch

    import attn_inputs as ai
    import exact_attention_13_amd as fa

    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(w.B, w.H, w.N, w.d, w.seed, w.k_scale)
    q, k, vt = q8.cuda(), k8.cuda(), v8.transpose(2, 3).contiguous().cuda()
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(), sq, sk, sv, w.B, w.H, w.N, w.d,
            int(w.causal), w.scale, stream.cuda_stream)

    def call():
        rc = fa.fa_fwd_fp8(*args)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_fp8 failed: {fa.fa_strerror(rc)}")
    wall, mean, durs = _time_region_calls(call, stream, steps, warmup, settle_s)
    return {"workload": w.name.replace("_bf16_", "_fp8_"), "dtype": "fp8 e4m3 (bf16 o)",
            "tflops": round(w.flops * steps / wall / 1e12, 2),
            "kernel_ms": {"mean": round(mean, 4), "median": round(statistics.median(durs), 4),
                          "min": round(min(durs), 4)},
            "roofline": {"bound": "mfma", "achieved": round(w.flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(w.flops / (mean * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)},
            "flops_per_launch": w.flops, "kernel": "fa_fwd_fp8_kernel",
            "traffic": traffic_from_profiles(w, "fp8_", FP8_SRCS),
            "kernel_src_sha256_16": kernel_src_hash(FP8_SRCS)}


def varlen_record(w, steps: int, warmup: int, settle_s: float = 0.0):
    """fa_fwd_varlen on a packed variable-length workload (inputs resident on the device)."""
    import torch

    import attn_inputs as ai
    import exact_attention_13_amd as fa

    q, k, v = (x.cuda() for x in ai.make_qkv_varlen(w.lens, w.H, w.d, w.seed, Hkv=w.Hkv or None))
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.H, w.T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu.data_ptr(), w.B, w.H, w.Hk,
            w.T, w.max_len, w.d, int(w.causal), w.scale, stream.cuda_stream)

    def call():
        rc = fa.fa_fwd_varlen(*args)
        if rc != 0:
            raise RuntimeError(f"fa_fwd_varlen failed: {fa.fa_strerror(rc)}")
    wall, mean, durs = _time_region_calls(call, stream, steps, warmup, settle_s)
    return {"workload": w.name, "lens": list(w.lens), "H": w.H, "H_kv": w.Hk, "d": w.d, "causal": w.causal,
            "tflops": round(w.flops * steps / wall / 1e12, 2),
            "kernel_ms": {"mean": round(mean, 4), "median": round(statistics.median(durs), 4),
                          "min": round(min(durs), 4)},
            "roofline": {"bound": "mfma", "achieved": round(w.flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(w.flops / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "flops_per_launch": w.flops, "algorithmic_bytes_per_launch": w.algorithmic_bytes,
            "kernel": "fa_fwd_bf16_kernel (VARLEN)", "kernel_src_sha256_16": kernel_src_hash()}


def varlen_backward_record(w, steps: int, warmup: int, settle_s: float = 0.0):
    """fa_bwd_varlen on a packed workload (o and lse from one fa_fwd_varlen call), FLOPs 2.5 x the forward's."""
    import torch

    import attn_inputs as ai
    import exact_attention_13_amd as fa

    q, k, v = (x.cuda() for x in ai.make_qkv_varlen(w.lens, w.H, w.d, w.seed, Hkv=w.Hkv or None))
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_len, causal=w.causal, scale=w.scale)
    g = torch.Generator("cpu").manual_seed(w.seed + 500)
    dout = torch.randn(tuple(q.shape), generator=g).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((fa.fa_bwd_workspace_bytes(w.B, w.H, w.Hk, w.max_len, w.d),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), cu.data_ptr(), w.B, w.H, w.Hk, w.T, w.max_len, w.d,
            int(w.causal), w.scale, stream.cuda_stream)

    def call():
        rc = fa.fa_bwd_varlen(*args)
        if rc != 0:
            raise RuntimeError(f"fa_bwd_varlen failed: {fa.fa_strerror(rc)}")
    wall, mean, durs = _time_region_calls(call, stream, steps, warmup, settle_s)
    flops = 2.5 * w.flops
    return {"workload": w.name, "call": "fa_bwd_varlen", "tflops": round(flops * steps / wall / 1e12, 2),
            "kernel_ms": {"mean": round(mean, 4), "median": round(statistics.median(durs), 4),
                          "min": round(min(durs), 4)},
            "roofline": {"bound": "mfma", "achieved": round(flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "flops_per_call": flops, "kernels": ["fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"],
            "kernel_src_sha256_16": kernel_src_hash(BWD_SRCS)}


ISSUE_MIX_MODES = ("8 MFMA", "8 MFMA + 8 exp2 (same wave)", "8 MFMA + 8 exp2 + 24 FMA (same wave)",
                   "waves 0-3: 8 MFMA; waves 4-7: 8 exp2 + 24 FMA", "8 exp2 + 24 FMA")


def issue_mix_probe(n_wg: int = 256, iters: int = 2048):
    """libfa_probe.so's issue-mix probe (include/fa_probe.h): per mode, the mean shader cycles per loop iteration
    of waves 0-3 and of waves 4-7 (the two waves of each SIMD), and the matrix cores' busy share per SIMD implied
    by the products issued (32 cycles per v_mfma_f32_32x32x16_bf16)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(str(ROOT / "exact_attention_13_amd" / "libfa_probe.so"))
    g = lib.fa_probe_issue_mix
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    sink = torch.empty((n_wg * lib.fa_probe_issue_mix_threads(),), dtype=torch.float32, device="cuda")
    cyc = torch.zeros((8 * n_wg,), dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    out = []
    for mode, name in enumerate(ISSUE_MIX_MODES):
        for _ in range(2):  # the second run is the one read
            if g(mode, sink.data_ptr(), cyc.data_ptr(), n_wg, iters, st.cuda_stream) != 0:
                raise RuntimeError("fa_probe_issue_mix failed")
        torch.cuda.synchronize()
        c = cyc.view(n_wg, 8).double()
        lo, hi = float(c[:, :4].mean()) / iters, float(c[:, 4:].mean()) / iters
        mfma_per_simd = {0: 16, 1: 16, 2: 16, 3: 8, 4: 0}[mode]  # products per iteration on a SIMD's two waves
        out.append({"mode": mode, "what": name, "cycles_per_iter_waves_0_3": round(lo, 1),
                    "cycles_per_iter_waves_4_7": round(hi, 1),
                    "matrix_busy": round(32 * mfma_per_simd / max(lo, hi), 3)})
    return out


ATOMIC_MODES = ("fp32 atomic add, tiles reached from any XCD", "fp32 atomic add, each tile from one XCD only",
                "fp32 atomic add, 32 workgroups on one tile at once", "plain stores, tiles as in mode 0")


def dq_partial_bytes(w) -> int:
    """fp32 bytes a single gradient pass with atomic dq updates would add into dq for workload w: one 128 x d block
    per (128-key block, 128-row query tile) pair that the mask leaves work in, for every query head."""
    nb = -(-w.N // 128)
    pairs = nb * (nb + 1) // 2 if w.causal else nb * nb
    return w.B * w.H * pairs * 128 * w.d * 4


def atomic_add_probe(n_wg: int = 2048, rounds: int = 8, tiles: int = 1024, reps: int = 10):
    """libfa_probe.so's atomic-add probe (include/fa_probe.h): GB/s of fp32 atomic adds into device memory in
    64 KiB tiles, per placement, against plain stores; each atomic mode's sum is checked. Then the time the dq
    partial blocks of the C3 and C4 shapes would take at the measured atomic rate."""
    import ctypes
    import torch

    import attn_inputs as ai
    lib = ctypes.CDLL(str(ROOT / "exact_attention_13_amd" / "libfa_probe.so"))
    g = lib.fa_probe_atomic_add
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    tf = lib.fa_probe_atomic_tile_floats()
    buf = torch.zeros((tiles * tf,), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    nbytes = n_wg * rounds * tf * 4
    out = []
    for mode, what in enumerate(ATOMIC_MODES):
        buf.zero_()
        for _ in range(2):
            if g(mode, buf.data_ptr(), tiles, n_wg, rounds, st.cuda_stream) != 0:
                raise RuntimeError("fa_probe_atomic_add failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            g(mode, buf.data_ptr(), tiles, n_wg, rounds, st.cuda_stream)
        b.record(st)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
        total = float(buf.double().sum())
        want = float(tiles * tf) if mode == 3 else float((2 + reps) * n_wg * rounds * tf)
        out.append({"mode": mode, "what": what, "bytes_per_launch": nbytes, "ms": round(ms, 4),
                    "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "sum_exact": total == want})
    rate = out[0]["GBps"] * 1e9
    for name in ("c3_bf16_b2h16n4096d128", "c4_bf16_b1h32n16384d128_causal"):
        nb = dq_partial_bytes(ai.WORKLOADS[name])
        out.append({"workload": name, "dq_partial_bytes": nb,
                    "atomic_ms_at_mode0_rate": round(nb / rate * 1e3, 3)})
    return out


def mfma_probe(n_wg: int = 2048, iters: int = 2048, reps: int = 5):
    """The dense bf16 rate the matrix cores of this GPU sustain, and the shader clock meanwhile
    (libfa_probe.so, include/fa_probe.h: v_mfma_f32_32x32x16_bf16 back to back on random register operands)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(str(ROOT / "exact_attention_13_amd" / "libfa_probe.so"))
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_flop_per_wg_iter.restype = ctypes.c_double
    lib.fa_probe_threads.restype = ctypes.c_int
    sink = torch.empty((n_wg * lib.fa_probe_threads(),), dtype=torch.float32, device="cuda")
    clk = torch.zeros((2 * n_wg,), dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream()
    args = (sink.data_ptr(), clk.data_ptr(), n_wg, iters, st.cuda_stream)
    for _ in range(2):
        if lib.fa_probe_mfma_bf16(*args) != 0:
            raise RuntimeError("fa_probe_mfma_bf16 failed")
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        lib.fa_probe_mfma_bf16(*args)
        b.record(st)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    c = clk.view(n_wg, 2).sum(dim=0).tolist()
    ghz = c[0] / c[1] * 0.1  # shader cycles per 100 MHz real-time tick
    tflops = n_wg * iters * lib.fa_probe_flop_per_wg_iter() / (statistics.median(ms) * 1e-3) / 1e12
    return {"tflops": round(tflops, 1), "sclk_ghz": round(ghz, 3), "pct_of_spec": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "note": "v_mfma_f32_32x32x16_bf16 back to back on random register operands, all CUs, 2 waves per SIMD"}


def traffic_from_profiles(w, prefix="", srcs=KERNEL_SRCS):
    """HBM bytes per launch from the committed PMC summary, if it was taken on the current kernel source."""
    f = PROFILES / f"{prefix}{w.name}_hbm_traffic.txt"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text())
    except json.JSONDecodeError:
        return None
    if rec.get("kernel_src_sha256_16") != kernel_src_hash(srcs):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, n_rows: int):
    """fp64 oracle on a seeded sample of the workload's query rows; TFLOP/s in the metric's FLOP count."""
    import numpy as np

    import attn_inputs as ai
    import oracle

    q, k, v = ai.make_workload(w)
    lens = ai.kv_len_of(w)
    total = w.B * w.H * w.N
    if n_rows <= 0 or n_rows >= total:
        rows = np.arange(total, dtype=np.int64)  # every query row of the workload
    else:
        rows = ai.sample_rows(w.B, w.H, w.N, n_rows, seed=w.seed + 7)
    threads = oracle.default_threads()
    oracle.attention_rows(q, k, v, w.causal, w.scale, rows=rows[:threads], threads=threads, kv_len=lens)  # warm
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, w.causal, w.scale, rows=rows, threads=threads, kv_len=lens)
    dt = time.perf_counter() - t0
    def sample_flops(r):
        i = r % w.N
        n_valid = np.array(lens)[r // (w.H * w.N)] if lens else np.full_like(i, w.N)
        keys = np.minimum(i + 1, n_valid) if w.causal else n_valid
        return float(np.sum(4.0 * keys * w.d))  # 2 FLOP per q.k product term + 2 per p.v term, per visible key
    # the metric counts 4*N*d per row (halved on average when causal); sampled rows use their real key counts
    flops = sample_flops(rows)
    # the same oracle on one thread, over the first 1/16 of the sample
    rows1 = rows[: max(1, len(rows) // 16)]
    t1 = time.perf_counter()
    oracle.attention_rows(q, k, v, w.causal, w.scale, rows=rows1, threads=1, kv_len=lens)
    dt1 = time.perf_counter() - t1
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"all {total} query rows of {w.name}" if len(rows) == total else
                       f"{len(rows)} seeded random query rows of {w.name} ({len(rows) / total:.1%} of the rows)")
                      + f", fp64, {dt:.2f} s wall on {threads} threads; FLOPs counted as 4*d per visible key",
            "single_thread": {"value": sample_flops(rows1) / dt1 / 1e12, "rows": len(rows1),
                              "seconds": round(dt1, 3)},
            "cpu_model": cpu, "host_cpus": os.cpu_count(), "seconds": dt}


def _copy_kernel_pass(reps: int) -> int:
    """A plain copy of known size (the calibration kernel of the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch

    n = 1 << 28  # 512 MiB of bf16 read + 512 MiB written by torch.neg
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    return n


def bwd_pmc_pass(w, reps: int):
    """Kernels for the rocprofv3 counter runs of the gradient call: the copy, then fa_bwd."""
    n = _copy_kernel_pass(reps)
    time_backward(w, steps=reps, warmup=0, region=False)
    print(json.dumps({"bwd_pmc_pass": w.name, "copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "reps": reps,
                      "kernel_src_sha256_16": kernel_src_hash(BWD_SRCS)}), flush=True)


def fp8_pmc_pass(w, reps: int):
    """Kernels for the rocprofv3 counter runs of the fp8 forward: the copy, then fa_fwd_fp8."""
    n = _copy_kernel_pass(reps)
    fp8_record(w, steps=reps, warmup=0)
    print(json.dumps({"fp8_pmc_pass": w.name, "copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "reps": reps,
                      "kernel_src_sha256_16": kernel_src_hash(FP8_SRCS)}), flush=True)


def pmc_pass(w, reps: int):
    """Kernels for the rocprofv3 counter runs: a plain copy of known size, then the workload kernel."""
    import torch

    n = _copy_kernel_pass(reps)
    q, k, v, o, lse, lens = _device_inputs(w)
    call = _caller(w, q, k, v, o, lse, lens, torch.cuda.current_stream().cuda_stream)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": w.name, "copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "reps": reps,
                      "kernel_src_sha256_16": kernel_src_hash()}), flush=True)


def summarize(d: str):
    """Summarise rocprofv3 CSV output under d: kernel stats and per-kernel counter means."""
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.setdefault("kernel_stats", []).append(
                    {"name": r.get("Name"), "calls": int(r.get("Calls", 0)),
                     "avg_us": float(r.get("AverageNs", 0)) / 1e3, "min_us": float(r.get("MinNs", 0)) / 1e3,
                     "max_us": float(r.get("MaxNs", 0)) / 1e3, "pct": float(r.get("Percentage", 0))})
    counters = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r.get("Kernel_Name"), r.get("Counter_Name"))
                counters.setdefault(key, {})
                did = r.get("Dispatch_Id")
                counters[key][did] = counters[key].get(did, 0.0) + float(r.get("Counter_Value", 0))
    if counters:
        out["counters"] = [{"kernel": k[0], "counter": k[1], "dispatches": len(v),
                            "mean_per_dispatch": statistics.fmean(v.values())} for k, v in sorted(counters.items())]
    print(json.dumps(out, indent=1))


def _timed_avg_us(trace_dir, name, cmd):
    """Mean duration (us) of the last K dispatches of kernel `name` in a --kernel-trace run of `cmd` (K = its
    --steps): the leg's timed steps, which follow its settle phase and warm-up. None without a per-dispatch trace."""
    m = re.search(r"--steps (\d+)", cmd)
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not m or not files:
        return None
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Kernel_Name"] == name]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    tail = rows[-int(m.group(1)):]
    if not tail:
        return None
    return statistics.fmean((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tail)


def _stats(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counters(d):
    """{(kernel substring match later), counter} -> list of per-dispatch values (summed over dimensions)."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (kname, cname, _), val in per.items():
        out.setdefault((kname, cname), []).append(val)
    return out


def _pick(counters, cname, needle):
    vals = [v for (k, c), v in counters.items() if c == cname and needle in k]
    if not vals:
        raise RuntimeError(f"no {cname} values for kernels matching {needle!r}")
    return statistics.fmean(vals[0])


def write_profiles(w):
    """Summaries of the PROFILE_COMMANDS outputs: profiles/<workload>_rocprof.md and ..._hbm_traffic.txt."""
    dirs = {k: f"gpurun_out/prof_{w.name}_{k}" for k in PROFILE_COMMANDS}
    kname = kernel_name(w).split("<")[0]
    trace = [r for r in _stats(dirs["trace"]) if kname in r["Name"]]
    if not trace:
        raise RuntimeError("no kernel statistics for the attention kernel")
    t = trace[0]
    avg_all = float(t["AverageNs"]) / 1e3
    avg_us = _timed_avg_us(dirs["trace"], t["Name"], PROFILE_COMMANDS["trace"]) or avg_all
    sq_us = _timed_avg_us(dirs["sq"], t["Name"], "--steps 1000000") or avg_us  # every dispatch of the counter run
    fetch, write = _counters(dirs["fetch"]), _counters(dirs["write"])
    copy = "neg_kernel"
    copy_read_kib = _pick(fetch, "FETCH_SIZE", copy)
    copy_write_kib = _pick(write, "WRITE_SIZE", copy)
    known_kib = 2 * (1 << 28) / 1024  # bytes read (and written) by the copy, in KiB
    f_fetch = known_kib / copy_read_kib
    f_write = known_kib / copy_write_kib
    k_read = _pick(fetch, "FETCH_SIZE", kname) * f_fetch * 1024
    k_write = _pick(write, "WRITE_SIZE", kname) * f_write * 1024
    sq = _counters(dirs["sq"])
    mfma_busy = _pick(sq, "SQ_VALU_MFMA_BUSY_CYCLES", kname)
    mops = _pick(sq, "SQ_INSTS_VALU_MFMA_MOPS_BF16", kname)
    conflict = _pick(sq, "SQ_LDS_BANK_CONFLICT", kname)
    lds_active = _pick(sq, "SQ_LDS_IDX_ACTIVE", kname)
    gui = _pick(sq, "GRBM_GUI_ACTIVE", kname)
    n_simd = 256 * 4
    util = mfma_busy / n_simd / (avg_us * 1e-6 * 2.4e9)
    traffic = {"kernel": kernel_name(w), "workload": w.name, "kernel_src_sha256_16": kernel_src_hash(),
               "hbm_bytes_per_launch": round(k_read + k_write), "read_bytes": round(k_read),
               "write_bytes": round(k_write), "algorithmic_bytes": w.algorithmic_bytes,
               "fetch_scale": round(f_fetch, 5), "write_scale": round(f_write, 5)}
    PROFILES.mkdir(exist_ok=True)
    (PROFILES / f"{w.name}_hbm_traffic.txt").write_text(json.dumps(traffic, indent=1) + "\n")
    cmds = "\n".join(f"    {PROFILE_COMMANDS[k].format(w=w.name)}" for k in PROFILE_COMMANDS)
    md = f"""# rocprofv3 summary: {kernel_name(w)} on {w.name}

Kernel code sha256[:16] (comments and layout excluded): `{kernel_src_hash()}` (exact_attention_13_amd/csrc/fa_fwd_kernel.hip and fa_gfx950.h).
Workload: B={w.B} H={w.H} H_kv={w.Hk} N={w.N} d={w.d} causal={w.causal} {w.dtype}{f' kv_len={list(w.kv_len)}' if w.kv_len else ''};
{w.flops:.4g} FLOP per launch (4*d*H per visible query-key pair, causal triangles counted as N^2/2),
{w.algorithmic_bytes} algorithmic HBM bytes per launch.

Commands (run from the repository root; outputs under gpurun_out/, summarised by `python bench.py --workload {w.name} --write-profiles`):

{cmds}

## Kernel trace (--kernel-trace --stats)

| kernel | calls | avg us, all calls | avg us, timed steps | min us | max us |
|---|---|---|---|---|---|
| {t['Name'][:90]} | {t['Calls']} | {avg_all:.1f} | {avg_us:.1f} | {float(t['MinNs']) / 1e3:.1f} | {float(t['MaxNs']) / 1e3:.1f} |

"Timed steps": the last --steps dispatches of the run, after its settle phase and warm-up (what bench.py's HIP-event
mean covers); the figures below use that average.

Attention TFLOP/s at the timed-step average: {w.flops / (avg_us * 1e-6) / 1e12:.1f}
({100 * w.flops / (avg_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of {PEAK_BF16_TFLOPS} dense bf16).

## HBM traffic (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)

Calibration: the copy kernel (torch.neg over 2^28 bf16) reads and writes {known_kib:.0f} KiB;
FETCH_SIZE reads {copy_read_kib:.1f} KiB (scale {f_fetch:.4f}), WRITE_SIZE reads {copy_write_kib:.1f} KiB (scale {f_write:.4f}).

| | counter KiB | scaled bytes | algorithmic bytes |
|---|---|---|---|
| read | {k_read / f_fetch / 1024:.1f} | {k_read:.0f} | {(w.B * w.H * w.N + 2 * w.kv_rows) * w.d * w.elt_bytes} (q, k, v) |
| write | {k_write / f_write / 1024:.1f} | {k_write:.0f} | {w.B * w.H * w.N * (w.d * w.elt_bytes + 4)} (o, lse) |

HBM bandwidth at the timed-step average: {(k_read + k_write) / (avg_us * 1e-6) / 1e9:.0f} GB/s.

## Matrix cores and LDS (SQ counters, per dispatch)

| counter | value |
|---|---|
| SQ_VALU_MFMA_BUSY_CYCLES | {mfma_busy:.4g} |
| SQ_INSTS_VALU_MFMA_MOPS_BF16 (x512 FLOP) | {mops:.4g} (= {mops * 512:.4g} FLOP) |
| SQ_INSTS_VALU | {_pick(sq, 'SQ_INSTS_VALU', kname):.4g} |
| SQ_INSTS_MFMA | {_pick(sq, 'SQ_INSTS_MFMA', kname):.4g} |
| SQ_LDS_BANK_CONFLICT | {conflict:.4g} |
| SQ_LDS_IDX_ACTIVE | {lds_active:.4g} |
| SQ_WAIT_INST_LDS | {_pick(sq, 'SQ_WAIT_INST_LDS', kname):.4g} |
| SQ_WAVE_CYCLES | {_pick(sq, 'SQ_WAVE_CYCLES', kname):.4g} |
| GRBM_GUI_ACTIVE | {gui:.4g} |

MFMA utilisation = MFMA busy cycles / 1024 SIMDs / (timed-step average x 2.4 GHz) = {100 * util:.1f} %;
over GRBM_GUI_ACTIVE / 8 (the GPU cycles counted during the kernel, summed over the 8 XCDs) = {100 * mfma_busy / n_simd / (gui / 8):.1f} %.
Clock during the kernel in the counter run, GRBM_GUI_ACTIVE / 8 / that run's kernel time ({sq_us:.1f} us; the
counter runs launch each dispatch on its own, after a pause, so this is not the settled clock): {gui / 8 / (sq_us * 1e-6) / 1e9:.2f} GHz.{
    "" if gui / 8 / (sq_us * 1e-6) <= 2.45e9 else " Above the 2.4 GHz maximum: for a launch this short GRBM_GUI_ACTIVE"
    " counts more than the kernel's own cycles (the counter run's dispatch and drain), so the shares over"
    " GRBM_GUI_ACTIVE and over SIMD-cycles below understate it; the 2.4 GHz-based utilisation is the one to read."}
LDS bank-conflict cycles / LDS active cycles = {100 * conflict / max(lds_active, 1):.1f} %.
""" + _cycle_breakdown(w, dirs, kname, avg_us)
    (PROFILES / f"{w.name}_rocprof.md").write_text(md)
    print(md)


def _cycle_breakdown(w, dirs, kname, avg_us):
    """Where the wave-cycles of the kernel go (the "stall" and "l2" passes), as markdown; empty if not run."""
    if not (glob.glob(os.path.join(dirs["stall"], "**", "*counter_collection.csv"), recursive=True) and
            glob.glob(os.path.join(dirs["l2"], "**", "*counter_collection.csv"), recursive=True)):
        return ""
    st, l2 = _counters(dirs["stall"]), _counters(dirs["l2"])
    g = lambda c, src=st: _pick(src, c, kname)  # noqa: E731
    wave_cyc = 4 * g("SQ_WAVE_CYCLES")          # quad-cycles, summed over waves
    wait_any, wait_inst = 4 * g("SQ_WAIT_ANY"), 4 * g("SQ_WAIT_INST_ANY")
    act_any, act_valu, act_lds = 4 * g("SQ_ACTIVE_INST_ANY"), 4 * g("SQ_ACTIVE_INST_VALU"), 4 * g("SQ_ACTIVE_INST_LDS")
    coexec = g("SQ_VALU_MFMA_COEXEC_CYCLES")
    busy = g("SQ_VALU_MFMA_BUSY_CYCLES", l2)
    gui = g("GRBM_GUI_ACTIVE", l2)
    hit, miss = g("TCC_HIT_sum", l2), g("TCC_MISS_sum", l2)
    valu2 = 4 * g("SQ_ACTIVE_INST_VALU2", l2)
    trans = g("SQ_INSTS_VALU_TRANS_F32", l2)
    fifo = g("SQ_LDS_DATA_FIFO_FULL", l2)
    simd_cyc = gui / 8 * 1024   # SIMD-cycles during the kernel (GPU cycles per XCD x 1024 SIMDs)
    rows = [("SQ_WAVE_CYCLES x4 (wave-cycles)", wave_cyc, ""),
            ("SQ_WAIT_ANY x4", wait_any, f"{100 * wait_any / wave_cyc:.1f} % of wave-cycles waiting (s_waitcnt, barrier)"),
            ("SQ_WAIT_INST_ANY x4", wait_inst, f"{100 * wait_inst / wave_cyc:.1f} % of wave-cycles waiting to issue"),
            ("SQ_ACTIVE_INST_ANY x4", act_any, f"{100 * act_any / wave_cyc:.1f} % of wave-cycles issuing"),
            ("SQ_ACTIVE_INST_VALU x4", act_valu, f"{100 * act_valu / wave_cyc:.1f} % of wave-cycles on vector/matrix instructions"),
            ("SQ_ACTIVE_INST_LDS x4", act_lds, f"{100 * act_lds / wave_cyc:.1f} % of wave-cycles on LDS instructions"),
            ("SQ_VALU_MFMA_BUSY_CYCLES", busy, f"{100 * busy / simd_cyc:.1f} % of SIMD-cycles"),
            ("SQ_VALU_MFMA_COEXEC_CYCLES", coexec, f"{100 * coexec / busy:.1f} % of the matrix-busy cycles also issue a vector instruction"),
            ("SQ_ACTIVE_INST_VALU2 x4", valu2, f"{100 * valu2 / simd_cyc:.1f} % of SIMD-cycles issue two vector instructions"),
            ("SQ_INSTS_VALU_TRANS_F32", trans, "transcendental (exp2, log, rcp) instructions"),
            ("SQ_LDS_DATA_FIFO_FULL", fifo, f"{100 * fifo / (gui / 8 * 256):.2f} % of CU-cycles with the LDS data queue full"),
            ("TCC_HIT_sum / TCC_MISS_sum", f"{hit:.4g} / {miss:.4g}", f"L2 hit rate {100 * hit / max(hit + miss, 1):.1f} %")]
    body = "\n".join(f"| {n} | {v if isinstance(v, str) else f'{v:.4g}'} | {d} |" for n, v, d in rows)
    return f"""
## Where the cycles go (SQ and TCC counters, per dispatch)

Wave-cycles are summed over every wave (two waves share each SIMD); SIMD-cycles = GRBM_GUI_ACTIVE / 8 x 1024 SIMDs.

| counter | value | share |
|---|---|---|
{body}
"""


def write_profiles_fp8(w):
    """Summary of the FP8_PROFILE_COMMANDS outputs: profiles/fp8_<workload>_rocprof.md and ..._hbm_traffic.txt."""
    dirs = {k: f"gpurun_out/prof_fp8_{w.name}_{k}" for k in FP8_PROFILE_COMMANDS}
    kname = "fa_fwd_fp8_kernel"
    trace = [r for r in _stats(dirs["trace"]) if kname in r["Name"]]
    if not trace:
        raise RuntimeError("no kernel statistics for the fp8 attention kernel")
    t = trace[0]
    avg_all = float(t["AverageNs"]) / 1e3
    avg_us = _timed_avg_us(dirs["trace"], t["Name"], FP8_PROFILE_COMMANDS["trace"]) or avg_all
    fetch, write, sq = _counters(dirs["fetch"]), _counters(dirs["write"]), _counters(dirs["sq"])
    known_kib = 2 * (1 << 28) / 1024
    copy_read_kib = _pick(fetch, "FETCH_SIZE", "neg_kernel")
    copy_write_kib = _pick(write, "WRITE_SIZE", "neg_kernel")
    f_fetch, f_write = known_kib / copy_read_kib, known_kib / copy_write_kib
    k_read = _pick(fetch, "FETCH_SIZE", kname) * f_fetch * 1024
    k_write = _pick(write, "WRITE_SIZE", kname) * f_write * 1024
    busy = _pick(sq, "SQ_VALU_MFMA_BUSY_CYCLES", kname)
    gui = _pick(sq, "GRBM_GUI_ACTIVE", kname)
    conflict = _pick(sq, "SQ_LDS_BANK_CONFLICT", kname)
    lds_active = _pick(sq, "SQ_LDS_IDX_ACTIVE", kname)
    n_simd = 256 * 4
    alg_read = (w.B * w.H * w.N + 2 * w.kv_rows) * w.d  # q, k, v: one byte per element
    alg_write = w.B * w.H * w.N * (2 * w.d + 4)         # o in bf16, lse in fp32
    tf = w.flops / (avg_us * 1e-6) / 1e12
    traffic = {"kernel": t["Name"][:120], "workload": w.name.replace("_bf16_", "_fp8_"),
               "kernel_src_sha256_16": kernel_src_hash(FP8_SRCS), "hbm_bytes_per_launch": round(k_read + k_write),
               "read_bytes": round(k_read), "write_bytes": round(k_write),
               "algorithmic_bytes": alg_read + alg_write, "fetch_scale": round(f_fetch, 5),
               "write_scale": round(f_write, 5)}
    PROFILES.mkdir(exist_ok=True)
    (PROFILES / f"fp8_{w.name}_hbm_traffic.txt").write_text(json.dumps(traffic, indent=1) + "\n")
    cmds = "\n".join(f"    {FP8_PROFILE_COMMANDS[k].format(w=w.name)}" for k in FP8_PROFILE_COMMANDS)
    md = f"""# rocprofv3 summary: fa_fwd_fp8_kernel on {w.name.replace('_bf16_', '_fp8_')}

Kernel code sha256[:16] (comments and layout excluded): `{kernel_src_hash(FP8_SRCS)}` (exact_attention_13_amd/csrc/fa_fwd_fp8_kernel.hip and fa_gfx950.h).
Workload: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}; q, k, v quantized per tensor to float8_e4m3fn from the
seeded bf16-shaped inputs (v passed transposed), o in bf16, lse in fp32;
{w.flops:.4g} FLOP per launch (4*d*H per visible query-key pair, causal triangles counted as N^2/2),
{alg_read + alg_write} algorithmic HBM bytes per launch.

Commands (run from the repository root; outputs under gpurun_out/, summarised by
`python bench.py --workload {w.name} --write-profiles-fp8`):

{cmds}

## Kernel trace (--kernel-trace --stats)

| kernel | calls | avg us, all calls | avg us, timed steps | min us | max us |
|---|---|---|---|---|---|
| {t['Name'][:90]} | {t['Calls']} | {avg_all:.1f} | {avg_us:.1f} | {float(t['MinNs']) / 1e3:.1f} | {float(t['MaxNs']) / 1e3:.1f} |

"Timed steps": the last --steps dispatches of the run, after its settle phase and warm-up (what bench.py's HIP-event
mean covers); the figures below use that average.

Attention TFLOP/s at the timed-step average: {tf:.1f} ({100 * tf / PEAK_FP8_TFLOPS:.1f} % of {PEAK_FP8_TFLOPS} dense fp8,
{100 * tf / PEAK_BF16_TFLOPS:.1f} % of {PEAK_BF16_TFLOPS} dense bf16).

## HBM traffic (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)

Calibration: the copy kernel (torch.neg over 2^28 bf16) reads and writes {known_kib:.0f} KiB;
FETCH_SIZE reads {copy_read_kib:.1f} KiB (scale {f_fetch:.4f}), WRITE_SIZE reads {copy_write_kib:.1f} KiB (scale {f_write:.4f}).

| | counter KiB | scaled bytes | algorithmic bytes |
|---|---|---|---|
| read | {k_read / f_fetch / 1024:.1f} | {k_read:.0f} | {alg_read} (q, k, v) |
| write | {k_write / f_write / 1024:.1f} | {k_write:.0f} | {alg_write} (o, lse) |

## Matrix cores and LDS (SQ counters, per dispatch)

| counter | value |
|---|---|
| SQ_VALU_MFMA_BUSY_CYCLES | {busy:.4g} |
| SQ_INSTS_VALU | {_pick(sq, 'SQ_INSTS_VALU', kname):.4g} |
| SQ_INSTS_MFMA | {_pick(sq, 'SQ_INSTS_MFMA', kname):.4g} |
| SQ_LDS_BANK_CONFLICT | {conflict:.4g} |
| SQ_LDS_IDX_ACTIVE | {lds_active:.4g} |
| SQ_WAIT_INST_LDS | {_pick(sq, 'SQ_WAIT_INST_LDS', kname):.4g} |
| SQ_WAVE_CYCLES | {_pick(sq, 'SQ_WAVE_CYCLES', kname):.4g} |
| GRBM_GUI_ACTIVE | {gui:.4g} |

MFMA busy = busy cycles / 1024 SIMDs over the timed-step average at 2.4 GHz: {100 * busy / n_simd / (avg_us * 1e-6 * 2.4e9):.1f} %;
over GRBM_GUI_ACTIVE / 8 (the clock measured during the kernel): {100 * busy / n_simd / (gui / 8):.1f} %.
LDS bank-conflict cycles / LDS active cycles = {100 * conflict / max(lds_active, 1):.1f} %.
"""
    (PROFILES / f"fp8_{w.name}_rocprof.md").write_text(md)
    print(md)


def write_profiles_varlen(w):
    """Summary of VARLEN_PROFILE_COMMAND's output: profiles/<packed workload>_rocprof.md."""
    trace = [r for r in _stats(f"gpurun_out/prof_{w.name}_trace") if "fa_fwd_bf16_kernel" in r["Name"]]
    if not trace:
        raise RuntimeError("no kernel statistics for the attention kernel")
    t = trace[0]
    avg_all = float(t["AverageNs"]) / 1e3
    avg_us = _timed_avg_us(f"gpurun_out/prof_{w.name}_trace", t["Name"], VARLEN_PROFILE_COMMAND) or avg_all
    tf = w.flops / (avg_us * 1e-6) / 1e12
    md = f"""# rocprofv3 summary: fa_fwd_varlen on {w.name}

Kernel code sha256[:16] (comments and layout excluded): `{kernel_src_hash()}` (exact_attention_13_amd/csrc/fa_fwd_kernel.hip and fa_gfx950.h).
Workload: {w.B} packed sequences of lengths {list(w.lens)} (total {w.T} tokens), H={w.H} H_kv={w.Hk} d={w.d}
causal={w.causal} bf16; {w.flops:.4g} FLOP per launch (4*H*d per visible query-key pair of every sequence, causal
triangles counted as L^2/2), {w.algorithmic_bytes} algorithmic HBM bytes per launch.

Command (run from the repository root; summarised by `python bench.py --write-profiles-varlen {w.name}`):

    {VARLEN_PROFILE_COMMAND.format(w=w.name)}

| kernel | calls | avg us, all calls | avg us, timed steps | min us | max us |
|---|---|---|---|---|---|
| {t['Name'][:100]} | {t['Calls']} | {avg_all:.1f} | {avg_us:.1f} | {float(t['MinNs']) / 1e3:.1f} | {float(t['MaxNs']) / 1e3:.1f} |

"Timed steps": the last --steps dispatches of the run, after its settle phase and warm-up (what bench.py's HIP-event
mean covers); the figures below use that average.

Attention TFLOP/s at the timed-step average: {tf:.1f} ({100 * tf / PEAK_BF16_TFLOPS:.1f} % of {PEAK_BF16_TFLOPS} dense bf16).
"""
    PROFILES.mkdir(exist_ok=True)
    (PROFILES / f"{w.name}_rocprof.md").write_text(md)
    print(md)


def write_profiles_bwd(w):
    """Summary of the BWD_PROFILE_COMMANDS outputs: profiles/bwd_<workload>_rocprof.md (the gradient kernels)."""
    dirs = {k: f"gpurun_out/prof_bwd_{w.name}_{k}" for k in BWD_PROFILE_COMMANDS}
    stats = _stats(dirs["trace"])
    fetch, write, sq = _counters(dirs["fetch"]), _counters(dirs["write"]), _counters(dirs["sq"])
    copy = "neg_kernel"
    known_kib = 2 * (1 << 28) / 1024
    f_fetch = known_kib / _pick(fetch, "FETCH_SIZE", copy)
    f_write = known_kib / _pick(write, "WRITE_SIZE", copy)
    n_simd = 256 * 4
    rows, total_us = [], 0.0
    # the reduction kernel runs only where the dk/dv kernel splits a group's query heads
    for kname in ("fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel", "fa_bwd_reduce_kernel"):
        t = [r for r in stats if kname in r["Name"]]
        if not t and kname == "fa_bwd_reduce_kernel":
            continue
        if not t:
            raise RuntimeError(f"no kernel statistics for {kname}")
        avg_us = (_timed_avg_us(dirs["trace"], t[0]["Name"], BWD_PROFILE_COMMANDS["trace"])
                  or float(t[0]["AverageNs"]) / 1e3)
        total_us += avg_us
        busy = _pick(sq, "SQ_VALU_MFMA_BUSY_CYCLES", kname)
        gui = _pick(sq, "GRBM_GUI_ACTIVE", kname)
        rows.append({"kernel": kname, "calls": t[0]["Calls"], "avg_us": avg_us,
                     "read": _pick(fetch, "FETCH_SIZE", kname) * f_fetch * 1024,
                     "write": _pick(write, "WRITE_SIZE", kname) * f_write * 1024,
                     "mfma_insts": _pick(sq, "SQ_INSTS_MFMA", kname), "mfma_busy": busy,
                     "util_spec": busy / n_simd / (avg_us * 1e-6 * 2.4e9),
                     "util_clock": busy / n_simd / (gui / 8),
                     "valu": _pick(sq, "SQ_INSTS_VALU", kname),
                     "lds_conflict": _pick(sq, "SQ_LDS_BANK_CONFLICT", kname),
                     "lds_active": _pick(sq, "SQ_LDS_IDX_ACTIVE", kname)})
    flops = 2.5 * w.flops
    cmds = "\n".join(f"    {BWD_PROFILE_COMMANDS[k].format(w=w.name)}" for k in BWD_PROFILE_COMMANDS)
    kb = w.B * w.Hk * w.N * w.d * 2
    qb = w.B * w.H * w.N * w.d * 2
    alg_read = 3 * qb + 2 * kb + 4 * w.B * w.H * w.N  # q, o, dout, k, v, lse
    alg_write = qb + 2 * kb                          # dq, dk, dv (the workspace pairs are extra)
    table = "\n".join(
        f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.1f} | {r['read']:.4g} | {r['write']:.4g} | "
        f"{r['mfma_insts']:.4g} | {100 * r['util_spec']:.1f} % | {100 * r['util_clock']:.1f} % | {r['valu']:.4g} | "
        f"{r['lds_conflict']:.4g} |" for r in rows)
    md = f"""# rocprofv3 summary: gradient call (fa_bwd) on {w.name}

Kernel code sha256[:16] (comments and layout excluded): `{kernel_src_hash(BWD_SRCS)}` (exact_attention_13_amd/csrc/fa_bwd_kernel.hip and fa_gfx950.h).
Workload: B={w.B} H={w.H} H_kv={w.Hk} N={w.N} d={w.d} causal={w.causal} bf16; {flops:.4g} FLOP per call in the usual
convention (2.5 x the forward's 4*B*H*N^2*d{', halved' if w.causal else ''}: five matrix products); the kernels
execute seven (S and dP are formed in both), {7 / 5 * flops:.4g} FLOP of MFMA work.

Commands (run from the repository root; outputs under gpurun_out/, summarised by
`python bench.py --workload {w.name} --write-profiles-bwd`):

{cmds}

| kernel | calls | avg us | HBM read B | HBM write B | MFMA insts | MFMA busy (2.4 GHz) | MFMA busy (measured clock) | VALU insts | LDS bank conflicts |
|---|---|---|---|---|---|---|---|---|---|
{table}

Gradient call at the timed-step averages: {total_us:.1f} us, {flops / (total_us * 1e-6) / 1e12:.1f} TFLOP/s
({100 * flops / (total_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of {PEAK_BF16_TFLOPS} dense bf16).
Algorithmic HBM bytes per call: read {alg_read} (q, o, dout, lse, k, v), write {alg_write} (dq, dk, dv).
FETCH_SIZE x {f_fetch:.4f} and WRITE_SIZE x {f_write:.4f} (calibrated on a copy of 2^28 bf16).
MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over the timed-step average at 2.4 GHz, and over GRBM_GUI_ACTIVE / 8
(the clock actually measured during the kernel).
"""
    PROFILES.mkdir(exist_ok=True)
    (PROFILES / f"bwd_{w.name}_rocprof.md").write_text(md)
    print(md)


def headline_line(w, steps: int, warmup: int, settle_s: float, wall: float, region_ms: float, durs, cold_wall: float,
                  cold_durs) -> dict:
    """The headline JSON line from the timed region (wall seconds and the event time of `steps` back-to-back calls),
    the per-call durations of the pass before it, and the cold leg; the legs added later (probe, other workloads,
    gradients, fp8, packed batches, CPU baseline) extend it."""
    ms_step = wall / steps * 1e3
    value = w.flops * steps / wall / 1e12
    k_mean = region_ms / steps  # average launch duration over the timed region (HIP events, launch stream)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = w.flops / (k_mean * 1e-3) / 1e12
    return {
        "metric": "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak (B,H,N,d,causal)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) q, k, v; no dataset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.Hk, "N": w.N, "d": w.d, "causal": w.causal,
                   "kv_len": list(w.kv_len) or None, "scale": w.scale, "input_dtype": w.dtype,
                   "accumulate": "fp32"},
        "pct_of_peak": round(100 * value / peak, 2),
        "kernel_ms": {"mean": round(k_mean, 4), "per_call_mean": round(statistics.fmean(durs), 4),
                      "median": round(statistics.median(durs), 4), "min": round(min(durs), 4),
                      "p90": round(sorted(durs)[int(0.9 * (len(durs) - 1))], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic_from_profiles(w),
                     "kernel": kernel_name(w), "flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes,
                     # the memory side of the same launch: algorithmic bytes over the kernel time, against HBM
                     "hbm_gbs": round(w.algorithmic_bytes / (k_mean * 1e-3) / 1e9, 1),
                     "hbm_frac": round(w.algorithmic_bytes / (k_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "kernel_src_sha256_16": kernel_src_hash(),
        "settle_s": settle_s,
        "cold_start": {"value": round(w.flops * steps / cold_wall / 1e12, 2),
                       "ms_per_step": round(cold_wall / steps * 1e3, 4),
                       "kernel_ms_mean": round(statistics.fmean(cold_durs), 4)},
    }


def main():
    import attn_inputs as ai

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(ai.WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows in the oracle's CPU sample (0: every row of the workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--write-profiles", action="store_true")
    ap.add_argument("--bwd-only", action="store_true")
    ap.add_argument("--bwd-pmc-pass", action="store_true")
    ap.add_argument("--write-profiles-bwd", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--fp8-only", action="store_true", help="time only fa_fwd_fp8 on --workload's shape")
    ap.add_argument("--fp8-pmc-pass", action="store_true")
    ap.add_argument("--varlen-only", metavar="WORKLOAD", choices=sorted(ai.VARLEN_WORKLOADS),
                    help="time only fa_fwd_varlen on a packed workload")
    ap.add_argument("--write-profiles-varlen", metavar="WORKLOAD", choices=sorted(ai.VARLEN_WORKLOADS))
    ap.add_argument("--write-profiles-fp8", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true")
    ap.add_argument("--issue-probe", action="store_true",
                    help="matrix cores against exp2/FMA work, in one wave or split over a SIMD's two waves")
    ap.add_argument("--atomic-probe", action="store_true",
                    help="fp32 atomic-add rate into device memory (64 KiB tiles) against plain stores")
    ap.add_argument("--clock-settle", action="store_true",
                    help="per-launch times of --workload after 2 s idle (300 launches, twice)")
    ap.add_argument("--settle", type=float, default=SETTLE_S, metavar="SECONDS",
                    help="untimed back-to-back calls before each leg's warm-up (0: time the leg as it comes)")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return 0
    if args.write_profiles:
        write_profiles(ai.WORKLOADS[args.workload])
        return 0
    if args.write_profiles_bwd:
        write_profiles_bwd(ai.WORKLOADS[args.workload])
        return 0
    if args.write_profiles_varlen:
        write_profiles_varlen(ai.VARLEN_WORKLOADS[args.write_profiles_varlen])
        return 0
    if args.write_profiles_fp8:
        write_profiles_fp8(ai.WORKLOADS[args.workload])
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); the attention "
              "forward shards over heads with no communication, so a multi-GPU figure is not measured here.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import exact_attention_13_amd  # noqa: F401  (fails loudly if libfa.so is missing)

    w = ai.WORKLOADS[args.workload]
    if args.pmc_pass:
        pmc_pass(w, reps=5)
        return 0
    if args.varlen_only:
        print(json.dumps(varlen_record(ai.VARLEN_WORKLOADS[args.varlen_only], args.steps, args.warmup, args.settle)), flush=True)
        return 0
    if args.fp8_only:
        print(json.dumps(fp8_record(w, args.steps, args.warmup, args.settle)), flush=True)
        return 0
    if args.bwd_pmc_pass:
        bwd_pmc_pass(w, reps=3)
        return 0
    if args.fp8_pmc_pass:
        fp8_pmc_pass(w, reps=5)
        return 0
    if args.issue_probe:
        for rec in issue_mix_probe():
            print(json.dumps(rec), flush=True)
        return 0
    if args.atomic_probe:
        for rec in atomic_add_probe():
            print(json.dumps(rec), flush=True)
        return 0
    if args.clock_settle:
        for rec in clock_settle(w):
            print(json.dumps({"workload": w.name, **rec}), flush=True)
        return 0
    if args.bwd_only:
        print(json.dumps(backward_record(w, args.steps, args.warmup, args.settle)), flush=True)
        return 0

    # The headline leg is timed twice on the same shape: as it comes (the W warm-up steps straight after the host
    # has made the inputs, the GPU idle until then, each call between events), reported as "cold_start", and after
    # `--settle` seconds of untimed back-to-back calls (time_region: K calls between events for their spread, W
    # warm-up calls, then the K timed calls with one event pair around them), which gives `value` and the
    # roofline's average launch duration: the throughput of a GPU kept busy.
    cold_wall, _, cold_durs = time_workload(w, args.steps, args.warmup, region=False)
    wall, region_ms, durs = time_region(w, args.steps, args.warmup, args.settle)
    line = headline_line(w, args.steps, args.warmup, args.settle, wall, region_ms, durs, cold_wall, cold_durs)
    achieved = w.flops / (region_ms / args.steps * 1e-3) / 1e12
    if not args.no_mfma_probe:
        # the same kernel time against what this GPU's matrix cores sustain (data-sheet peak: 2516.6 at 2.4 GHz)
        probe = mfma_probe()
        line["mfma_probe"] = probe
        line["roofline"]["frac_of_probe"] = round(achieved / probe["tflops"], 4)
    if not args.no_other_workloads:
        others = {}
        for name, ow in ai.WORKLOADS.items():
            if name == w.name or ow.dtype != "bf16":
                continue
            _, om, _ = time_workload(ow, steps=20, warmup=3, settle_s=args.settle)
            others[name] = {"kernel_ms_mean": round(om, 4), "tflops": round(ow.flops / (om * 1e-3) / 1e12, 2),
                            "pct_of_peak": round(100 * ow.flops / (om * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        line["other_workloads"] = others
    if not args.no_backward:
        st = args.settle
        line["backward"] = [backward_record(ai.WORKLOADS[n], steps=20, warmup=3, settle_s=st) for n in BWD_WORKLOADS]
        line["fp8"] = [fp8_record(ai.WORKLOADS[n], steps=20, warmup=3, settle_s=st) for n in FP8_WORKLOADS]
        line["varlen"] = [varlen_record(vw, steps=20, warmup=3, settle_s=st) for vw in ai.VARLEN_WORKLOADS.values()]
        line["varlen_backward"] = [varlen_backward_record(vw, steps=10, warmup=2, settle_s=st)
                                   for vw in ai.VARLEN_WORKLOADS.values()]
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_rows)
        cb.pop("seconds")
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
