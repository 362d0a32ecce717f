"""The C-ABI library on the host: it loads, exports every symbol include/fa.h declares, and rejects bad
arguments before any HIP call (so these run without a GPU). No call here reaches a kernel launch."""
import re
import subprocess
from pathlib import Path

import pytest

import exact_attention_13_amd as fa
from exact_attention_13_amd import binding

HEADER = Path(__file__).resolve().parent.parent / "include" / "fa.h"
A = 0x10000  # 16-byte aligned fake device addresses, far apart so that nothing overlaps
B_ = 0x20000000


def _declared():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\s*\**\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert _declared() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for sym in _declared():
        assert sym in exported, sym
        assert hasattr(binding._lib, sym)


def test_probe_library_exports_what_its_header_declares():
    """libfa_probe.so (the matrix-core probe bench.py quotes the kernels against) is built beside libfa.so and
    exports every function include/fa_probe.h declares; its argument checks run without a GPU."""
    import ctypes
    header = HEADER.parent / "fa_probe.h"
    declared = sorted(set(re.findall(r"^(?:const\s+)?\w+\s*\**\s*(fa_probe_\w+)\s*\(", header.read_text(),
                                     flags=re.M)))
    assert declared == ["fa_probe_atomic_add", "fa_probe_atomic_tile_floats", "fa_probe_flop_per_wg_iter",
                        "fa_probe_issue_mix", "fa_probe_issue_mix_threads", "fa_probe_mfma_bf16", "fa_probe_threads"]
    path = Path(fa.library_path()).parent / "libfa_probe.so"
    out = subprocess.run(["nm", "-D", "--defined-only", str(path)], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert set(declared) <= exported
    lib = ctypes.CDLL(str(path))
    lib.fa_probe_flop_per_wg_iter.restype = ctypes.c_double
    assert lib.fa_probe_flop_per_wg_iter() == 4 * 8 * 2 * 32 * 32 * 16
    assert lib.fa_probe_threads() == 256
    f = lib.fa_probe_mfma_bf16
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert f(None, A, 1, 1, None) == 1 and f(A, None, 1, 1, None) == 1
    assert f(A, B_, 0, 1, None) == 2 and f(A, B_, 1, 0, None) == 2 and f(A, B_, (1 << 20) + 1, 1, None) == 2
    assert lib.fa_probe_issue_mix_threads() == 512
    g = lib.fa_probe_issue_mix
    g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert g(0, None, A, 1, 1, None) == 1 and g(0, A, None, 1, 1, None) == 1
    assert g(-1, A, B_, 1, 1, None) == 2 and g(5, A, B_, 1, 1, None) == 2
    assert g(0, A, B_, 0, 1, None) == 2 and g(0, A, B_, 1, 0, None) == 2
    assert lib.fa_probe_atomic_tile_floats() == 16384
    h = lib.fa_probe_atomic_add
    h.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert h(0, None, 8, 1, 1, None) == 1
    assert h(-1, A, 8, 1, 1, None) == 2 and h(4, A, 8, 1, 1, None) == 2
    assert h(1, A, 0, 1, 1, None) == 2 and h(1, A, 12, 1, 1, None) == 2 and h(1, A, 1 << 17, 1, 1, None) == 2
    assert h(0, A, 8, 0, 1, None) == 2 and h(0, A, 8, 1, 0, None) == 2


def test_version_and_strerror():
    assert fa.fa_version() == 10700
    for code in range(9):
        assert isinstance(fa.fa_strerror(code), str) and fa.fa_strerror(code)
    assert fa.fa_strerror(99) == "unknown error code"


def test_noalloc_gradient_refuses_problems_beyond_its_scratch_buffer():
    """fa_bwd_noalloc checks everything fa_bwd checks, then that the workspace fits the library's 64 MiB buffer,
    all before any HIP call."""
    args = (A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000, B_, B_ + 0x10000000,
            B_ + 0x20000000)
    assert fa.fa_bwd_workspace_bytes(1, 32, 1, 16384, 128) > 64 << 20  # one key/value head: split dk/dv partials
    assert fa.fa_bwd_noalloc(*args, 1, 32, 1, 16384, 128, 1, 0.088, 0) == fa.FA_ERR_SCRATCH
    assert "scratch" in fa.fa_strerror(fa.FA_ERR_SCRATCH)
    assert fa.fa_bwd_noalloc(*args[:6], 0, *args[7:], 1, 4, 4, 64, 64, 0, 0.125, 0) == fa.FA_ERR_NULL
    assert fa.fa_bwd_noalloc(*args, 1, 4, 4, 64, 96, 0, 0.125, 0) == fa.FA_ERR_HEADDIM
    assert fa.fa_bwd_noalloc(*args, 1, 4, 4, 64, 64, 0, 0.0, 0) == fa.FA_ERR_ARG
    assert fa.fa_bwd_noalloc(*args, 0, 4, 4, 64, 64, 0, 0.125, 0) == fa.FA_OK  # empty: nothing enqueued


def test_instance_query():
    """fa_fwd_instance names the kernel instance the bf16 forward launches, from the grid size alone: 256-row
    workgroups when they give the 256 CUs two each, else 128-row ones when those do, else the split-key shape."""
    assert fa.fa_fwd_instance(2, 16, 4096, 128, 0, 0) == "fa_fwd_bf16_kernel<128, false, 8, 2, 2, false, 1>"
    assert fa.fa_fwd_instance(1, 32, 16384, 128, 1, 0) == "fa_fwd_bf16_kernel<128, true, 8, 2, 2, false, 1>"
    assert fa.fa_fwd_instance(2, 32, 1000, 64, 1, 0) == "fa_fwd_bf16_kernel<64, true, 4, 2, 1, false, 1>"
    assert fa.fa_fwd_instance(4, 8, 1024, 64, 0, 0) == "fa_fwd_bf16_kernel<64, false, 8, 2, 2, false, 2>"
    assert fa.fa_fwd_instance(4, 32, 1000, 128, 0, 1) == "fa_fwd_bf16_kernel<128, false, 8, 2, 2, true, 1>"
    # the boundaries: 128 heads of 1024 rows (4 x 128 = 512 wide workgroups), 127 of them (8 x 127 narrow ones),
    # 63 (8 x 63 = 504 narrow ones: split)
    assert fa.fa_fwd_instance(1, 128, 1024, 64, 0, 0).endswith("8, 2, 2, false, 1>")
    assert fa.fa_fwd_instance(1, 127, 1024, 64, 0, 0).endswith("4, 2, 1, false, 1>")
    assert fa.fa_fwd_instance(1, 64, 1024, 64, 0, 0).endswith("4, 2, 1, false, 1>")
    assert fa.fa_fwd_instance(1, 63, 1024, 64, 0, 0).endswith("8, 2, 2, false, 2>")
    # causal d = 64 grids whose 64-row blocks fit two per CU (16 x 32 = 512): the 64-row split shape; not at d = 128,
    # not past 512 such blocks, not for packed batches
    assert fa.fa_fwd_instance(4, 8, 1024, 64, 1, 0) == "fa_fwd_bf16_kernel<64, true, 4, 2, 2, false, 2>"
    assert fa.fa_fwd_instance(4, 8, 1024, 128, 1, 0).endswith("8, 2, 2, false, 2>")
    assert fa.fa_fwd_instance(1, 33, 1024, 64, 1, 0).endswith("8, 2, 2, false, 2>")
    assert fa.fa_fwd_instance(4, 8, 1024, 64, 1, 1).endswith("8, 2, 2, true, 2>")
    for bad in ((0, 1, 64, 64, 0, 0), (1, 0, 64, 64, 0, 0), (1, 1, 0, 64, 0, 0), (1, 1, 64, 96, 0, 0),
                (1, 1, 64, 64, 2, 0), (1, 1, 64, 64, 0, 2), (70000, 1, 64, 64, 0, 0), (1, 1, (1 << 30) + 1, 64, 0, 0)):
        assert fa.fa_fwd_instance(*bad) is None, bad


LEN = A + 0x5000000  # fake device address of kv_len


def _gqa_same_heads(q, k, v, o, lse, B, H, N, d, causal, scale, stream):
    return fa.fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream)


def _kpad_same_heads(q, k, v, o, lse, B, H, N, d, causal, scale, stream):
    return fa.fa_fwd_kpad(q, k, v, o, lse, LEN, B, H, H, N, d, causal, scale, stream)


ENTRIES = [fa.fa_fwd, fa.fa_fwd_f32, _gqa_same_heads, _kpad_same_heads]


def _call(fn=None, q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000, B=1, H=2, N=64,
          d=64, causal=0, scale=0.125):
    fn = fn or fa.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, causal, scale, 0)


@pytest.mark.parametrize("fn", ENTRIES)
def test_error_codes(fn):
    assert _call(fn, q=0) == fa.FA_ERR_NULL
    assert _call(fn, lse=0) == fa.FA_ERR_NULL
    assert _call(fn, N=-1) == fa.FA_ERR_SHAPE
    assert _call(fn, B=-3) == fa.FA_ERR_SHAPE
    assert _call(fn, B=300, H=300) == fa.FA_ERR_SHAPE
    assert _call(fn, N=(1 << 30) + 1) == fa.FA_ERR_SHAPE
    for d in (0, 32, 96, 256):
        assert _call(fn, d=d) == fa.FA_ERR_HEADDIM
    for s in (0.0, -0.125, float("inf"), float("nan")):
        assert _call(fn, scale=s) == fa.FA_ERR_ARG
    assert _call(fn, causal=2) == fa.FA_ERR_ARG
    assert _call(fn, causal=-1) == fa.FA_ERR_ARG
    assert _call(fn, q=A + 8) == fa.FA_ERR_ALIGN
    assert _call(fn, o=A + 0x3000000 + 4) == fa.FA_ERR_ALIGN
    assert _call(fn, lse=A + 0x4000000 + 2) == fa.FA_ERR_ALIGN
    assert _call(fn, o=A) == fa.FA_ERR_ALIAS                     # o is q
    assert _call(fn, o=A + 0x2000000 + 64) == fa.FA_ERR_ALIAS     # o starts inside v
    assert _call(fn, lse=A + 0x1000000 + 16) == fa.FA_ERR_ALIAS  # lse inside k
    assert _call(fn, lse=A + 0x3000000 + 256) == fa.FA_ERR_ALIAS  # lse inside o


def test_grouped_heads_error_codes():
    def gqa(H=4, H_kv=2, o=A + 0x3000000, N=64, B=1):
        return fa.fa_fwd_gqa(A, A + 0x1000000, A + 0x2000000, o, A + 0x4000000, B, H, H_kv, N, 64, 0, 0.125, 0)
    assert gqa(H_kv=0) == fa.FA_ERR_SHAPE
    assert gqa(H_kv=-1) == fa.FA_ERR_SHAPE
    assert gqa(H_kv=3) == fa.FA_ERR_SHAPE     # 3 does not divide 4
    assert gqa(H_kv=8) == fa.FA_ERR_SHAPE     # more key/value heads than query heads
    # k holds H_kv = 1 head of 64 x 64 bf16 = 8192 bytes: o starting 8000 bytes into k overlaps it
    assert gqa(H_kv=1, o=A + 0x1000000 + 8000) == fa.FA_ERR_ALIAS
    assert gqa(H_kv=0, N=0) == fa.FA_OK       # empty problem: nothing to check the grouping against
    assert gqa(H_kv=-1, N=0) == fa.FA_ERR_SHAPE


def test_key_padding_error_codes():
    def kpad(kv_len=LEN, o=A + 0x3000000, lse=A + 0x4000000, N=64):
        return fa.fa_fwd_kpad(A, A + 0x1000000, A + 0x2000000, o, lse, kv_len, 2, 4, 2, N, 64, 1, 0.125, 0)
    assert kpad(kv_len=0) == fa.FA_ERR_NULL
    assert kpad(kv_len=LEN + 2) == fa.FA_ERR_ALIGN
    assert kpad(o=LEN - 64) == fa.FA_ERR_ALIAS       # o's last bytes cover kv_len
    assert kpad(lse=LEN + 4 - 4 * 2 * 4 * 64) == fa.FA_ERR_ALIAS  # lse ends on kv_len's first element
    assert kpad(kv_len=0, N=0) == fa.FA_OK           # empty problem ignores the pointers


@pytest.mark.parametrize("fn", ENTRIES)
def test_empty_problem_is_a_no_op_that_ignores_pointers(fn):
    assert _call(fn, q=0, k=0, v=0, o=0, lse=0, N=0) == fa.FA_OK
    assert _call(fn, q=0, k=0, v=0, o=0, lse=0, B=0) == fa.FA_OK
    assert _call(fn, q=0, k=0, v=0, o=0, lse=0, H=0, d=128, causal=1) == fa.FA_OK
    # scalar arguments are still checked on an empty problem
    assert _call(fn, N=0, d=80) == fa.FA_ERR_HEADDIM
    assert _call(fn, N=0, scale=0.0) == fa.FA_ERR_ARG


BWD = dict(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000, dout=A + 0x5000000,
           dq=A + 0x6000000, dk=A + 0x7000000, dv=A + 0x8000000, ws=A + 0x9000000)


def _bwd(B=1, H=2, H_kv=2, N=64, d=64, causal=0, scale=0.125, **ptrs):
    p = dict(BWD, **ptrs)
    return fa.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"], p["ws"], B, H,
                     H_kv, N, d, causal, scale, 0)


def test_backward_error_codes():
    for name in BWD:
        assert _bwd(**{name: 0}) == fa.FA_ERR_NULL, name
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv", "ws"):
        assert _bwd(**{name: BWD[name] + 8}) == fa.FA_ERR_ALIGN, name
    assert _bwd(lse=BWD["lse"] + 2) == fa.FA_ERR_ALIGN
    assert _bwd(d=96) == fa.FA_ERR_HEADDIM
    assert _bwd(H_kv=3) == fa.FA_ERR_SHAPE
    assert _bwd(N=-1) == fa.FA_ERR_SHAPE
    # the workspace planes are addressed with 32-bit byte offsets: 2^28 rows at most
    assert _bwd(N=(1 << 28) + 1) == fa.FA_ERR_SHAPE
    assert _bwd(scale=0.0) == fa.FA_ERR_ARG
    assert _bwd(causal=3) == fa.FA_ERR_ARG
    assert _bwd(dq=BWD["q"]) == fa.FA_ERR_ALIAS                  # dq is q
    assert _bwd(dk=BWD["dv"] + 4096) == fa.FA_ERR_ALIAS           # dk overlaps dv (16 KiB each)
    assert _bwd(ws=BWD["o"] + 1024) == fa.FA_ERR_ALIAS            # workspace inside o
    assert _bwd(dv=BWD["lse"] - 16) == fa.FA_ERR_ALIAS            # dv runs into lse
    assert _bwd(ws=BWD["dq"] - 16) == fa.FA_ERR_ALIAS             # workspace runs into dq
    # empty problem: success, pointers ignored
    assert _bwd(N=0, **{name: 0 for name in BWD}) == fa.FA_OK


def _bwd_kpad(B=1, H=2, H_kv=2, N=64, d=64, causal=0, scale=0.125, kv_len=A + 0xA000000, **ptrs):
    p = dict(BWD, **ptrs)
    return fa.fa_bwd_kpad(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"], p["ws"],
                          kv_len, B, H, H_kv, N, d, causal, scale, 0)


def test_backward_kpad_error_codes():
    for name in BWD:
        assert _bwd_kpad(**{name: 0}) == fa.FA_ERR_NULL, name
    assert _bwd_kpad(kv_len=0) == fa.FA_ERR_NULL
    assert _bwd_kpad(kv_len=A + 0xA000000 + 2) == fa.FA_ERR_ALIGN
    assert _bwd_kpad(dq=BWD["dq"] + 8) == fa.FA_ERR_ALIGN
    assert _bwd_kpad(kv_len=BWD["dk"] + 64) == fa.FA_ERR_ALIAS     # lengths inside dk
    assert _bwd_kpad(kv_len=BWD["ws"] + 16) == fa.FA_ERR_ALIAS     # lengths inside the workspace
    assert _bwd_kpad(H_kv=3) == fa.FA_ERR_SHAPE
    assert _bwd_kpad(N=(1 << 28) + 1) == fa.FA_ERR_SHAPE
    assert _bwd_kpad(d=80) == fa.FA_ERR_HEADDIM
    assert _bwd_kpad(causal=2) == fa.FA_ERR_ARG
    assert _bwd_kpad(N=0, kv_len=0, **{name: 0 for name in BWD}) == fa.FA_OK


def test_varlen_error_codes():
    def vl(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000, cu=A + 0x5000000, B=2, H=4,
           Hkv=2, total=100, max_seqlen=60, d=64, causal=0, scale=0.125):
        return fa.fa_fwd_varlen(q, k, v, o, lse, cu, B, H, Hkv, total, max_seqlen, d, causal, scale, 0)
    for name in ("q", "k", "v", "o", "lse", "cu"):
        assert vl(**{name: 0}) == fa.FA_ERR_NULL, name
    assert vl(cu=A + 0x5000000 + 2) == fa.FA_ERR_ALIGN
    assert vl(lse=A + 0x4000000 + 2) == fa.FA_ERR_ALIGN
    assert vl(o=A + 0x3000000 + 8) == fa.FA_ERR_ALIGN
    assert vl(max_seqlen=0) == fa.FA_ERR_SHAPE and vl(max_seqlen=101) == fa.FA_ERR_SHAPE
    assert vl(Hkv=3) == fa.FA_ERR_SHAPE and vl(total=-1) == fa.FA_ERR_SHAPE
    assert vl(d=96) == fa.FA_ERR_HEADDIM and vl(scale=float("nan")) == fa.FA_ERR_ARG
    assert vl(lse=A + 0x3000000 + 1024) == fa.FA_ERR_ALIAS        # lse inside o (100*4*64*2 bytes)
    assert vl(o=A + 0x5000000) == fa.FA_ERR_ALIAS and vl(lse=A + 0x4000000, cu=A + 0x4000000 + 64) == fa.FA_ERR_ALIAS
    assert vl(o=A + 0x1000000 + 16) == fa.FA_ERR_ALIAS            # o inside k
    assert vl(total=0, q=0, k=0, v=0, o=0, lse=0, cu=0) == fa.FA_OK  # no token: nothing to do
    assert vl(B=0, q=0, cu=0) == fa.FA_OK


def test_varlen_backward_error_codes():
    P = dict(q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000, dout=A + 0x5000000,
             dq=A + 0x6000000, dk=A + 0x7000000, dv=A + 0x8000000, ws=A + 0x9000000, cu=A + 0xA000000)

    def bv(B=2, H=4, Hkv=2, total=100, max_seqlen=60, d=64, causal=0, scale=0.125, **kw):
        p = dict(P, **kw)
        return fa.fa_bwd_varlen(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"],
                                p["ws"], p["cu"], B, H, Hkv, total, max_seqlen, d, causal, scale, 0)
    for name in P:
        assert bv(**{name: 0}) == fa.FA_ERR_NULL, name
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv", "ws"):
        assert bv(**{name: P[name] + 8}) == fa.FA_ERR_ALIGN, name
    assert bv(cu=P["cu"] + 2) == fa.FA_ERR_ALIGN and bv(lse=P["lse"] + 2) == fa.FA_ERR_ALIGN
    assert bv(max_seqlen=101) == fa.FA_ERR_SHAPE and bv(Hkv=3) == fa.FA_ERR_SHAPE
    assert bv(total=(1 << 28) + 5, max_seqlen=(1 << 28) + 1) == fa.FA_ERR_SHAPE
    assert bv(dq=P["q"]) == fa.FA_ERR_ALIAS and bv(ws=P["cu"] - 16) == fa.FA_ERR_ALIAS
    assert bv(dk=P["dv"] + 64) == fa.FA_ERR_ALIAS
    assert bv(total=0, **{name: 0 for name in P}) == fa.FA_OK


def test_fp8_error_codes():
    def f8(q=A, k=A + 0x1000000, vt=A + 0x2000000, o=A + 0x3000000, lse=A + 0x4000000, sq=0.01, sk=0.01, sv=0.01,
           B=1, H=2, N=64, d=64, causal=0, scale=0.125):
        return fa.fa_fwd_fp8(q, k, vt, o, lse, sq, sk, sv, B, H, N, d, causal, scale, 0)
    assert f8(N=70) == fa.FA_ERR_SHAPE                 # v^T rows must be 16-byte multiples
    assert f8(N=(1 << 24) + 16) == fa.FA_ERR_SHAPE
    assert f8(d=96) == fa.FA_ERR_HEADDIM
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert f8(sq=bad) == fa.FA_ERR_ARG and f8(sk=bad) == fa.FA_ERR_ARG and f8(sv=bad) == fa.FA_ERR_ARG
    assert f8(vt=0) == fa.FA_ERR_NULL
    assert f8(vt=A + 0x2000000 + 4) == fa.FA_ERR_ALIGN
    assert f8(o=A + 0x2000000 + 4096) == fa.FA_ERR_ALIAS    # o inside v^T (8 KiB of fp8)
    assert f8(lse=A + 0x3000000 + 1024) == fa.FA_ERR_ALIAS  # lse inside o (16 KiB of bf16)
    assert f8(N=0, q=0, k=0, vt=0, o=0, lse=0) == fa.FA_OK


def test_backward_workspace_bytes():
    ws = fa.fa_bwd_workspace_bytes
    # (D, lse*log2e) float pairs per query row, rows rounded up to 128 per head
    assert ws(2, 3, 3, 100, 64) == 2 * 3 * 128 * 8
    assert ws(1, 1, 1, 64, 128) == 128 * 8
    assert ws(1, 32, 32, 16384, 128) == 32 * 16384 * 8
    # grouped heads whose key/value heads already give 512 dk/dv workgroups (2 x 8 heads x 32 key blocks): no split
    assert ws(2, 32, 8, 4096, 128) == 2 * 32 * 4096 * 8
    # one key/value head of 16384 keys: 128 workgroups, so the 32 query heads split 4 ways (the smallest divisor
    # reaching 512), each way with fp32 partial dk and dv of every key row
    assert ws(1, 32, 1, 16384, 128) == 32 * 16384 * 8 + 2 * 4 * 16384 * 128 * 4
    # a tiny grid: 2 workgroups would need 256 parts, but a block has only 2 visits (2 heads x 1 query tile)
    assert ws(1, 4, 2, 100, 64) == 4 * 128 * 8 + 2 * 2 * 2 * 100 * 64 * 4
    # one head of 32768 keys: 256 key blocks, so each block's query tiles split 2 ways
    assert ws(1, 1, 1, 32768, 128) == 32768 * 8 + 2 * 2 * 32768 * 128 * 4
    # 8 heads of 1000 keys: 8 blocks x 8 heads = 64 workgroups, 8 parts; at most 64 parts however small the grid
    assert ws(1, 8, 8, 1000, 64) == 8 * 1024 * 8 + 2 * 8 * 8 * 1000 * 64 * 4
    assert ws(1, 64, 1, 128, 64) == 64 * 128 * 8 + 2 * 64 * 128 * 64 * 4
    assert ws(0, 3, 3, 100, 64) == 0 and ws(1, 1, 1, -5, 64) == 0
    assert ws(1, 4, 3, 100, 64) == 0 and ws(1, 4, 0, 100, 64) == 0 and ws(1, 4, 4, 100, 96) == 0


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_one_hip_runtime_in_the_process():
    """libfa.so must share torch's HIP runtime: exactly one libamdhip64 mapped after importing the package."""
    code = ("import exact_attention_13_amd, torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, check=True,
                         cwd=str(HEADER.parent.parent)).stdout
    assert out.strip() == "1"
