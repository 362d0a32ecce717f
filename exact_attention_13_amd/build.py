"""Build libfa.so (the C-ABI library) and libfa_probe.so (a matrix-core throughput probe used by bench.py)
from csrc/ with hipcc for gfx950, in-tree.

    python exact_attention_13_amd/build.py

Run it as a script (or load it by path): importing the package itself loads libfa.so, which may not exist yet.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libfa.so"
SOURCES = [CSRC / "fa_fwd_kernel.hip", CSRC / "fa_fwd_fp8_kernel.hip", CSRC / "fa_bwd_kernel.hip",
           CSRC / "fa_scratch.hip", CSRC / "fa_api.hip"]
PROBE_LIB = PKG / "libfa_probe.so"
PROBE_SOURCES = [CSRC / "fa_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def compile_cmd(out: Path, sources: list[Path] = SOURCES) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            f"-I{ROOT / 'include'}", f"-I{CSRC}",
            *map(str, sources), "-o", str(out)]


def build(verbose: bool = False) -> Path:
    """Build both libraries; returns the path of libfa.so."""
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose)
    return _build_one(LIB, SOURCES, verbose)


def _build_one(lib: Path, sources: list[Path], verbose: bool) -> Path:
    tmp = lib.with_suffix(".so.tmp")
    cmd = compile_cmd(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag and says so; anything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
