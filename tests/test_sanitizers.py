"""Sanitizer tier of the CPU tests: the host code built with AddressSanitizer and UndefinedBehaviorSanitizer.

* The C ABI's host-side validation (exact_attention_13_amd/csrc/fa_api.hip compiled as plain C++ with g++, the
  kernel launchers replaced by the recording stubs of tests/sanitize/launch_stubs.cpp) runs the checks of
  tests/sanitize/abi_host_check.cpp: every entry point, every error code, the largest accepted sizes.
* The fp64 oracle (oracle/*.c) built the same way runs every oracle pin test (tests/test_oracle_pins*.py) in a
  child process that preloads the sanitizer runtime and loads that build through FA_ORACLE_LIB.
Any sanitizer report fails the test (UB checks do not recover; leak checks are off in the Python child, whose
interpreter and libraries keep memory until exit by design). Built with g++/gcc only: no GPU code is compiled
with a sanitizer.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not available")


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not installed")
    return path


def _no_report(text: str):
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior"):
        assert marker not in text, text[-4000:]


def test_abi_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_check"
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT / 'include'}",
           f"-I{ROOT / 'exact_attention_13_amd' / 'csrc'}", "-x", "c++",
           str(ROOT / "exact_attention_13_amd" / "csrc" / "fa_api.hip"), "-x", "none",
           str(ROOT / "tests" / "sanitize" / "launch_stubs.cpp"), str(ROOT / "tests" / "sanitize" / "abi_host_check.cpp"),
           "-o", str(exe)]
    if not Path("/opt/rocm/include/hip/hip_runtime_api.h").exists():
        pytest.skip("HIP headers not installed")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    print(out[-2000:])
    _no_report(out)
    assert res.returncode == 0 and "abi_host_check: 0 failed" in out, out[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    srcs = [str(ROOT / "oracle" / "attn_oracle.c"), str(ROOT / "oracle" / "attn_bwd_oracle.c")]
    subprocess.run(["gcc", "-std=c11", *SAN, "-fPIC", "-shared", "-pthread", *srcs, "-o", str(lib), "-lm"],
                   check=True, capture_output=True, text=True)
    # the sanitizer runtimes go first in the preload list; whatever the environment already preloads stays
    preload = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")] +
                       [p for p in os.environ.get("LD_PRELOAD", "").split(":") if p])
    env = dict(os.environ, LD_PRELOAD=preload, FA_ORACLE_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    probe = ("import oracle\noracle._load()\n"
             "maps = open('/proc/self/maps').read()\n"
             "print('liboracle_san.so' in maps, 'libasan' in maps, 'liboracle.so' in maps)\n")
    res = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env, cwd=str(ROOT),
                         timeout=120)
    assert res.stdout.split() == ["True", "True", "False"], res.stdout + res.stderr  # the sanitized build is the one
    tests = sorted(str(p) for p in (ROOT / "tests").glob("test_oracle_pins*.py"))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                         capture_output=True, text=True, env=env, cwd=str(ROOT), timeout=900)
    out = res.stdout + res.stderr
    print(out[-3000:])
    _no_report(out)
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
