"""Host code under the sanitizers (CPU only, no GPU needed).

``tests/oracle_sanitize.c`` links ``oracle/topk_oracle.c`` directly and
checks every entry point against a rank definition on edge-heavy random
batches. It is built twice: with AddressSanitizer + UndefinedBehaviorSanitizer
(out-of-bounds reads and writes, leaks, signed overflow, bad shifts) and with
ThreadSanitizer (the per-row worker threads of ``oracle_select``).

``tests/abi_sanitize.c`` drives the C-ABI library's host code, built with
AddressSanitizer + UndefinedBehaviorSanitizer on the host pass only (the
device code is built as usual and never runs): argument checks, status codes
and plan sizes, every call returning before any HIP call.

Any sanitizer report makes the program exit non-zero.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
DRIVER = ROOT / "tests" / "oracle_sanitize.c"
ORACLE_C = ROOT / "oracle" / "topk_oracle.c"
ABI_DRIVER = ROOT / "tests" / "abi_sanitize.c"
HIP_SRC = ROOT / "row_top_selection_amd" / "csrc" / "dsatopk.hip"
ROCM = Path(os.environ.get("ROCM_PATH", "/opt/rocm"))

FLAVOURS = {
    "address_undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                          "-fno-omit-frame-pointer"],
    "thread": ["-fsanitize=thread"],
}


@pytest.mark.parametrize("flavour", sorted(FLAVOURS))
def test_oracle_clean_under_sanitizer(flavour, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / f"oracle_{flavour}"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pthread",
           *FLAVOURS[flavour], str(ORACLE_C), str(DRIVER), "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "cannot find" in build.stderr:
        pytest.skip(f"sanitizer runtime missing: {build.stderr.strip()}")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1:exitcode=66"
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout


@pytest.mark.slow
def test_abi_host_code_clean_under_address_and_undefined_sanitizers(tmp_path):
    hipcc = ROCM / "bin" / "hipcc"
    clang = ROCM / "llvm" / "bin" / "clang"
    if not hipcc.exists() or not clang.exists():
        pytest.skip("hipcc or ROCm clang not found")
    lib = tmp_path / "libdsatopk_host_sanitized.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    cmd = [str(hipcc), "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
           "-fno-omit-frame-pointer", f"-I{ROOT / 'include'}", str(HIP_SRC), "-o", str(lib)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    exe = tmp_path / "abi_sanitize"
    cmd = [str(clang), "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           f"-I{ROOT / 'include'}", str(ABI_DRIVER), f"-L{tmp_path}", "-ldsatopk_host_sanitized",
           f"-Wl,-rpath,{tmp_path}", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    # the HIP runtime's own start-up allocations are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
