"""The C ABI's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer: the library built
with the sanitizers on its host code (device code unchanged), and tests/abi_sanitize_driver.c calling every entry
point with arguments the header says are rejected on the host. No GPU is used: every call returns before a launch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_argument_checks_run_clean_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc or the ROCm clang is not installed")
    csrc = os.path.join(ROOT, "tile_binned_gaussian_amd", "csrc")
    sources = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    lib = str(tmp_path / "libgs_host_sanitized.so")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-shared", "-std=c++17", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-I", os.path.join(ROOT, "include"),
           *sources, "-o", lib]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    exe = str(tmp_path / "abi_sanitize")
    link = [clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_sanitize_driver.c"),
            f"-L{tmp_path}", "-lgs_host_sanitized", f"-Wl,-rpath,{tmp_path}", f"-L{ROCM}/lib", "-lamdhip64",
            f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    build = subprocess.run(link, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    # the HIP runtime's own allocations are not ours to account for: no leak report
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "abi sanitizer run ok" in run.stdout
