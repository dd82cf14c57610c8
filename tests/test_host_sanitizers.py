"""libfmd's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU needed).

The C ABI source is compiled again with both sanitizers on its host code only
(the device code is compiled as usual; no sanitizer runs on a GPU), linked
with the kernels' objects from the in-tree build and with a seeded sweep
driver (tests/host_sanitize/planner_sweep.cpp) that runs the workspace
planners and the argument validation on a few hundred random ring states,
session counts (1..64), head counts and query counts.  Any sanitizer report
aborts the driver; the driver's own checks (determinism, planner agreement,
rejected calls leave every cache untouched) set its exit status."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "flow_matching_denoising_amd")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "planner_sweep.cpp")


def _tool(path_or_name):
    if os.path.exists(path_or_name):
        return path_or_name
    return shutil.which(os.path.basename(path_or_name))


def test_planner_sweep_under_asan_and_ubsan(tmp_path):
    hipcc = _tool("/opt/rocm/bin/hipcc")
    clangxx = _tool("/opt/rocm/llvm/bin/clang++")
    kernels = [os.path.join(PKG, "_build", f"{n}.hip.o")
               for n in ("attention", "kv_append", "proj_euler", "gemm_wide")]
    if not hipcc or not clangxx or not all(os.path.exists(k) for k in kernels):
        pytest.skip("ROCm toolchain or the in-tree kernel objects are missing")
    abi_o = str(tmp_path / "abi_asan.o")
    drv_o = str(tmp_path / "sweep.o")
    exe = str(tmp_path / "planner_sweep")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-c",
                    os.path.join(PKG, "csrc", "abi.hip"), "-o", abi_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-c", DRIVER,
                    "-o", drv_o], check=True, capture_output=True, text=True)
    subprocess.run([clangxx, "-fsanitize=address,undefined", abi_o, *kernels, drv_o,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "300"], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failed checks" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
