"""Builds libfmd.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every HIP source is compiled to its own object (in parallel) and linked into
``flow_matching_denoising_amd/libfmd.so``.  Packed-FP32 code generation is
switched off for the device code, and the build fails if the gfx950 code of
any object still holds a packed-FP32 add, multiply or FMA (its disassembly is
checked after every compile)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfmd.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libfmd")


_PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _llvm_tool(name: str) -> str:
    for cand in (os.path.join("/opt/rocm/llvm/bin", name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError(f"{name} not found (ROCm LLVM tools are required to check the build)")


def check_device_code(obj: str) -> int:
    """Disassemble the gfx950 code object inside a compiled HIP object and
    raise if it holds packed-FP32 arithmetic.  Returns the number of MFMA
    instructions found (a sanity check that the code was disassembled)."""
    sections = subprocess.run([_llvm_tool("llvm-readelf"), "-S", obj], check=True,
                              capture_output=True, text=True).stdout
    if ".hip_fatbin" not in sections:
        return 0   # host code only
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        co = os.path.join(tmp, "device.co")
        subprocess.run([_llvm_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj],
                       check=True, capture_output=True)
        subprocess.run([_llvm_tool("clang-offload-bundler"), "--type=o", f"--input={fat}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}",
                        "--unbundle"], check=True, capture_output=True)
        asm = subprocess.run([_llvm_tool("llvm-objdump"), "-d", co], check=True,
                             capture_output=True, text=True).stdout
    bad = [l.strip() for l in asm.splitlines() if _PACKED_FP32.search(l)]
    if bad:
        raise RuntimeError(f"{os.path.basename(obj)}: {len(bad)} packed-FP32 instruction(s) in "
                           f"the {ARCH} code, e.g. {bad[0]}")
    return sum(1 for l in asm.splitlines() if "v_mfma" in l)


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *COMMON, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l and "--hip-link" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        check_device_code(obj)
        return obj

    with cf.ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load time.
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
