"""The build's own checks (CPU only): the gfx950 code of every compiled HIP
object holds no packed-FP32 add, multiply or FMA, and the objects that hold
the MFMA kernels were really disassembled."""
import glob
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "flow_matching_denoising_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("_fmd_build_check",
                                                  os.path.join(PKG, "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_packed_fp32_pattern():
    b = _build_module()
    assert b._PACKED_FP32.search("v_pk_mul_f32 v[4:5], v[0:1], v[2:3]")
    assert b._PACKED_FP32.search("  v_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]")
    assert b._PACKED_FP32.search("v_pk_add_f32 v[0:1], v[0:1], v[2:3]")
    assert not b._PACKED_FP32.search("v_pk_mul_f16 v0, v1, v2")
    assert not b._PACKED_FP32.search("v_pk_mov_b32 v[0:1], v[2:3], v[4:5]")


def test_device_code_has_no_packed_fp32():
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    if not objs:
        pytest.skip("library not built in-tree")
    b = _build_module()
    mfma = {os.path.basename(o): b.check_device_code(o) for o in objs}
    for name in ("attention.hip.o", "proj_euler.hip.o", "gemm_wide.hip.o"):
        assert mfma.get(name, 0) > 0, (name, mfma)
