"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):
the library loads and exports every function fmd.h declares, argument
validation returns the documented codes without touching cache state, and the
workspace sizing is consistent.  Pointers here are fake, aligned integers:
every call is rejected before anything would touch device memory."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import flow_matching_denoising_amd as fmd
from flow_matching_denoising_amd import _Cache, _UnitIO, _UnitStep, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmd.h")

FAKE = 0x10000000        # 256-byte aligned, never dereferenced


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fmd_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(_lib, n), f"libfmd.so does not export {n}"
    assert set(names) == set(fmd.EXPORTED)


def test_strerror_and_version():
    for code, name in fmd.STATUS.items():
        assert fmd.strerror(code) and isinstance(fmd.strerror(code), str)
    assert fmd.strerror(12345) == "unknown status"
    assert re.match(r"^\d+\.\d+\.\d+$", fmd.version())


def _cache(H=2, hd=64, cap=128, ln=96, head=96, k=FAKE, v=FAKE + 0x100000):
    return _Cache(k, v, H, hd, cap, ln, head)


def _append(c, T, ks=FAKE + 0x200000, vs=FAKE + 0x300000):
    return fmd._kv_append(ctypes.byref(c), ks, vs, T, None)


@pytest.mark.parametrize("mut,code", [
    (dict(hd=96), -2), (dict(hd=0), -2), (dict(cap=100), -2), (dict(cap=0), -2),
    (dict(hd=128, cap=1 << 23, ln=0, head=0), -2),
    (dict(H=0), -2), (dict(ln=129), -1), (dict(head=128), -1), (dict(head=-1), -1),
    (dict(k=FAKE + 8), -4), (dict(v=0), -1),
])
def test_append_rejects_bad_cache(mut, code):
    c = _cache(**mut)
    before = (c.len_tokens, c.head_tokens)
    assert _append(c, 32) == code
    assert (c.len_tokens, c.head_tokens) == before
    assert fmd._last_error().decode()


@pytest.mark.parametrize("T,code", [(0, -1), (-5, -1), (129, -3)])
def test_append_rejects_bad_slice(T, code):
    c = _cache()
    assert _append(c, T) == code
    assert (c.len_tokens, c.head_tokens) == (96, 96)


def test_append_rejects_misaligned_or_null_slice():
    c = _cache()
    assert _append(c, 32, ks=FAKE + 2) == -4
    assert _append(c, 32, vs=0) == -1
    assert (c.len_tokens, c.head_tokens) == (96, 96)


def test_batched_append_rejects_mismatch_and_duplicates():
    a, b = _cache(), _cache(H=3)
    arr = (ctypes.POINTER(_Cache) * 2)(ctypes.pointer(a), ctypes.pointer(b))
    ks = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ts = (ctypes.c_int64 * 2)(16, 16)
    assert fmd._kv_append_batched(arr, ks, ks, ts, 2, None) == -2
    arr2 = (ctypes.POINTER(_Cache) * 2)(ctypes.pointer(a), ctypes.pointer(a))
    assert fmd._kv_append_batched(arr2, ks, ks, ts, 2, None) == -1
    assert fmd._kv_append_batched(arr2, ks, ks, ts, 0, None) == -1
    assert fmd._kv_append_batched(arr2, ks, ks, ts, 65, None) == -1
    assert (a.len_tokens, a.head_tokens) == (96, 96)


def _step(c, n_video=12, n_audio=4, h=1.0, q=FAKE, z=FAKE):
    return _UnitStep(ctypes.pointer(c), q, FAKE, FAKE, z, n_video, n_audio, h)


def _ws(units):
    arr = (_UnitStep * len(units))(*units)
    out = ctypes.c_size_t(0)
    rc = fmd._workspace_bytes(arr, len(units), ctypes.byref(out))
    return rc, out.value


def test_workspace_bytes_is_host_arithmetic():
    c = _cache(H=40, hd=128, cap=60416, ln=60416, head=0)
    rc, n1 = _ws([_step(c, 920, 8)])
    assert rc == 0 and n1 > 0
    # Staged unit K and V (2 x 40 x 928 x 128 bf16) + O (928 x 5120 bf16).
    assert n1 >= 2 * 40 * 928 * 128 * 2 + 928 * 5120 * 2
    rc, n2 = _ws([_step(c, 920, 8), _step(_cache(H=40, hd=128, cap=944, ln=944, head=0), 920, 8)])
    assert rc == 0 and n2 > n1


@pytest.mark.parametrize("kw,code", [
    (dict(n_video=0, n_audio=0), -1), (dict(n_video=-1), -1), (dict(q=FAKE + 4), -4),
    (dict(n_video=1 << 22, n_audio=1), -1),
    (dict(q=0), -1),
])
def test_step_validation(kw, code):
    c = _cache()
    rc, _ = _ws([_step(c, **kw)])
    assert rc == code


def test_denoise_step_checks_h_z_and_workspace():
    c = _cache()
    for kw, code in [(dict(h=0.0), -1), (dict(h=float("nan")), -1), (dict(z=0), -1)]:
        arr = (_UnitStep * 1)(_step(c, **kw))
        assert fmd._denoise_step(arr, 1, FAKE, FAKE, 1 << 30, None) == code
    arr = (_UnitStep * 1)(_step(c))
    assert fmd._denoise_step(arr, 1, FAKE, None, 0, None) == -5          # no workspace
    assert fmd._denoise_step(arr, 1, FAKE, FAKE, 16, None) == -5         # too small
    assert fmd._denoise_step(arr, 1, FAKE, FAKE + 16, 1 << 30, None) == -4   # misaligned
    assert fmd._denoise_step(arr, 1, 0, FAKE, 1 << 30, None) == -1       # no W_o
    # Mismatched heads across sessions.
    arr2 = (_UnitStep * 2)(_step(c), _step(_cache(H=3)))
    assert fmd._denoise_step(arr2, 2, FAKE, FAKE, 1 << 30, None) == -2


def test_denoise_unit_validation_leaves_state():
    c = _cache()
    h = (ctypes.c_float * 2)(0.5, -0.5)
    io = _UnitIO(ctypes.pointer(c), FAKE, FAKE, 32, FAKE, FAKE, FAKE, 0, FAKE, 12, 4,
                 ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    arr = (_UnitIO * 1)(io)
    assert fmd._denoise_unit(arr, 1, 2, FAKE, FAKE, 1 << 30, None) == -1   # h[1] < 0
    assert fmd._denoise_unit(arr, 1, 0, FAKE, FAKE, 1 << 30, None) == -1   # no steps
    assert (c.len_tokens, c.head_tokens) == (96, 96)
    io.slice_tokens = 200
    arr = (_UnitIO * 1)(io)
    h[1] = 0.5
    assert fmd._denoise_unit(arr, 1, 2, FAKE, FAKE, 1 << 30, None) == -3   # slice > cap
    io.slice_tokens = 32
    io.step_stride_elems = 3
    arr = (_UnitIO * 1)(io)
    assert fmd._denoise_unit(arr, 1, 2, FAKE, FAKE, 1 << 30, None) == -4   # unaligned stride
    assert (c.len_tokens, c.head_tokens) == (96, 96)
    io.step_stride_elems = 0
    arr = (_UnitIO * 1)(io)
    out = ctypes.c_size_t(0)
    assert fmd._unit_workspace_bytes(arr, 1, 2, ctypes.byref(out)) == 0 and out.value > 0


def test_profile_read_rejects_bad_class():
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    assert fmd._profile_read(99, ctypes.byref(ms), ctypes.byref(n)) == -1


def test_device_code_has_no_packed_fp32_arithmetic():
    # The kernels are built with packed-FP32 generation switched off; check
    # the gfx950 assembly of our own sources for v_pk_{add,mul,fma}_f32.
    from flow_matching_denoising_amd import _build
    hipcc = _build._hipcc()
    with tempfile.TemporaryDirectory() as td:
        for name in ("attention.hip", "proj_euler.hip", "kv_append.hip", "gemm_wide.hip"):
            out = os.path.join(td, name + ".s")
            cmd = [hipcc, *_build.COMMON, "--cuda-device-only", "-S",
                   os.path.join(_build.CSRC, name), "-o", out]
            subprocess.run(cmd, check=True, capture_output=True)
            asm = open(out).read()
            assert not re.search(r"v_pk_(add|mul|fma)_f32", asm), name
            assert "scratch_" not in asm, f"{name}: register spills to scratch"
            # M0 is set by the LDS-DMA helpers' inline assembly; the compiler
            # ignores it in their clobber lists, so none of its own code may use it.
            outside, inside = [], False
            for line in asm.splitlines():
                if ";;#ASMSTART" in line:
                    inside = True
                elif ";;#ASMEND" in line:
                    inside = False
                elif not inside and not line.lstrip().startswith(";"):
                    outside.append(line)
            assert not [l for l in outside if re.search(r"\bm0\b", l)], f"{name}: compiler uses M0"


def test_denoise_unit_qkv_validation_leaves_state():
    from flow_matching_denoising_amd import _UnitQkvIO
    c = _cache()
    h = (ctypes.c_float * 2)(0.5, -0.5)
    io = _UnitQkvIO(ctypes.pointer(c), FAKE, FAKE, 32, FAKE, 12, 4,
                    ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    arr = (_UnitQkvIO * 1)(io)
    run = fmd._denoise_unit_qkv
    assert run(arr, 1, 2, FAKE, FAKE, FAKE, 1 << 30, None) == -1       # h[1] < 0
    assert run(arr, 1, 0, FAKE, FAKE, FAKE, 1 << 30, None) == -1       # no steps
    h[1] = 0.5
    assert run(arr, 1, 2, 0, FAKE, FAKE, 1 << 30, None) == -1          # no W_qkv
    assert run(arr, 1, 2, FAKE + 8, FAKE, FAKE, 1 << 30, None) == -4   # misaligned W_qkv
    assert run(arr, 1, 2, FAKE, FAKE, FAKE, 16, None) == -5            # workspace too small
    io.slice_tokens = 200
    arr = (_UnitQkvIO * 1)(io)
    assert run(arr, 1, 2, FAKE, FAKE, FAKE, 1 << 30, None) == -3       # slice > cap
    io.slice_tokens = 32
    io.z = 0
    arr = (_UnitQkvIO * 1)(io)
    assert run(arr, 1, 2, FAKE, FAKE, FAKE, 1 << 30, None) == -1       # no z
    assert (c.len_tokens, c.head_tokens) == (96, 96)


def test_unit_qkv_workspace_holds_projections_and_step():
    from flow_matching_denoising_amd import _UnitQkvIO
    c = _cache(H=40, hd=128, cap=60416, ln=60416, head=0)
    h = (ctypes.c_float * 1)(1.0)
    io = _UnitQkvIO(ctypes.pointer(c), 0, 0, 0, FAKE, 920, 8,
                    ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    out = ctypes.c_size_t(0)
    assert fmd._unit_qkv_workspace_bytes((_UnitQkvIO * 1)(io), 1, ctypes.byref(out)) == 0
    _, step = _ws([_step(c, 920, 8)])
    # bf16 z and Q (2 x 928 x 5120 bf16) on top of the step workspace, whose
    # unit key/value slots take K_u and V_u straight from the projection.
    assert out.value == step + 2 * 928 * 5120 * 2


def _cfg_io(cond, uncond, h, g=5.0, ct=32, ut=0, z=FAKE):
    from flow_matching_denoising_amd import _UnitCfgIO
    return _UnitCfgIO(ctypes.pointer(cond), ctypes.pointer(uncond), FAKE, FAKE, ct, FAKE, FAKE,
                      ut, z, 12, 4, ctypes.cast(h, ctypes.POINTER(ctypes.c_float)), g)


def test_denoise_unit_cfg_validation_leaves_state():
    from flow_matching_denoising_amd import _UnitCfgIO
    a, b, c = _cache(), _cache(), _cache()
    h = (ctypes.c_float * 2)(0.5, 0.5)
    run = fmd._denoise_unit_cfg

    def call(ios, n_steps=2, wq=FAKE, ws=1 << 30):
        arr = (_UnitCfgIO * len(ios))(*ios)
        return run(arr, len(ios), n_steps, wq, FAKE, FAKE, ws, None)
    assert call([_cfg_io(a, a, h)]) == -1                      # same cache for both branches
    assert call([_cfg_io(a, b, h), _cfg_io(c, a, h)]) == -1    # cache shared across units
    assert call([_cfg_io(a, b, h, g=float("nan"))]) == -1      # guidance not finite
    assert call([_cfg_io(a, b, h, g=float("inf"))]) == -1
    assert call([_cfg_io(a, b, h, ct=200)]) == -3              # slice > cap
    assert call([_cfg_io(a, b, h, ut=-1)]) == -1               # negative slice
    assert call([_cfg_io(a, _cache(H=3), h)]) == -2            # branch shapes differ
    assert call([_cfg_io(a, b, h, z=0)]) == -1                 # no z
    assert call([_cfg_io(a, b, h)], n_steps=0) == -1
    assert call([_cfg_io(a, b, h)], wq=0) == -1                # no W_qkv
    assert call([_cfg_io(a, b, h)], ws=16) == -5               # workspace too small
    many = [_cache() for _ in range(66)]
    assert call([_cfg_io(many[2 * i], many[2 * i + 1], h) for i in range(33)]) == -1
    h[1] = -0.5
    assert call([_cfg_io(a, b, h)]) == -1                      # h[1] < 0
    for x in (a, b, c):
        assert (x.len_tokens, x.head_tokens) == (96, 96)


def test_unit_cfg_workspace_holds_both_branches():
    from flow_matching_denoising_amd import _UnitCfgIO, _UnitQkvIO
    a = _cache(H=40, hd=128, cap=60416, ln=60416, head=0)
    b = _cache(H=40, hd=128, cap=60416, ln=60416, head=0)
    h = (ctypes.c_float * 1)(1.0)
    io = _cfg_io(a, b, h, ct=0)
    io.n_video, io.n_audio = 920, 8
    out = ctypes.c_size_t(0)
    assert fmd._unit_cfg_workspace_bytes((_UnitCfgIO * 1)(io), 1, ctypes.byref(out)) == 0
    qio = _UnitQkvIO(ctypes.pointer(a), 0, 0, 0, FAKE, 920, 8,
                     ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    q = ctypes.c_size_t(0)
    assert fmd._unit_qkv_workspace_bytes((_UnitQkvIO * 1)(qio), 1, ctypes.byref(q)) == 0
    # A second attention output (928 x 5120 bf16) and staging on top of the
    # single-branch workspace.
    assert out.value >= q.value + 928 * 5120 * 2


def _layers_io(caches, h, T=0, z=FAKE, with_slices=True):
    from flow_matching_denoising_amd import _UnitLayersIO
    L = len(caches)
    arr = (ctypes.POINTER(_Cache) * L)(*[ctypes.pointer(c) for c in caches])
    sl = (ctypes.c_void_p * L)(*([FAKE] * L)) if with_slices else None
    io = _UnitLayersIO(arr, sl, sl, T, z, 12, 4, ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    io._keep = (arr, sl)
    return io


def test_denoise_unit_layers_validation_leaves_state():
    from flow_matching_denoising_amd import _UnitLayersIO
    h = (ctypes.c_float * 2)(0.5, 0.5)
    a, b, c = _cache(), _cache(), _cache()
    w = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    run = fmd._denoise_unit_layers

    def call(ios, L, n_steps=2, ws=1 << 30, wq=w):
        arr = (_UnitLayersIO * len(ios))(*ios)
        return run(arr, len(ios), L, n_steps, wq, w, FAKE, ws, None)
    assert call([_layers_io([a, a], h)], 2) == -1                    # one ring in two layers
    assert call([_layers_io([a, b], h), _layers_io([c, a], h)], 2) == -1   # shared across sessions
    assert call([_layers_io([a, _cache(H=3)], h)], 2) == -2          # layer shapes differ
    assert call([_layers_io([a, b], h, T=8, with_slices=False)], 2) == -1   # no slice arrays
    assert call([_layers_io([a, b], h, T=200)], 2) == -3             # slice > cap
    assert call([_layers_io([a, b], h)], 0) == -1                    # no layers
    assert call([_layers_io([a, b], h)], 2, n_steps=0) == -1
    assert call([_layers_io([a, b], h, z=0)], 2) == -1               # no z
    assert call([_layers_io([a, b], h)], 2, ws=16) == -5             # workspace too small
    assert call([_layers_io([a, b], h)], 2, wq=None) == -1           # no weight array
    h[1] = -1.0
    assert call([_layers_io([a, b], h)], 2) == -1                    # h[1] < 0
    for x in (a, b, c):
        assert (x.len_tokens, x.head_tokens) == (96, 96)


def test_unit_layers_workspace():
    from flow_matching_denoising_amd import _UnitLayersIO, _UnitQkvIO
    h = (ctypes.c_float * 1)(1.0)
    rings = [_cache(H=40, hd=128, cap=60416, ln=60416, head=0) for _ in range(3)]

    def ws(L):
        io = _layers_io(rings[:L], h)
        io.n_video, io.n_audio = 920, 8
        out = ctypes.c_size_t(0)
        assert fmd._unit_layers_workspace_bytes((_UnitLayersIO * 1)(io), 1, L,
                                                ctypes.byref(out)) == 0
        return out.value
    qio = _UnitQkvIO(ctypes.pointer(rings[0]), 0, 0, 0, FAKE, 920, 8,
                     ctypes.cast(h, ctypes.POINTER(ctypes.c_float)))
    q = ctypes.c_size_t(0)
    assert fmd._unit_qkv_workspace_bytes((_UnitQkvIO * 1)(qio), 1, ctypes.byref(q)) == 0
    assert ws(1) == q.value                              # one layer: the z-dependent solver
    assert ws(3) == ws(2) >= q.value + 928 * 5120 * 4    # plus the fp32 residual, rings alike


def test_overlapping_latents_are_rejected():
    # Two sessions whose fp32 latents overlap would race in the in-place
    # update: every solver entry point rejects them before anything runs.
    from flow_matching_denoising_amd import _UnitCfgIO, _UnitLayersIO, _UnitQkvIO
    a, b, c, e = _cache(), _cache(), _cache(), _cache()
    h = (ctypes.c_float * 1)(0.5)
    hp = ctypes.cast(h, ctypes.POINTER(ctypes.c_float))
    d = 2 * 64
    near = FAKE + 8 * d * 4            # inside the first session's 16 x d floats
    apart = FAKE + 16 * d * 4          # right after it: allowed
    arr = (_UnitStep * 2)(_step(a, z=FAKE), _step(b, z=near))
    assert fmd._denoise_step(arr, 2, FAKE, FAKE, 1 << 30, None) == -1
    q = (_UnitQkvIO * 2)(_UnitQkvIO(ctypes.pointer(a), FAKE, FAKE, 0, FAKE, 12, 4, hp),
                         _UnitQkvIO(ctypes.pointer(b), FAKE, FAKE, 0, near, 12, 4, hp))
    assert fmd._denoise_unit_qkv(q, 2, 1, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    g = (_UnitCfgIO * 2)(_cfg_io(a, b, h, ct=0, z=FAKE), _cfg_io(c, e, h, ct=0, z=near))
    assert fmd._denoise_unit_cfg(g, 2, 1, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    lay = (_UnitLayersIO * 2)(_layers_io([a], h, z=FAKE), _layers_io([b], h, z=near))
    w = (ctypes.c_void_p * 1)(FAKE)
    assert fmd._denoise_unit_layers(lay, 2, 1, 1, w, w, FAKE, 1 << 30, None) == -1
    assert "overlap" in fmd._last_error().decode()
    out = ctypes.c_size_t(0)
    ok = (_UnitQkvIO * 2)(_UnitQkvIO(ctypes.pointer(a), FAKE, FAKE, 0, FAKE, 12, 4, hp),
                          _UnitQkvIO(ctypes.pointer(b), FAKE, FAKE, 0, apart, 12, 4, hp))
    assert fmd._unit_qkv_workspace_bytes(ok, 2, ctypes.byref(out)) == 0
    for x in (a, b, c, e):
        assert (x.len_tokens, x.head_tokens) == (96, 96)


def test_profile_select_rejects_unknown_classes():
    n = len(fmd.KERNEL_CLASSES)
    assert fmd._profile_select(1 << n) == -1
    assert fmd._last_error().decode()
    assert fmd._profile_select(0xFFFFFFFF) == -1
    assert fmd._profile_select((1 << n) - 1) == 0
    assert fmd._profile_select(0) == 0
    assert fmd._profile_select((1 << n) - 1) == 0


def _model_pieces(H, per_head, lanes, groups):
    """Pieces per lane of one launch, from the definition: the window
    sequence (head-major, then session) is cut into `groups` ranges
    [g*T//G, (g+1)*T//G); a lane's pieces are its windows cut at every range
    start inside it and at the start of each non-empty segment after the first.
    lanes: per session (lane0, [n0, n1, n2])."""
    T = H * per_head
    starts = {g * T // groups for g in range(1, groups)}
    out = []
    for lane0, segs in lanes:
        most = 1
        for h in range(H):
            first = h * per_head + lane0
            W = sum(segs)
            cuts = {c for c in starts if first < c < first + W}
            if segs[0] > 0:
                cuts.add(first + segs[0])
            if segs[1] > 0:
                cuts.add(first + segs[0] + segs[1])
            cuts = {c for c in cuts if first < c < first + W}
            most = max(most, len(cuts) + 1)
        out.append(most)
    return out


def _proj_part_bytes(n_q, d):
    """fp32 partial products of a split projection: 160 x 128 output tiles;
    when they fill less than half of 256 CUs, the k range (d / 64 steps) is
    cut into as many parts as fit the chip, at most 4 and at least two k
    steps each."""
    tiles = -(-n_q // 160) * -(-d // 128)
    if tiles * 2 >= 256:
        return 0
    splits = max(1, min(256 // tiles, 4, (d // 64) // 2))
    return splits * n_q * d * 4 if splits > 1 else 0


def test_projection_split_workspace():
    # The 192x336-class unit (12 heads x 128, 260 queries): 2 x 12 tiles, so
    # the k range of 24 steps is cut into 4 parts of fp32 partials.
    c = _cache(H=12, hd=128, cap=8576, ln=8576, head=0)
    rc, n_split = _ws([_step(c, 252, 8)])
    assert rc == 0
    assert _proj_part_bytes(260, 1536) == 4 * 260 * 1536 * 4
    big = _cache(H=40, hd=128, cap=60416, ln=60416, head=0)
    rc, n_big = _ws([_step(big, 920, 8)])
    assert rc == 0 and _proj_part_bytes(928, 5120) == 0
    # Staged unit K and V (npad = 272), O and the partials; the 8,836 keys per
    # query make few windows, so no lane is cut into pieces here or the
    # pieces' bytes come on top.
    base = 2 * 12 * 272 * 128 * 2 + 260 * 1536 * 2 + 4 * 260 * 1536 * 4
    assert n_split >= base


@pytest.mark.parametrize("H,head", [(5, 59472), (10, 59472), (40, 59472), (40, 0), (12, 8304),
                                     (3, 59472), (20, 0), (24, 59472)])
def test_group_planner_pieces(H, head):
    # A full 60,416-key ring and a 928-query unit (4 query blocks): 8 XCDs x
    # 8 groups of 4 work-groups (60 for 5, 10, 12 and 20 heads, 63 for 3; 24
    # heads keep 64, as 48 is below 85 % of it).  The partial slots the workspace holds (one
    # bf16 piece of O and one fp32 log-sum-exp each) equal the most pieces any
    # lane is cut into, by an independent model of the partition.
    n_q, hd, cap = 928, 128, 60416
    c = _cache(H=H, hd=hd, cap=cap, ln=cap, head=head)
    rc, nbytes = _ws([_step(c, 920, 8)])
    assert rc == 0

    def a256(x):
        return (x + 255) // 256 * 256

    def layout(npart):
        # unit K and V (npad = n_q), O, then the pieces and their log-sum-exps,
        # then the projection's partials; every region starts 256-byte aligned
        size = 2 * a256(H * n_q * hd * 2) + a256(n_q * H * hd * 2)
        if npart:
            size = a256(size + npart * n_q * H * hd * 2)
            size = a256(size + npart * n_q * H * 4)
        return size + a256(_proj_part_bytes(n_q, H * hd))
    start = head % cap                                     # the valid range starts at head
    seg0 = cap - start
    n0 = (cap - (start & ~15) + 63) // 64
    n1 = (start + 63) // 64 if start else 0
    n2 = (n_q + 63) // 64
    assert seg0 > 0
    per_head = n0 + n1 + n2
    # 8 XCDs x 8 groups of 4 work-groups, at least 8 windows per group; the
    # largest multiple of H instead when it is at least 85 % of that.
    groups = min(64, H * per_head // 8)
    if groups // H * H * 20 >= groups * 17:
        groups = groups // H * H
    want = _model_pieces(H, per_head, [(0, [n0, n1, n2])], groups)[0]
    assert nbytes == layout(want if want > 1 else 0)


def test_noalloc_rejects_units_beyond_the_static_scratch():
    # Two sessions of the 640x368-class unit over wrapped 256-unit (241,664-key)
    # rings need more scratch than FMD_NOALLOC_SCRATCH_BYTES: rejected with
    # FMD_E_WORKSPACE before anything touches a device, cache state unchanged.
    # One such session fits (its workspace size is below the limit).
    h = (ctypes.c_float * 4)(0.25, 0.25, 0.25, 0.25)
    hp = ctypes.cast(h, ctypes.POINTER(ctypes.c_float))
    cap = 256 * 944
    for n, fits in ((2, False), (1, True)):
        cs = [_Cache(FAKE + i * 0x1000000, FAKE + 0x100000 + i * 0x1000000, 40, 128, cap, cap,
                     100 * 944) for i in range(n)]
        ios = [_UnitIO(ctypes.pointer(c), FAKE, FAKE, 944, FAKE, FAKE, FAKE, 928 * 5120,
                       FAKE + 0x40000000 + i * 0x2000000, 920, 8, hp) for i, c in enumerate(cs)]
        arr = (_UnitIO * n)(*ios)
        need = ctypes.c_size_t(0)
        assert fmd._unit_workspace_bytes(arr, n, 4, ctypes.byref(need)) == 0
        assert (need.value <= fmd.FMD_NOALLOC_SCRATCH_BYTES) == fits, need.value
        if not fits:
            assert fmd._denoise_unit_noalloc(arr, n, 4, FAKE, None) == -5
            assert b"static scratch" in fmd._last_error()
            assert all((c.len_tokens, c.head_tokens) == (cap, 100 * 944) for c in cs)
        # Validation comes first, as for fmd_denoise_unit.
        assert fmd._denoise_unit_noalloc(arr, n, 0, FAKE, None) == -1


@pytest.mark.parametrize("n_sessions,steps_per_launch", [(1, 4), (3, 4), (5, 2), (8, 2), (17, 1)])
def test_unit_workspace_batches_the_steps_attention(n_sessions, steps_per_launch):
    # fmd_denoise_unit runs the attention of B steps as one launch whose
    # sessions are the (step, session) pairs, step-major (B: the largest
    # divisor of the 4 steps with B * sessions <= 16).  Its workspace is, per
    # session, the 4 steps' staged unit values (the keys are read in place),
    # and per (step of the batch, session) O and the pieces of the lanes that
    # the launch's group ranges cut, by an independent model of the partition.
    H, hd, n_q, cap, head = 40, 128, 928, 60416, 59472
    h = (ctypes.c_float * 4)(0.25, 0.25, 0.25, 0.25)
    hp = ctypes.cast(h, ctypes.POINTER(ctypes.c_float))
    cs = [_Cache(FAKE + i * 0x1000000, FAKE + 0x100000 + i * 0x1000000, H, hd, cap, cap, head)
          for i in range(n_sessions)]
    ios = [_UnitIO(ctypes.pointer(c), None, None, 0, FAKE, FAKE, FAKE, n_q * H * hd,
                   FAKE + 0x40000000 + i * 0x2000000, 920, 8, hp) for i, c in enumerate(cs)]
    arr = (_UnitIO * n_sessions)(*ios)
    need = ctypes.c_size_t(0)
    assert fmd._unit_workspace_bytes(arr, n_sessions, 4, ctypes.byref(need)) == 0

    def a256(x):
        return (x + 255) // 256 * 256
    start = head % cap
    n0 = (cap - (start & ~15) + 63) // 64
    n1 = (start + 63) // 64
    n2 = (n_q + 63) // 64
    B = steps_per_launch
    m = B * n_sessions                                 # attention sessions per launch
    per_head = m * (n0 + n1 + n2)
    groups = min(64, H * per_head // 8)                # 8 XCDs x 8 groups of 4 work-groups
    if groups // H * H * 20 >= groups * 17:
        groups = groups // H * H
    if m <= 16:
        pieces = _model_pieces(H, per_head, [(k * (n0 + n1 + n2), [n0, n1, n2])
                                             for k in range(m)], groups)
    else:                                              # several launches of at most 16
        pieces = []
        for c0 in range(0, m, 16):
            cn = min(16, m - c0)
            ph = cn * (n0 + n1 + n2)
            g = min(64, H * ph // 8)
            if g // H * H * 20 >= g * 17:
                g = g // H * H
            pieces += _model_pieces(H, ph, [(k * (n0 + n1 + n2), [n0, n1, n2])
                                            for k in range(cn)], g)
    size = n_sessions * 4 * a256(H * n_q * hd * 2)      # 4 steps' staged values
    for npart in pieces:
        size += a256(n_q * H * hd * 2)                  # O
        if npart > 1:
            size += a256(npart * n_q * H * hd * 2) + a256(npart * n_q * H * 4)
    assert need.value == size, (need.value, size)
