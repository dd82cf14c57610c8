"""Python binding of libfmd, the MI355X (gfx950) performer denoise step.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libfmd.so`` behind the C ABI declared in ``include/fmd.h``.  PyTorch is used
for device memory and streams.  There is no fallback: if the library is not
built, importing this package raises ``ImportError``.

Names follow the C ABI: ``kv_append``, ``kv_append_batched``, ``attention``,
``denoise_step``, ``denoise_unit``, ``denoise_unit_qkv``, ``workspace_bytes``,
``unit_workspace_bytes``, ``unit_qkv_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfmd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc for gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

FMD_MAX_SESSIONS = 64
FMD_CACHE_BLOCK = 16
STATUS = {0: "FMD_OK", -1: "FMD_E_INVAL", -2: "FMD_E_SHAPE", -3: "FMD_E_CAPACITY",
          -4: "FMD_E_ALIGN", -5: "FMD_E_WORKSPACE", -6: "FMD_E_HIP"}
KERNEL_CLASSES = {"append": 0, "vt": 1, "attn": 2, "combine": 3, "proj": 4, "qkv": 5, "cvt": 6,
                  "mix": 7}


class FmdError(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__(f"{self.name} ({code}): {detail}")


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("cap_tokens", ctypes.c_int64),
                ("len_tokens", ctypes.c_int64), ("head_tokens", ctypes.c_int64)]


class _UnitStep(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(_Cache)), ("q", ctypes.c_void_p),
                ("k_u", ctypes.c_void_p), ("v_u", ctypes.c_void_p),
                ("z", ctypes.c_void_p), ("n_video", ctypes.c_int32),
                ("n_audio", ctypes.c_int32), ("h", ctypes.c_float)]


class _UnitIO(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(_Cache)), ("k_slice", ctypes.c_void_p),
                ("v_slice", ctypes.c_void_p), ("slice_tokens", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("k_u", ctypes.c_void_p), ("v_u", ctypes.c_void_p),
                ("step_stride_elems", ctypes.c_int64), ("z", ctypes.c_void_p),
                ("n_video", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("h", ctypes.POINTER(ctypes.c_float))]


class _UnitQkvIO(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(_Cache)), ("k_slice", ctypes.c_void_p),
                ("v_slice", ctypes.c_void_p), ("slice_tokens", ctypes.c_int64),
                ("z", ctypes.c_void_p), ("n_video", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("h", ctypes.POINTER(ctypes.c_float))]


class _UnitCfgIO(ctypes.Structure):
    _fields_ = [("cond", ctypes.POINTER(_Cache)), ("uncond", ctypes.POINTER(_Cache)),
                ("cond_k_slice", ctypes.c_void_p), ("cond_v_slice", ctypes.c_void_p),
                ("cond_slice_tokens", ctypes.c_int64),
                ("uncond_k_slice", ctypes.c_void_p), ("uncond_v_slice", ctypes.c_void_p),
                ("uncond_slice_tokens", ctypes.c_int64),
                ("z", ctypes.c_void_p), ("n_video", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("h", ctypes.POINTER(ctypes.c_float)), ("guidance", ctypes.c_float)]


class _UnitLayersIO(ctypes.Structure):
    _fields_ = [("caches", ctypes.POINTER(ctypes.POINTER(_Cache))),
                ("k_slices", ctypes.POINTER(ctypes.c_void_p)),
                ("v_slices", ctypes.POINTER(ctypes.c_void_p)),
                ("slice_tokens", ctypes.c_int64), ("z", ctypes.c_void_p),
                ("n_video", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("h", ctypes.POINTER(ctypes.c_float))]


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_kv_append = _sig("fmd_kv_append", ctypes.c_int, ctypes.POINTER(_Cache), _vp, _vp, _i64, _vp)
_kv_append_batched = _sig("fmd_kv_append_batched", ctypes.c_int,
                          ctypes.POINTER(ctypes.POINTER(_Cache)), ctypes.POINTER(_vp),
                          ctypes.POINTER(_vp), ctypes.POINTER(_i64), _i32, _vp)
_workspace_bytes = _sig("fmd_workspace_bytes", ctypes.c_int, ctypes.POINTER(_UnitStep), _i32,
                        ctypes.POINTER(_sz))
_denoise_step = _sig("fmd_denoise_step", ctypes.c_int, ctypes.POINTER(_UnitStep), _i32, _vp, _vp,
                     _sz, _vp)
_attention = _sig("fmd_attention", ctypes.c_int, ctypes.POINTER(_UnitStep), _i32, _vp, _vp, _sz,
                  _vp)
_unit_workspace_bytes = _sig("fmd_unit_workspace_bytes", ctypes.c_int, ctypes.POINTER(_UnitIO),
                             _i32, _i32, ctypes.POINTER(_sz))
_denoise_unit = _sig("fmd_denoise_unit", ctypes.c_int, ctypes.POINTER(_UnitIO), _i32, _i32, _vp,
                     _vp, _sz, _vp)
_denoise_unit_noalloc = _sig("fmd_denoise_unit_noalloc", ctypes.c_int, ctypes.POINTER(_UnitIO),
                            _i32, _i32, _vp, _vp)
FMD_NOALLOC_SCRATCH_BYTES = 256 << 20
_unit_qkv_workspace_bytes = _sig("fmd_unit_qkv_workspace_bytes", ctypes.c_int,
                                 ctypes.POINTER(_UnitQkvIO), _i32, ctypes.POINTER(_sz))
_denoise_unit_qkv = _sig("fmd_denoise_unit_qkv", ctypes.c_int, ctypes.POINTER(_UnitQkvIO), _i32,
                         _i32, _vp, _vp, _vp, _sz, _vp)
_unit_cfg_workspace_bytes = _sig("fmd_unit_cfg_workspace_bytes", ctypes.c_int,
                                 ctypes.POINTER(_UnitCfgIO), _i32, ctypes.POINTER(_sz))
_denoise_unit_cfg = _sig("fmd_denoise_unit_cfg", ctypes.c_int, ctypes.POINTER(_UnitCfgIO), _i32,
                         _i32, _vp, _vp, _vp, _sz, _vp)
_unit_layers_workspace_bytes = _sig("fmd_unit_layers_workspace_bytes", ctypes.c_int,
                                    ctypes.POINTER(_UnitLayersIO), _i32, _i32,
                                    ctypes.POINTER(_sz))
_denoise_unit_layers = _sig("fmd_denoise_unit_layers", ctypes.c_int, ctypes.POINTER(_UnitLayersIO),
                            _i32, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _sz,
                            _vp)
_strerror = _sig("fmd_strerror", ctypes.c_char_p, ctypes.c_int)
_last_error = _sig("fmd_last_error", ctypes.c_char_p)
_profile_enable = _sig("fmd_profile_enable", ctypes.c_int, ctypes.c_int)
_profile_select = _sig("fmd_profile_select", ctypes.c_int, ctypes.c_uint32)
_profile_read = _sig("fmd_profile_read", ctypes.c_int, ctypes.c_int,
                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64))
_version = _sig("fmd_version", ctypes.c_char_p)
_test_force_attn_groups = _sig("fmd_test_force_attn_groups", ctypes.c_int, _i32)

EXPORTED = ["fmd_kv_append", "fmd_kv_append_batched", "fmd_workspace_bytes", "fmd_denoise_step",
            "fmd_attention", "fmd_unit_workspace_bytes", "fmd_denoise_unit",
            "fmd_denoise_unit_noalloc",
            "fmd_unit_qkv_workspace_bytes", "fmd_denoise_unit_qkv",
            "fmd_unit_cfg_workspace_bytes", "fmd_denoise_unit_cfg",
            "fmd_unit_layers_workspace_bytes", "fmd_denoise_unit_layers", "fmd_strerror",
            "fmd_last_error", "fmd_profile_enable", "fmd_profile_select", "fmd_profile_read",
            "fmd_version", "fmd_test_force_attn_groups"]


def _check(rc: int):
    if rc != 0:
        raise FmdError(rc, _last_error().decode(errors="replace") or _strerror(rc).decode())


def strerror(code: int) -> str:
    return _strerror(code).decode()


def version() -> str:
    return _version().decode()


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect_shape(t, shape, name):
    """Raise ValueError unless tensor t has exactly this shape.  The C ABI
    receives bare pointers, so every extent it relies on is checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _expect_slices(k_slice, v_slice, H, hd, name="slice"):
    if (k_slice is None) != (v_slice is None):
        raise ValueError(f"k_{name} and v_{name} must both be given or both be None")
    if k_slice is None:
        return 0
    if k_slice.dim() != 3:
        raise ValueError(f"k_{name} must be [T][H][hd], got {tuple(k_slice.shape)}")
    T = k_slice.shape[0]
    _expect_shape(k_slice, (T, H, hd), f"k_{name}")
    _expect_shape(v_slice, (T, H, hd), f"v_{name}")
    return T


def _sync_workspace(workspace, stream):
    # A workspace allocated on torch's current stream but used on another one
    # must not be recycled by the caching allocator before that stream is done.
    if stream is not None and stream != torch.cuda.current_stream(workspace.device):
        workspace.record_stream(stream)


class KVCache:
    """One session's ring: device tensors k [H][cap][hd] and v
    [H][cap/16][hd][16] (bf16), plus the host-side (len, head) state that the
    library advances on every append."""

    def __init__(self, n_heads: int, head_dim: int, cap_tokens: int, device="cuda",
                 k: torch.Tensor | None = None, v: torch.Tensor | None = None,
                 len_tokens: int = 0, head_tokens: int = 0):
        if k is None:
            k = torch.empty((n_heads, cap_tokens, head_dim), dtype=torch.bfloat16, device=device)
        if v is None:
            v = torch.empty((n_heads, cap_tokens // FMD_CACHE_BLOCK, head_dim, FMD_CACHE_BLOCK),
                            dtype=torch.bfloat16, device=device)
        _expect_shape(k, (n_heads, cap_tokens, head_dim), "k")
        if cap_tokens % FMD_CACHE_BLOCK:
            raise ValueError(f"cap_tokens {cap_tokens} must be a multiple of {FMD_CACHE_BLOCK}")
        _expect_shape(v, (n_heads, cap_tokens // FMD_CACHE_BLOCK, head_dim, FMD_CACHE_BLOCK), "v")
        self.k, self.v = k, v
        self._c = _Cache(_ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"), n_heads,
                         head_dim, cap_tokens, len_tokens, head_tokens)

    n_heads = property(lambda self: self._c.n_heads)
    head_dim = property(lambda self: self._c.head_dim)
    cap_tokens = property(lambda self: self._c.cap_tokens)

    @property
    def len_tokens(self):
        return self._c.len_tokens

    @property
    def head_tokens(self):
        return self._c.head_tokens

    def set_state(self, len_tokens: int, head_tokens: int):
        self._c.len_tokens = len_tokens
        self._c.head_tokens = head_tokens

    @staticmethod
    def logical_to_device_v(v_logical: torch.Tensor) -> torch.Tensor:
        """[H][cap][hd] -> [H][cap/16][hd][16] (the device layout of the V ring)."""
        H, cap, hd = v_logical.shape
        return v_logical.reshape(H, cap // 16, 16, hd).transpose(2, 3).contiguous()

    @staticmethod
    def device_to_logical_v(v_dev: torch.Tensor) -> torch.Tensor:
        H, nb, hd, b = v_dev.shape
        return v_dev.transpose(2, 3).reshape(H, nb * b, hd).contiguous()


def kv_append(cache: KVCache, k_slice, v_slice, stream=None):
    """Append one slice [T][H][hd] (bf16) to the ring; advances len/head."""
    if k_slice is None or v_slice is None:
        raise ValueError("k_slice and v_slice are required")
    _expect_slices(k_slice, v_slice, cache.n_heads, cache.head_dim)
    _check(_kv_append(ctypes.byref(cache._c), _ptr(k_slice, torch.bfloat16, "k_slice"),
                      _ptr(v_slice, torch.bfloat16, "v_slice"), k_slice.shape[0],
                      _stream_ptr(stream)))


def kv_append_batched(caches, k_slices, v_slices, stream=None):
    n = len(caches)
    if len(k_slices) != n or len(v_slices) != n:
        raise ValueError("one K and one V slice per cache")
    for c, k, v in zip(caches, k_slices, v_slices):
        if k is None or v is None:
            raise ValueError("k_slices and v_slices must not hold None")
        _expect_slices(k, v, c.n_heads, c.head_dim)
    arr_c = (ctypes.POINTER(_Cache) * n)(*[ctypes.pointer(c._c) for c in caches])
    arr_k = (_vp * n)(*[_ptr(t, torch.bfloat16, "k_slice") for t in k_slices])
    arr_v = (_vp * n)(*[_ptr(t, torch.bfloat16, "v_slice") for t in v_slices])
    arr_t = (_i64 * n)(*[t.shape[0] for t in k_slices])
    _check(_kv_append_batched(arr_c, arr_k, arr_v, arr_t, n, _stream_ptr(stream)))


class PreparedAppend:
    """``kv_append_batched`` with its argument arrays built once, for loops
    that append from the same slice buffers into the same caches every time:
    ``launch()`` only enqueues.  The caches' host state (len, head) is read and
    advanced by each launch, as with ``kv_append_batched``."""

    def __init__(self, caches, k_slices, v_slices):
        n = len(caches)
        if len(k_slices) != n or len(v_slices) != n:
            raise ValueError("one K and one V slice per cache")
        for c, k, v in zip(caches, k_slices, v_slices):
            if k is None or v is None:
                raise ValueError("k_slices and v_slices must not hold None")
            _expect_slices(k, v, c.n_heads, c.head_dim)
        self._keep = (list(caches), list(k_slices), list(v_slices))
        self._args = ((ctypes.POINTER(_Cache) * n)(*[ctypes.pointer(c._c) for c in caches]),
                      (_vp * n)(*[_ptr(t, torch.bfloat16, "k_slice") for t in k_slices]),
                      (_vp * n)(*[_ptr(t, torch.bfloat16, "v_slice") for t in v_slices]),
                      (_i64 * n)(*[t.shape[0] for t in k_slices]), n)

    def launch(self, stream=None):
        _check(_kv_append_batched(*self._args, _stream_ptr(stream)))


class UnitStep:
    """One session's inputs for one solver step (see ``fmd_unit_step``)."""

    def __init__(self, cache: KVCache, q, k_u, v_u, z=None, n_video=None, n_audio=0, h=1.0):
        self.cache, self.q, self.k_u, self.v_u, self.z = cache, q, k_u, v_u, z
        H, hd = cache.n_heads, cache.head_dim
        if q.dim() != 3:
            raise ValueError(f"q must be [n_q][H][hd], got {tuple(q.shape)}")
        n_q = q.shape[0]
        for t, nm in ((q, "q"), (k_u, "k_u"), (v_u, "v_u")):
            _expect_shape(t, (n_q, H, hd), nm)
        _expect_shape(z, (n_q, H * hd), "z")
        self.n_video = n_q - n_audio if n_video is None else n_video
        self.n_audio = n_audio
        if self.n_video + self.n_audio != n_q:
            raise ValueError(f"n_video + n_audio = {self.n_video + self.n_audio} != n_q = {n_q}")
        self.h = h

    def _struct(self):
        return _UnitStep(ctypes.pointer(self.cache._c), _ptr(self.q, torch.bfloat16, "q"),
                         _ptr(self.k_u, torch.bfloat16, "k_u"),
                         _ptr(self.v_u, torch.bfloat16, "v_u"),
                         _ptr(self.z, torch.float32, "z", allow_none=True),
                         self.n_video, self.n_audio, self.h)


def _steps_array(units):
    n = len(units)
    return (_UnitStep * n)(*[u._struct() for u in units]), n


def workspace_bytes(units) -> int:
    arr, n = _steps_array(units)
    out = _sz(0)
    _check(_workspace_bytes(arr, n, ctypes.byref(out)))
    return out.value


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to 512 bytes.
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def attention(units, o_out=None, workspace=None, stream=None):
    """O = attention of every session (bf16 [sum n_q][H][hd]).  Test entry."""
    arr, n = _steps_array(units)
    H, hd = units[0].cache.n_heads, units[0].cache.head_dim
    rows = sum(u.q.shape[0] for u in units)
    if o_out is None:
        o_out = torch.empty((rows, H, hd), dtype=torch.bfloat16, device=units[0].q.device)
    _expect_shape(o_out, (rows, H, hd), "o_out")
    need = _sz(0)
    _check(_workspace_bytes(arr, n, ctypes.byref(need)))
    if workspace is None:
        workspace = alloc_workspace(need.value, units[0].q.device)
    _sync_workspace(workspace, stream)
    _check(_attention(arr, n, _ptr(o_out, torch.bfloat16, "o_out"),
                      workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
    return o_out


def denoise_step(units, w_o, workspace=None, stream=None):
    """One solver step for every session: z <- z - h * (attention(...) W_o^T)."""
    d = units[0].cache.n_heads * units[0].cache.head_dim
    _expect_shape(w_o, (d, d), "w_o")
    if any(u.z is None for u in units):
        raise ValueError("every unit needs its latent z for a solver step")
    arr, n = _steps_array(units)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(units), units[0].q.device)
    _sync_workspace(workspace, stream)
    _check(_denoise_step(arr, n, _ptr(w_o, torch.bfloat16, "w_o"), workspace.data_ptr(),
                         workspace.numel(), _stream_ptr(stream)))


class UnitIO:
    """One session's inputs for a whole unit (see ``fmd_unit_io``).

    q, k_u, v_u: bf16 [S][n_q][H][hd] (one set per step) or [n_q][H][hd]
    (reused for every step); z: float32 [n_q][d], eps in, final latent out;
    h: step sizes."""

    def __init__(self, cache: KVCache, k_slice, v_slice, q, k_u, v_u, z, h, n_audio=0):
        self.cache, self.k_slice, self.v_slice = cache, k_slice, v_slice
        self.q, self.k_u, self.v_u, self.z = q, k_u, v_u, z
        self.h = (ctypes.c_float * len(h))(*[float(x) for x in h])
        self.n_steps = len(h)
        H, hd = cache.n_heads, cache.head_dim
        if q.dim() not in (3, 4):
            raise ValueError(f"q must be [S][n_q][H][hd] or [n_q][H][hd], got {tuple(q.shape)}")
        per_step = q.dim() == 4
        self.n_q = q.shape[1] if per_step else q.shape[0]
        if per_step and q.shape[0] < self.n_steps:
            raise ValueError(f"q holds {q.shape[0]} steps, {self.n_steps} step sizes given")
        for t, nm in ((q, "q"), (k_u, "k_u"), (v_u, "v_u")):
            _expect_shape(t, tuple(q.shape[:-2]) + (H, hd), nm)
        _expect_shape(z, (self.n_q, H * hd), "z")
        _expect_slices(k_slice, v_slice, H, hd)
        if not 0 <= n_audio <= self.n_q:
            raise ValueError(f"n_audio {n_audio} outside 0..n_q={self.n_q}")
        self.stride = q[0].numel() if per_step else 0
        self.n_audio = n_audio

    def _struct(self):
        T = 0 if self.k_slice is None else self.k_slice.shape[0]
        return _UnitIO(ctypes.pointer(self.cache._c),
                       _ptr(self.k_slice, torch.bfloat16, "k_slice", allow_none=True),
                       _ptr(self.v_slice, torch.bfloat16, "v_slice", allow_none=True), T,
                       _ptr(self.q, torch.bfloat16, "q"), _ptr(self.k_u, torch.bfloat16, "k_u"),
                       _ptr(self.v_u, torch.bfloat16, "v_u"), self.stride,
                       _ptr(self.z, torch.float32, "z"), self.n_q - self.n_audio, self.n_audio,
                       ctypes.cast(self.h, ctypes.POINTER(ctypes.c_float)))


def _io_array(sessions):
    n = len(sessions)
    return (_UnitIO * n)(*[s._struct() for s in sessions]), n


def unit_workspace_bytes(sessions) -> int:
    arr, n = _io_array(sessions)
    out = _sz(0)
    _check(_unit_workspace_bytes(arr, n, sessions[0].n_steps, ctypes.byref(out)))
    return out.value


def denoise_unit(sessions, w_o, workspace=None, stream=None):
    """Append every session's slice, then run the S solver steps."""
    n_steps = sessions[0].n_steps
    if any(s.n_steps != n_steps for s in sessions):
        raise ValueError("all sessions must have the same number of steps")
    d = sessions[0].cache.n_heads * sessions[0].cache.head_dim
    _expect_shape(w_o, (d, d), "w_o")
    if workspace is None:
        workspace = alloc_workspace(unit_workspace_bytes(sessions), sessions[0].z.device)
    _sync_workspace(workspace, stream)
    arr, n = _io_array(sessions)
    _check(_denoise_unit(arr, n, n_steps, _ptr(w_o, torch.bfloat16, "w_o"), workspace.data_ptr(),
                         workspace.numel(), _stream_ptr(stream)))
    # The library advanced each cache's (len, head) in the struct array it was
    # given; the array holds pointers to the caches' own structs, so nothing to copy.


def denoise_unit_noalloc(sessions, w_o, stream=None):
    """denoise_unit without a workspace: the library's static device scratch
    (FMD_NOALLOC_SCRATCH_BYTES per GPU) holds the kernels' scratch, so the call
    allocates no device memory.  Calls that overlap on one GPU race."""
    n_steps = sessions[0].n_steps
    if any(s.n_steps != n_steps for s in sessions):
        raise ValueError("all sessions must have the same number of steps")
    d = sessions[0].cache.n_heads * sessions[0].cache.head_dim
    _expect_shape(w_o, (d, d), "w_o")
    arr, n = _io_array(sessions)
    _check(_denoise_unit_noalloc(arr, n, n_steps, _ptr(w_o, torch.bfloat16, "w_o"),
                                 _stream_ptr(stream)))


class UnitQkvIO:
    """One session's inputs for a unit of the z-dependent solver (see
    ``fmd_unit_qkv_io``): Q, K_u, V_u are projected from z by the library at
    every step.  z: float32 [n_q][d], eps in, final latent out; h: step sizes."""

    def __init__(self, cache: KVCache, k_slice, v_slice, z, h, n_audio=0):
        self.cache, self.k_slice, self.v_slice, self.z = cache, k_slice, v_slice, z
        self.h = (ctypes.c_float * len(h))(*[float(x) for x in h])
        self.n_steps = len(h)
        self.n_q = z.shape[0]
        _expect_shape(z, (self.n_q, cache.n_heads * cache.head_dim), "z")
        _expect_slices(k_slice, v_slice, cache.n_heads, cache.head_dim)
        if not 0 <= n_audio <= self.n_q:
            raise ValueError(f"n_audio {n_audio} outside 0..n_q={self.n_q}")
        self.n_audio = n_audio

    def _struct(self):
        T = 0 if self.k_slice is None else self.k_slice.shape[0]
        return _UnitQkvIO(ctypes.pointer(self.cache._c),
                          _ptr(self.k_slice, torch.bfloat16, "k_slice", allow_none=True),
                          _ptr(self.v_slice, torch.bfloat16, "v_slice", allow_none=True), T,
                          _ptr(self.z, torch.float32, "z"), self.n_q - self.n_audio, self.n_audio,
                          ctypes.cast(self.h, ctypes.POINTER(ctypes.c_float)))


def _qkv_array(sessions):
    n = len(sessions)
    return (_UnitQkvIO * n)(*[s._struct() for s in sessions]), n


def unit_qkv_workspace_bytes(sessions) -> int:
    arr, n = _qkv_array(sessions)
    out = _sz(0)
    _check(_unit_qkv_workspace_bytes(arr, n, ctypes.byref(out)))
    return out.value


def denoise_unit_qkv(sessions, w_qkv, w_o, workspace=None, stream=None):
    """Append every session's slice, then run the S solver steps, each
    projecting the unit's Q, K_u, V_u from the current latent (W_qkv bf16
    [3d][d])."""
    n_steps = sessions[0].n_steps
    if any(s.n_steps != n_steps for s in sessions):
        raise ValueError("all sessions must have the same number of steps")
    d = sessions[0].cache.n_heads * sessions[0].cache.head_dim
    _expect_shape(w_qkv, (3 * d, d), "w_qkv")
    _expect_shape(w_o, (d, d), "w_o")
    if workspace is None:
        workspace = alloc_workspace(unit_qkv_workspace_bytes(sessions), sessions[0].z.device)
    _sync_workspace(workspace, stream)
    arr, n = _qkv_array(sessions)
    _check(_denoise_unit_qkv(arr, n, n_steps, _ptr(w_qkv, torch.bfloat16, "w_qkv"),
                             _ptr(w_o, torch.bfloat16, "w_o"), workspace.data_ptr(),
                             workspace.numel(), _stream_ptr(stream)))


class UnitCfgIO:
    """One unit's inputs for the classifier-free-guided solver (see
    ``fmd_unit_cfg_io``): the conditional and the unconditional branch's caches
    and slices, the latent z (float32 [n_q][d], eps in, final latent out), the
    step sizes h and the guidance scale g."""

    def __init__(self, cond: KVCache, uncond: KVCache, z, h, guidance, cond_slice=(None, None),
                 uncond_slice=(None, None), n_audio=0):
        self.cond, self.uncond, self.z = cond, uncond, z
        self.cond_slice, self.uncond_slice = cond_slice, uncond_slice
        self.h = (ctypes.c_float * len(h))(*[float(x) for x in h])
        self.n_steps = len(h)
        self.n_q = z.shape[0]
        H, hd = cond.n_heads, cond.head_dim
        _expect_shape(z, (self.n_q, H * hd), "z")
        _expect_slices(*cond_slice, H, hd, "cond_slice")
        _expect_slices(*uncond_slice, uncond.n_heads, uncond.head_dim, "uncond_slice")
        if not 0 <= n_audio <= self.n_q:
            raise ValueError(f"n_audio {n_audio} outside 0..n_q={self.n_q}")
        self.n_audio = n_audio
        self.guidance = float(guidance)

    def _struct(self):
        def sl(pair, name):
            k, v = pair
            T = 0 if k is None else k.shape[0]
            return (_ptr(k, torch.bfloat16, name + "_k_slice", allow_none=True),
                    _ptr(v, torch.bfloat16, name + "_v_slice", allow_none=True), T)
        return _UnitCfgIO(ctypes.pointer(self.cond._c), ctypes.pointer(self.uncond._c),
                          *sl(self.cond_slice, "cond"), *sl(self.uncond_slice, "uncond"),
                          _ptr(self.z, torch.float32, "z"), self.n_q - self.n_audio, self.n_audio,
                          ctypes.cast(self.h, ctypes.POINTER(ctypes.c_float)), self.guidance)


def _cfg_array(sessions):
    n = len(sessions)
    return (_UnitCfgIO * n)(*[s._struct() for s in sessions]), n


def unit_cfg_workspace_bytes(sessions) -> int:
    arr, n = _cfg_array(sessions)
    out = _sz(0)
    _check(_unit_cfg_workspace_bytes(arr, n, ctypes.byref(out)))
    return out.value


def denoise_unit_cfg(sessions, w_qkv, w_o, workspace=None, stream=None):
    """Append every branch's slice, then run the S guided solver steps: per
    step one Q/K/V projection of each unit's latent, attention over both
    branches' caches, the guided mix and one projection with the Euler
    update."""
    n_steps = sessions[0].n_steps
    if any(s.n_steps != n_steps for s in sessions):
        raise ValueError("all sessions must have the same number of steps")
    d = sessions[0].cond.n_heads * sessions[0].cond.head_dim
    _expect_shape(w_qkv, (3 * d, d), "w_qkv")
    _expect_shape(w_o, (d, d), "w_o")
    if workspace is None:
        workspace = alloc_workspace(unit_cfg_workspace_bytes(sessions), sessions[0].z.device)
    _sync_workspace(workspace, stream)
    arr, n = _cfg_array(sessions)
    _check(_denoise_unit_cfg(arr, n, n_steps, _ptr(w_qkv, torch.bfloat16, "w_qkv"),
                             _ptr(w_o, torch.bfloat16, "w_o"), workspace.data_ptr(),
                             workspace.numel(), _stream_ptr(stream)))


class UnitLayersIO:
    """One session's inputs for a unit of the layer-stack solver (see
    ``fmd_unit_layers_io``): one ring per layer, one K/V slice per layer (or
    none), the latent z (float32 [n_q][d], eps in, final latent out) and the
    step sizes h."""

    def __init__(self, caches, z, h, k_slices=None, v_slices=None, n_audio=0):
        self.caches, self.z = list(caches), z
        self.k_slices = list(k_slices) if k_slices is not None else None
        self.v_slices = list(v_slices) if v_slices is not None else None
        self.h = (ctypes.c_float * len(h))(*[float(x) for x in h])
        self.n_steps = len(h)
        self.n_q = z.shape[0]
        H, hd = self.caches[0].n_heads, self.caches[0].head_dim
        _expect_shape(z, (self.n_q, H * hd), "z")
        if (self.k_slices is None) != (self.v_slices is None):
            raise ValueError("k_slices and v_slices must both be given or both be None")
        if self.k_slices is not None:
            if len(self.k_slices) != len(self.caches) or len(self.v_slices) != len(self.caches):
                raise ValueError("one K and one V slice per layer")
            Ts = {_expect_slices(k, v, c.n_heads, c.head_dim, "slices")
                  for k, v, c in zip(self.k_slices, self.v_slices, self.caches)}
            if len(Ts) != 1:
                raise ValueError("every layer appends the same number of tokens")
        if not 0 <= n_audio <= self.n_q:
            raise ValueError(f"n_audio {n_audio} outside 0..n_q={self.n_q}")
        self.n_audio = n_audio

    def _struct(self):
        L = len(self.caches)
        self._c_arr = (ctypes.POINTER(_Cache) * L)(*[ctypes.pointer(c._c) for c in self.caches])
        T = 0
        if self.k_slices is not None:
            if len(self.k_slices) != L or len(self.v_slices) != L:
                raise ValueError("one K and one V slice per layer")
            T = self.k_slices[0].shape[0]
            if any(k.shape[0] != T for k in self.k_slices + self.v_slices):
                raise ValueError("every layer appends the same number of tokens")
            self._k_arr = (_vp * L)(*[_ptr(k, torch.bfloat16, "k_slice") for k in self.k_slices])
            self._v_arr = (_vp * L)(*[_ptr(v, torch.bfloat16, "v_slice") for v in self.v_slices])
            kp, vp = self._k_arr, self._v_arr
        else:
            kp = vp = None
        return _UnitLayersIO(self._c_arr, kp, vp, T, _ptr(self.z, torch.float32, "z"),
                             self.n_q - self.n_audio, self.n_audio,
                             ctypes.cast(self.h, ctypes.POINTER(ctypes.c_float)))


def _layers_array(sessions):
    n = len(sessions)
    L = len(sessions[0].caches)
    if any(len(s.caches) != L for s in sessions):
        raise ValueError("every session has the same number of layers")
    return (_UnitLayersIO * n)(*[s._struct() for s in sessions]), n, L


def unit_layers_workspace_bytes(sessions) -> int:
    arr, n, L = _layers_array(sessions)
    out = _sz(0)
    _check(_unit_layers_workspace_bytes(arr, n, L, ctypes.byref(out)))
    return out.value


def denoise_unit_layers(sessions, w_qkv, w_o, workspace=None, stream=None):
    """Append every layer's slice, then run the S solver steps through the
    layer stack (w_qkv, w_o: one bf16 weight tensor per layer)."""
    n_steps = sessions[0].n_steps
    if any(s.n_steps != n_steps for s in sessions):
        raise ValueError("all sessions must have the same number of steps")
    L = len(sessions[0].caches)
    if len(w_qkv) != L or len(w_o) != L:
        raise ValueError("one W_qkv and one W_o per layer")
    d = sessions[0].caches[0].n_heads * sessions[0].caches[0].head_dim
    for w in w_qkv:
        _expect_shape(w, (3 * d, d), "w_qkv")
    for w in w_o:
        _expect_shape(w, (d, d), "w_o")
    if workspace is None:
        workspace = alloc_workspace(unit_layers_workspace_bytes(sessions), sessions[0].z.device)
    _sync_workspace(workspace, stream)
    arr, n, L = _layers_array(sessions)
    wq = (_vp * L)(*[_ptr(w, torch.bfloat16, "w_qkv") for w in w_qkv])
    wo = (_vp * L)(*[_ptr(w, torch.bfloat16, "w_o") for w in w_o])
    _check(_denoise_unit_layers(arr, n, L, n_steps, wq, wo, workspace.data_ptr(),
                                workspace.numel(), _stream_ptr(stream)))


class forced_attn_groups:
    """Test helper: ``with forced_attn_groups(n): ...`` runs the enclosed calls
    with every attention launch's window sequence cut into n ranges (see
    ``fmd_test_force_attn_groups``); ``None`` leaves the planner's choice."""

    def __init__(self, n_groups):
        self.n = n_groups

    def __enter__(self):
        if self.n is not None:
            _check(_test_force_attn_groups(int(self.n)))
        return self

    def __exit__(self, *exc):
        if self.n is not None:
            _check(_test_force_attn_groups(0))
        return False


def profile_enable(on: bool = True, classes=None):
    """Turn per-launch event timing on (clearing earlier records) or off.
    `classes`: names from KERNEL_CLASSES to record (default: all)."""
    mask = (1 << len(KERNEL_CLASSES)) - 1
    if classes is not None:
        mask = 0
        for c in classes:
            mask |= 1 << KERNEL_CLASSES[c]
    _check(_profile_select(mask))
    _check(_profile_enable(1 if on else 0))


def profile_read(kernel: str):
    ms, n = ctypes.c_double(0), _i64(0)
    _check(_profile_read(KERNEL_CLASSES[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
