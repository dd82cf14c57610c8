"""Seeded synthetic inputs for the performer's per-unit denoise step.

This module only draws random numbers, rounds them to bf16 and lays them out.
It holds none of the method's arithmetic (no append, no attention, no
projection, no Euler update), so both the CPU oracle and the GPU path can take
their inputs from it without sharing any of the computation.

Recipe (the pages publish no dataset or trained weights; these tensors stand in
for the thinker's K/V and the VAE latents at the pages' shapes):

* every tensor is drawn per (session, tensor name, head) from its own
  ``numpy.random.PCG64`` stream, seeded by ``SeedSequence([seed, session,
  tensor_id, head])``, so heads can be drawn in parallel threads and any single
  head can be regenerated alone;
* values are standard normal float32, rounded to bf16 with round-to-nearest-even
  (the projection weight is scaled by ``d**-0.5`` before rounding, i.e. its
  variance is ``1/d``); the start latent ``eps`` stays float32;
* ring slots that are not valid before the append may be filled with a bf16 NaN
  (``0x7FC0``) so that any read of them shows in the output;
* a guided unit's unconditional branch has the conditional branch's shapes
  and ring state, its ring and slice drawn from streams of their own
  (``uncond_*`` tensor ids).

Shapes follow the two resolutions the pages name (192x336 and 640x368 at 25 FPS,
160 ms units) with the token-count assumptions stated beside each workload.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# Stable ids so the stream of a tensor never depends on the draw order.
_TENSOR_IDS = {
    "ring_k": 1, "ring_v": 2, "slice_k": 3, "slice_v": 4,
    "q": 5, "k_u": 6, "v_u": 7, "eps": 8, "z0": 9, "w_o": 10, "w_qkv": 11,
    "uncond_ring_k": 12, "uncond_ring_v": 13, "uncond_slice_k": 14, "uncond_slice_v": 15,
}

# Guidance scale of the guided (teacher) sampler's workloads.  The pages give
# none; the cost of a step does not depend on it.
CFG_GUIDANCE = 5.0


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite normals, so no NaN/Inf handling is needed here."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _stream(seed: int, session: int, name: str, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, session, _TENSOR_IDS[name], head])))


def _normal_f32(seed, session, name, head, shape, scale=1.0):
    g = _stream(seed, session, name, head)
    a = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def _per_head(fn, n_heads):
    """Run fn(h) for every head, in threads (numpy releases the GIL)."""
    if n_heads == 1:
        return [fn(0)]
    with _cf.ThreadPoolExecutor(min(_threads(), n_heads)) as ex:
        return list(ex.map(fn, range(n_heads)))


@dataclass(frozen=True)
class SessionShape:
    """One session's shapes and ring state for one denoised unit.

    ``len_before``/``head_before`` are the ring state before the unit's append;
    ``slice_tokens == 0`` means the unit appends nothing."""
    n_heads: int
    head_dim: int
    n_video: int
    n_audio: int
    slice_tokens: int
    cap_tokens: int
    len_before: int
    head_before: int
    h: tuple  # step sizes, one per solver step (positive magnitudes)

    @property
    def n_q(self) -> int:
        return self.n_video + self.n_audio

    @property
    def d(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_steps(self) -> int:
        return len(self.h)

    @property
    def len_after(self) -> int:
        return min(self.len_before + self.slice_tokens, self.cap_tokens)

    @property
    def head_after(self) -> int:
        return (self.head_before + self.slice_tokens) % self.cap_tokens

    @property
    def keys_per_query(self) -> int:
        return self.len_after + self.n_q


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    seed: int
    sessions: tuple

    @property
    def n_heads(self):
        return self.sessions[0].n_heads

    @property
    def head_dim(self):
        return self.sessions[0].head_dim

    @property
    def d(self):
        return self.sessions[0].d

    @property
    def n_steps(self):
        return self.sessions[0].n_steps

    def attention_flops_per_step(self) -> float:
        return float(sum(4 * s.n_q * s.keys_per_query * s.d for s in self.sessions))

    def projection_flops_per_step(self) -> float:
        return float(sum(2 * s.n_q * s.d * s.d for s in self.sessions))

    def kv_bytes_per_step(self) -> float:
        """K and V of every key each query attends to, read once, bf16."""
        return float(sum(2 * 2 * s.keys_per_query * s.d for s in self.sessions))

    def append_bytes(self) -> float:
        """Bytes read plus written by the unit's append (K and V, bf16)."""
        return float(sum(2 * 2 * 2 * s.slice_tokens * s.d for s in self.sessions))


def _unit_session(n_heads, head_dim, n_video, n_audio, T, units_cap, units_before,
                  head_units, h):
    return SessionShape(n_heads, head_dim, n_video, n_audio, T, units_cap * T,
                        units_before * T, (head_units * T) % (units_cap * T), tuple(h))


def _batch8_sessions(seed: int):
    # Ring lengths and offsets come from their own stream, so shapes never
    # shift the tensor values.
    g = np.random.Generator(np.random.PCG64(seed + 1000))
    out = []
    for _ in range(8):
        L = int(g.integers(8, 129))            # units, inclusive 8..128
        head_u = int(g.integers(0, L))          # units, 0..L-1
        out.append(_unit_session(40, 128, 920, 8, 944, L, L, head_u,
                                 (0.4, 0.3, 0.2, 0.1)))
    return tuple(out)


def _build():
    w = {}
    w["tiny"] = Workload(
        "tiny",
        "2 heads x 64, 12 video + 4 audio queries, full 128-key cache "
        "(4 prior units x 32 tokens), no append, one Euler step of size 1",
        0, (SessionShape(2, 64, 12, 4, 0, 128, 128, 0, (1.0,)),))
    w["v01_unit"] = Workload(
        "v01_unit",
        "192x336-class unit: 12x21=252 video (16x spatial, 1 latent frame per "
        "160 ms unit) + 8 audio queries, 12 heads x 128, 32-unit ring of 268-token "
        "slices filled by this unit's append, 4 steps of 0.25",
        1, (_unit_session(12, 128, 252, 8, 268, 32, 31, 31, (0.25,) * 4),))
    w["v02_unit"] = Workload(
        "v02_unit",
        "640x368-class unit: 40x23=920 video + 8 audio queries, 40 heads x 128 "
        "(d=5120), 64-unit ring of 944-token slices (60,416 keys) filled by this "
        "unit's append, 4 steps of 0.25",
        2, (_unit_session(40, 128, 920, 8, 944, 64, 63, 63, (0.25,) * 4),))
    w["v02_long"] = Workload(
        "v02_long",
        "640x368-class unit against a 256-unit ring (241,664 keys) that has "
        "wrapped, append offset 100 units, 4 steps of 0.25",
        3, (_unit_session(40, 128, 920, 8, 944, 256, 256, 100, (0.25,) * 4),))
    w["v02_cfg_unit"] = Workload(
        "v02_cfg_unit",
        "640x368-class unit sampled by the guided teacher: conditional and "
        "unconditional 64-unit rings of 944-token slices (60,416 keys each) filled "
        "by this unit's appends, 16 steps of 1/16, guidance scale 5",
        5, (_unit_session(40, 128, 920, 8, 944, 64, 63, 63, (1.0 / 16,) * 16),))
    w["v02_batch8"] = Workload(
        "v02_batch8",
        "8 independent 640x368-class sessions, full rings of 8..128 units of 944 "
        "tokens drawn per session, per-session append offsets, 4 steps "
        "[0.4, 0.3, 0.2, 0.1]",
        4, _batch8_sessions(4))
    return w


WORKLOADS = _build()


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# Tensor draws.  bf16 tensors are returned as uint16 bit patterns.
# ---------------------------------------------------------------------------

def ring_logical(seed, session, s: SessionShape, which: str, poison_invalid=False):
    """Ring content in logical layout [H][cap][hd] (bf16 bits)."""
    assert which in ("ring_k", "ring_v", "uncond_ring_k", "uncond_ring_v")

    def one(h):
        return round_to_bf16_bits(
            _normal_f32(seed, session, which, h, (s.cap_tokens, s.head_dim)))
    out = np.stack(_per_head(one, s.n_heads))
    if poison_invalid and s.len_before < s.cap_tokens:
        valid = np.zeros(s.cap_tokens, dtype=bool)
        idx = (s.head_before - s.len_before + np.arange(s.len_before)) % s.cap_tokens
        valid[idx] = True
        out[:, ~valid, :] = BF16_NAN
    return out


def token_major(seed, session, s: SessionShape, name: str, n_tokens: int, step=None):
    """A [n_tokens][H][hd] bf16 tensor (slice K/V, or per-step Q/K_u/V_u)."""
    sess_key = session if step is None else session * 1000 + step

    def one(h):
        return round_to_bf16_bits(
            _normal_f32(seed, sess_key, name, h, (n_tokens, s.head_dim)))
    return np.ascontiguousarray(np.stack(_per_head(one, s.n_heads), axis=1))


def latent(seed, session, s: SessionShape, name: str):
    """float32 [n_q][d]: eps (start latent) or z0 (clean target)."""
    assert name in ("eps", "z0")

    def one(h):
        return _normal_f32(seed, session, name, h, (s.n_q, s.head_dim))
    return np.ascontiguousarray(np.concatenate(_per_head(one, s.n_heads), axis=1))


def projection_weight(seed, d: int, head_dim: int):
    """bf16 [d_out][d_in], N(0, 1/d); drawn per block of head_dim output rows."""
    n_blocks = d // head_dim

    def one(b):
        return round_to_bf16_bits(
            _normal_f32(seed, 0, "w_o", b, (head_dim, d), scale=d ** -0.5))
    return np.ascontiguousarray(np.concatenate(_per_head(one, n_blocks), axis=0))


def qkv_weight(seed, d: int, head_dim: int):
    """bf16 [3d][d] ([d_out][d_in]), N(0, 1/d): the map from the latent to the
    unit's Q, K_u, V_u; drawn per block of head_dim output rows."""
    n_blocks = 3 * d // head_dim

    def one(b):
        return round_to_bf16_bits(
            _normal_f32(seed, 0, "w_qkv", b, (head_dim, d), scale=d ** -0.5))
    return np.ascontiguousarray(np.concatenate(_per_head(one, n_blocks), axis=0))


@dataclass
class SessionInputs:
    shape: SessionShape
    ring_k: np.ndarray            # [H][cap][hd] bf16 bits, state before the append
    ring_v: np.ndarray
    slice_k: np.ndarray | None    # [T][H][hd]
    slice_v: np.ndarray | None
    q: list = field(default_factory=list)      # per step [n_q][H][hd]
    k_u: list = field(default_factory=list)
    v_u: list = field(default_factory=list)
    eps: np.ndarray | None = None              # [n_q][d] float32


@dataclass
class UnitInputs:
    workload: Workload
    sessions: list
    w_o: np.ndarray                            # [d][d] bf16 bits, [out][in]


def make_inputs(wl: Workload, poison_invalid=False, reuse_step_inputs=False,
                sessions=None) -> UnitInputs:
    """Draw every input of one denoised unit of ``wl``.

    ``reuse_step_inputs`` draws Q/K_u/V_u once and reuses them for every step
    (the step-stride-0 mode); otherwise each step gets independent tensors."""
    seed = wl.seed
    idx = range(len(wl.sessions)) if sessions is None else sessions
    out = []
    for si in idx:
        s = wl.sessions[si]
        rk = ring_logical(seed, si, s, "ring_k", poison_invalid)
        rv = ring_logical(seed, si, s, "ring_v", poison_invalid)
        if s.slice_tokens:
            sk = token_major(seed, si, s, "slice_k", s.slice_tokens)
            sv = token_major(seed, si, s, "slice_v", s.slice_tokens)
        else:
            sk = sv = None
        si_in = SessionInputs(s, rk, rv, sk, sv)
        n_draw = 1 if reuse_step_inputs else s.n_steps
        for st in range(n_draw):
            si_in.q.append(token_major(seed, si, s, "q", s.n_q, step=st))
            si_in.k_u.append(token_major(seed, si, s, "k_u", s.n_q, step=st))
            si_in.v_u.append(token_major(seed, si, s, "v_u", s.n_q, step=st))
        si_in.eps = latent(seed, si, s, "eps")
        out.append(si_in)
    return UnitInputs(wl, out, projection_weight(seed, wl.d, wl.head_dim))


@dataclass
class BranchInputs:
    """The unconditional branch of a guided unit: ring before the append and
    the slice appended to it (same shapes as the conditional branch)."""
    ring_k: np.ndarray
    ring_v: np.ndarray
    slice_k: np.ndarray | None
    slice_v: np.ndarray | None


def uncond_inputs(wl: Workload, session: int, poison_invalid=False) -> BranchInputs:
    s = wl.sessions[session]
    rk = ring_logical(wl.seed, session, s, "uncond_ring_k", poison_invalid)
    rv = ring_logical(wl.seed, session, s, "uncond_ring_v", poison_invalid)
    if s.slice_tokens:
        sk = token_major(wl.seed, session, s, "uncond_slice_k", s.slice_tokens)
        sv = token_major(wl.seed, session, s, "uncond_slice_v", s.slice_tokens)
    else:
        sk = sv = None
    return BranchInputs(rk, rv, sk, sv)


def custom_session(n_heads, head_dim, n_video, n_audio, slice_tokens, cap_tokens,
                   len_before, head_before, h):
    return SessionShape(n_heads, head_dim, n_video, n_audio, slice_tokens, cap_tokens,
                        len_before, head_before, tuple(h))


def custom_workload(name, seed, sessions):
    return Workload(name, name, seed, tuple(sessions))
