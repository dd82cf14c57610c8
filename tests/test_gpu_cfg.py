"""GPU parity of the classifier-free-guided solver (two branches per unit that
differ only in their K/V cache, guided velocity v_u + g (v_c - v_u)) against
the oracle, its g = 1 / g = 0 limits against the single-branch solver, and a
closed form on the GPU."""
import numpy as np
import pytest

import oracle
import workload
from tests.pins import random_bits

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import (DEV, assert_close, cache_logical, dev_bf16, host_f64,  # noqa: E402
                            make_cache)

pytestmark = pytest.mark.gpu


def _branch(si_ring_k, si_ring_v, slice_k, slice_v, s):
    return dict(ring_k=si_ring_k, ring_v=si_ring_v, length=s.len_before, head=s.head_before,
                slice_k=slice_k, slice_v=slice_v)


def _inputs(wl):
    ui = workload.make_inputs(wl, poison_invalid=True, reuse_step_inputs=True)
    uns = [workload.uncond_inputs(wl, i, poison_invalid=True) for i in range(len(wl.sessions))]
    w_qkv = workload.qkv_weight(wl.seed, wl.d, wl.head_dim)
    return ui, uns, w_qkv


def _run(wl, ui, uns, w_qkv, hs, gs):
    out = []
    ios = []
    for si, un, g in zip(ui.sessions, uns, gs):
        s = si.shape
        cc = make_cache(fmd, s, si.ring_k, si.ring_v)
        uc = make_cache(fmd, s, un.ring_k, un.ring_v)
        z = torch.from_numpy(si.eps.copy()).to(DEV)
        cs = (dev_bf16(si.slice_k), dev_bf16(si.slice_v)) if si.slice_k is not None else (None,
                                                                                          None)
        us = (dev_bf16(un.slice_k), dev_bf16(un.slice_v)) if un.slice_k is not None else (None,
                                                                                          None)
        ios.append(fmd.UnitCfgIO(cc, uc, z, list(hs or s.h), g, cond_slice=cs, uncond_slice=us,
                                 n_audio=s.n_audio))
        out.append((cc, uc, z))
    fmd.denoise_unit_cfg(ios, dev_bf16(w_qkv), dev_bf16(ui.w_o))
    torch.cuda.synchronize()
    return out


def _check_caches(c, ref_branch):
    rk, rv, ln, hd_ = ref_branch
    gk, gv = cache_logical(fmd, c)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert (c.len_tokens, c.head_tokens) == (ln, hd_)


def _check(wl, g, hs=None):
    ui, uns, w_qkv = _inputs(wl)
    gs = [g] * len(ui.sessions)
    res = _run(wl, ui, uns, w_qkv, hs, gs)
    for b, (si, un, (cc, uc, z)) in enumerate(zip(ui.sessions, uns, res)):
        s = si.shape
        ref = oracle.denoise_unit_cfg(_branch(si.ring_k, si.ring_v, si.slice_k, si.slice_v, s),
                                      _branch(un.ring_k, un.ring_v, un.slice_k, un.slice_v, s),
                                      si.eps, list(hs or s.h), g, w_qkv, ui.w_o, s.n_heads)
        zg = host_f64(z)
        assert_close(zg, ref["z"], f"{wl.name} unit {b} z (g={g})")
        assert_close(zg - si.eps, ref["z"] - si.eps, f"{wl.name} unit {b} dz (g={g})")
        _check_caches(cc, ref["cond"])
        _check_caches(uc, ref["uncond"])


@pytest.mark.parametrize("name,g", [("tiny", 5.0), ("v01_unit", 5.0), ("v01_unit", -0.5)])
def test_unit_cfg_matches_oracle(name, g):
    _check(workload.get(name), g)


def test_unit_cfg_640x368_first_step_every_row():
    # The guided teacher's 640x368-class unit at full size (both branches
    # append 944 tokens to full 60,416-token rings), one step, in the launch
    # configuration the benchmark times.  The oracle computes every row of
    # both branches' attention, the guided velocity and the Euler step.
    wl = workload.get("v02_cfg_unit")
    g = workload.CFG_GUIDANCE
    h = wl.sessions[0].h[0]
    ui, uns, w_qkv = _inputs(wl)
    (cc, uc, z), = _run(wl, ui, uns, w_qkv, [h], [g])
    si, un = ui.sessions[0], uns[0]
    s = si.shape
    q, k_u, v_u = oracle.qkv_projection(si.eps, w_qkv, s.n_heads)
    vs = []
    for rk, rv, sk, sv in ((si.ring_k, si.ring_v, si.slice_k, si.slice_v),
                           (un.ring_k, un.ring_v, un.slice_k, un.slice_v)):
        ring = oracle.kv_append(rk, rv, s.len_before, s.head_before, sk, sv)
        o = oracle.attention(q, *ring, k_u, v_u)
        vs.append(oracle.velocity(o.reshape(s.n_q, -1), ui.w_o))
        print("branch done", flush=True)
    want = oracle.euler_step(si.eps.astype(np.float64), h,
                             oracle.guided_velocity(vs[0], vs[1], g))
    zg = host_f64(z)
    assert_close(zg - si.eps, want - si.eps, "v02 cfg dz (every row)")
    for c, (rk, rv, sk, sv) in ((cc, (si.ring_k, si.ring_v, si.slice_k, si.slice_v)),
                                (uc, (un.ring_k, un.ring_v, un.slice_k, un.slice_v))):
        _check_caches(c, oracle.kv_append(rk, rv, s.len_before, s.head_before, sk, sv))


def test_guidance_limits_are_the_single_branch_solver():
    # g = 1: the conditional branch alone; g = 0: the unconditional one.  The
    # single-branch runs use the z-dependent solver on fresh copies of the
    # same caches.
    wl = workload.get("v01_unit")
    ui, uns, w_qkv = _inputs(wl)
    si, un = ui.sessions[0], uns[0]
    s = si.shape
    for g, (rk, rv, sk, sv) in ((1.0, (si.ring_k, si.ring_v, si.slice_k, si.slice_v)),
                                (0.0, (un.ring_k, un.ring_v, un.slice_k, un.slice_v))):
        (_, _, z), = _run(wl, ui, uns, w_qkv, None, [g])
        c = make_cache(fmd, s, rk, rv)
        z1 = torch.from_numpy(si.eps.copy()).to(DEV)
        fmd.denoise_unit_qkv([fmd.UnitQkvIO(c, dev_bf16(sk), dev_bf16(sv), z1, list(s.h),
                                            n_audio=s.n_audio)], dev_bf16(w_qkv),
                             dev_bf16(ui.w_o))
        torch.cuda.synchronize()
        assert_close(host_f64(z) - si.eps, host_f64(z1) - si.eps, f"g={g} vs single branch")


def test_uniform_attention_closed_form_on_gpu():
    # W_q = W_v = 0: in each branch O_b is the mean of its valid ring values
    # and slice over (len_b + T + n_q); the guided velocity is then known in
    # closed form: z_final = eps - sum(h) (v_u + g (v_c - v_u)).
    rng = np.random.default_rng(5)
    H, hd, cap, n_q, g = 2, 64, 96, 37, 3.0
    d = H * hd
    hs = [0.5, 0.25]
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[d:2 * d] = random_bits(rng, (d, d))
    w_o = random_bits(rng, (d, d), scale=d ** -0.5)
    eps = rng.standard_normal((n_q, d)).astype(np.float32)
    caches, slices, means = [], [], []
    for length, head, T in ((40, 70, 16), (53, 9, 5)):
        ring_k = random_bits(rng, (H, cap, hd))
        ring_v = random_bits(rng, (H, cap, hd))
        sk = random_bits(rng, (T, H, hd))
        sv = random_bits(rng, (T, H, hd))
        slots = [(head - length + i) % cap for i in range(length)]
        total = (oracle.bf16_bits_to_f64(ring_v)[:, slots, :].sum(axis=1)
                 + oracle.bf16_bits_to_f64(sv).sum(axis=0))
        means.append(total / (length + T + n_q))
        caches.append(fmd.KVCache(H, hd, cap, device=DEV, k=dev_bf16(ring_k),
                                  v=fmd.KVCache.logical_to_device_v(dev_bf16(ring_v)),
                                  len_tokens=length, head_tokens=head))
        slices.append((dev_bf16(sk), dev_bf16(sv)))
    z = torch.from_numpy(eps.copy()).to(DEV)
    fmd.denoise_unit_cfg([fmd.UnitCfgIO(caches[0], caches[1], z, hs, g, cond_slice=slices[0],
                                        uncond_slice=slices[1], n_audio=5)],
                         dev_bf16(w), dev_bf16(w_o))
    torch.cuda.synchronize()
    W = oracle.bf16_bits_to_f64(w_o)
    v_c, v_u = (np.tile(m.reshape(1, d), (n_q, 1)) @ W.T for m in means)
    want = eps - sum(hs) * (v_u + g * (v_c - v_u))
    assert_close(host_f64(z) - eps, want - eps, "guided uniform closed form dz")
    assert (caches[0].len_tokens, caches[0].head_tokens) == (56, 86 % cap)
    assert (caches[1].len_tokens, caches[1].head_tokens) == (58, 14)


def test_nine_units_span_two_launches():
    # Nine guided units are 18 attention sessions: two launch chunks.  Ragged
    # unit sizes, wrapped and partly filled rings, units without slices and
    # per-unit guidance scales (negative included).
    rng = np.random.default_rng(12)
    shapes = []
    for i in range(9):
        n_v, n_a = int(rng.integers(1, 70)), int(rng.integers(0, 9))
        cap = int(rng.integers(3, 9)) * 32
        T = int(rng.integers(0, 2)) * int(rng.integers(1, 40))
        ln = int(rng.integers(0, cap + 1))
        head = int(rng.integers(0, cap))
        shapes.append(workload.custom_session(2, 64, n_v, n_a, T, cap, ln, head, (0.5, 0.3)))
    wl = workload.custom_workload("cfg_nine", 21, shapes)
    ui, uns, w_qkv = _inputs(wl)
    gs = [float(x) for x in rng.uniform(-1.0, 6.0, 9)]
    res = _run(wl, ui, uns, w_qkv, None, gs)
    for b, (si, un, g, (cc, uc, z)) in enumerate(zip(ui.sessions, uns, gs, res)):
        s = si.shape
        ref = oracle.denoise_unit_cfg(_branch(si.ring_k, si.ring_v, si.slice_k, si.slice_v, s),
                                      _branch(un.ring_k, un.ring_v, un.slice_k, un.slice_v, s),
                                      si.eps, list(s.h), g, w_qkv, ui.w_o, s.n_heads)
        assert_close(host_f64(z) - si.eps, ref["z"] - si.eps, f"unit {b} dz (g={g:.2f})")
        _check_caches(cc, ref["cond"])
        _check_caches(uc, ref["uncond"])


def test_unit_cfg_deterministic():
    wl = workload.get("v01_unit")
    ui, uns, w_qkv = _inputs(wl)
    (_, _, za), = _run(wl, ui, uns, w_qkv, None, [5.0])
    (_, _, zb), = _run(wl, ui, uns, w_qkv, None, [5.0])
    assert torch.equal(za, zb)
