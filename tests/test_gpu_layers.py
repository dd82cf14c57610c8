"""GPU parity of the layer-stack solver (one ring and one pair of weights per
layer, residual stream, v = sum of the layers' updates) against the oracle,
its one-layer case against the z-dependent solver, and two closed forms on
the GPU."""
import dataclasses

import numpy as np
import pytest

import oracle
import workload
from tests.pins import bits, random_bits

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import (DEV, assert_close, cache_logical, dev_bf16, host_f64,  # noqa: E402
                            make_cache)

pytestmark = pytest.mark.gpu


def _layer_inputs(wl, n_layers):
    """Per layer: the workload drawn with its own seed (ring, slice) and its
    own weights; eps of layer 0's draw."""
    per = []
    for l in range(n_layers):
        wl_l = dataclasses.replace(wl, seed=wl.seed + 1000 * (l + 1))
        ui = workload.make_inputs(wl_l, poison_invalid=True, reuse_step_inputs=True)
        per.append((ui, workload.qkv_weight(wl_l.seed, wl.d, wl.head_dim), ui.w_o))
    return per


def _run(wl, per, hs=None, sessions=None):
    idx = range(len(wl.sessions)) if sessions is None else sessions
    ios, out = [], []
    for si_i in idx:
        s = wl.sessions[si_i]
        caches, ks, vs = [], [], []
        for ui, _, _ in per:
            si = ui.sessions[si_i]
            caches.append(make_cache(fmd, s, si.ring_k, si.ring_v))
            if si.slice_k is not None:
                ks.append(dev_bf16(si.slice_k))
                vs.append(dev_bf16(si.slice_v))
        z = torch.from_numpy(per[0][0].sessions[si_i].eps.copy()).to(DEV)
        ios.append(fmd.UnitLayersIO(caches, z, list(hs or s.h), ks or None, vs or None,
                                    n_audio=s.n_audio))
        out.append((caches, z))
    fmd.denoise_unit_layers(ios, [dev_bf16(w) for _, w, _ in per], [dev_bf16(w) for _, _, w in per])
    torch.cuda.synchronize()
    return out


def _oracle(wl, per, si_i, hs=None):
    s = wl.sessions[si_i]
    layers = []
    for ui, _, _ in per:
        si = ui.sessions[si_i]
        layers.append(dict(ring_k=si.ring_k, ring_v=si.ring_v, length=s.len_before,
                           head=s.head_before, slice_k=si.slice_k, slice_v=si.slice_v))
    return oracle.denoise_unit_layers(layers, per[0][0].sessions[si_i].eps, list(hs or s.h),
                                      [w for _, w, _ in per], [w for _, _, w in per], s.n_heads)


@pytest.mark.parametrize("name,n_layers", [("tiny", 3), ("v01_unit", 3)])
def test_unit_layers_match_oracle(name, n_layers):
    wl = workload.get(name)
    per = _layer_inputs(wl, n_layers)
    res = _run(wl, per)
    for b, (caches, z) in enumerate(res):
        ref = _oracle(wl, per, b)
        eps = per[0][0].sessions[b].eps
        assert_close(host_f64(z) - eps, ref["z"] - eps, f"{name} L={n_layers} dz")
        for c, (rk, rv, ln, hd_) in zip(caches, ref["rings"]):
            gk, gv = cache_logical(fmd, c)
            assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
            assert (c.len_tokens, c.head_tokens) == (ln, hd_)


def test_ragged_sessions_and_layers():
    shapes = [workload.custom_session(2, 64, 37, 3, 16, 128, 100, 90, (0.5, 0.5)),
              workload.custom_session(2, 64, 5, 0, 0, 64, 64, 17, (0.5, 0.5)),
              workload.custom_session(2, 64, 160, 8, 40, 256, 0, 0, (0.5, 0.5))]
    wl = workload.custom_workload("layers_ragged", 31, shapes)
    per = _layer_inputs(wl, 2)
    res = _run(wl, per)
    for b, (caches, z) in enumerate(res):
        ref = _oracle(wl, per, b)
        eps = per[0][0].sessions[b].eps
        assert_close(host_f64(z) - eps, ref["z"] - eps, f"session {b} dz")


def test_one_layer_is_the_z_dependent_solver_bitwise():
    wl = workload.get("v01_unit")
    per = _layer_inputs(wl, 1)
    (caches, z), = _run(wl, per)
    ui, w_qkv, w_o = per[0]
    si = ui.sessions[0]
    s = si.shape
    c = make_cache(fmd, s, si.ring_k, si.ring_v)
    z1 = torch.from_numpy(si.eps.copy()).to(DEV)
    fmd.denoise_unit_qkv([fmd.UnitQkvIO(c, dev_bf16(si.slice_k), dev_bf16(si.slice_v), z1,
                                        list(s.h), n_audio=s.n_audio)],
                         dev_bf16(w_qkv), dev_bf16(w_o))
    torch.cuda.synchronize()
    assert torch.equal(z, z1)


def test_640x368_two_layers_one_step_every_row():
    # The 640x368-class unit through two layers at full size (each layer's
    # ring takes its 944-token slice: 61,344 keys per query).  The oracle
    # computes both layers on every row.
    wl = workload.get("v02_unit")
    h = 0.25
    per = _layer_inputs(wl, 2)
    (caches, z), = _run(wl, per, hs=[h])
    s = wl.sessions[0]
    eps = per[0][0].sessions[0].eps.astype(np.float64)
    rings = []
    for ui, _, _ in per:
        si = ui.sessions[0]
        rings.append(oracle.kv_append(si.ring_k, si.ring_v, s.len_before, s.head_before,
                                      si.slice_k, si.slice_v))
    (_, wq0, wo0), (_, wq1, wo1) = per
    q, k, v = oracle.qkv_projection(eps, wq0, s.n_heads)
    o0 = oracle.attention(q, *rings[0], k, v)
    r1 = oracle.velocity(o0.reshape(s.n_q, -1), wo0)
    print("layer 0 done", flush=True)
    q, k, v = oracle.qkv_projection(eps + r1, wq1, s.n_heads)
    o1 = oracle.attention(q, *rings[1], k, v)
    vel = r1 + oracle.velocity(o1.reshape(s.n_q, -1), wo1)
    want = eps - h * vel
    assert_close(host_f64(z) - eps, want - eps, "v02 two layers dz (every row)")


def test_uniform_attention_closed_form_on_gpu():
    # Every layer W_q = W_v = 0: layer l's attention is the mean of its own
    # ring and slice; v = sum_l mean_l W_o,l^T.
    rng = np.random.default_rng(9)
    H, hd, cap, n_q = 2, 64, 96, 21
    d = H * hd
    hs = [0.5, 0.25]
    eps = rng.standard_normal((n_q, d)).astype(np.float32)
    caches, ks, vs, wqs, wos, v = [], [], [], [], [], np.zeros((n_q, d))
    for length, head, T in ((30, 40, 8), (77, 3, 8), (0, 0, 8)):
        rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
        sk, sv = random_bits(rng, (T, H, hd)), random_bits(rng, (T, H, hd))
        slots = [(head - length + i) % cap for i in range(length)]
        total = oracle.bf16_bits_to_f64(rv)[:, slots, :].sum(axis=1) + \
            oracle.bf16_bits_to_f64(sv).sum(axis=0)
        w = np.zeros((3 * d, d), dtype=np.uint16)
        w[d:2 * d] = random_bits(rng, (d, d))
        wo = random_bits(rng, (d, d), scale=d ** -0.5)
        v += np.tile((total / (length + T + n_q)).reshape(1, d), (n_q, 1)) @ \
            oracle.bf16_bits_to_f64(wo).T
        caches.append(fmd.KVCache(H, hd, cap, device=DEV, k=dev_bf16(rk),
                                  v=fmd.KVCache.logical_to_device_v(dev_bf16(rv)),
                                  len_tokens=length, head_tokens=head))
        ks.append(dev_bf16(sk))
        vs.append(dev_bf16(sv))
        wqs.append(dev_bf16(w))
        wos.append(dev_bf16(wo))
    z = torch.from_numpy(eps.copy()).to(DEV)
    fmd.denoise_unit_layers([fmd.UnitLayersIO(caches, z, hs, ks, vs, n_audio=4)], wqs, wos)
    torch.cuda.synchronize()
    want = eps - sum(hs) * v
    assert_close(host_f64(z) - eps, want - eps, "layers uniform closed form dz")


def test_residual_chain_closed_form_on_gpu():
    # Two identity layers over empty rings: v = 3 mean(z), the mean decays by
    # (1 - 3h) per step, deviations from it stay.
    rng = np.random.default_rng(10)
    H, hd, n_q = 2, 64, 32
    d = H * hd
    hs = [0.25, 0.25]
    eps = (rng.standard_normal((n_q, d)) + 0.5).astype(np.float32)
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[2 * d:] = bits(np.eye(d))
    eye = dev_bf16(bits(np.eye(d)))
    caches = [fmd.KVCache(H, hd, 64, device=DEV) for _ in range(2)]
    z = torch.from_numpy(eps.copy()).to(DEV)
    fmd.denoise_unit_layers([fmd.UnitLayersIO(caches, z, hs)], [dev_bf16(w)] * 2, [eye, eye])
    torch.cuda.synchronize()
    e = eps.astype(np.float64)
    mean0 = e.mean(axis=0, keepdims=True)
    want = (e - mean0) + np.prod([1 - 3 * h for h in hs]) * mean0
    got = host_f64(z)
    assert np.max(np.abs(got - want)) <= 3e-2
    assert np.max(np.abs(got.mean(axis=0) - 0.0625 * mean0[0])) <= 3e-2


def test_unit_layers_deterministic():
    wl = workload.get("v01_unit")
    per = _layer_inputs(wl, 2)
    (_, za), = _run(wl, per)
    (_, zb), = _run(wl, per)
    assert torch.equal(za, zb)
