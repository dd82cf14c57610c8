"""GPU parity of the z-dependent solver (Q, K_u, V_u projected from the
current latent every step) against the oracle, and its closed forms on the
GPU."""
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


def _run(wl, hs=None, poison=True):
    ui = workload.make_inputs(wl, poison_invalid=poison, reuse_step_inputs=True)
    w_qkv = workload.qkv_weight(wl.seed, wl.d, wl.head_dim)
    caches, ios, zs = [], [], []
    for si in ui.sessions:
        s = si.shape
        c = make_cache(fmd, s, si.ring_k, si.ring_v)
        z = torch.from_numpy(si.eps.copy()).to(DEV)
        sk = dev_bf16(si.slice_k) if si.slice_k is not None else None
        sv = dev_bf16(si.slice_v) if si.slice_v is not None else None
        caches.append(c)
        zs.append(z)
        ios.append(fmd.UnitQkvIO(c, sk, sv, z, list(hs or s.h), n_audio=s.n_audio))
    fmd.denoise_unit_qkv(ios, dev_bf16(w_qkv), dev_bf16(ui.w_o))
    torch.cuda.synchronize()
    return ui, w_qkv, caches, zs


def _check(name, hs=None):
    wl = workload.get(name)
    ui, w_qkv, caches, zs = _run(wl, hs)
    for b, (si, c, z) in enumerate(zip(ui.sessions, caches, zs)):
        s = si.shape
        ref = oracle.denoise_unit_qkv(si.ring_k, si.ring_v, s.len_before, s.head_before,
                                      si.slice_k, si.slice_v, si.eps, list(hs or s.h), w_qkv,
                                      ui.w_o, s.n_heads)
        zg = host_f64(z)
        assert_close(zg, ref["z"], f"{name} session {b} z")
        assert_close(zg - si.eps, ref["z"] - si.eps, f"{name} session {b} dz")
        gk, gv = cache_logical(fmd, c)
        assert np.array_equal(gk, ref["ring_k"]) and np.array_equal(gv, ref["ring_v"])
        assert (c.len_tokens, c.head_tokens) == (ref["length"], ref["head"])


@pytest.mark.parametrize("name", ["tiny", "v01_unit"])
def test_unit_qkv_matches_oracle(name):
    _check(name)


def test_unit_qkv_640x368_two_steps_full():
    # The 640x368-class unit at full size (append, 40 heads x 928 queries x
    # 61,344 keys); two steps so that the second projects from a z the first
    # step produced.  The oracle computes every row.
    _check("v02_unit", hs=[0.25, 0.25])


def _closed_form_session(H, hd, cap, length, head, n_q):
    s = workload.custom_session(H, hd, n_q, 0, 0, cap, length, head, (1.0,))
    return s


def test_uniform_attention_closed_form_on_gpu():
    # W_q = W_v = 0: uniform attention over the valid ring and the unit (whose
    # values are 0), whatever z is; z_final = eps - sum(h) * O W_o^T.
    rng = np.random.default_rng(3)
    H, hd, cap, length, head, n_q = 2, 64, 64, 48, 20, 24
    d = H * hd
    hs = [0.5, 0.25, 0.125]
    ring_k = random_bits(rng, (H, cap, hd))
    ring_v = random_bits(rng, (H, cap, hd))
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[d:2 * d] = random_bits(rng, (d, d))
    w_o = random_bits(rng, (d, d), scale=d ** -0.5)
    eps = rng.standard_normal((n_q, d)).astype(np.float32)
    c = fmd.KVCache(H, hd, cap, device=DEV, k=dev_bf16(ring_k),
                    v=fmd.KVCache.logical_to_device_v(dev_bf16(ring_v)), len_tokens=length,
                    head_tokens=head)
    z = torch.from_numpy(eps.copy()).to(DEV)
    fmd.denoise_unit_qkv([fmd.UnitQkvIO(c, None, None, z, hs)], dev_bf16(w), dev_bf16(w_o))
    torch.cuda.synchronize()
    slots = [(head - length + i) % cap for i in range(length)]
    mean_v = oracle.bf16_bits_to_f64(ring_v)[:, slots, :].sum(axis=1) / (length + n_q)
    v = np.tile(mean_v.reshape(1, d), (n_q, 1)) @ oracle.bf16_bits_to_f64(w_o).T
    want = eps - sum(hs) * v
    assert_close(host_f64(z) - eps, want - eps, "uniform closed form dz")


def test_mean_decay_closed_form_on_gpu():
    # Empty cache, W_v = W_o = I: each step maps z_i -> z_i - h mean(bf16(z)),
    # so the mean decays by prod(1 - h) while deviations from it stay.
    rng = np.random.default_rng(4)
    H, hd, n_q = 2, 64, 32
    d = H * hd
    hs = [0.5, 0.5]
    eps = (rng.standard_normal((n_q, d)) + 0.5).astype(np.float32)
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[2 * d:] = bits(np.eye(d))
    w_o = bits(np.eye(d))
    c = fmd.KVCache(H, hd, 64, device=DEV, len_tokens=0, head_tokens=0)
    z = torch.from_numpy(eps.copy()).to(DEV)
    fmd.denoise_unit_qkv([fmd.UnitQkvIO(c, None, None, z, hs)], dev_bf16(w), dev_bf16(w_o))
    torch.cuda.synchronize()
    e = eps.astype(np.float64)
    mean0 = e.mean(axis=0, keepdims=True)
    want = (e - mean0) + np.prod([1 - h for h in hs]) * mean0
    got = host_f64(z)
    assert np.max(np.abs(got - want)) <= 2e-2
    # The decay factor itself: prod(1 - h) = 0.25, not 1 - sum(h) = 0.
    assert np.max(np.abs(got.mean(axis=0) - 0.25 * mean0[0])) <= 2e-2


def test_unit_qkv_deterministic():
    wl = workload.get("v01_unit")
    _, _, _, za = _run(wl)
    _, _, _, zb = _run(wl)
    assert torch.equal(za[0], zb[0])
