"""Pins for the oracle's classifier-free-guided sampler: a closed form in which
each branch's attention is a plain mean (so the guided velocity is known
exactly), a closed form in which guidance must change nothing, and the two
limits g = 1 and g = 0, which are the single-branch solver on the conditional
and on the unconditional cache."""
import numpy as np

import oracle
import workload
from tests.pins import check_cfg_mean_decay, check_cfg_uniform_closed_form


def test_uniform_attention_closed_form():
    for g in (3.0, 0.5, -1.0):
        assert check_cfg_uniform_closed_form(oracle.denoise_unit_cfg, g=g) <= 1e-12


def test_equal_branches_make_guidance_inert():
    assert check_cfg_mean_decay(oracle.denoise_unit_cfg) <= 2e-2


def _two_branches(seed=7, H=2, hd=16, cap=48, n_q=9):
    rng = np.random.default_rng(seed)
    d = H * hd
    mk = lambda *s: workload.round_to_bf16_bits(rng.standard_normal(s).astype(np.float32))  # noqa: E731
    cond = dict(ring_k=mk(H, cap, hd), ring_v=mk(H, cap, hd), length=40, head=11,
                slice_k=mk(5, H, hd), slice_v=mk(5, H, hd))
    uncond = dict(ring_k=mk(H, cap, hd), ring_v=mk(H, cap, hd), length=17, head=30,
                  slice_k=None, slice_v=None)
    w = workload.round_to_bf16_bits((rng.standard_normal((3 * d, d)) / np.sqrt(d)).astype(np.float32))
    w_o = workload.round_to_bf16_bits((rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32))
    eps = rng.standard_normal((n_q, d))
    return cond, uncond, eps, w, w_o, H


def test_guidance_one_is_the_conditional_solver_and_zero_the_unconditional():
    cond, uncond, eps, w, w_o, H = _two_branches()
    hs = [0.5, 0.3, 0.2]
    for g, b in ((1.0, cond), (0.0, uncond)):
        got = oracle.denoise_unit_cfg(cond, uncond, eps, hs, g, w, w_o, H)
        want = oracle.denoise_unit_qkv(b["ring_k"], b["ring_v"], b["length"], b["head"],
                                       b["slice_k"], b["slice_v"], eps, hs, w, w_o, H)
        assert np.max(np.abs(got["z"] - want["z"])) <= 1e-12
    # Each branch's cache takes its own slice (and only its own).
    got = oracle.denoise_unit_cfg(cond, uncond, eps, hs, 2.0, w, w_o, H)
    assert got["cond"][2:] == (45, 16) and got["uncond"][2:] == (17, 30)


def test_guidance_extrapolates_beyond_the_conditional():
    # With g > 1 the first step moves z further along v_c - v_u than g = 1 does:
    # dz(g) - dz(1) = -(g - 1) h (v_c - v_u), exactly, after one step.
    cond, uncond, eps, w, w_o, H = _two_branches(seed=8)
    z1 = oracle.denoise_unit_cfg(cond, uncond, eps, [0.5], 1.0, w, w_o, H)["z"]
    z0 = oracle.denoise_unit_cfg(cond, uncond, eps, [0.5], 0.0, w, w_o, H)["z"]
    z3 = oracle.denoise_unit_cfg(cond, uncond, eps, [0.5], 3.0, w, w_o, H)["z"]
    assert np.max(np.abs((z3 - z1) - 2.0 * (z1 - z0))) <= 1e-12
    assert np.max(np.abs(z1 - z0)) > 1e-3
