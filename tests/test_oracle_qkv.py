"""Pins for the oracle's per-step Q/K/V projection from z: bf16 rounding
against torch's conversion, the projection against a scalar loop, and two
closed forms of the whole z-dependent solver."""
import numpy as np
import torch

import oracle
from tests.pins import (brute_qkv, check_qkv_mean_decay, check_qkv_uniform_closed_form,
                        random_bits)


def test_round_to_bf16_matches_torch_on_float32_values():
    # For inputs that are float32 values, one rounding to bf16 is what
    # torch's float32 -> bfloat16 conversion does (nearest, ties to even).
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x), ref)


def test_round_to_bf16_ties_to_even():
    # bf16 spacing at 1 is 2^-7: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    # (goes to the even 1); 1 + 3*2^-8 is halfway between 1 + 2^-7 and
    # 1 + 2^-6 (goes to the even 1 + 2^-6).
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 + 2.0 ** -7, 0.0])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 3.0, 0.0])
    assert np.array_equal(oracle.round_to_bf16(x), want)


def test_qkv_projection_matches_scalar_loop():
    rng = np.random.default_rng(1)
    H, hd, n = 2, 3, 4
    d = H * hd
    z = rng.standard_normal((n, d))
    w = random_bits(rng, (3 * d, d))
    got = oracle.qkv_projection(z, w, H)
    want = brute_qkv(z, w, H)
    for g, w_ in zip(got, want):
        assert g.shape == (n, H, hd)
        assert np.array_equal(oracle.bf16_bits_to_f64(g), w_)


def test_qkv_projection_orientation():
    # Row t*d + c of W_qkv produces column c of the t-th output (Q, K_u, V_u),
    # which is head c // hd, feature c % hd.
    H, hd = 2, 2
    d = H * hd
    z = np.arange(1, d + 1, dtype=np.float64)[None, :]          # one token
    w = np.zeros((3 * d, d), dtype=np.uint16)
    one = 0x3F80
    w[0 * d + 3, 0] = one          # Q head 1 feature 1 <- z[0] = 1
    w[1 * d + 1, 2] = one          # K head 0 feature 1 <- z[2] = 3
    w[2 * d + 2, 3] = one          # V head 1 feature 0 <- z[3] = 4
    q, k, v = (oracle.bf16_bits_to_f64(t) for t in oracle.qkv_projection(z, w, H))
    assert q[0, 1, 1] == 1.0 and k[0, 0, 1] == 3.0 and v[0, 1, 0] == 4.0
    assert np.count_nonzero(q) == np.count_nonzero(k) == np.count_nonzero(v) == 1


def test_uniform_attention_closed_form():
    assert check_qkv_uniform_closed_form(oracle.denoise_unit_qkv) <= 1e-12


def test_mean_decay_closed_form_depends_on_current_z():
    assert check_qkv_mean_decay(oracle.denoise_unit_qkv) <= 2e-2
