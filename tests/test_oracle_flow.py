"""Pins for the oracle's projection and Euler solver: the rectified-flow closed
form, step linearity, and scalar brute force for the projection."""
import os

import numpy as np
import pytest

import oracle
import workload
from tests.pins import (bits, brute_velocity, check_closed_form_flow, random_bits,
                        widen)

SCHEDULES = [
    [1.0],
    [0.5, 0.5],
    [0.25] * 4,
    [0.4, 0.3, 0.2, 0.1],
    [1.0 / 7] * 7,
]


@pytest.mark.parametrize("hs", SCHEDULES)
def test_closed_form_recovers_clean_latent(hs):
    # With the exact constant velocity eps - z0 the Euler solver lands on z0
    # for any step count and any schedule summing to one.
    err = check_closed_form_flow(oracle.denoise_unit, hs)
    assert err <= 1e-14, err


def test_golden_closed_form_fixture():
    # Hand-derived numbers, stored as text (see the fixture's header).
    path = os.path.join(os.path.dirname(__file__), "golden", "rectified_flow_closed_form.txt")
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split("=")
            rows[key.strip()] = np.array([float(x) for x in vals.split()])
    z = rows["eps"].copy()
    v = rows["eps"] - rows["z0"]
    for i, h in enumerate(rows["h"]):
        z = oracle.euler_step(z, h, v)
        assert np.allclose(z, rows[f"z_after_{i + 1}"], atol=1e-15, rtol=0)
    assert np.allclose(z, rows["z0"], atol=1e-15, rtol=0)


def test_velocity_matches_brute_force_non_symmetric():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((3, 6))
    w = random_bits(rng, (6, 6))
    assert not np.array_equal(w, w.T)
    got = oracle.velocity(o, w)
    assert np.max(np.abs(got - brute_velocity(o, w))) <= 1e-13


def test_velocity_rectangular_orientation():
    # W is [d_out][d_in]: a 2x3 weight maps 3 input features to 2 outputs.
    o = np.array([[1.0, 2.0, 3.0]])
    w = bits(np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 2.0]]))
    assert np.array_equal(oracle.velocity(o, w), np.array([[1.0, 6.0]]))


def test_reused_step_inputs_equal_one_big_step():
    # The velocity does not depend on z in this step, so with the same inputs
    # every step, S steps of sizes h equal one step of size sum(h).
    wl = workload.get("tiny")
    ui = workload.make_inputs(wl, reuse_step_inputs=True)
    s = ui.sessions[0]
    sh = s.shape
    args = (s.ring_k, s.ring_v, sh.len_before, sh.head_before, None, None,
            s.q, s.k_u, s.v_u, s.eps)
    a = oracle.denoise_unit(*args, [0.4, 0.3, 0.2, 0.1], ui.w_o)["z"]
    b = oracle.denoise_unit(*args, [1.0], ui.w_o)["z"]
    assert np.max(np.abs(a - b)) <= 1e-14


def test_denoise_unit_appends_before_attending():
    # The slice is in the cache before the first solver step: attention at
    # step 0 must see the slice's keys (append-then-denoise order).
    rng = np.random.default_rng(8)
    H, hd, cap, T, n_q = 1, 8, 16, 4, 2
    rk = random_bits(rng, (H, cap, hd))
    sk = random_bits(rng, (T, H, hd))
    sv = random_bits(rng, (T, H, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    eye = bits(np.eye(H * hd))
    res = oracle.denoise_unit(rk, rk, 12, 12, sk, sv, [q], [ku], [vu],
                              np.zeros((n_q, H * hd)), [1.0], eye)
    assert res["length"] == 16 and res["head"] == 0
    # z = 0 - 1 * (O @ I) = -O, with O over the post-append ring.
    o = oracle.attention(q, res["ring_k"], res["ring_v"], 16, 0, ku, vu)
    assert np.max(np.abs(res["z"] + o.reshape(n_q, -1))) <= 1e-15
    assert np.array_equal(res["ring_k"][0, 12:16], sk[:, 0])


def test_widen_matches_library_conversion():
    rng = np.random.default_rng(9)
    b = random_bits(rng, (1000,))
    b[:3] = [0x7FC0, 0x0000, 0x8000]
    a = oracle.bf16_bits_to_f64(b)
    ref = widen(b)
    assert np.array_equal(np.isnan(a), np.isnan(ref))
    assert np.array_equal(a[3:], ref[3:])


def test_tiny_workload_matches_frozen_oracle_output():
    # Regression guard: the oracle's output on the tiny workload as frozen by
    # tests/golden/make_golden.py.
    import importlib.util
    here = os.path.dirname(__file__)
    spec = importlib.util.spec_from_file_location("make_golden",
                                                  os.path.join(here, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    O, dz = mg.compute()
    ref = {}
    with open(os.path.join(here, "golden", "tiny_oracle.txt")) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=")
            ref[k.strip()] = np.array([float(x) for x in v.split()])
    for r in (0, 15):
        for h in (0, 1):
            assert np.allclose(O[r, h, :8], ref[f"O_{r}_{h}"], rtol=1e-13, atol=1e-15)
        assert np.allclose(dz[r, :8], ref[f"dz_{r}"], rtol=1e-13, atol=1e-15)
    assert abs(np.linalg.norm(O) - ref["O_norm"][0]) <= 1e-12
    assert abs(np.linalg.norm(dz) - ref["dz_norm"][0]) <= 1e-12
