"""Pins for the oracle's layer stack: one layer is the single-layer
z-dependent solver; a closed form in which every layer's attention is a plain
mean of its own ring; a closed form that fixes the residual chaining; and
planted mistakes."""
import importlib

import numpy as np

import oracle
import workload
from tests.pins import check_layers_residual_chain, check_layers_uniform_closed_form

lay = importlib.import_module("oracle.layers")


def test_one_layer_is_the_z_dependent_solver():
    rng = np.random.default_rng(0)
    H, hd, cap, n_q = 2, 16, 48, 7
    d = H * hd
    mk = lambda *s: workload.round_to_bf16_bits(rng.standard_normal(s).astype(np.float32))  # noqa: E731
    b = dict(ring_k=mk(H, cap, hd), ring_v=mk(H, cap, hd), length=33, head=40,
             slice_k=mk(6, H, hd), slice_v=mk(6, H, hd))
    w = workload.round_to_bf16_bits((rng.standard_normal((3 * d, d)) / np.sqrt(d)).astype(np.float32))
    wo = workload.round_to_bf16_bits((rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32))
    eps = rng.standard_normal((n_q, d))
    hs = [0.5, 0.3, 0.2]
    got = oracle.denoise_unit_layers([b], eps, hs, [w], [wo], H)
    want = oracle.denoise_unit_qkv(b["ring_k"], b["ring_v"], b["length"], b["head"], b["slice_k"],
                                   b["slice_v"], eps, hs, w, wo, H)
    assert np.max(np.abs(got["z"] - want["z"])) <= 1e-12
    assert got["rings"][0][2:] == (39, 46 % cap)


def test_uniform_attention_closed_form():
    assert check_layers_uniform_closed_form(oracle.denoise_unit_layers) <= 1e-12


def test_residual_chain_closed_form():
    assert check_layers_residual_chain(oracle.denoise_unit_layers) <= 3e-2


def test_layer_input_without_residual_is_caught(monkeypatch):
    # mistake: layer 1 projects from z (layer 0's input), ignoring the
    # residual stream (two layers per step: even calls are layer 0)
    orig = lay.qkv_projection
    calls = {"n": 0, "z": None}

    def layer_from_z(a, w, H):
        if calls["n"] % 2 == 0:
            calls["z"] = np.array(a)
        calls["n"] += 1
        return orig(calls["z"], w, H)
    monkeypatch.setattr(lay, "qkv_projection", layer_from_z)
    assert check_layers_residual_chain(oracle.denoise_unit_layers) > 0.1


def test_swapped_layer_rings_is_caught(monkeypatch):
    # mistake: the layers read each other's rings (order reversed)
    orig = lay.layer_stack_velocity
    monkeypatch.setattr(lay, "layer_stack_velocity",
                        lambda z, rings, wq, wo, H: orig(z, rings[::-1], wq, wo, H))
    assert check_layers_uniform_closed_form(oracle.denoise_unit_layers) > 1e-3


def test_velocity_from_last_layer_only_is_caught(monkeypatch):
    # mistake: v is the last layer's update alone instead of the sum
    def last_only(z, rings, wq, wo, H):
        z = np.asarray(z, dtype=np.float64)
        r = np.zeros_like(z)
        upd = None
        for ring, a, b in zip(rings, wq, wo):
            q, k, v = lay.qkv_projection(z + r, a, H)
            o = lay.attention(q, *ring, k, v)
            upd = lay.velocity(o.reshape(o.shape[0], -1), b)
            r = r + upd
        return upd
    monkeypatch.setattr(lay, "layer_stack_velocity", last_only)
    assert check_layers_uniform_closed_form(oracle.denoise_unit_layers) > 1e-3
