"""Planted mistakes: each plausible slip in the oracle (made here, on the CPU,
by patching the oracle module) must make at least one pin fail.  This shows the
pins constrain the oracle rather than restate it."""
import importlib

import numpy as np
import pytest

import oracle
from tests.pins import (brute_velocity, check_attention_vs_history, check_closed_form_flow,
                        check_values_one, random_bits)

att_mod = importlib.import_module("oracle.attention")
flow_mod = importlib.import_module("oracle.flow")
ring_mod = importlib.import_module("oracle.ring")


class _Math:
    @staticmethod
    def sqrt(x):
        return x                       # mistake: scale 1/hd instead of 1/sqrt(hd)


def test_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(att_mod, "math", _Math)
    assert check_attention_vs_history(oracle.attention, oracle.kv_append) > 1e-3


def test_wrong_valid_slots_is_caught(monkeypatch):
    # mistake: the slots *from* head on instead of the ones before it
    monkeypatch.setattr(att_mod, "valid_slots",
                        lambda length, head, cap: [(head + j) % cap for j in range(length)])
    assert check_attention_vs_history(oracle.attention, oracle.kv_append) > 1e-3


def test_dropped_unit_keys_is_caught(monkeypatch):
    orig = att_mod._gather_head

    def ring_only(ring_k, ring_v, length, head, k_u, v_u, h, *rest):
        K, V = orig(ring_k, ring_v, length, head, k_u, v_u, h, *rest)
        n = k_u.shape[0]
        return K[:-n], V[:-n]
    monkeypatch.setattr(att_mod, "_gather_head", ring_only)
    assert check_attention_vs_history(oracle.attention, oracle.kv_append) > 1e-3


def test_missing_normalisation_is_caught(monkeypatch):
    def unnormalised(sc):
        return np.exp(sc - sc.max(axis=1, keepdims=True))     # mistake: no division
    monkeypatch.setattr(att_mod, "_softmax_rows", unnormalised)
    assert check_values_one(oracle.attention) > 1e-3


def test_append_off_by_one_is_caught(monkeypatch):
    orig = ring_mod.kv_append

    def shifted(ring_k, ring_v, length, head, slice_k, slice_v):
        return orig(ring_k, ring_v, length, (head + 1) % ring_k.shape[1], slice_k, slice_v)
    assert check_attention_vs_history(oracle.attention, shifted) > 1e-3


def test_euler_sign_is_caught(monkeypatch):
    monkeypatch.setattr(flow_mod, "euler_step", lambda z, h, v: np.asarray(z) + h * np.asarray(v))
    assert check_closed_form_flow(oracle.denoise_unit, [0.25] * 4) > 1e-2


def test_untransposed_projection_is_caught():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((3, 6))
    w = random_bits(rng, (6, 6))
    wrong = o @ oracle.bf16_bits_to_f64(w)           # mistake: O @ W instead of O @ W^T
    assert np.max(np.abs(wrong - brute_velocity(o, w))) > 1e-3


qkv_mod = importlib.import_module("oracle.qkv")


def test_projection_from_eps_is_caught(monkeypatch):
    # mistake: every step projects Q, K, V from the starting latent eps
    from tests.pins import check_qkv_mean_decay
    orig = qkv_mod.qkv_projection
    first = {}

    def from_first(z, w, n_heads):
        key = id(w)
        first.setdefault(key, np.array(z, dtype=np.float64))
        return orig(first[key], w, n_heads)
    monkeypatch.setattr(qkv_mod, "qkv_projection", from_first)
    assert check_qkv_mean_decay(oracle.denoise_unit_qkv) > 5e-2


def test_swapped_query_and_key_thirds_is_caught(monkeypatch):
    # mistake: the first third of W_qkv taken as the keys, the second as queries
    from tests.pins import check_qkv_uniform_closed_form
    orig = qkv_mod.qkv_projection

    def swapped(z, w, n_heads):
        q, k, v = orig(z, w, n_heads)
        return k, q, v
    monkeypatch.setattr(qkv_mod, "qkv_projection", swapped)
    assert check_qkv_uniform_closed_form(oracle.denoise_unit_qkv) > 1e-3


def test_unrounded_latent_in_projection_is_caught(monkeypatch):
    # mistake: z fed to the projection in full precision (no bf16 rounding)
    from tests.pins import brute_qkv
    monkeypatch.setattr(qkv_mod, "round_to_bf16", lambda x: np.asarray(x, dtype=np.float64))
    rng = np.random.default_rng(1)
    z = rng.standard_normal((4, 6))
    w = random_bits(rng, (18, 6))
    got = qkv_mod.qkv_projection(z, w, 2)
    want = brute_qkv(z, w, 2)
    assert max(np.max(np.abs(oracle.bf16_bits_to_f64(g) - w_)) for g, w_ in zip(got, want)) > 0


cfg_mod = importlib.import_module("oracle.cfg")


def test_swapped_guidance_branches_is_caught(monkeypatch):
    # mistake: the guidance extrapolates from the conditional branch instead
    from tests.pins import check_cfg_uniform_closed_form
    monkeypatch.setattr(cfg_mod, "guided_velocity", lambda v_c, v_u, g: v_c + g * (v_u - v_c))
    assert check_cfg_uniform_closed_form(oracle.denoise_unit_cfg) > 1e-3


def test_other_guidance_convention_is_caught(monkeypatch):
    # mistake: v_c + g (v_c - v_u), the convention whose scale is offset by one
    from tests.pins import check_cfg_uniform_closed_form
    monkeypatch.setattr(cfg_mod, "guided_velocity", lambda v_c, v_u, g: v_c + g * (v_c - v_u))
    assert check_cfg_uniform_closed_form(oracle.denoise_unit_cfg) > 1e-3


def test_slice_appended_to_one_branch_only_is_caught(monkeypatch):
    # mistake: the unconditional branch skips its slice
    from tests.pins import check_cfg_uniform_closed_form
    orig = cfg_mod._branch
    calls = []

    def first_only(b):
        calls.append(1)
        if len(calls) % 2 == 0:
            b = dict(b, slice_k=None, slice_v=None)
        return orig(b)
    monkeypatch.setattr(cfg_mod, "_branch", first_only)
    assert check_cfg_uniform_closed_form(oracle.denoise_unit_cfg) > 1e-3


def test_guided_projection_from_eps_is_caught(monkeypatch):
    # mistake: Q, K_u, V_u projected from eps at every step
    from tests.pins import check_cfg_mean_decay
    orig = cfg_mod.qkv_projection
    first = {}

    def from_first(z, w, H):
        first.setdefault("z", np.array(z))
        return orig(first["z"], w, H)
    monkeypatch.setattr(cfg_mod, "qkv_projection", from_first)
    assert check_cfg_mean_decay(oracle.denoise_unit_cfg) > 5e-2
