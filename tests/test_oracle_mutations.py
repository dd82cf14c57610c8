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

    def ring_only(ring_k, ring_v, length, head, k_u, v_u, h):
        K, V = orig(ring_k, ring_v, length, head, k_u, v_u, h)
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
