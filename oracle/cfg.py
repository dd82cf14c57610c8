"""Oracle: classifier-free-guided sampling of one unit (the teacher's sampler).

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the deployed few-step performer is distilled from a stronger teacher
that samples with classifier-free guidance and more flow-matching solver steps
[Wan-Streamer (gongshangzheng blog), training stages, Stage 3 低延迟蒸馏].
Classifier-free guidance evaluates the velocity network with and without the
conditioning at every solver step and extrapolates from the unconditional
velocity towards the conditional one by the guidance scale g:
v = v_u + g (v_c - v_u)  (g = 1: conditional only; g = 0: unconditional only).

Readings where the pages are silent:
* the conditioning reaches the unit only through its clean context, so the two
  branches differ only in the K/V cache they attend to (conditional ring c,
  unconditional ring u); the unit's own Q, K_u, V_u are common to both,
  projected from the one latent z as in ``qkv.denoise_unit_qkv``;
* each branch's velocity is the same dense projection of its own attention
  output, v_b = O_b W_o^T, in float64 like ``flow.velocity``;
* one guidance scale g per unit, the same at every step.
"""
from __future__ import annotations

import numpy as np

from .attention import attention
from .flow import euler_step, velocity
from .qkv import qkv_projection
from .ring import kv_append


def guided_velocity(v_c, v_u, g: float):
    """Classifier-free guidance: extrapolate from v_u through v_c by g."""
    return v_u + g * (v_c - v_u)


def _branch(b):
    rk, rv, ln, hd_ = b["ring_k"], b["ring_v"], b["length"], b["head"]
    if b.get("slice_k") is not None:
        rk, rv, ln, hd_ = kv_append(rk, rv, ln, hd_, b["slice_k"], b["slice_v"])
    return rk, rv, ln, hd_


def denoise_unit_cfg(cond, uncond, eps, hs, g: float, w_qkv_bits, w_o_bits, n_heads: int):
    """cond / uncond: dicts with ring_k, ring_v, length, head and optional
    slice_k, slice_v (each branch's cache and the slice appended to it first).
    Runs len(hs) guided Euler steps from eps, projecting Q, K_u, V_u from the
    current z at every step.  Returns dict(z, Oc, Ou, cond=(ring_k, ring_v,
    length, head), uncond=(...)); Oc / Ou hold each step's attention outputs."""
    bc, bu = _branch(cond), _branch(uncond)
    z = np.asarray(eps, dtype=np.float64)
    Ocs, Ous = [], []
    for h in hs:
        q, k_u, v_u = qkv_projection(z, w_qkv_bits, n_heads)
        o_c = attention(q, *bc, k_u, v_u)
        o_u = attention(q, *bu, k_u, v_u)
        n = o_c.shape[0]
        v = guided_velocity(velocity(o_c.reshape(n, -1), w_o_bits),
                            velocity(o_u.reshape(n, -1), w_o_bits), g)
        z = euler_step(z, h, v)
        Ocs.append(o_c)
        Ous.append(o_u)
    return dict(z=z, Oc=Ocs, Ou=Ous, cond=bc, uncond=bu)
