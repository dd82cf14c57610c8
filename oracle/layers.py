"""Oracle: the z-dependent solver with a stack of L attention layers, each
with its own K/V ring.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the velocity network f_theta is a block-causal transformer evaluated
on the unit's noisy latents together with the clean context at every solver
step [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal Transformer and
3.4 条件流匹配]; the thinker hands the performer a K/V slice for the cache it
keeps [Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
方法概述和架构].  The pages give no layer count and no layer structure.

Readings:
* layer l has its own ring (the clean context's keys and values of that
  layer), its own W_qkv,l ([3d][d]) and W_o,l ([d][d]); every layer's ring
  takes the same number of slice tokens per unit (one slice per layer);
* residual stream: r_0 = 0; layer l reads a_l = z + r_l, rounded to bf16,
  projects [Q_l | K_l | V_l] = bf16(bf16(a_l) W_qkv,l^T), attends over its ring
  and its own K_l, V_l, and adds r_{l+1} = r_l + O_l W_o,l^T;
* the velocity is the sum of the layers' updates, v = r_L, and the Euler step
  is z <- z - h v; with L = 1 this is exactly ``qkv.denoise_unit_qkv``.
"""
from __future__ import annotations

import numpy as np

from .attention import attention
from .flow import euler_step, velocity
from .qkv import qkv_projection
from .ring import kv_append


def _layer_ring(b):
    rk, rv, ln, hd_ = b["ring_k"], b["ring_v"], b["length"], b["head"]
    if b.get("slice_k") is not None:
        rk, rv, ln, hd_ = kv_append(rk, rv, ln, hd_, b["slice_k"], b["slice_v"])
    return rk, rv, ln, hd_


def layer_stack_velocity(z, rings, w_qkv_bits, w_o_bits, n_heads: int):
    """v = r_L for the latent z over the layers' (post-append) rings."""
    z = np.asarray(z, dtype=np.float64)
    r = np.zeros_like(z)
    for ring, wq, wo in zip(rings, w_qkv_bits, w_o_bits):
        q, k_u, v_u = qkv_projection(z + r, wq, n_heads)
        o = attention(q, *ring, k_u, v_u)
        r = r + velocity(o.reshape(o.shape[0], -1), wo)
    return r


def denoise_unit_layers(layers, eps, hs, w_qkv_bits, w_o_bits, n_heads: int):
    """layers: per layer a dict with ring_k, ring_v, length, head and optional
    slice_k, slice_v; w_qkv_bits / w_o_bits: per layer.  Appends every layer's
    slice, then len(hs) Euler steps from eps.  Returns dict(z, rings)."""
    rings = [_layer_ring(b) for b in layers]
    z = np.asarray(eps, dtype=np.float64)
    for h in hs:
        z = euler_step(z, h, layer_stack_velocity(z, rings, w_qkv_bits, w_o_bits, n_heads))
    return dict(z=z, rings=rings)
