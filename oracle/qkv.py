"""Oracle: the unit's queries, keys and values projected from the latent at
every solver step (the step the velocity network takes first).

Source: the velocity field is f_theta evaluated on the current noisy latents
of the unit, together with the clean context, at every flow time the solver
visits [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配: one network
predicts the velocities of both modalities from the noisy latents; 3.3
Block-Causal Transformer: the unit's tokens attend to the clean history and to
each other].  Each solver step therefore re-derives the unit's own Q, K and V
from the latent z it has reached.

Readings where the pages are silent (they give no architecture):
* the unit's Q, K, V are one linear map of z: [Q | K_u | V_u] = z W_qkv^T with
  W_qkv stored [3d][d] ([d_out][d_in]); output column h*hd + e of each third is
  head h, feature e;
* activations are bf16: z is rounded to bf16 (round to nearest, ties to even)
  before the map, and Q, K_u, V_u are rounded to bf16 after it; the cache, W_o
  and the rest of the step are unchanged;
* no positional terms, norms or biases.
"""
from __future__ import annotations

import numpy as np

from .flow import denoise_step
from .ring import bf16_bits_to_f64, kv_append


def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    A bf16 keeps 8 significant bits: x = m * 2^e with m in [0.5, 1) is rounded
    to (round-half-even(m * 2^8)) * 2^(e - 8).  Returns float64 values that are
    exactly representable in bf16 (normal range; zero stays zero)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def f64_to_bf16_bits(x):
    """bf16 bit patterns of values that are already bf16-representable."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def qkv_projection(z, w_qkv_bits, n_heads: int):
    """Q, K_u, V_u (bf16 bits, each [n][H][hd]) of the latent z [n][d]."""
    z = np.asarray(z, dtype=np.float64)
    n, d = z.shape
    W = bf16_bits_to_f64(w_qkv_bits)
    assert W.shape == (3 * d, d), W.shape
    y = round_to_bf16(round_to_bf16(z) @ W.T)
    hd = d // n_heads
    parts = [f64_to_bf16_bits(y[:, t * d:(t + 1) * d]).reshape(n, n_heads, hd) for t in range(3)]
    return parts[0], parts[1], parts[2]


def denoise_unit_qkv(ring_k, ring_v, length, head, slice_k, slice_v, eps, hs, w_qkv_bits,
                     w_o_bits, n_heads: int):
    """Append the slice (if any), then len(hs) Euler steps from eps, each
    projecting Q, K_u, V_u from the current z.  Returns dict(z, Os, qkv, ring_k,
    ring_v, length, head); qkv holds each step's (Q, K_u, V_u) bits."""
    if slice_k is not None:
        ring_k, ring_v, length, head = kv_append(ring_k, ring_v, length, head, slice_k, slice_v)
    z = np.asarray(eps, dtype=np.float64)
    Os, qkv = [], []
    for h in hs:
        q, k_u, v_u = qkv_projection(z, w_qkv_bits, n_heads)
        qkv.append((q, k_u, v_u))
        z, O = denoise_step(q, ring_k, ring_v, length, head, k_u, v_u, z, h, w_o_bits)
        Os.append(O)
    return dict(z=z, Os=Os, qkv=qkv, ring_k=ring_k, ring_v=ring_v, length=length, head=head)
