"""Oracle: attention of the unit's noisy tokens over [clean cache || own tokens].

Source: a single block-causal Transformer; every block attends to all earlier
blocks and to itself [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal
Transformer].  For the unit being denoised this means: its noisy audio and
video latents see the whole clean history (3.4, clean context) and each other
in both directions (3.4, cross-modal conditioning).  The multi-GPU version
splits this over ranks and still computes the same global attention
[Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
方法概述和架构], so the one-GPU result is the same function.

Readings where the pages are silent: scale 1/sqrt(head_dim); no mask inside
the unit or over the valid cache; no positional terms inside this step (any
rotary encoding is already in the given Q and K); sessions never see each other.

The definition used is the textbook one: scores, the row maximum, exponentials
of the shifted scores, their sum, and the weighted mean of the values
(the maximum is subtracted only to keep exp finite; it cancels exactly).

``dtype`` selects the arithmetic: float64 (the default, the parity reference)
or float32 (the same steps with BLAS in single precision, used only to time
the oracle as a CPU baseline; pinned against float64 in the tests).
"""
from __future__ import annotations

import math

import numpy as np

from .ring import bf16_bits_to_f64, valid_slots


def _softmax_rows(s):
    """Row-wise softmax of a score block: shift by the row max, exponentiate,
    divide by the row sum (two passes over each row)."""
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def _widen(bits, dtype):
    return bf16_bits_to_f64(bits).astype(dtype, copy=False)


def _gather_head(ring_k, ring_v, length, head, k_u, v_u, h, dtype=np.float64):
    """Keys/values one head attends to: the valid ring slots, then the unit."""
    cap = ring_k.shape[1]
    slots = np.asarray(valid_slots(length, head, cap), dtype=np.int64)
    K = np.concatenate([_widen(ring_k[h][slots], dtype), _widen(k_u[:, h, :], dtype)])
    V = np.concatenate([_widen(ring_v[h][slots], dtype), _widen(v_u[:, h, :], dtype)])
    return K, V


def attention(q, ring_k, ring_v, length: int, head: int, k_u, v_u,
              rows=None, heads=None, row_chunk: int = 64, dtype=np.float64):
    """Attention output O [n_rows][H][hd] for one session (float64 unless
    ``dtype`` says otherwise).

    q, k_u, v_u: [n_q][H][hd] bf16 bits; ring_k/ring_v: [H][cap][hd] bf16 bits
    holding the post-append ring; (length, head) its state.
    ``rows``/``heads`` restrict the computation to a subset (for spot checks at
    full size); the returned array then has only those rows, and zeros in the
    heads that were skipped.
    """
    n_q, H, hd = q.shape
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    heads = range(H) if heads is None else heads
    scale = dtype(1.0 / math.sqrt(hd))
    out = np.zeros((len(rows), H, hd), dtype=dtype)
    for h in heads:
        K, V = _gather_head(ring_k, ring_v, length, head, k_u, v_u, h, dtype)
        Q = _widen(q[rows, h, :], dtype)
        for r0 in range(0, len(rows), row_chunk):
            s = (Q[r0:r0 + row_chunk] @ K.T) * scale          # scores
            out[r0:r0 + row_chunk, h, :] = _softmax_rows(s) @ V
    return out


def attention_naive(q, ring_k, ring_v, length: int, head: int, k_u, v_u):
    """Same definition with scalar Python loops.  Tiny inputs only."""
    n_q, H, hd = q.shape
    cap = ring_k.shape[1]
    f = bf16_bits_to_f64
    slots = valid_slots(length, head, cap)
    out = np.zeros((n_q, H, hd))
    for h in range(H):
        keys = [f(ring_k[h, p]) for p in slots] + [f(k_u[j, h]) for j in range(n_q)]
        vals = [f(ring_v[h, p]) for p in slots] + [f(v_u[j, h]) for j in range(n_q)]
        for i in range(n_q):
            qi = f(q[i, h])
            s = [sum(qi[e] * kj[e] for e in range(hd)) / math.sqrt(hd) for kj in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for e in range(hd):
                out[i, h, e] = sum(w[j] * vals[j][e] for j in range(len(w))) / tot
    return out
