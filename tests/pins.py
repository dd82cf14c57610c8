"""Pin checks for the oracle, written as functions of the oracle entry points so
that the planted-mistake tests can run the same checks against a broken oracle.

Each check derives its expected value without the oracle's own code path:
from the append history (not from slot arithmetic), from a library attention
routine, or from a closed form.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from workload import round_to_bf16_bits


def bits(x):
    return round_to_bf16_bits(np.asarray(x, dtype=np.float32))


def widen(b):
    # Independent of the oracle's own widening: go through torch's bf16 type.
    t = torch.from_numpy(np.ascontiguousarray(b).astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def random_bits(rng, shape, scale=1.0):
    return bits(rng.standard_normal(shape).astype(np.float32) * scale)


def build_ring_by_history(rng, H, hd, cap, slice_lens, head0=0):
    """Empty ring (NaN-filled), then append the given slices through ``append_fn``
    later; returns the slices and the concatenated history [N][H][hd] for K, V."""
    ks = [random_bits(rng, (T, H, hd)) for T in slice_lens]
    vs = [random_bits(rng, (T, H, hd)) for T in slice_lens]
    return ks, vs


def apply_history(append_fn, H, hd, cap, ks, vs, head0):
    nan = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)
    rk, rv, length, head = nan.copy(), nan.copy(), 0, head0
    for k, v in zip(ks, vs):
        rk, rv, length, head = append_fn(rk, rv, length, head, k, v)
    return rk, rv, length, head


def sdpa_reference(q_bits, hist_k, hist_v, length, k_u, v_u):
    """torch SDPA in float64 over the last ``length`` tokens of history plus the
    unit's own tokens (no mask).  Returns [n_q][H][hd]."""
    tail_k = hist_k[len(hist_k) - length:] if length else hist_k[:0]
    tail_v = hist_v[len(hist_v) - length:] if length else hist_v[:0]
    K = np.concatenate([tail_k, k_u])          # [Lk][H][hd]
    V = np.concatenate([tail_v, v_u])
    qt = torch.from_numpy(widen(q_bits)).permute(1, 0, 2)[None]   # [1][H][n][hd]
    kt = torch.from_numpy(widen(K)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(widen(V)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o[0].permute(1, 0, 2).numpy()


def check_attention_vs_history(attention_fn, append_fn, seed=0, H=3, hd=16, cap=48,
                               slice_lens=(20, 13), head0=30, n_q=9):
    """max |oracle - SDPA(history tail || unit)| for a ring filled by appends
    (default: a partly filled ring whose valid range wraps; unwritten slots are
    NaN, so reading one gives an infinite error)."""
    rng = np.random.default_rng(seed)
    ks, vs = build_ring_by_history(rng, H, hd, cap, slice_lens)
    rk, rv, length, head = apply_history(append_fn, H, hd, cap, ks, vs, head0)
    hist_k, hist_v = np.concatenate(ks), np.concatenate(vs)
    q = random_bits(rng, (n_q, H, hd))
    k_u = random_bits(rng, (n_q, H, hd))
    v_u = random_bits(rng, (n_q, H, hd))
    got = attention_fn(q, rk, rv, length, head, k_u, v_u)
    ref = sdpa_reference(q, hist_k, hist_v, min(sum(slice_lens), cap), k_u, v_u)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref)))


def expected_ring_from_history(init, hist, head0, cap):
    """Closed form of the ring after writing history token n at (head0+n) mod cap:
    each slot holds the latest token that maps to it, else its initial bytes."""
    N = hist.shape[0]
    out = init.copy()
    p = np.arange(cap)
    r = (p - head0) % cap                      # first history index landing on p
    touched = r < N
    last = r + cap * ((N - 1 - r) // cap)      # latest index landing on p
    out[:, p[touched], :] = np.transpose(hist[last[touched]], (1, 0, 2))
    return out


def check_closed_form_flow(denoise_unit_fn, hs, seed=0, H=2, hd=8, n_q=5, cap=32, length=24):
    """K == 0 (uniform weights), every V row == w, W = I, start at eps.
    The velocity is exactly w = eps - z0 with z0 := eps - w, so Euler over any
    schedule summing to 1 must land on z0.  Returns max |z - z0|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    w = bits(rng.standard_normal(d).astype(np.float32))       # bf16-exact values
    w_f = widen(w)
    zero = np.zeros((H, cap, hd), dtype=np.uint16)             # +0.0 bits
    ring_v = np.broadcast_to(w.reshape(H, 1, hd), (H, cap, hd)).copy()
    q = random_bits(rng, (n_q, H, hd))
    k_u = np.zeros((n_q, H, hd), dtype=np.uint16)
    v_u = np.broadcast_to(w.reshape(1, H, hd), (n_q, H, hd)).copy()
    eye = bits(np.eye(d, dtype=np.float32))
    eps = rng.standard_normal((n_q, d))
    z0 = eps - w_f[None, :]
    res = denoise_unit_fn(zero, ring_v, length, 3, None, None, [q], [k_u], [v_u],
                          eps, hs, eye)
    return float(np.max(np.abs(res["z"] - z0)))


def brute_velocity(o, w_bits):
    """v[i][n] = sum_k O[i][k] * W[n][k], scalar loops (tiny sizes only)."""
    W = widen(w_bits)
    n_rows, d = o.shape
    v = np.zeros((n_rows, W.shape[0]))
    for i in range(n_rows):
        for n in range(W.shape[0]):
            acc = 0.0
            for k in range(d):
                acc += o[i, k] * W[n, k]
            v[i, n] = acc
    return v


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def softmax_scale(hd):
    return 1.0 / math.sqrt(hd)


def check_values_one(attention_fn, seed=2, H=2, hd=16, cap=40, n_q=7):
    """V == 1 everywhere => O == 1 (softmax weights sum to one).  Returns max |O - 1|."""
    rng = np.random.default_rng(seed)
    one = bits(np.ones(1))[0]
    rk = random_bits(rng, (H, cap, hd))
    rv = np.full((H, cap, hd), one, dtype=np.uint16)
    q, ku = random_bits(rng, (n_q, H, hd)), random_bits(rng, (n_q, H, hd))
    vu = np.full((n_q, H, hd), one, dtype=np.uint16)
    o = attention_fn(q, rk, rv, 33, 5, ku, vu)
    return float(np.max(np.abs(o - 1.0)))


# ---------------------------------------------------------------------------
# Per-step Q/K/V projected from z.
# ---------------------------------------------------------------------------
def brute_qkv(z, w_bits, n_heads):
    """Scalar-loop [Q | K_u | V_u] = bf16(bf16(z) W^T), bf16 rounding by torch."""
    def rb(x):
        return torch.tensor(float(x), dtype=torch.float64).to(torch.float32).to(
            torch.bfloat16).to(torch.float64).item()
    z = np.asarray(z, dtype=np.float64)
    n, d = z.shape
    W = widen(w_bits)
    zb = [[rb(z[i, k]) for k in range(d)] for i in range(n)]
    out = np.zeros((3, n, d))
    for t in range(3):
        for i in range(n):
            for c in range(d):
                out[t, i, c] = rb(sum(zb[i][k] * W[t * d + c, k] for k in range(d)))
    hd = d // n_heads
    return [out[t].reshape(n, n_heads, hd) for t in range(3)]


def check_qkv_uniform_closed_form(unit_qkv_fn, hs=(0.5, 0.25, 0.125), seed=3, H=2, hd=8,
                                  cap=32, length=24, head=5, n_q=6):
    """W_q = 0 and W_v = 0: every query scores 0 on every key, so O is the plain
    mean of all seen values, the unit's own values being 0: O = (sum of the
    valid ring values) / (length + n_q), the same at every step whatever z is.
    Then z_final = eps - (sum h) * O_flat W_o^T.  Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    ring_k = random_bits(rng, (H, cap, hd))
    ring_v = random_bits(rng, (H, cap, hd))
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[d:2 * d] = random_bits(rng, (d, d))          # W_k nonzero: must not matter
    w_o = random_bits(rng, (d, d), scale=d ** -0.5)
    eps = rng.standard_normal((n_q, d))
    slots = [(head - length + i) % cap for i in range(length)]
    mean_v = widen(ring_v)[:, slots, :].sum(axis=1) / (length + n_q)   # [H][hd]
    v = np.tile(mean_v.reshape(1, d), (n_q, 1)) @ widen(w_o).T
    expect = eps - sum(hs) * v
    got = unit_qkv_fn(ring_k, ring_v, length, head, None, None, eps, list(hs), w, w_o, H)["z"]
    return float(np.max(np.abs(got - expect)))


def check_qkv_mean_decay(unit_qkv_fn, hs=(0.5, 0.5), seed=4, H=2, hd=8, n_q=16):
    """Empty cache, W_q = W_k = 0, W_v = I, W_o = I: every query attends
    uniformly to the unit's own values V_u = bf16(z), so the velocity of every
    row is the column mean of bf16(z) and each step maps z_i -> z_i - h mean(z).
    The deviations from the mean are invariant and the mean decays by (1 - h)
    per step: after the steps it is prod(1 - h) * mean(eps) (rounding of z to
    bf16 perturbs this by ~2^-9 of |z|).  A solver that kept projecting from
    eps would decay it by (1 - sum h) instead.  Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    eps = rng.standard_normal((n_q, d)) + 0.5
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[2 * d:] = bits(np.eye(d))
    w_o = bits(np.eye(d))
    ring = np.zeros((H, 16, hd), dtype=np.uint16)
    mean0 = eps.mean(axis=0, keepdims=True)
    expect = (eps - mean0) + np.prod([1.0 - h for h in hs]) * mean0
    got = unit_qkv_fn(ring, ring, 0, 0, None, None, eps, list(hs), w, w_o, H)["z"]
    return float(np.max(np.abs(got - expect)))


# ---------------------------------------------------------------------------
# Classifier-free-guided sampling (two branches, guidance scale g).
# ---------------------------------------------------------------------------
def check_cfg_uniform_closed_form(unit_cfg_fn, g=3.0, hs=(0.5, 0.25), seed=5, H=2, hd=8,
                                  cap=64, n_q=6):
    """W_q = 0 and W_v = 0: in each branch every query attends uniformly to all
    seen values, the unit's own being 0, so O_b = (sum of the branch's valid
    ring values + its appended slice) / (len_b + T_b + n_q) at every step.  The
    branches differ in length, start and slice; nothing is evicted (cap is
    large).  Then z_final = eps - (sum h) (v_u + g (v_c - v_u)), v_b = O_b W_o^T.
    Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[d:2 * d] = random_bits(rng, (d, d))          # W_k nonzero: must not matter
    w_o = random_bits(rng, (d, d), scale=d ** -0.5)
    eps = rng.standard_normal((n_q, d))
    branches, means = [], []
    for length, head, T in ((20, 50, 7), (33, 9, 4)):
        ring_k = random_bits(rng, (H, cap, hd))
        ring_v = random_bits(rng, (H, cap, hd))
        sk = random_bits(rng, (T, H, hd))
        sv = random_bits(rng, (T, H, hd))
        slots = [(head - length + i) % cap for i in range(length)]
        total = widen(ring_v)[:, slots, :].sum(axis=1) + widen(sv).sum(axis=0)   # [H][hd]
        means.append(total / (length + T + n_q))
        branches.append(dict(ring_k=ring_k, ring_v=ring_v, length=length, head=head,
                             slice_k=sk, slice_v=sv))
    W = widen(w_o)
    v_c, v_u = (np.tile(m.reshape(1, d), (n_q, 1)) @ W.T for m in means)
    expect = eps - sum(hs) * (v_u + g * (v_c - v_u))
    got = unit_cfg_fn(branches[0], branches[1], eps, list(hs), g, w, w_o, H)["z"]
    return float(np.max(np.abs(got - expect)))


def check_cfg_mean_decay(unit_cfg_fn, g=4.0, hs=(0.5, 0.5), seed=6, H=2, hd=8, n_q=16):
    """Both caches empty, W_q = W_k = 0, W_v = I, W_o = I: both branches see only
    the unit's own values, so v_c = v_u = mean(bf16(z)) and guidance changes
    nothing whatever g is; each step maps z_i -> z_i - h mean(z), the mean decays
    by prod(1 - h) (up to the bf16 rounding of z).  Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    eps = rng.standard_normal((n_q, d)) + 0.5
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[2 * d:] = bits(np.eye(d))
    w_o = bits(np.eye(d))
    empty = dict(ring_k=np.zeros((H, 16, hd), dtype=np.uint16),
                 ring_v=np.zeros((H, 16, hd), dtype=np.uint16), length=0, head=3)
    mean0 = eps.mean(axis=0, keepdims=True)
    expect = (eps - mean0) + np.prod([1.0 - h for h in hs]) * mean0
    got = unit_cfg_fn(empty, dict(empty), eps, list(hs), g, w, w_o, H)["z"]
    return float(np.max(np.abs(got - expect)))


# ---------------------------------------------------------------------------
# Stack of L attention layers with a residual stream.
# ---------------------------------------------------------------------------
def check_layers_uniform_closed_form(unit_layers_fn, hs=(0.5, 0.25), seed=9, H=2, hd=8,
                                     cap=64, n_q=5):
    """Every layer has W_q = 0 and W_v = 0: layer l's attention is the plain
    mean of its own valid ring values and slice over (len_l + T_l + n_q),
    whatever its input, so v = sum_l mean_l W_o,l^T and z_final = eps -
    (sum h) v.  The three layers have different rings, states, slices and
    W_o; nothing is evicted (len + T <= cap).  Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    eps = rng.standard_normal((n_q, d))
    layers, w_qkv, w_o, v = [], [], [], np.zeros((n_q, d))
    for length, head, T in ((30, 40, 6), (12, 3, 0), (47, 20, 9)):
        ring_k = random_bits(rng, (H, cap, hd))
        ring_v = random_bits(rng, (H, cap, hd))
        sk = random_bits(rng, (T, H, hd)) if T else None
        sv = random_bits(rng, (T, H, hd)) if T else None
        slots = [(head - length + i) % cap for i in range(length)]
        total = widen(ring_v)[:, slots, :].sum(axis=1)
        if T:
            total = total + widen(sv).sum(axis=0)
        mean = total / (length + T + n_q)
        w = np.zeros((3 * d, d), dtype=np.uint16)
        w[d:2 * d] = random_bits(rng, (d, d))
        wo = random_bits(rng, (d, d), scale=d ** -0.5)
        v = v + np.tile(mean.reshape(1, d), (n_q, 1)) @ widen(wo).T
        layers.append(dict(ring_k=ring_k, ring_v=ring_v, length=length, head=head,
                           slice_k=sk, slice_v=sv))
        w_qkv.append(w)
        w_o.append(wo)
    expect = eps - sum(hs) * v
    got = unit_layers_fn(layers, eps, list(hs), w_qkv, w_o, H)["z"]
    return float(np.max(np.abs(got - expect)))


def check_layers_residual_chain(unit_layers_fn, hs=(0.25, 0.25), seed=10, H=2, hd=8, n_q=16):
    """Two layers, empty rings, W_q = W_k = 0, W_v = I, W_o = I: layer 0 sees
    z and adds mean(z) to every row; layer 1 sees z + mean(z), whose mean is
    2 mean(z), and adds it; so v = 3 mean(z) (up to bf16 rounding of the layer
    inputs), deviations from the mean are invariant and the mean decays by
    (1 - 3h) per step.  Layer 1 fed with z instead of z + r would give (1 - 2h).
    Returns max |error|."""
    rng = np.random.default_rng(seed)
    d = H * hd
    eps = rng.standard_normal((n_q, d)) + 0.5
    w = np.zeros((3 * d, d), dtype=np.uint16)
    w[2 * d:] = bits(np.eye(d))
    eye = bits(np.eye(d))
    empty = dict(ring_k=np.zeros((H, 16, hd), dtype=np.uint16),
                 ring_v=np.zeros((H, 16, hd), dtype=np.uint16), length=0, head=0)
    mean0 = eps.mean(axis=0, keepdims=True)
    expect = (eps - mean0) + np.prod([1.0 - 3.0 * h for h in hs]) * mean0
    got = unit_layers_fn([empty, dict(empty)], eps, list(hs), [w, w], [eye, eye], H)["z"]
    return float(np.max(np.abs(got - expect)))
