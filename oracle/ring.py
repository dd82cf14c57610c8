"""Oracle: the performer's K/V ring cache.

Source: the performer keeps a preallocated local K/V cache; each unit the
thinker sends a compact K/V slice and the performer writes it into the cache
at the matching position before running the solver
[Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
方法概述和架构; Wan-Streamer v0.2 (zhao9797 blog), Infra; Wan-Streamer
(gongshangzheng blog), Fig. 2].

Reading: the cache is a ring of ``cap`` token slots per head.  A slice of T
tokens goes to slots ``(head + t) mod cap``; the oldest tokens are overwritten
once the ring is full.  The cache is held in logical layout ``[H][cap][hd]``
(bf16 bit patterns); the device may store it in another layout, and the tests
map that layout back to this one before comparing bytes.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns: a bf16 is the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def kv_append(ring_k, ring_v, length: int, head: int, slice_k, slice_v):
    """Write one slice into the ring, token by token.

    ring_k, ring_v: [H][cap][hd] bf16 bits (not modified; copies are returned).
    slice_k, slice_v: [T][H][hd] bf16 bits, token-major as a projection emits them.
    Returns (new_k, new_v, new_length, new_head).

    Slot of token t is (head + t) mod cap; afterwards head advances by T
    (mod cap) and the valid length saturates at cap.  T must be 1..cap.
    """
    cap = ring_k.shape[1]
    T = slice_k.shape[0]
    if T < 1 or T > cap:
        raise ValueError(f"slice of {T} tokens does not fit a ring of {cap}")
    if not (0 <= length <= cap and 0 <= head < cap):
        raise ValueError("ring state out of range")
    k = ring_k.copy()
    v = ring_v.copy()
    for t in range(T):
        p = (head + t) % cap
        k[:, p, :] = slice_k[t]
        v[:, p, :] = slice_v[t]
    return k, v, min(length + T, cap), (head + T) % cap


def valid_slots(length: int, head: int, cap: int) -> list:
    """The ``length`` slots written most recently: the ones just before ``head``."""
    return [(head - length + j) % cap for j in range(length)]
