"""Pins for the oracle's ring append: the ring after a sequence of appends must
equal what the append history implies (each slot holds the latest token that
maps to it), derived here with vectorised index arithmetic instead of the
oracle's token loop."""
import numpy as np
import pytest

import oracle
from tests.pins import expected_ring_from_history, random_bits


def _run(H, hd, cap, slice_lens, head0, len0=0, seed=0):
    rng = np.random.default_rng(seed)
    init_k = random_bits(rng, (H, cap, hd))
    init_v = random_bits(rng, (H, cap, hd))
    ks = [random_bits(rng, (T, H, hd)) for T in slice_lens]
    vs = [random_bits(rng, (T, H, hd)) for T in slice_lens]
    rk, rv, length, head = init_k, init_v, len0, head0
    for k, v in zip(ks, vs):
        rk, rv, length, head = oracle.kv_append(rk, rv, length, head, k, v)
    hist_k, hist_v = np.concatenate(ks), np.concatenate(vs)
    N = hist_k.shape[0]
    assert np.array_equal(rk, expected_ring_from_history(init_k, hist_k, head0, cap))
    assert np.array_equal(rv, expected_ring_from_history(init_v, hist_v, head0, cap))
    assert length == min(len0 + N, cap)
    assert head == (head0 + N) % cap
    return rk, rv, length, head, hist_k


@pytest.mark.parametrize("H,hd,cap,slice_lens,head0,len0", [
    (2, 64, 128, [32], 0, 96),            # fills the last free unit
    (2, 64, 128, [32], 112, 96),          # straddles the wrap point (112+32 > 128)
    (3, 16, 48, [48], 5, 0),              # T == cap at an unaligned head
    (2, 8, 40, [7, 7, 7, 7, 7, 7, 7], 3, 0),  # repeated appends past a full ring
    (1, 4, 16, [1] * 20, 15, 0),          # single-token appends wrapping
    (4, 32, 64, [17, 30, 1, 64], 63, 10),
])
def test_append_matches_history(H, hd, cap, slice_lens, head0, len0):
    _run(H, hd, cap, slice_lens, head0, len0)


def test_after_many_appends_ring_holds_last_slices():
    # cap/T slices of T tokens: after m >= cap/T appends the ring holds exactly
    # the last cap/T slices, each at its own unit position.
    H, hd, T, units = 2, 8, 12, 5
    cap = T * units
    rk, _, length, head, hist = _run(H, hd, cap, [T] * 13, 0, 0, seed=3)
    assert length == cap and head == (13 * T) % cap
    last = hist[-cap:]                                        # last `units` slices
    for j in range(cap):                                      # token j of the tail
        slot = (13 * T - cap + j) % cap
        assert np.array_equal(rk[:, slot, :], last[j])


def test_valid_slots_hold_latest_tokens():
    # Encode the history index in the data, then check the valid slots contain
    # exactly the last `length` indices (as a multiset; order is irrelevant).
    H, hd, cap = 1, 1, 37
    rk = np.zeros((H, cap, hd), dtype=np.uint16)
    length, head, n = 0, 11, 0
    for T in (5, 9, 20, 3, 14):
        sk = np.arange(n + 1, n + T + 1, dtype=np.uint16).reshape(T, 1, 1)
        rk, _, length, head = oracle.kv_append(rk, rk, length, head, sk, sk)
        n += T
        got = sorted(int(rk[0, p, 0]) for p in oracle.valid_slots(length, head, cap))
        assert got == list(range(n - length + 1, n + 1))


@pytest.mark.parametrize("T", [0, 129])
def test_append_rejects_bad_sizes(T):
    rk = np.zeros((1, 128, 8), dtype=np.uint16)
    s = np.zeros((T, 1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.kv_append(rk, rk, 0, 0, s, s)


def test_append_does_not_modify_inputs():
    rng = np.random.default_rng(1)
    rk = random_bits(rng, (2, 32, 8))
    before = rk.copy()
    s = random_bits(rng, (5, 2, 8))
    oracle.kv_append(rk, rk, 0, 30, s, s)
    assert np.array_equal(rk, before)
