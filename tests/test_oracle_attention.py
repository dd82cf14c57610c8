"""Pins for the oracle's attention: a library routine (torch SDPA, float64) on
keys gathered from the append history, scalar brute force, and invariants."""
import numpy as np
import pytest

import oracle
import workload
from tests.pins import (apply_history, bits, check_attention_vs_history, check_values_one,
                        random_bits, rel_l2, widen)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(H=3, hd=16, cap=48, slice_lens=(20, 20, 13), head0=7, n_q=9),   # full ring
    dict(H=2, hd=64, cap=128, slice_lens=(32, 32, 32, 32, 32), head0=0, n_q=16),
    dict(H=1, hd=8, cap=20, slice_lens=(3,), head0=19, n_q=1),        # short history
    dict(H=2, hd=32, cap=40, slice_lens=(40, 40), head0=13, n_q=12),  # full, wrapped
])
def test_attention_matches_sdpa_on_history(kw):
    err = check_attention_vs_history(oracle.attention, oracle.kv_append, **kw)
    assert err <= 1e-12, err


def test_naive_matches_vectorised_on_tiny_workload():
    wl = workload.get("tiny")
    ui = workload.make_inputs(wl)
    s = ui.sessions[0]
    sh = s.shape
    a = oracle.attention(s.q[0], s.ring_k, s.ring_v, sh.len_after, sh.head_after,
                         s.k_u[0], s.v_u[0])
    b = oracle.attention_naive(s.q[0], s.ring_k, s.ring_v, sh.len_after, sh.head_after,
                               s.k_u[0], s.v_u[0])
    assert np.max(np.abs(a - b)) <= 1e-12


def test_rows_and_heads_subset_equals_full():
    rng = np.random.default_rng(5)
    H, hd, cap, n_q = 3, 16, 64, 20
    rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    full = oracle.attention(q, rk, rv, 50, 9, ku, vu)
    rows = [0, 7, 19]
    part = oracle.attention(q, rk, rv, 50, 9, ku, vu, rows=rows, heads=[1])
    assert np.array_equal(part[:, 1], full[rows, 1])
    assert not part[:, 0].any() and not part[:, 2].any()


def test_values_all_one_give_one():
    # Softmax weights sum to one: V == 1 everywhere => O == 1.
    assert check_values_one(oracle.attention) <= 1e-15


def test_uniform_keys_give_mean_of_values():
    # K == c for every key => equal weights => O is the plain mean of the
    # values the query sees (the history tail and the unit).
    rng = np.random.default_rng(3)
    H, hd, cap, n_q = 2, 8, 30, 6
    c = bits(np.full(1, 0.375))[0]
    hist_v = random_bits(rng, (45, H, hd))
    hist_k = np.full((45, H, hd), c, dtype=np.uint16)
    rk, rv, length, head = apply_history(oracle.kv_append, H, hd, cap,
                                         [hist_k[:20], hist_k[20:]],
                                         [hist_v[:20], hist_v[20:]], head0=4)
    q = random_bits(rng, (n_q, H, hd))
    ku = np.full((n_q, H, hd), c, dtype=np.uint16)
    vu = random_bits(rng, (n_q, H, hd))
    o = oracle.attention(q, rk, rv, length, head, ku, vu)
    seen = np.concatenate([widen(hist_v[-length:]), widen(vu)])     # [Lk][H][hd]
    mean = seen.mean(axis=0)
    assert np.max(np.abs(o - mean[None])) <= 1e-14


def test_single_key_returns_its_value():
    # Empty cache and a single query: the only key is the query's own.
    rng = np.random.default_rng(4)
    H, hd, cap = 3, 32, 16
    rk = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)             # all invalid
    q, ku, vu = (random_bits(rng, (1, H, hd)) for _ in range(3))
    o = oracle.attention(q, rk, rk, 0, 0, ku, vu)
    assert np.array_equal(o, widen(vu))


def test_ring_rotation_and_poison_do_not_change_output():
    # Same valid content at a different head offset, and NaN in every slot that
    # is not valid: the output must be identical and finite.
    rng = np.random.default_rng(6)
    H, hd, cap, n_q, length = 2, 16, 50, 8, 31
    content_k = random_bits(rng, (H, length, hd))
    content_v = random_bits(rng, (H, length, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    outs = []
    for head in (31, 0, 17, 49):
        rk = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)
        rv = rk.copy()
        slots = (head - length + np.arange(length)) % cap
        rk[:, slots, :] = content_k
        rv[:, slots, :] = content_v
        outs.append(oracle.attention(q, rk, rv, length, head, ku, vu))
    assert np.all(np.isfinite(outs[0]))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-12


def test_sessions_workload_shapes():
    # The shapes the pages imply (two resolutions, 160 ms units) as drawn.
    w = workload.get("v02_unit").sessions[0]
    assert (w.n_q, w.d, w.keys_per_query) == (928, 5120, 61344)
    w1 = workload.get("v01_unit").sessions[0]
    assert (w1.n_q, w1.d, w1.keys_per_query) == (260, 1536, 8836)
    b = workload.get("v02_batch8").sessions
    assert len(b) == 8 and all(8 * 944 <= s.cap_tokens <= 128 * 944 for s in b)


def test_attention_vs_sdpa_random_shapes():
    # Small randomised sweep of shapes and ring states.
    rng = np.random.default_rng(11)
    for trial in range(8):
        H = int(rng.integers(1, 4))
        hd = int(rng.choice([8, 16, 64]))
        cap = int(rng.integers(4, 60))
        n_q = int(rng.integers(1, 20))
        lens = [int(rng.integers(1, cap + 1)) for _ in range(int(rng.integers(1, 4)))]
        head0 = int(rng.integers(0, cap))
        err = check_attention_vs_history(oracle.attention, oracle.kv_append, seed=trial,
                                         H=H, hd=hd, cap=cap, slice_lens=tuple(lens),
                                         head0=head0, n_q=n_q)
        assert err <= 1e-12, (trial, err)
        _ = rel_l2  # noqa


@pytest.mark.parametrize("H,hd,cap,length,head,n_q", [
    (2, 64, 128, 128, 0, 16), (3, 128, 1024, 700, 913, 77), (1, 128, 4096, 4096, 1234, 130)])
def test_float32_mode_matches_float64(H, hd, cap, length, head, n_q):
    # The float32 mode (used only to time the oracle on the CPU) computes the
    # same steps: against the float64 reference its error is single-precision
    # rounding, and its dtype really is float32.
    rng = np.random.default_rng(hd + cap)
    rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    a = oracle.attention(q, rk, rv, length, head, ku, vu)
    b = oracle.attention(q, rk, rv, length, head, ku, vu, dtype=np.float32)
    assert b.dtype == np.float32
    assert rel_l2(b, a) <= 1e-5, rel_l2(b, a)
    w = random_bits(rng, (H * hd, H * hd), scale=(H * hd) ** -0.5)
    va = oracle.velocity(a.reshape(n_q, -1), w)
    vb = oracle.velocity(b.reshape(n_q, -1), w, dtype=np.float32)
    assert vb.dtype == np.float32 and rel_l2(vb, va) <= 1e-5
    z = rng.standard_normal((n_q, H * hd)).astype(np.float32)
    za, zb = oracle.euler_step(z, 0.25, va), oracle.euler_step(z, 0.25, vb, dtype=np.float32)
    assert zb.dtype == np.float32 and np.max(np.abs(zb - za)) <= 1e-5
