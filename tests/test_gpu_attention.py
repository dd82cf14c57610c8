"""GPU parity of the attention kernel (through fmd_attention) against the
oracle, plus the oracle's invariants checked on the GPU."""

import numpy as np
import pytest

import oracle
import workload
from tests.pins import bits, random_bits

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import (DEV, assert_close, dev_bf16, host_f64, make_cache,  # noqa: E402
                            rel_l2)

pytestmark = pytest.mark.gpu


def _attn_case(H, hd, cap, length, head, n_q, seed=0, poison=True, split=None, n_audio=0):
    rng = np.random.default_rng(seed)
    rk = random_bits(rng, (H, cap, hd))
    rv = random_bits(rng, (H, cap, hd))
    if poison:
        valid = np.zeros(cap, bool)
        valid[(head - length + np.arange(length)) % cap] = True
        rk[:, ~valid, :] = 0x7FC0
        rv[:, ~valid, :] = 0x7FC0
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    shape = workload.custom_session(H, hd, n_q - n_audio, n_audio, 0, cap, length, head, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    unit = fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu), n_audio=n_audio)
    with fmd.forced_attn_groups(split):
        o = fmd.attention([unit])
        torch.cuda.synchronize()
    ref = oracle.attention(q, rk, rv, length, head, ku, vu)
    return host_f64(o), ref


CASES = [
    # H, hd, cap, len, head, n_q
    (2, 64, 128, 128, 0, 16),          # the tiny workload's shape
    (2, 128, 128, 100, 37, 16),        # partial ring, unaligned segment
    (3, 128, 256, 200, 50, 33),        # wrapped valid range, two segments
    (2, 128, 64, 0, 0, 1),             # empty cache, single query
    (1, 128, 1024, 777, 913, 260),     # v0.1-class query count, ragged tail
    (2, 64, 512, 300, 17, 300),        # hd 64, two query blocks
    (4, 128, 2048, 2048, 1000, 257),   # full ring, one row into the second block
]


@pytest.mark.parametrize("case", CASES)
def test_attention_matches_oracle(case):
    got, ref = _attn_case(*case)
    assert_close(got, ref, f"O {case}")


@pytest.mark.parametrize("H", [3, 20])
def test_attention_head_aligned_groups(H):
    # A full, wrapped 16,384-key ring and 300 queries (two query blocks): the
    # default planner takes a multiple of the head count (96 groups for 3
    # heads, 120 for 20), so group boundaries fall on lane boundaries and on
    # window boundaries inside lanes; every row of every head is compared.
    got, ref = _attn_case(H, 128, 16384, 16384, 5000, 300, seed=11 + H)
    assert_close(got, ref, f"O H={H}")


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_attention_key_splits_agree(split):
    got, ref = _attn_case(2, 128, 4096, 3000, 100, 100, seed=5, split=split)
    assert_close(got, ref, f"O split={split}")


@pytest.mark.parametrize("length", [1, 59, 64, 130, 200, 250, 320, 400, 450, 510, 580, 640, 700,
                                    760, 1000])
def test_attention_window_counts(length):
    # One split per key segment; the ring segment starts off a 16-slot block
    # so that its first and last 64-key windows are partial.  1..17 windows
    # walk the pipeline's prologue, steady and last-step paths.
    head = (5 + length) % 2048
    got, ref = _attn_case(1, 128, 2048, length, head, 40, seed=length, split=1)
    assert_close(got, ref, f"O length={length}")


def test_single_key_returns_value_exactly():
    rng = np.random.default_rng(1)
    H, hd = 3, 128
    q, ku, vu = (random_bits(rng, (1, H, hd)) for _ in range(3))
    rk = np.full((H, 32, hd), 0x7FC0, dtype=np.uint16)
    shape = workload.custom_session(H, hd, 1, 0, 0, 32, 0, 0, (1.0,))
    cache = make_cache(fmd, shape, rk, rk)
    o = fmd.attention([fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu))])
    torch.cuda.synchronize()
    assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), vu)


def test_values_one_give_one():
    rng = np.random.default_rng(2)
    H, hd, cap, n_q = 2, 128, 256, 40
    one = bits(np.ones(1))[0]
    rk = random_bits(rng, (H, cap, hd))
    rv = np.full((H, cap, hd), one, dtype=np.uint16)
    q, ku = random_bits(rng, (n_q, H, hd)), random_bits(rng, (n_q, H, hd))
    vu = np.full((n_q, H, hd), one, dtype=np.uint16)
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, 190, 70, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    o = host_f64(fmd.attention([fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu))]))
    assert np.max(np.abs(o - 1.0)) <= 2 ** -8


def test_uniform_keys_give_mean():
    rng = np.random.default_rng(3)
    H, hd, cap, n_q, length, head = 2, 128, 192, 20, 150, 20
    c = bits(np.full(1, 0.5))[0]
    rk = np.full((H, cap, hd), c, dtype=np.uint16)
    rv = random_bits(rng, (H, cap, hd))
    q = random_bits(rng, (n_q, H, hd))
    ku = np.full((n_q, H, hd), c, dtype=np.uint16)
    vu = random_bits(rng, (n_q, H, hd))
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, length, head, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    o = host_f64(fmd.attention([fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu))]))
    slots = (head - length + np.arange(length)) % cap
    seen = np.concatenate([oracle.bf16_bits_to_f64(rv[:, slots, :]).transpose(1, 0, 2),
                           oracle.bf16_bits_to_f64(vu)])
    assert_close(o, np.broadcast_to(seen.mean(axis=0), o.shape), "uniform keys")


def test_ring_rotation_invariance():
    rng = np.random.default_rng(4)
    H, hd, cap, n_q, length = 2, 128, 320, 24, 230
    ck, cv = random_bits(rng, (H, length, hd)), random_bits(rng, (H, length, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    outs = []
    for head in (230, 0, 77, 319):
        rk = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)
        rv = rk.copy()
        slots = (head - length + np.arange(length)) % cap
        rk[:, slots], rv[:, slots] = ck, cv
        shape = workload.custom_session(H, hd, n_q, 0, 0, cap, length, head, (1.0,))
        cache = make_cache(fmd, shape, rk, rv)
        outs.append(host_f64(fmd.attention(
            [fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu))])))
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) <= 1e-2 and np.max(np.abs(o - outs[0])) <= 2e-2


def test_attention_deterministic():
    a, _ = _attn_case(2, 128, 1024, 900, 300, 70, seed=9)
    b, _ = _attn_case(2, 128, 1024, 900, 300, 70, seed=9)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("hd,length,split", [(128, 1000, 1), (128, 1000, None), (64, 1000, 1),
                                             (128, 300, 1), (128, 130, 1)])
def test_rising_scores_move_the_running_maximum(hd, length, split):
    # Keys along the ring order carry a growing component along the queries'
    # common direction, so the scores rise by about 10 (exp2 units) per
    # 64-key window: the running maximum passes the lazy-rescale threshold in
    # nearly every window, in the first window, the steady steps and the last
    # steps, and O is dominated by the newest keys.
    rng = np.random.default_rng(100 + hd + length)
    H, cap, n_q = 2, 2048, 40
    head = (5 + length) % cap
    u = np.ones(hd)
    step_per_key = 10.0 / (64 * np.sqrt(hd) * np.log2(np.e))
    alpha = step_per_key * np.arange(length)
    ck = bits((rng.standard_normal((H, length, hd)) + alpha[None, :, None] * u).astype(np.float32))
    cv = random_bits(rng, (H, length, hd))
    rk = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)
    rv = rk.copy()
    slots = (head - length + np.arange(length)) % cap
    rk[:, slots], rv[:, slots] = ck, cv
    q = bits((u + 0.1 * rng.standard_normal((n_q, H, hd))).astype(np.float32))
    ku, vu = random_bits(rng, (n_q, H, hd)), random_bits(rng, (n_q, H, hd))
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, length, head, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    with fmd.forced_attn_groups(split):
        got = host_f64(fmd.attention([fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu))]))
    ref = oracle.attention(q, rk, rv, length, head, ku, vu)
    # The newest keys dominate: O is far from the plain mean of the values.
    assert np.max(np.abs(ref - oracle.bf16_bits_to_f64(cv).mean(axis=1)[None])) > 0.5
    assert_close(got, ref, f"O rising scores hd={hd} length={length} split={split}")


@pytest.mark.parametrize("length", [400, 640, 1000])
def test_attention_window_counts_hd64(length):
    # 64-wide heads through the steady loop (8, 11 and 17 windows).
    head = (5 + length) % 2048
    got, ref = _attn_case(1, 64, 2048, length, head, 40, seed=length, split=1)
    assert_close(got, ref, f"O hd=64 length={length}")
