"""GPU parity of the ring append (bit-exact against the oracle)."""
import numpy as np
import pytest

import oracle
import workload
from tests.pins import random_bits

pytestmark = pytest.mark.gpu

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import DEV, cache_logical, dev_bf16, make_cache  # noqa: E402


def _run_case(H, hd, cap, slices, head0, len0, seed=0):
    rng = np.random.default_rng(seed)
    rk = np.full((H, cap, hd), 0x7FC0, dtype=np.uint16)          # NaN poison
    rv = rk.copy()
    valid = (head0 - len0 + np.arange(len0)) % cap
    rk[:, valid, :] = random_bits(rng, (H, len0, hd))
    rv[:, valid, :] = random_bits(rng, (H, len0, hd))
    shape = workload.custom_session(H, hd, 1, 0, 0, cap, len0, head0, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    ok, ov, ol, oh = rk, rv, len0, head0
    for T in slices:
        sk = random_bits(rng, (T, H, hd))
        sv = random_bits(rng, (T, H, hd))
        fmd.kv_append(cache, dev_bf16(sk), dev_bf16(sv))
        ok, ov, ol, oh = oracle.kv_append(ok, ov, ol, oh, sk, sv)
    torch.cuda.synchronize()
    gk, gv = cache_logical(fmd, cache)
    print(f"append H={H} hd={hd} cap={cap} slices={slices} head0={head0} len0={len0}", flush=True)
    assert (cache.len_tokens, cache.head_tokens) == (ol, oh)
    assert np.array_equal(gk, ok), "K ring bytes differ"
    assert np.array_equal(gv, ov), "V ring bytes differ"


@pytest.mark.parametrize("H,hd,cap,slices,head0,len0", [
    (2, 64, 128, [32], 96, 96),                 # tiny ring, fills the last unit
    (2, 64, 128, [32], 112, 96),                # straddles the wrap point
    (3, 128, 64, [64], 5, 10),                  # T == cap at an unaligned head
    (2, 128, 48, [48], 47, 0),                  # T == cap, head just before the end
    (1, 64, 32, [1] * 40, 31, 0),               # single tokens, repeated wraps
    (2, 128, 80, [7, 9, 13, 3, 30, 50], 3, 0),  # ragged slices, partial blocks
    (4, 128, 16, [16, 5], 8, 16),               # smallest ring
])
def test_append_bit_exact(H, hd, cap, slices, head0, len0):
    _run_case(H, hd, cap, slices, head0, len0)


def test_append_batched_matches_single():
    rng = np.random.default_rng(3)
    specs = [(96, 40, 17), (160, 0, 64), (48, 47, 48)]   # (cap, head0, T)
    H, hd = 3, 128
    caches, ks, vs, refs = [], [], [], []
    for cap, head0, T in specs:
        rk = random_bits(rng, (H, cap, hd))
        rv = random_bits(rng, (H, cap, hd))
        shape = workload.custom_session(H, hd, 1, 0, 0, cap, cap, head0, (1.0,))
        caches.append(make_cache(fmd, shape, rk, rv))
        sk, sv = random_bits(rng, (T, H, hd)), random_bits(rng, (T, H, hd))
        ks.append(dev_bf16(sk))
        vs.append(dev_bf16(sv))
        refs.append(oracle.kv_append(rk, rv, cap, head0, sk, sv))
    fmd.kv_append_batched(caches, ks, vs)
    torch.cuda.synchronize()
    for c, (ok, ov, ol, oh) in zip(caches, refs):
        gk, gv = cache_logical(fmd, c)
        assert (c.len_tokens, c.head_tokens) == (ol, oh)
        assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


def test_prepared_append_matches_oracle_twice():
    # The prepared call reads the caches' current state at every launch: two
    # launches without resetting it append twice, as two batched calls would.
    rng = np.random.default_rng(4)
    specs = [(96, 40, 17), (64, 63, 30)]   # (cap, head0, T)
    H, hd = 2, 64
    caches, ks, vs, refs = [], [], [], []
    for cap, head0, T in specs:
        rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
        shape = workload.custom_session(H, hd, 1, 0, 0, cap, cap, head0, (1.0,))
        caches.append(make_cache(fmd, shape, rk, rv))
        sk, sv = random_bits(rng, (T, H, hd)), random_bits(rng, (T, H, hd))
        ks.append(dev_bf16(sk))
        vs.append(dev_bf16(sv))
        k1, v1, l1, h1 = oracle.kv_append(rk, rv, cap, head0, sk, sv)
        refs.append(oracle.kv_append(k1, v1, l1, h1, sk, sv))
    prep = fmd.PreparedAppend(caches, ks, vs)
    prep.launch()
    prep.launch()
    torch.cuda.synchronize()
    for c, (ok, ov, ol, oh) in zip(caches, refs):
        gk, gv = cache_logical(fmd, c)
        assert (c.len_tokens, c.head_tokens) == (ol, oh)
        assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


@pytest.mark.parametrize("name", ["v01_unit", "v02_unit"])
def test_append_full_size(name):
    # The unit's append at the full shapes (poisoned last unit gets overwritten).
    wl = workload.get(name)
    s = wl.sessions[0]
    si = workload.make_inputs(wl, poison_invalid=True).sessions[0]
    cache = make_cache(fmd, s, si.ring_k, si.ring_v)
    fmd.kv_append(cache, dev_bf16(si.slice_k), dev_bf16(si.slice_v))
    ok, ov, ol, oh = oracle.kv_append(si.ring_k, si.ring_v, s.len_before, s.head_before,
                                      si.slice_k, si.slice_v)
    torch.cuda.synchronize()
    gk, gv = cache_logical(fmd, cache)
    print(f"append full size {name}", flush=True)
    assert (cache.len_tokens, cache.head_tokens) == (ol, oh)
    assert np.array_equal(gk, ok) and np.array_equal(gv, ov)


def test_append_rejects_oversize_and_keeps_state():
    shape = workload.custom_session(2, 64, 1, 0, 0, 32, 10, 10, (1.0,))
    z = np.zeros((2, 32, 64), dtype=np.uint16)
    cache = make_cache(fmd, shape, z, z)
    big = torch.zeros((33, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fmd.FmdError) as e:
        fmd.kv_append(cache, big, big)
    assert e.value.name == "FMD_E_CAPACITY"
    assert (cache.len_tokens, cache.head_tokens) == (10, 10)
