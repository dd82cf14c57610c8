"""GPU attention at the largest sizes the C ABI accepts: a ring of the maximum
capacity (one head's storage just under 2^31 bytes, wrapped, full) and a unit
of the maximum query count (2^22 queries).  With all keys zero every score is
zero, so every query attends uniformly: O = (sum of the valid ring values +
sum of the unit's values) / (len + n_q), the same for every query.  Values are
small multiples of 1/16 (exact in bf16) whose sums have closed forms, so the
expected output needs no full-size reference and the kernels' fp32 sums of
them are exact; only the final division and the bf16 store round."""
import numpy as np
import pytest

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import DEV, host_f64  # noqa: E402

pytestmark = pytest.mark.gpu


def _pattern_ring(n, hd, mult, period, offset):
    """bf16 [1][n][hd]: value (((slot * mult) % period - offset) + (e % 5 - 2)) / 16."""
    a = ((torch.arange(n, device=DEV, dtype=torch.int64) * mult) % period - offset).to(torch.int8)
    b = (torch.arange(hd, device=DEV, dtype=torch.int64) % 5 - 2).to(torch.int8)
    v = (a[:, None] + b[None, :]).to(torch.bfloat16)
    del a
    return v.div_(16)[None]


def _sum_a(slots, mult, period, offset):
    return int((((np.asarray(slots, dtype=np.int64) * mult) % period) - offset).sum())


def _expect(hd, ring_slots, n_q, ring_n):
    b = (np.arange(hd) % 5 - 2).astype(np.float64)
    tot = (_sum_a(ring_slots, 7, 9, 4) + len(ring_slots) * b
           + _sum_a(np.arange(n_q), 5, 7, 3) + n_q * b) / 16.0
    return tot / (len(ring_slots) + n_q)


def _check(o, want):
    # bf16 store of a value computed with one rounding: |err| <= 2^-8 |want|.
    got = o.float()
    w = torch.from_numpy(want).to(DEV, torch.float32).view(1, 1, -1)
    err = (got - w).abs().amax().item()
    bound = float(np.abs(want).max()) * 2.0 ** -8 + 1e-6
    print(f"max |O - closed form| = {err:.3e} (bound {bound:.3e})", flush=True)
    assert torch.isfinite(got).all()
    assert err <= bound


def test_attention_at_maximum_ring_capacity():
    H, hd, n_q = 1, 128, 40
    cap = ((2 ** 31 - 1) // (hd * 2)) // 16 * 16
    assert cap * hd * 2 < 2 ** 31 <= (cap + 16) * hd * 2
    head = 5_000_003                       # full ring, wrapped at an unaligned slot
    k = torch.zeros((H, cap, hd), dtype=torch.bfloat16, device=DEV)
    v = fmd.KVCache.logical_to_device_v(_pattern_ring(cap, hd, 7, 9, 4))
    cache = fmd.KVCache(H, hd, cap, device=DEV, k=k, v=v, len_tokens=cap, head_tokens=head)
    g = torch.Generator(device=DEV).manual_seed(1)
    q = torch.randn((n_q, H, hd), generator=g, device=DEV).to(torch.bfloat16)
    k_u = torch.zeros((n_q, H, hd), dtype=torch.bfloat16, device=DEV)
    v_u = _pattern_ring(n_q, hd, 5, 7, 3).reshape(n_q, H, hd).contiguous()
    print(f"cap {cap} head {head} n_q {n_q}", flush=True)
    o = fmd.attention([fmd.UnitStep(cache, q, k_u, v_u)])
    torch.cuda.synchronize()
    _check(o, _expect(hd, np.arange(cap), n_q, cap))


def test_attention_at_maximum_query_count():
    H, hd, n_q = 1, 64, 1 << 22
    cap, length, head = 64, 48, 20         # valid slots 36..63 and 0..19
    k = torch.zeros((H, cap, hd), dtype=torch.bfloat16, device=DEV)
    v = fmd.KVCache.logical_to_device_v(_pattern_ring(cap, hd, 7, 9, 4))
    cache = fmd.KVCache(H, hd, cap, device=DEV, k=k, v=v, len_tokens=length, head_tokens=head)
    g = torch.Generator(device=DEV).manual_seed(2)
    q = torch.randn((n_q, H, hd), generator=g, device=DEV).to(torch.bfloat16)
    k_u = torch.zeros((n_q, H, hd), dtype=torch.bfloat16, device=DEV)
    v_u = _pattern_ring(n_q, hd, 5, 7, 3).reshape(n_q, H, hd).contiguous()
    print(f"n_q {n_q} cap {cap} len {length} head {head}", flush=True)
    o = fmd.attention([fmd.UnitStep(cache, q, k_u, v_u)])
    torch.cuda.synchronize()
    slots = [(head - length + i) % cap for i in range(length)]
    _check(o, _expect(hd, slots, n_q, cap))
