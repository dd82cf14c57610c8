"""The per-rank kernel of Ulysses context parallel at its real shape, on one
GPU: after the sequence -> head exchange, rank r of P holds every token of the
unit for its H/P heads and the head shard of the (pre-sharded) ring, so its
attention is this library's attention on a head slice.  Running all P ranks'
shares one after another and stacking their outputs must give global
attention (checked against the oracle on sampled rows); the exchange itself
is pinned on the CPU by the oracle's Ulysses simulation."""
import numpy as np
import pytest

import oracle
import workload

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import DEV, assert_close, dev_bf16, host_f64  # noqa: E402

pytestmark = pytest.mark.gpu


def _full_ring_640x368():
    # The 640x368-class unit's shape with its ring full (60,416 keys) and
    # wrapped: valid slots start at the append position.
    cap = 64 * 944
    s = workload.custom_session(40, 128, 920, 8, 0, cap, cap, 63 * 944, (1.0,))
    seed = 7
    rk = workload.ring_logical(seed, 0, s, "ring_k")
    rv = workload.ring_logical(seed, 0, s, "ring_v")
    q, ku, vu = (workload.token_major(seed, 0, s, n, s.n_q, step=0) for n in ("q", "k_u", "v_u"))
    return s, rk, rv, q, ku, vu


@pytest.mark.parametrize("P", [8, 4])
def test_ulysses_rank_shares_give_global_attention(P):
    s, rk, rv, q, ku, vu = _full_ring_640x368()
    H, hd = s.n_heads, s.head_dim
    hp = H // P
    print(f"P={P}: {hp} heads per rank, {s.n_q} queries x {s.cap_tokens + s.n_q} keys", flush=True)
    o = torch.empty((s.n_q, H, hd), dtype=torch.bfloat16, device=DEV)
    for r in range(P):
        h0, h1 = r * hp, (r + 1) * hp
        cache = fmd.KVCache(hp, hd, s.cap_tokens, device=DEV, k=dev_bf16(rk[h0:h1]),
                            v=fmd.KVCache.logical_to_device_v(dev_bf16(rv[h0:h1])),
                            len_tokens=s.len_before, head_tokens=s.head_before)
        unit = fmd.UnitStep(cache, dev_bf16(np.ascontiguousarray(q[:, h0:h1])),
                            dev_bf16(np.ascontiguousarray(ku[:, h0:h1])),
                            dev_bf16(np.ascontiguousarray(vu[:, h0:h1])), n_audio=s.n_audio)
        o[:, h0:h1] = fmd.attention([unit])
        del cache, unit
    torch.cuda.synchronize()
    rng = np.random.default_rng(P)
    rows = np.unique(np.concatenate([[0, 114, 115, 255, 256, 919, 920, 927],
                                     rng.choice(s.n_q, 24, replace=False)]))
    ref = oracle.attention(q, rk, rv, s.len_before, s.head_before, ku, vu, rows=rows)
    assert_close(host_f64(o)[rows], ref, f"P={P} rank shares stacked, sampled rows")
