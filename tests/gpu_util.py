"""Helpers for the GPU tests: move seeded inputs to the device, run the C ABI
through the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

DEV = torch.device("cuda:0")

# Tolerances: bf16 attention outputs and final latents, fp32 accumulation.
MAX_ABS = 2e-2
REL_L2 = 1e-2


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t):
    return t.float().cpu().double().numpy()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def make_cache(fmd, shape, ring_k, ring_v, after_append=False):
    """Device ring holding the given logical content and state."""
    ln = shape.len_after if after_append else shape.len_before
    hd_ = shape.head_after if after_append else shape.head_before
    return fmd.KVCache(shape.n_heads, shape.head_dim, shape.cap_tokens, device=DEV,
                       k=dev_bf16(ring_k),
                       v=fmd.KVCache.logical_to_device_v(dev_bf16(ring_v)),
                       len_tokens=ln, head_tokens=hd_)


def cache_logical(fmd, cache):
    """(K, V) bytes of a device ring in logical [H][cap][hd] layout."""
    return host_u16(cache.k), host_u16(fmd.KVCache.device_to_logical_v(cache.v))


def stack_steps(xs):
    return dev_bf16(np.stack(xs)) if len(xs) > 1 else dev_bf16(xs[0])


def assert_close(got, ref, what, max_abs=MAX_ABS, rel=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    ma = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rl = rel_l2(got, ref)
    print(f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}", flush=True)
    assert ma <= max_abs and rl <= rel, f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}"
    return ma, rl
