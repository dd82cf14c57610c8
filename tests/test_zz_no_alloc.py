"""fmd_denoise_unit_noalloc (scratch in the library's static device array)
against fmd_denoise_unit (scratch in a caller workspace), through the C ABI:
two calls in a row on the same GPU, the second with a smaller unit, each
compared with the workspace entry point on the same inputs.  Both run the same
kernels on the same plan, so the latents and rings must agree bit for bit, and
both stay within the parity tolerance of the oracle-checked path."""
import numpy as np
import pytest

import workload

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import DEV, assert_close, cache_logical, dev_bf16, host_f64, make_cache  # noqa: E402

pytestmark = pytest.mark.gpu


def _ios(ui):
    caches, ios, zs = [], [], []
    for si in ui.sessions:
        s = si.shape
        c = make_cache(fmd, s, si.ring_k, si.ring_v)
        z = torch.from_numpy(si.eps.copy()).to(DEV)
        sk = dev_bf16(si.slice_k) if si.slice_k is not None else None
        sv = dev_bf16(si.slice_v) if si.slice_v is not None else None
        ios.append(fmd.UnitIO(c, sk, sv, dev_bf16(np.stack(si.q)), dev_bf16(np.stack(si.k_u)),
                              dev_bf16(np.stack(si.v_u)), z, list(s.h), n_audio=s.n_audio))
        caches.append(c)
        zs.append(z)
    return caches, ios, zs


def _compare(name, wl):
    ui = workload.make_inputs(wl, poison_invalid=True)
    w_o = dev_bf16(ui.w_o)
    ref_c, ref_io, ref_z = _ios(ui)
    fmd.denoise_unit(ref_io, w_o)
    new_c, new_io, new_z = _ios(ui)
    fmd.denoise_unit_noalloc(new_io, w_o)
    torch.cuda.synchronize()
    for b, (rc, nc, rz, nz, si) in enumerate(zip(ref_c, new_c, ref_z, new_z, ui.sessions)):
        assert_close(host_f64(nz) - si.eps, host_f64(rz) - si.eps, f"{name} session {b} dz")
        assert torch.equal(nz, rz), f"{name} session {b}: latents differ"
        assert (nc.len_tokens, nc.head_tokens) == (rc.len_tokens, rc.head_tokens)
        gk, gv = cache_logical(fmd, nc)
        rk, rv = cache_logical(fmd, rc)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


def test_noalloc_two_calls_second_smaller():
    # First the 640x368-class unit (about 192 MB of scratch), then three small
    # ragged sessions reusing the same scratch with the first call's contents
    # left in it.
    big = workload.get("v02_unit")
    small = workload.custom_workload("noalloc_small", 31, [
        workload.custom_session(4, 128, 60, 4, 48, 480, 480, 96, (0.4, 0.3, 0.2, 0.1)),
        workload.custom_session(4, 128, 30, 2, 48, 192, 150, 150, (0.4, 0.3, 0.2, 0.1)),
        workload.custom_session(4, 128, 120, 8, 0, 960, 912, 912, (0.4, 0.3, 0.2, 0.1))])
    _compare("v02_unit", big)
    _compare("small", small)


def test_noalloc_rejects_a_unit_beyond_the_scratch_untouched():
    # Two sessions over wrapped 242k-key rings of the 640x368-class shape,
    # four steps with their own Q/K/V, need more scratch than the static
    # array (384 MB against 256 MiB): FMD_E_WORKSPACE, no kernel, ring states
    # unchanged.
    H, hd, units = 40, 128, 256
    cap = units * 944
    ios, caches = [], []
    w = torch.zeros((H * hd, H * hd), dtype=torch.bfloat16, device=DEV)
    for _ in range(2):
        cache = fmd.KVCache(H, hd, cap, device=DEV, len_tokens=cap, head_tokens=100 * 944)
        q = torch.zeros((4, 928, H, hd), dtype=torch.bfloat16, device=DEV)
        z = torch.zeros((928, H * hd), dtype=torch.float32, device=DEV)
        ks = torch.zeros((944, H, hd), dtype=torch.bfloat16, device=DEV)
        ios.append(fmd.UnitIO(cache, ks, ks, q, q, q, z, [0.25] * 4, n_audio=8))
        caches.append(cache)
    assert fmd.unit_workspace_bytes(ios) > fmd.FMD_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fmd.FmdError) as e:
        fmd.denoise_unit_noalloc(ios, w)
    assert e.value.code == -5
    assert all((c.len_tokens, c.head_tokens) == (cap, 100 * 944) for c in caches)
