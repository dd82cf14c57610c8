"""The Python binding checks every tensor extent the C ABI relies on (the
library receives bare device pointers, so a wrong shape would become an
out-of-bounds device access).  CPU only: each case raises ValueError before
any pointer is taken."""
import pytest
import torch

import flow_matching_denoising_amd as fmd

BF, F32 = torch.bfloat16, torch.float32


class _Shape:
    """Stands in for a KVCache where only (n_heads, head_dim) are read."""
    n_heads, head_dim = 2, 64


def _t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


C = _Shape()
H, HD, D, NQ = 2, 64, 128, 20


def test_kv_cache_shapes():
    with pytest.raises(ValueError, match="k must have shape"):
        fmd.KVCache(H, HD, 64, k=_t(H, 48, HD), v=_t(H, 4, HD, 16))
    with pytest.raises(ValueError, match="v must have shape"):
        fmd.KVCache(H, HD, 64, k=_t(H, 64, HD), v=_t(H, 64, HD))
    with pytest.raises(ValueError, match="multiple of 16"):
        fmd.KVCache(H, HD, 40, k=_t(H, 40, HD), v=_t(H, 2, HD, 16))


@pytest.mark.parametrize("bad", ["q4d", "ku", "vu", "z", "split"])
def test_unit_step_shapes(bad):
    q, ku, vu, z = _t(NQ, H, HD), _t(NQ, H, HD), _t(NQ, H, HD), _t(NQ, D, dtype=F32)
    if bad == "q4d":
        q = _t(2, NQ, H, HD)
    elif bad == "ku":
        ku = _t(NQ + 1, H, HD)
    elif bad == "vu":
        vu = _t(NQ, H, HD * 2)
    elif bad == "z":
        z = _t(NQ, D + 8, dtype=F32)
    kw = dict(n_video=NQ - 3, n_audio=2) if bad == "split" else {}
    with pytest.raises(ValueError):
        fmd.UnitStep(C, q, ku, vu, z, **kw)


@pytest.mark.parametrize("bad", ["few_steps", "ku_3d", "z_width", "z_rows", "slice",
                                 "one_slice", "audio"])
def test_unit_io_shapes(bad):
    S = 4
    q, ku, vu = _t(S, NQ, H, HD), _t(S, NQ, H, HD), _t(S, NQ, H, HD)
    z = _t(NQ, D, dtype=F32)
    ks, vs = _t(8, H, HD), _t(8, H, HD)
    h, n_audio = [0.25] * S, 2
    if bad == "few_steps":
        h = [0.2] * (S + 1)
    elif bad == "ku_3d":
        ku = _t(NQ, H, HD)
    elif bad == "z_width":
        z = _t(NQ, D // 2, dtype=F32)
    elif bad == "z_rows":
        z = _t(NQ - 1, D, dtype=F32)
    elif bad == "slice":
        vs = _t(9, H, HD)
    elif bad == "one_slice":
        vs = None
    elif bad == "audio":
        n_audio = NQ + 1
    with pytest.raises(ValueError):
        fmd.UnitIO(C, ks, vs, q, ku, vu, z, h, n_audio=n_audio)


def test_unit_qkv_cfg_layers_shapes():
    z = _t(NQ, D, dtype=F32)
    with pytest.raises(ValueError):
        fmd.UnitQkvIO(C, None, None, _t(NQ, D + 1, dtype=F32), [0.5])
    with pytest.raises(ValueError):
        fmd.UnitQkvIO(C, _t(8, H, HD), _t(8, H + 1, HD), z, [0.5])
    with pytest.raises(ValueError):
        fmd.UnitCfgIO(C, C, _t(NQ, 3 * D, dtype=F32), [0.5], 5.0)
    with pytest.raises(ValueError):
        fmd.UnitCfgIO(C, C, z, [0.5], 5.0, cond_slice=(_t(8, H, HD), _t(7, H, HD)))
    with pytest.raises(ValueError):
        fmd.UnitLayersIO([C, C], z, [0.5], [_t(8, H, HD)], [_t(8, H, HD)])
    with pytest.raises(ValueError):
        fmd.UnitLayersIO([C, C], z, [0.5], [_t(8, H, HD), _t(9, H, HD)],
                         [_t(8, H, HD), _t(9, H, HD)])
    with pytest.raises(ValueError):
        fmd.UnitLayersIO([C], _t(NQ, D, dtype=BF).float()[:, :D - 8], [0.5])


def test_weight_shapes_checked_before_any_pointer():
    z = _t(NQ, D, dtype=F32)
    unit = fmd.UnitStep(C, _t(NQ, H, HD), _t(NQ, H, HD), _t(NQ, H, HD), z)
    with pytest.raises(ValueError, match="w_o"):
        fmd.denoise_step([unit], _t(D, D + 16))
    io = fmd.UnitIO(C, None, None, _t(NQ, H, HD), _t(NQ, H, HD), _t(NQ, H, HD), z, [0.5])
    with pytest.raises(ValueError, match="w_o"):
        fmd.denoise_unit([io], _t(D + 16, D))
    qio = fmd.UnitQkvIO(C, None, None, z, [0.5])
    with pytest.raises(ValueError, match="w_qkv"):
        fmd.denoise_unit_qkv([qio], _t(D, D), _t(D, D))
    cio = fmd.UnitCfgIO(C, C, z, [0.5], 2.0)
    with pytest.raises(ValueError, match="w_qkv"):
        fmd.denoise_unit_cfg([cio], _t(2 * D, D), _t(D, D))
    lio = fmd.UnitLayersIO([C, C], z, [0.5])
    with pytest.raises(ValueError, match="w_o"):
        fmd.denoise_unit_layers([lio], [_t(3 * D, D)] * 2, [_t(D, D), _t(D, 2 * D)])
    with pytest.raises(ValueError, match="per layer"):
        fmd.denoise_unit_layers([lio], [_t(3 * D, D)], [_t(D, D)])


def test_forced_split_entry_rejects_negative():
    assert fmd._test_force_attn_groups(-1) == -1
    assert fmd._test_force_attn_groups(0) == 0


def test_prepared_append_shapes():
    with pytest.raises(ValueError, match="one K and one V slice per cache"):
        fmd.PreparedAppend([C], [], [])
    with pytest.raises(ValueError):
        fmd.PreparedAppend([C], [_t(5, H + 1, HD)], [_t(5, H + 1, HD)])
    with pytest.raises(ValueError):
        fmd.PreparedAppend([C], [_t(5, H, HD)], [_t(6, H, HD)])

