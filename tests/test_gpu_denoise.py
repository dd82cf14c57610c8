"""GPU parity of the whole step and unit (append + S Euler steps) against the
oracle, and the rectified-flow closed form on the GPU."""
import numpy as np
import pytest

import oracle
import workload
from tests.pins import bits, random_bits

import flow_matching_denoising_amd as fmd  # noqa: E402  (no fallback: fails if not built)
import torch  # noqa: E402
from tests.gpu_util import (DEV, assert_close, cache_logical, dev_bf16, host_f64,  # noqa: E402
                            make_cache, rel_l2, stack_steps)

pytestmark = pytest.mark.gpu


def _unit_io(ui, si, cache, z):
    s = si.shape
    q = stack_steps(si.q)
    ku = stack_steps(si.k_u)
    vu = stack_steps(si.v_u)
    sk = dev_bf16(si.slice_k) if si.slice_k is not None else None
    sv = dev_bf16(si.slice_v) if si.slice_v is not None else None
    return fmd.UnitIO(cache, sk, sv, q, ku, vu, z, list(s.h), n_audio=s.n_audio)


def _run_unit(wl, poison=True, reuse=False):
    ui = workload.make_inputs(wl, poison_invalid=poison, reuse_step_inputs=reuse)
    caches, ios, zs = [], [], []
    for si in ui.sessions:
        c = make_cache(fmd, si.shape, si.ring_k, si.ring_v)
        z = torch.from_numpy(si.eps.copy()).to(DEV)
        caches.append(c)
        zs.append(z)
        ios.append(_unit_io(ui, si, c, z))
    fmd.denoise_unit(ios, dev_bf16(ui.w_o))
    torch.cuda.synchronize()
    return ui, caches, zs


def _oracle_unit(ui, si):
    s = si.shape
    return oracle.denoise_unit(si.ring_k, si.ring_v, s.len_before, s.head_before, si.slice_k,
                               si.slice_v, si.q, si.k_u, si.v_u, si.eps, list(s.h), ui.w_o)


@pytest.mark.parametrize("name", ["tiny", "v01_unit"])
def test_unit_matches_oracle(name):
    wl = workload.get(name)
    ui, caches, zs = _run_unit(wl)
    for si, c, z in zip(ui.sessions, caches, zs):
        ref = _oracle_unit(ui, si)
        zg = host_f64(z)
        assert_close(zg, ref["z"], f"{name} z")
        assert_close(zg - si.eps, ref["z"] - si.eps, f"{name} dz", max_abs=2e-2, rel=1e-2)
        gk, gv = cache_logical(fmd, c)
        assert np.array_equal(gk, ref["ring_k"]) and np.array_equal(gv, ref["ring_v"])
        assert (c.len_tokens, c.head_tokens) == (ref["length"], ref["head"])


def test_small_batch_sessions_independent():
    # Three ragged sessions in one call.  The attention launch cuts its window
    # sequence (over all sessions) into equal ranges, so where a session's
    # lanes are cut depends on the batch: alone, a session matches its batched
    # result within the parity tolerance.  With one range the lanes are cut
    # only at their own segment boundaries, and a session alone is equal to
    # its batched result bit for bit.
    sess = [workload.custom_session(4, 128, 60, 4, 48, 480, 480, 96, (0.4, 0.3, 0.2, 0.1)),
            workload.custom_session(4, 128, 30, 2, 48, 192, 150, 150, (0.4, 0.3, 0.2, 0.1)),
            workload.custom_session(4, 128, 120, 8, 48, 960, 912, 912, (0.4, 0.3, 0.2, 0.1))]
    wl = workload.custom_workload("batch3", 21, sess)
    for groups in (None, 1):
        with fmd.forced_attn_groups(groups):
            ui, caches, zs = _run_unit(wl)
            for i, si in enumerate(ui.sessions):
                ref = _oracle_unit(ui, si)
                assert_close(host_f64(zs[i]) - si.eps, ref["z"] - si.eps,
                             f"batch session {i} dz (groups {groups})")
                ui1 = workload.make_inputs(wl, poison_invalid=True, sessions=[i])
                c1 = make_cache(fmd, ui1.sessions[0].shape, ui1.sessions[0].ring_k,
                                ui1.sessions[0].ring_v)
                z1 = torch.from_numpy(ui1.sessions[0].eps.copy()).to(DEV)
                fmd.denoise_unit([_unit_io(ui1, ui1.sessions[0], c1, z1)], dev_bf16(ui1.w_o))
                torch.cuda.synchronize()
                if groups == 1:
                    assert torch.equal(z1, zs[i]), f"session {i} differs when run alone"
                else:
                    assert_close(host_f64(z1) - si.eps, host_f64(zs[i]) - si.eps,
                                 f"session {i} alone vs batched dz")


@pytest.mark.parametrize("H", [2, 8])
@pytest.mark.parametrize("hs", [[1.0], [0.5, 0.5], [0.25] * 4, [0.4, 0.3, 0.2, 0.1],
                                [1.0 / 7] * 7])
def test_closed_form_rectified_flow(hs, H):
    # K == 0, every V row == w (bf16), W_o = I, z starts at eps: the velocity
    # is exactly w = eps - z0, and Euler must land on z0 for any schedule.
    # With 8 heads (d = 512, 8 k steps) the unit's steps batch their split
    # projections into one launch whose reduce applies the updates in order.
    rng = np.random.default_rng(0)
    hd, n_q, cap, length = 64, 40, 256, 200
    d = H * hd
    w = bits(rng.standard_normal(d).astype(np.float32))
    wf = oracle.bf16_bits_to_f64(w)
    zero = np.zeros((H, cap, hd), dtype=np.uint16)
    ring_v = np.broadcast_to(w.reshape(H, 1, hd), (H, cap, hd)).copy()
    q = random_bits(rng, (n_q, H, hd))
    ku = np.zeros((n_q, H, hd), dtype=np.uint16)
    vu = np.broadcast_to(w.reshape(1, H, hd), (n_q, H, hd)).copy()
    eps = rng.standard_normal((n_q, d)).astype(np.float32)
    z0 = eps.astype(np.float64) - wf[None, :]
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, length, 17, tuple(hs))
    cache = make_cache(fmd, shape, zero, ring_v)
    z = torch.from_numpy(eps.copy()).to(DEV)
    io = fmd.UnitIO(cache, None, None, dev_bf16(q), dev_bf16(ku), dev_bf16(vu), z, hs)
    fmd.denoise_unit([io], dev_bf16(bits(np.eye(d, dtype=np.float32))))
    torch.cuda.synchronize()
    err = np.max(np.abs(host_f64(z) - z0))
    print(f"closed form H={H} S={len(hs)}: max |z - z0| = {err:.3e}", flush=True)
    assert err <= 1e-5


def test_reused_inputs_equal_one_big_step():
    # step stride 0: four steps of [0.4, 0.3, 0.2, 0.1] == one step of 1.0
    s4 = workload.custom_session(4, 128, 90, 6, 0, 512, 400, 300, (0.4, 0.3, 0.2, 0.1))
    s1 = workload.custom_session(4, 128, 90, 6, 0, 512, 400, 300, (1.0,))
    ui4, _, z4 = _run_unit(workload.custom_workload("lin", 5, [s4]), reuse=True)
    ui1, _, z1 = _run_unit(workload.custom_workload("lin", 5, [s1]), reuse=True)
    a, b = host_f64(z4[0]), host_f64(z1[0])
    assert np.max(np.abs(a - b)) <= 1e-5


def test_projection_isolated_from_attention_rounding():
    # Take the GPU's own O, run one step with z = 0 and h = 1: z must equal
    # -(O W^T) computed in float64 from that same O.
    rng = np.random.default_rng(6)
    H, hd, n_q, cap = 8, 128, 200, 512
    d = H * hd
    rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    w = random_bits(rng, (d, d), scale=d ** -0.5)
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, 333, 100, (1.0,))
    cache = make_cache(fmd, shape, rk, rv)
    unit = fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu),
                        z=torch.zeros((n_q, d), dtype=torch.float32, device=DEV), h=1.0)
    o = fmd.attention([unit])
    fmd.denoise_step([unit], dev_bf16(w))
    torch.cuda.synchronize()
    v_ref = host_f64(o).reshape(n_q, d) @ oracle.bf16_bits_to_f64(w).T
    got = -host_f64(unit.z)
    assert rel_l2(got, v_ref) <= 1e-5, rel_l2(got, v_ref)


@pytest.mark.parametrize("H,hd,n_q", [(41, 64, 1000), (40, 128, 497)])
def test_projection_euler_epilogue_full_tiles(H, hd, n_q):
    # Unsplit projections (at least 128 output tiles) whose z values are loaded
    # during the k loop: 41 x 64 features leave half a feature tile at the end
    # and 1000 or 497 rows a partial row tile.  With z and h given, the step
    # must equal z - h * (O W^T) computed in float64 from the GPU's own O.
    rng = np.random.default_rng(H * 1000 + n_q)
    d, cap = H * hd, 256
    rk, rv = random_bits(rng, (H, cap, hd)), random_bits(rng, (H, cap, hd))
    q, ku, vu = (random_bits(rng, (n_q, H, hd)) for _ in range(3))
    w = random_bits(rng, (d, d), scale=d ** -0.5)
    z0 = rng.standard_normal((n_q, d)).astype(np.float32)
    h = 0.37
    shape = workload.custom_session(H, hd, n_q, 0, 0, cap, 200, 31, (h,))
    cache = make_cache(fmd, shape, rk, rv)
    unit = fmd.UnitStep(cache, dev_bf16(q), dev_bf16(ku), dev_bf16(vu),
                        z=torch.from_numpy(z0.copy()).to(DEV), h=h)
    o = fmd.attention([unit])
    fmd.denoise_step([unit], dev_bf16(w))
    torch.cuda.synchronize()
    v_ref = host_f64(o).reshape(n_q, d) @ oracle.bf16_bits_to_f64(w).T
    z_ref = z0.astype(np.float64) - h * v_ref
    got = host_f64(unit.z)
    assert rel_l2(got - z0, z_ref - z0) <= 1e-5, rel_l2(got - z0, z_ref - z0)
    assert np.max(np.abs(got - z_ref)) <= 1e-5


def test_unit_deterministic():
    wl = workload.get("v01_unit")
    _, _, za = _run_unit(wl)
    _, _, zb = _run_unit(wl)
    assert torch.equal(za[0], zb[0])


def test_maximum_session_count_four_launch_chunks():
    # FMD_MAX_SESSIONS sessions in one call: four launches of 16 sessions
    # each, ragged query counts, ring states (empty, partial, wrapped, full)
    # and slices, every session checked against the oracle.
    rng = np.random.default_rng(64)
    shapes = []
    for i in range(64):
        n_v, n_a = int(rng.integers(1, 48)), int(rng.integers(0, 5))
        cap = int(rng.integers(2, 9)) * 32
        T = int(rng.integers(0, 2)) * int(rng.integers(1, 33))
        ln = int(rng.integers(0, cap + 1)) if i % 5 else 0
        head = int(rng.integers(0, cap))
        shapes.append(workload.custom_session(2, 64, n_v, n_a, T, cap, ln, head, (0.6, 0.4)))
    wl = workload.custom_workload("max_sessions", 64, shapes)
    ui, caches, zs = _run_unit(wl)
    for i, (si, c, z) in enumerate(zip(ui.sessions, caches, zs)):
        ref = _oracle_unit(ui, si)
        assert_close(host_f64(z) - si.eps, ref["z"] - si.eps, f"session {i} dz")
        gk, gv = cache_logical(fmd, c)
        assert np.array_equal(gk, ref["ring_k"]) and np.array_equal(gv, ref["ring_v"])
        assert (c.len_tokens, c.head_tokens) == (ref["length"], ref["head"])


def test_profiling_records_only_the_selected_classes():
    # One unit = one append, one staging of every step's unit values, one
    # attention launch for all 4 steps (one session: the steps are the
    # launch's sessions), the merge of cut lanes (if any), then one
    # projection record for all 4 steps (the 192x336-class projection splits
    # its k range, so the steps' partial products are one launch and one
    # reduce applies the Euler updates in step order).  Recording is on for
    # the attention class only, then for every class.
    wl = workload.get("v01_unit")
    n_steps = len(wl.sessions[0].h)
    try:
        fmd.profile_enable(True, classes=("attn",))
        _, _, z_sel = _run_unit(wl)
        rec = {k: fmd.profile_read(k) for k in fmd.KERNEL_CLASSES}
        assert rec["attn"][1] == 1 and rec["attn"][0] > 0
        assert all(n == 0 for k, (_, n) in rec.items() if k != "attn")
        fmd.profile_enable(True)
        _, _, z_all = _run_unit(wl)
        rec = {k: fmd.profile_read(k) for k in fmd.KERNEL_CLASSES}
        assert rec["append"][1] == 1
        assert rec["attn"][1] == 1 and rec["combine"][1] <= 1
        assert rec["proj"][1] == 1
        assert rec["vt"][1] == 1
        assert rec["qkv"][1] == rec["mix"][1] == 0
    finally:
        fmd.profile_enable(False)
    # Timing events do not change the result.
    assert torch.equal(z_sel[0], z_all[0])
