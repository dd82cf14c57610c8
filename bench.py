"""Benchmark: denoised units per second on one MI355X.

One step = one denoised unit of the 640x368-class workload (40 heads x 128,
920 video + 8 audio queries, a 64-unit ring of 944-token slices = 60,416 keys):
the slice append, then 4 Euler solver steps, each attention over
[60,416 cached keys || 928 unit keys] -> projection (5120 x 5120) -> Euler
update.  The steps' Q, K_u, V_u are inputs, so the unit runs the 4 steps'
attention as one launch, then the projections and updates in step order.  Inputs are seeded synthetic tensors (no weights or data were
released for the method), resident in HBM before the timed region.

Prints ONE JSON line (rank 0, N=1).  Besides throughput it reports:
* roofline: the attention kernel (the dominant kernel), algorithmic flops per
  launch / its mean launch duration measured with HIP events recorded on the
  launch stream during the timed region, against the bf16 dense MFMA peak;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same workload
  (one full solver step: attention of every head, the projection and the Euler
  update), scaled to the unit's solver steps;
* qkv_unit: the same unit with the z-dependent solver (Q, K_u, V_u projected
  from the latent at every step);
* cfg_unit: the guided teacher's sampler (conditional + unconditional rings,
  16 steps, guidance 5) on the 640x368-class unit;
* ulysses_rank_p8: one rank's attention under 8-way Ulysses context parallel
  (5 heads, all 928 tokens, the head shard of the ring);
* layers_unit: the layer-stack solver with 4 layers (one ring and one pair of
  weights per layer) on the 640x368-class unit;
* append_batch8: the batched ring append at the 8-session shape.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 (published)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E (published)
UNIT_BUDGET_S = 0.160              # one streaming unit
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_v02_unit_traffic.json")
ATTN_SRC = os.path.join(ROOT, "flow_matching_denoising_amd", "csrc", "attention.hip")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    # Under sustained MFMA load the GPU's clock settles only after a few hundred
    # ms (the first launches run up to 30 % slower); 60 units of the
    # 640x368-class workload are about 0.3 s.
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="v02_unit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the z-dependent, guided and batched-append probes")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (three "
                         "launches), the known-size reference for HBM byte counters")
    return ap.parse_args()


def copy_probe(nbytes):
    """A plain copy kernel of known size: each launch reads and writes nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    t = min(times)
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3, "best_s": t,
                      "read_plus_write_GBps": round(2 * nbytes / t / 1e9, 1)}), flush=True)


def _log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def _attn_traffic(workload_name, steps_per_launch):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    valid only for the workload and the solver steps per launch they were
    taken on and while attention.hip is unchanged since then."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("workload", "").split(" ")[0] != workload_name:
            return None
        if t.get("steps_per_launch") != steps_per_launch:
            return None
        with open(ATTN_SRC, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
        if t.get("attention_hip_sha256") != h:
            return None
        return float(t["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def qkv_unit_probe(wl, ui, caches, states, w_o, units=20, warmup=5):
    """The z-dependent solver on the same workload: every step first projects
    the unit's Q, K_u, V_u from the current latent (bf16 [3d][d] weights, one
    GEMM of n_q x 3d x d), then runs the step.  Same rings, same append."""
    import numpy as np
    import torch

    import flow_matching_denoising_amd as fmd
    import workload

    dev = torch.device("cuda:0")
    w_qkv = torch.from_numpy(workload.qkv_weight(wl.seed, wl.d, wl.head_dim).view(np.int16)).view(
        torch.bfloat16).to(dev)
    ios = []
    for si, c in zip(ui.sessions, caches):
        s = si.shape
        z = torch.from_numpy(si.eps.copy()).to(dev)
        sk = torch.from_numpy(si.slice_k.view(np.int16)).view(torch.bfloat16).to(dev)
        sv = torch.from_numpy(si.slice_v.view(np.int16)).view(torch.bfloat16).to(dev)
        ios.append(fmd.UnitQkvIO(c, sk, sv, z, list(s.h), n_audio=s.n_audio))
    ws = fmd.alloc_workspace(fmd.unit_qkv_workspace_bytes(ios), dev)

    def one():
        for c, (ln, hd_) in zip(caches, states):
            c.set_state(ln, hd_)
        fmd.denoise_unit_qkv(ios, w_qkv, w_o, ws)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    fmd.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(units):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms, n = fmd.profile_read("qkv")
    fmd.profile_enable(False)
    s0 = wl.sessions[0]
    qkv_flops = 2.0 * sum(s.n_q for s in wl.sessions) * 3 * s0.d * s0.d
    return {"workload": wl.name, "units_per_s": round(len(ui.sessions) * units / wall, 3),
            "ms_per_unit": round(wall / units * 1e3, 4),
            "qkv_gemm_us": round(ms / n * 1e3, 2),
            "qkv_gemm_TFLOPs": round(qkv_flops / (ms / n / 1e3) / 1e12, 1)}


def cfg_unit_probe(units=4, warmup=2):
    """The guided (teacher) sampler on its 640x368-class workload: conditional
    and unconditional 60,416-key rings, both appended, 16 steps; per step one
    Q/K/V projection, attention over both branches (one launch), the guided
    mix and one projection with the Euler update."""
    import numpy as np
    import torch

    import flow_matching_denoising_amd as fmd
    import workload

    wl = workload.get("v02_cfg_unit")
    dev = torch.device("cuda:0")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    ui = workload.make_inputs(wl, reuse_step_inputs=True)
    w_qkv = bf(workload.qkv_weight(wl.seed, wl.d, wl.head_dim))
    w_o = bf(ui.w_o)
    ios, caches = [], []
    for i, si in enumerate(ui.sessions):
        s = si.shape
        un = workload.uncond_inputs(wl, i)
        st = dict(len_tokens=s.len_before, head_tokens=s.head_before)
        cc = fmd.KVCache(s.n_heads, s.head_dim, s.cap_tokens, device=dev, k=bf(si.ring_k),
                         v=fmd.KVCache.logical_to_device_v(bf(si.ring_v)), **st)
        uc = fmd.KVCache(s.n_heads, s.head_dim, s.cap_tokens, device=dev, k=bf(un.ring_k),
                         v=fmd.KVCache.logical_to_device_v(bf(un.ring_v)), **st)
        z = torch.from_numpy(si.eps.copy()).to(dev)
        ios.append(fmd.UnitCfgIO(cc, uc, z, list(s.h), workload.CFG_GUIDANCE,
                                 cond_slice=(bf(si.slice_k), bf(si.slice_v)),
                                 uncond_slice=(bf(un.slice_k), bf(un.slice_v)),
                                 n_audio=s.n_audio))
        caches.append((cc, uc, (s.len_before, s.head_before), z, si.eps))
    ws = fmd.alloc_workspace(fmd.unit_cfg_workspace_bytes(ios), dev)

    def one():
        for cc, uc, (ln, hd_), z, eps in caches:
            cc.set_state(ln, hd_)
            uc.set_state(ln, hd_)
        fmd.denoise_unit_cfg(ios, w_qkv, w_o, ws)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    fmd.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(units):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = {k: fmd.profile_read(k) for k in ("attn", "mix", "proj", "qkv", "combine")}
    fmd.profile_enable(False)
    attn_ms, attn_n = kt["attn"]
    attn_flops = 2 * wl.attention_flops_per_step()        # both branches in one launch
    s0 = wl.sessions[0]
    return {"workload": wl.name, "solver_steps": s0.n_steps, "guidance": workload.CFG_GUIDANCE,
            "units_per_s": round(len(ui.sessions) * units / wall, 3),
            "ms_per_unit": round(wall / units * 1e3, 3),
            "attn_us": round(attn_ms / attn_n * 1e3, 2),
            "attn_TFLOPs": round(attn_flops / (attn_ms / attn_n / 1e3) / 1e12, 1),
            "per_kernel_us": {k: (round(v[0] / v[1] * 1e3, 2) if v[1] else None)
                              for k, v in kt.items()}}


def layers_unit_probe(n_layers=4, units=4, warmup=2):
    """The layer-stack solver on the 640x368-class unit: n_layers attention
    layers, each with its own 60,416-key ring (filled by this unit's append of
    a 944-token slice per layer) and its own W_qkv / W_o, 4 solver steps.
    Contents do not change the work, so tensors are drawn on the device
    (weights scaled by d^-1/2)."""
    import torch

    import flow_matching_denoising_amd as fmd

    H, hd, cap, T, n_q, n_audio = 40, 128, 64 * 944, 944, 928, 8
    d = H * hd
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    rnd = lambda *shape, scale=1.0: (torch.randn(shape, generator=g, device=dev) * scale).to(  # noqa: E731
        torch.bfloat16)
    caches, ks, vs, wq, wo = [], [], [], [], []
    for _ in range(n_layers):
        caches.append(fmd.KVCache(H, hd, cap, device=dev, k=rnd(H, cap, hd),
                                  v=fmd.KVCache.logical_to_device_v(rnd(H, cap, hd)),
                                  len_tokens=cap - T, head_tokens=cap - T))
        ks.append(rnd(T, H, hd))
        vs.append(rnd(T, H, hd))
        wq.append(rnd(3 * d, d, scale=d ** -0.5))
        wo.append(rnd(d, d, scale=d ** -0.5))
    z = torch.randn((n_q, d), generator=g, device=dev)
    hs = [0.25] * 4
    io = fmd.UnitLayersIO(caches, z, hs, ks, vs, n_audio=n_audio)
    ws = fmd.alloc_workspace(fmd.unit_layers_workspace_bytes([io]), dev)

    def one():
        for c in caches:
            c.set_state(cap - T, cap - T)
        fmd.denoise_unit_layers([io], wq, wo, ws)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    fmd.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(units):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = {k: fmd.profile_read(k) for k in ("attn", "proj", "qkv", "append")}
    fmd.profile_enable(False)
    ring_bytes = 2 * H * cap * hd * 2
    return {"layers": n_layers, "solver_steps": len(hs),
            "units_per_s": round(units / wall, 3), "ms_per_unit": round(wall / units * 1e3, 3),
            "layer_steps_per_s": round(units * n_layers * len(hs) / wall, 1),
            "ring_GB_per_layer": round(ring_bytes / 1e9, 3),
            "per_kernel_us": {k: (round(v[0] / v[1] * 1e3, 2) if v[1] else None)
                              for k, v in kt.items()}}


def ulysses_rank_probe(P=8, launches=20, warmup=10):
    """One Ulysses rank's attention at the 640x368-class shape: after the
    sequence -> head exchange a rank of P holds all 928 tokens for H/P heads
    and the head shard of the 60,416-key ring.  Contents do not change the
    work, so the tensors are drawn on the device."""
    import torch

    import flow_matching_denoising_amd as fmd

    H, hd, cap, n_q, n_audio = 40 // P, 128, 64 * 944, 928, 8
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(9)
    rnd = lambda *shape: torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)  # noqa: E731
    cache = fmd.KVCache(H, hd, cap, device=dev, k=rnd(H, cap, hd),
                        v=fmd.KVCache.logical_to_device_v(rnd(H, cap, hd)), len_tokens=cap,
                        head_tokens=63 * 944)
    unit = fmd.UnitStep(cache, rnd(n_q, H, hd), rnd(n_q, H, hd), rnd(n_q, H, hd), n_audio=n_audio)
    o = torch.empty((n_q, H, hd), dtype=torch.bfloat16, device=dev)
    ws = fmd.alloc_workspace(fmd.workspace_bytes([unit]), dev)
    for _ in range(warmup):
        fmd.attention([unit], o, ws)
    torch.cuda.synchronize()
    fmd.profile_enable(True)
    for _ in range(launches):
        fmd.attention([unit], o, ws)
    torch.cuda.synchronize()
    ms, n = fmd.profile_read("attn")
    c_ms, c_n = fmd.profile_read("combine")
    fmd.profile_enable(False)
    flops = 4.0 * n_q * (cap + n_q) * H * hd
    return {"ranks": P, "heads_per_rank": H, "queries": n_q, "keys_per_query": cap + n_q,
            "attn_us": round(ms / n * 1e3, 2),
            "attn_TFLOPs": round(flops / (ms / n / 1e3) / 1e12, 1),
            "combine_us": round(c_ms / c_n * 1e3, 2) if c_n else None}


def append_batch_probe(launches=20):
    """The batched ring append at the 8-session shape (rings of 8..128 units of
    944 tokens, 40 heads x 128, per-session append offsets): one launch appends
    all 8 slices (309 MB read + written).  Timed with HIP events recorded on the
    launch stream.  Launches alternate between two sets of slices and two append
    offsets per ring (half a ring apart), so consecutive launches touch disjoint
    bytes: 618 MB per cycle, more than the 256 MB Infinity Cache holds, so the
    rate is not one of that cache.  The rings' contents do not affect the
    append, so they are left uninitialised."""
    import torch

    import flow_matching_denoising_amd as fmd
    import workload

    wl = workload.get("v02_batch8")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    caches, sets = [], [([], [], []), ([], [], [])]
    for s in wl.sessions:
        caches.append(fmd.KVCache(s.n_heads, s.head_dim, s.cap_tokens, device=dev,
                                  len_tokens=s.len_before, head_tokens=s.head_before))
        shape = (s.slice_tokens, s.n_heads, s.head_dim)
        assert 2 * s.slice_tokens <= s.cap_tokens, "the two offsets' blocks must not overlap"
        for k, (ks, vs, states) in enumerate(sets):
            ks.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
            vs.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
            head = (s.head_before + k * (s.cap_tokens // 2)) % s.cap_tokens
            states.append((s.len_before, head))

    prepared = [fmd.PreparedAppend(caches, ks, vs) for ks, vs, _ in sets]

    def once(k):
        for c, (ln, hd_) in zip(caches, sets[k][2]):
            c.set_state(ln, hd_)
        prepared[k].launch()

    for i in range(4):
        once(i & 1)
    torch.cuda.synchronize()
    # The argument arrays are built once, so the host enqueues far faster than
    # a launch runs and the launches run back to back: one pair of events
    # around all of them times the kernels alone.
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(launches):
        once(i & 1)
    b.record()
    torch.cuda.synchronize()
    n = launches
    avg_s = a.elapsed_time(b) / n / 1e3
    nbytes = wl.append_bytes()
    del caches, sets, prepared
    torch.cuda.empty_cache()
    return {"workload": "v02_batch8", "bytes_per_launch": nbytes, "launches": n,
            "bytes_touched_per_cycle": 2 * nbytes,
            "avg_launch_us": round(avg_s * 1e6, 2), "GBps": round(nbytes / avg_s / 1e9, 1),
            "frac_hbm": round(nbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4)}


CPU_THREADS_MAX = 16   # the host cores one GPU's share of the box provides


def _cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(CPU_THREADS_MAX, n))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# Bounded samples of each configuration for the CPU baseline: the sessions,
# heads and solver steps the oracle computes, scaled to whole units.
CPU_SAMPLES = (
    ("v01_unit", None, 12, None),    # the whole unit: every head, every step
    ("v02_unit", None, 4, 1),        # 4 of 40 heads, 1 of 4 steps
    ("v02_long", None, 2, 1),        # 2 of 40 heads, 1 of 4 steps
    ("v02_batch8", None, 1, 1),      # every session, 1 of 40 heads, 1 of 4 steps
)


def cpu_baseline(args, reps=3):
    """The oracle in its float32 mode (numpy + BLAS, the textbook two-pass
    softmax, keys gathered per head) timed on this host's cores for every
    configuration, on a bounded sample of each unit (some heads and steps;
    the projection and Euler update at full size), scaled to whole units.
    Median of `reps` repetitions; inputs drawn before the timed region."""
    import dataclasses

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import workload

    threads = _cpu_threads()
    out = {}
    with threadpool_limits(limits=threads):
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        for name, sess, heads, steps in CPU_SAMPLES:
            wl = workload.get(name)
            s0 = wl.sessions[0]
            H, S = s0.n_heads, s0.n_steps
            k = min(heads, H)
            n_st = S if steps is None else min(steps, S)
            idx = list(range(len(wl.sessions))) if sess is None else list(sess)
            # The first k heads of each session: the workload draws every head
            # from its own stream, so these are exactly the full unit's values.
            sub = workload.custom_workload(
                name, wl.seed, [dataclasses.replace(wl.sessions[i], n_heads=k) for i in idx])
            ui = workload.make_inputs(sub)
            w_o = workload.projection_weight(wl.seed, wl.d, wl.head_dim)
            rng = np.random.default_rng(0)
            o_full = rng.standard_normal((s0.n_q, wl.d)).astype(np.float32)
            z_full = rng.standard_normal((s0.n_q, wl.d)).astype(np.float32)
            rep_s = []
            for _ in range(reps):
                t_attn = t_app = 0.0
                for si in ui.sessions:
                    sh = si.shape
                    t0 = time.perf_counter()
                    rk, rv, ln, hd_ = oracle.kv_append(si.ring_k, si.ring_v, sh.len_before,
                                                       sh.head_before, si.slice_k, si.slice_v)[:4]
                    t_app += time.perf_counter() - t0
                    t0 = time.perf_counter()
                    for st in range(n_st):
                        oracle.attention(si.q[st], rk, rv, ln, hd_, si.k_u[st], si.v_u[st],
                                         dtype=np.float32)
                    t_attn += time.perf_counter() - t0
                # The projection and Euler update of one session and step at
                # full size (their cost does not depend on the values).
                t0 = time.perf_counter()
                v = oracle.velocity(o_full, w_o, dtype=np.float32)
                oracle.euler_step(z_full, s0.h[0], v, dtype=np.float32)
                t_proj = time.perf_counter() - t0
                scale_h = H / k
                n_all = len(wl.sessions)
                t_unit = (t_app * scale_h * n_all / len(idx)
                          + t_attn * scale_h * (S / n_st) * n_all / len(idx)
                          + t_proj * S * n_all)
                rep_s.append(t_unit)
            med = float(np.median(rep_s))
            out[name] = {
                "units_per_s": round(len(wl.sessions) / med, 6),
                "s_per_unit_reps": [round(x, 3) for x in rep_s],
                "sample": (f"{len(idx)} of {len(wl.sessions)} session(s), {k} of {H} heads, "
                           f"{n_st} of {S} steps of attention (+ the append of those heads); "
                           f"projection and Euler update at full size"),
            }
            _log(args, f"cpu oracle {name}: {med:.2f} s per unit (reps {rep_s})")
            del ui
    c2 = out["v02_unit"]
    return {"value": c2["units_per_s"], "unit": "units/s", "cores": threads, "kind": "oracle",
            "dtype": "f32",
            "sample": "float32 oracle on v02_unit: " + c2["sample"] + f"; median of {reps} reps",
            "cpu_model": _cpu_model(),
            "blas": [{"vendor": b.get("internal_api"), "version": b.get("version"),
                      "threads": b.get("num_threads")} for b in blas],
            "per_config": out}


def main():
    args = _args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the denoise step here is a single-GPU "
              "kernel path (multi-GPU sharding is design-only); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import flow_matching_denoising_amd as fmd
    import workload

    wl = workload.get(args.workload)
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    ui = workload.make_inputs(wl)
    _log(args, f"inputs drawn in {time.perf_counter() - t0:.1f}s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    caches, ios, states = [], [], []
    for si in ui.sessions:
        s = si.shape
        c = fmd.KVCache(s.n_heads, s.head_dim, s.cap_tokens, device=dev, k=bf(si.ring_k),
                        v=fmd.KVCache.logical_to_device_v(bf(si.ring_v)),
                        len_tokens=s.len_before, head_tokens=s.head_before)
        z = torch.from_numpy(si.eps.copy()).to(dev)
        q = bf(np.stack(si.q))
        ku = bf(np.stack(si.k_u))
        vu = bf(np.stack(si.v_u))
        io = fmd.UnitIO(c, bf(si.slice_k), bf(si.slice_v), q, ku, vu, z, list(s.h),
                        n_audio=s.n_audio)
        caches.append(c)
        ios.append(io)
        states.append((s.len_before, s.head_before))
    w_o = bf(ui.w_o)
    ws = fmd.alloc_workspace(fmd.unit_workspace_bytes(ios), dev)
    torch.cuda.synchronize()

    def one_unit():
        # Every timed unit appends at the same offset into the same ring state.
        for c, (ln, hd_) in zip(caches, states):
            c.set_state(ln, hd_)
        fmd.denoise_unit(ios, w_o, ws)

    for _ in range(args.warmup):
        one_unit()
    torch.cuda.synchronize()

    # Inside the timed region only the attention launches (the roofline's
    # kernel) carry events: every recorded launch adds queue time around it.
    fmd.profile_enable(True, classes=("attn",))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_unit()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_rec = fmd.profile_read("attn")
    fmd.profile_enable(False)
    # Per-unit median and p90: an untimed pass with one pair of events per
    # unit on the launch stream.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        one_unit()
        b.record()
    torch.cuda.synchronize()
    unit_ms = sorted(a.elapsed_time(b) for a, b in evs)
    # The other kernels' durations: a second, untimed pass over the same
    # units with every class recorded.
    fmd.profile_enable(True)
    for _ in range(min(args.steps, 10)):
        one_unit()
    torch.cuda.synchronize()
    kt = {k: fmd.profile_read(k) for k in fmd.KERNEL_CLASSES}
    kt["attn"] = attn_rec
    fmd.profile_enable(False)

    n_sess = len(ui.sessions)
    ms_per_step = wall / args.steps * 1e3
    units_per_s = n_sess * args.steps / wall
    attn_ms, attn_n = kt["attn"]
    attn_avg_s = attn_ms / attn_n / 1e3
    # One launch covers the attention of every session for one or several
    # solver steps (the unit driver batches steps whose inputs are given).
    s0 = wl.sessions[0]
    attn_launches_per_unit = attn_n / args.steps
    steps_per_launch = s0.n_steps / attn_launches_per_unit
    attn_flops_launch = wl.attention_flops_per_step() * steps_per_launch
    attn_tflops = attn_flops_launch / attn_avg_s / 1e12
    traffic = _attn_traffic(wl.name, round(steps_per_launch, 3))
    per_kernel_us = {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in kt.items()}
    app_ms, app_n = kt["append"]
    append_gbs = wl.append_bytes() / (app_ms / app_n / 1e3) / 1e9 if app_n else None
    proj_ms, proj_n = kt["proj"]
    # A projection record covers one solver step, or every step of a batch
    # when small units chain their split projections into one launch.
    proj_steps = s0.n_steps * min(args.steps, 10) / proj_n if proj_n else 0
    proj_tflops = (wl.projection_flops_per_step() * proj_steps / (proj_ms / proj_n / 1e3) / 1e12
                   if proj_n else None)

    out = {
        "metric": "denoised units/sec (1 GPU) at 640×368-class shape; attn TFLOP/s vs MFMA peak",
        "value": round(units_per_s, 3),
        "unit": "units/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "sessions": n_sess,
            "heads": s0.n_heads, "head_dim": s0.head_dim,
            "queries_per_unit": s0.n_q, "cached_keys": s0.len_after,
            "keys_per_query": s0.keys_per_query, "slice_tokens": s0.slice_tokens,
            "solver_steps": s0.n_steps,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "attn_kernel<128>",
            "flops_per_launch": attn_flops_launch,
            "avg_launch_us": round(attn_avg_s * 1e6, 2),
            "solver_steps_per_launch": round(steps_per_launch, 3),
        },
        "per_kernel_us": {k: (round(v, 2) if v is not None else None)
                          for k, v in per_kernel_us.items()},
        # launches of each class per unit (the staging launch covers every step)
        "launches_per_unit": dict({k: (round(v[1] / min(args.steps, 10), 2) if v[1] else 0)
                                   for k, v in kt.items() if k != "attn"},
                                  attn=round(attn_launches_per_unit, 2)),
        "append_GBps": round(append_gbs, 1) if append_gbs else None,
        "append_frac_hbm": round(append_gbs / HBM_PEAK_GBS, 4) if append_gbs else None,
        "proj_TFLOPs": round(proj_tflops, 1) if proj_tflops else None,
        "proj_steps_per_record": round(proj_steps, 3),
        "unit_layers_per_160ms": round(UNIT_BUDGET_S / (ms_per_step / 1e3 / n_sess), 2),
        "step_ms_median": round(unit_ms[len(unit_ms) // 2], 4),
        "step_ms_p90": round(unit_ms[min(len(unit_ms) - 1, (9 * len(unit_ms)) // 10)], 4),
    }
    if not args.no_probes:
        out["qkv_unit"] = qkv_unit_probe(wl, ui, caches, states, w_o)
        del caches, ios
        torch.cuda.empty_cache()
        out["cfg_unit"] = cfg_unit_probe()
        torch.cuda.empty_cache()
        out["ulysses_rank_p8"] = ulysses_rank_probe(8)
        torch.cuda.empty_cache()
        out["layers_unit"] = layers_unit_probe(4)
        torch.cuda.empty_cache()
        out["append_batch8"] = append_batch_probe()
    if not args.no_cpu_baseline:
        del ui
        out["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
