"""CPU oracle for the performer's per-unit flow-matching denoise step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
product path (``flow_matching_denoising_amd``) never imports it and shares no
code with it; the two meet only in the seeded input module ``workload``.

What it computes, in the pages' order (sources are the pages' titles and
sections):

1. ``ring.kv_append`` -- the performer writes the thinker's K/V slice into its
   local, preallocated cache at the slice's position
   [Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
   方法概述和架构; Wan-Streamer v0.2 (zhao9797 blog), Infra].
2. ``attention.attention`` -- the unit's noisy audio and video tokens attend to
   all clean history plus the unit's own tokens, bidirectionally inside the
   unit [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal Transformer and
   3.4 条件流匹配: cross-modal conditioning, clean context].
3. ``flow.velocity`` -- one dense output projection gives the velocity of both
   modalities [same page, 3.4: one f_theta predicts both velocity fields].
4. ``flow.euler_step`` / ``flow.denoise_unit`` -- the linear (rectified-flow)
   path has a constant velocity, integrated by an ODE solver over a few steps
   [same page, 3.4; Fig. 2: the performer receives the slice, then only runs
   the flow-matching solver].
5. ``qkv.qkv_projection`` / ``qkv.denoise_unit_qkv`` -- the same solver with
   the unit's Q, K, V projected from the current latent at every step
   [same page, 3.4: f_theta is evaluated on the noisy latents it integrates].
6. ``cfg.denoise_unit_cfg`` -- the classifier-free-guided sampler of the
   teacher: conditional and unconditional branches, guided velocity
   v_u + g (v_c - v_u) [same page, training stages, Stage 3].
7. ``ulysses.ulysses_attention`` -- the attention computed over P performer
   ranks: head-sharded cache, sequence-sharded video rows, all-to-all between
   sequence and head dimensions, gather [Wan-Streamer v0.2: Higher
   Resolution, Same Latency (nanless digest), 方法概述和架构].
8. ``layers.denoise_unit_layers`` -- the z-dependent solver over a stack of
   L attention layers with per-layer rings and a residual stream
   [Wan-Streamer (gongshangzheng blog), 3.3 and 3.4].

Everything is float64 unless a function says otherwise.  bf16 inputs arrive as
uint16 bit patterns and are widened exactly by ``ring.bf16_bits_to_f64``.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (brute force on tiny inputs, a library attention
routine on independently gathered keys, closed forms, invariants).  The
end-to-end composition on random N(0,1) inputs has no pin beyond its parts:
parity unpinned for that composition as a whole.
"""
from .ring import bf16_bits_to_f64, kv_append, valid_slots  # noqa: F401
from .attention import attention, attention_naive  # noqa: F401
from .flow import velocity, euler_step, denoise_step, denoise_unit  # noqa: F401
from .qkv import round_to_bf16, f64_to_bf16_bits, qkv_projection, denoise_unit_qkv  # noqa: F401
from .cfg import guided_velocity, denoise_unit_cfg  # noqa: F401
from .ulysses import ulysses_attention  # noqa: F401
from .layers import layer_stack_velocity, denoise_unit_layers  # noqa: F401
