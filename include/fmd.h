/*
 * fmd.h -- C ABI of the performer's per-unit flow-matching denoise step
 * (Wan-Streamer v0.2), built for one MI355X (gfx950).
 *
 * What the calls implement, by source page and section:
 *  - fmd_kv_append / fmd_kv_append_batched: the performer writes the thinker's
 *    compact K/V slice into its own preallocated cache at the slice's position
 *    [Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
 *    方法概述和架构; Wan-Streamer v0.2 (zhao9797 blog), Infra].
 *  - fmd_attention / fmd_denoise_step: the unit's noisy video and audio latent
 *    tokens attend to all clean history and to each other (bidirectional inside
 *    the unit) [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal
 *    Transformer; 3.4 条件流匹配, cross-modal conditioning and clean context];
 *    one dense projection gives the velocity of both modalities and an Euler
 *    step moves z along the rectified-flow path [same page, 3.4].
 *  - fmd_denoise_unit: one unit = the append, then the flow-matching solver
 *    [same page, Fig. 2: the performer receives the slice and only runs the
 *    solver].
 *  - fmd_denoise_unit_qkv: the solver with the unit's Q, K, V projected from
 *    the current latent at every step [same page, 3.4].
 *  - fmd_denoise_unit_cfg: the classifier-free-guided sampler of the teacher
 *    the deployed performer is distilled from [same page, training stages,
 *    Stage 3].
 *  - fmd_denoise_unit_layers: the solver over a stack of attention layers,
 *    one ring per layer [same page, 3.3 and 3.4].
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains device memory; scratch space is the
 *    caller's `workspace`.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work and return; results are valid once the stream reaches that point.
 *  - Every argument is validated before anything is enqueued.  A non-zero
 *    return other than FMD_E_HIP means no kernel was launched and no host
 *    state (a cache's len_tokens/head_tokens) changed.  fmd_last_error() then
 *    describes the first failed check.  FMD_E_HIP means the HIP runtime
 *    refused a launch: the launches before it stay enqueued, and a ring
 *    whose append was among them has advanced (the others are unchanged).
 *  - All tensor pointers must be 16-byte aligned (FMD_E_ALIGN otherwise).
 *  - bf16 = IEEE binary32's upper 16 bits; fp32 = IEEE binary32.
 *  - Calls on different caches are independent; one cache must not be used
 *    by two host threads at once.
 */
#ifndef FMD_H
#define FMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMD_MAX_SESSIONS 64   /* sessions per call */
#define FMD_CACHE_BLOCK 16    /* tokens per block of the V cache layout */

typedef enum {
  FMD_OK = 0,
  FMD_E_INVAL = -1,      /* null pointer, non-positive count, bad ring state */
  FMD_E_SHAPE = -2,      /* head_dim not 64/128, heads or d mismatched, cap not a multiple of 16 */
  FMD_E_CAPACITY = -3,   /* slice longer than the ring */
  FMD_E_ALIGN = -4,      /* a pointer is not 16-byte aligned */
  FMD_E_WORKSPACE = -5,  /* workspace missing or smaller than required */
  FMD_E_HIP = -6         /* the HIP runtime reported an error */
} fmd_status;

/*
 * One session's K/V ring.  The struct lives in host memory and is owned by
 * the caller; k and v point to device memory the caller allocated.
 *   k : bf16 [n_heads][cap_tokens][head_dim]              (token rows per head)
 *   v : bf16 [n_heads][cap_tokens/16][head_dim][16]       (16-token blocks, each
 *       stored feature-major: element (h, slot p, e) is at
 *       ((h*(cap/16) + p/16)*head_dim + e)*16 + p%16)
 *   The pages fix no layout; they pre-shard the cache so that no step has to
 *   rearrange it [精读笔记 (paper.gecl.asia), Key Insight].  V is kept in
 *   16-token feature-major blocks so that the attention's P*V product reads
 *   its operand straight from the stored bytes, hence cap_tokens % 16 == 0.
 *   head_dim   : 64 or 128
 *   cap_tokens : ring capacity in tokens, a positive multiple of 16, with
 *                cap_tokens*head_dim*2 < 2^31 (one head's slice is addressed
 *                with 32-bit byte offsets)
 *   len_tokens : valid tokens, 0..cap_tokens
 *   head_tokens: slot the next token goes to, 0..cap_tokens-1
 * The valid tokens are the len_tokens slots just before head_tokens (mod cap).
 * The library updates len_tokens/head_tokens when it enqueues an append.
 */
typedef struct fmd_kv_cache {
  void* k;
  void* v;
  int32_t n_heads;
  int32_t head_dim;
  int64_t cap_tokens;
  int64_t len_tokens;
  int64_t head_tokens;
} fmd_kv_cache;

/*
 * Append one slice of n_tokens tokens to a ring: token t goes to slot
 * (head + t) mod cap of every head; then head += n_tokens (mod cap) and
 * len = min(len + n_tokens, cap).  Oldest tokens are overwritten.
 *   k_slice, v_slice: bf16 [n_tokens][n_heads][head_dim], contiguous,
 *                     token-major as the thinker's projection emits them.
 * Errors: FMD_E_INVAL (null, n_tokens < 1, bad ring state), FMD_E_CAPACITY
 * (n_tokens > cap), FMD_E_SHAPE, FMD_E_ALIGN, FMD_E_HIP.
 */
int fmd_kv_append(fmd_kv_cache* cache, const void* k_slice, const void* v_slice,
                  int64_t n_tokens, void* stream);

/* The same for n_sessions rings in one launch (sessions may differ in
 * capacity, state and slice length; n_heads and head_dim must match).
 * caches[i] is updated as by fmd_kv_append.  Same errors. */
int fmd_kv_append_batched(fmd_kv_cache* const* caches, const void* const* k_slices,
                          const void* const* v_slices, const int64_t* n_tokens,
                          int32_t n_sessions, void* stream);

/*
 * One session's inputs for ONE solver step.
 *   cache     : the session's ring in its post-append state (read only)
 *   q, k_u, v_u: bf16 [n_q][n_heads][head_dim], the unit's queries and its own
 *               keys/values, n_q = n_video + n_audio (1..2^22), rows video then audio
 *   z         : fp32 [n_q][n_heads*head_dim], updated in place
 *   h         : positive step size; the step is z <- z - h * v
 */
typedef struct fmd_unit_step {
  const fmd_kv_cache* cache;
  const void* q;
  const void* k_u;
  const void* v_u;
  float* z;
  int32_t n_video;
  int32_t n_audio;
  float h;
} fmd_unit_step;

/* Workspace bytes fmd_attention / fmd_denoise_step need for these units.
 * Pure host arithmetic. Errors: FMD_E_INVAL, FMD_E_SHAPE. */
int fmd_workspace_bytes(const fmd_unit_step* units, int32_t n_units, size_t* out_bytes);

/*
 * One solver step for n_units sessions:
 *   O = attention(q, [valid ring || k_u], [valid ring || v_u]) per head, scale
 *       1/sqrt(head_dim), no mask; q is multiplied by log2(e)/sqrt(head_dim)
 *       and rounded to bf16 once, scores, softmax and accumulation are fp32,
 *       the probabilities enter the value product as bf16, O is rounded to
 *       bf16.  The keys of one launch are cut into equal ranges, one per
 *       group of work-groups; the rows of a (head, session) whose keys a cut
 *       splits get each piece's normalised output stored as bf16 (with an
 *       fp32 log-sum-exp) and merged, and the merged O is rounded to bf16
 *       again: one extra bf16 rounding (<= 2^-9 relative) for those rows;
 *   v = O_flat * W_o^T with O_flat [n_q][d] (heads concatenated);
 *   z <- z - h * v  (fp32).
 *   w_o: bf16 [d][d] stored [d_out][d_in], d = n_heads*head_dim, shared.
 *   workspace: device scratch of at least fmd_workspace_bytes() bytes.
 * Errors: FMD_E_INVAL (also when two sessions' latents z overlap: each is
 * updated in place), FMD_E_SHAPE, FMD_E_ALIGN, FMD_E_WORKSPACE, FMD_E_HIP.
 */
int fmd_denoise_step(const fmd_unit_step* units, int32_t n_units, const void* w_o,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The attention part of fmd_denoise_step alone (z and h unused), writing
 * O as bf16 [sum n_q][n_heads][head_dim], sessions in order.  Same errors. */
int fmd_attention(const fmd_unit_step* units, int32_t n_units, void* o_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * One session's inputs for a whole unit.
 *   cache          : the session's ring (state before the append; updated)
 *   k_slice/v_slice: bf16 [slice_tokens][n_heads][head_dim]; slice_tokens = 0
 *                    means the unit appends nothing
 *   q, k_u, v_u    : bf16 base pointers of step 0's [n_q][n_heads][head_dim]
 *                    tensors; step s uses base + s*step_stride_elems
 *                    (0 = the same tensors for every step)
 *   z              : fp32 [n_q][d], holds eps on entry, the final latent on exit
 *   h              : HOST array [n_steps] of positive step sizes, read during
 *                    the call
 */
typedef struct fmd_unit_io {
  fmd_kv_cache* cache;
  const void* k_slice;
  const void* v_slice;
  int64_t slice_tokens;
  const void* q;
  const void* k_u;
  const void* v_u;
  int64_t step_stride_elems;
  float* z;
  int32_t n_video;
  int32_t n_audio;
  const float* h;
} fmd_unit_io;

/* Workspace bytes fmd_denoise_unit needs for n_steps steps (pure host
 * arithmetic).  The unit values of all n_steps steps are staged in the
 * attention's 16-key blocked layout by one launch before the first step; the
 * attention reads the unit keys where the caller keeps them (they are staged
 * too, in [H][npad][hd], only when n_q * d * 2 bytes reach 2^31).  The
 * workspace holds n_steps copies of room for what is staged (one when every
 * session's step_stride_elems is 0).  Errors: as fmd_denoise_unit's
 * validation. */
int fmd_unit_workspace_bytes(const fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps,
                             size_t* out_bytes);

/*
 * One denoised unit for n_sessions sessions: one batched append, then
 * n_steps solver steps, each as fmd_denoise_step with h[s].  The steps' Q,
 * K_u and V_u are inputs, so no step's attention reads the latent: the
 * attention of B steps runs as one launch whose sessions are the (step,
 * session) pairs (B: the largest divisor of n_steps with B * n_sessions <= 16,
 * else 1), then the B projections and Euler updates follow in step order.
 * The workspace holds O and the pieces of cut lanes for each of the B steps.
 * Errors: as fmd_kv_append and fmd_denoise_step; n_steps < 1 -> FMD_E_INVAL.
 */
int fmd_denoise_unit(fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps,
                     const void* w_o, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * fmd_denoise_unit without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics, validation
 * and errors as fmd_denoise_unit, and the same kernels; their scratch is a
 * static device array of FMD_NOALLOC_SCRATCH_BYTES (256 MiB) that the
 * library holds on every GPU it runs on until the process ends.  The call
 * allocates no device memory.
 *   - A unit whose scratch need (fmd_unit_workspace_bytes) exceeds
 *     FMD_NOALLOC_SCRATCH_BYTES -> FMD_E_WORKSPACE, nothing enqueued.  One
 *     640x368-class session (40 heads x 928 queries, 4 steps with their own
 *     Q/K/V) needs 192 MB with 60,416 cached keys and 230 MB with the wrapped
 *     241,664-key ring, and fits; two such sessions do not.
 *   - `stream` must belong to the current device (FMD_E_INVAL otherwise).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on
 *     one GPU (different streams or host threads without ordering) race and
 *     give wrong results.  Calls ordered on one stream are safe.  Nothing in
 *     the scratch needs to start at zero; it keeps the last call's contents.
 */
#define FMD_NOALLOC_SCRATCH_BYTES (256u << 20)
int fmd_denoise_unit_noalloc(fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps,
                             const void* w_o, void* stream);

/*
 * The solver with the unit's queries, keys and values re-derived from the
 * latent at every step: the velocity network is evaluated on the noisy
 * latents it integrates [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配:
 * f_theta on the unit's noisy audio and video latents; 3.3 Block-Causal
 * Transformer: those tokens attend to the clean history and to each other].
 * Per step s, for every session:
 *   [Q | K_u | V_u] = bf16( bf16(z) * W_qkv^T ),  W_qkv bf16 [3d][d] stored
 *       [d_out][d_in]; output column h*hd + e of each third is head h,
 *       feature e (bf16 rounding: nearest, ties to even);
 *   then the step of fmd_denoise_step with those Q, K_u, V_u and h[s].
 * One session's inputs (no per-step Q/K/V: they come from z):
 *   cache          : the session's ring (state before the append; updated)
 *   k_slice/v_slice: bf16 [slice_tokens][n_heads][head_dim]; 0 tokens = no append
 *   z              : fp32 [n_q][d], eps on entry, the final latent on exit
 *   h              : HOST array [n_steps] of positive step sizes
 */
typedef struct fmd_unit_qkv_io {
  fmd_kv_cache* cache;
  const void* k_slice;
  const void* v_slice;
  int64_t slice_tokens;
  float* z;
  int32_t n_video;
  int32_t n_audio;
  const float* h;
} fmd_unit_qkv_io;

/* Workspace bytes fmd_denoise_unit_qkv needs (pure host arithmetic). */
int fmd_unit_qkv_workspace_bytes(const fmd_unit_qkv_io* sessions, int32_t n_sessions,
                                 size_t* out_bytes);

/* One denoised unit of the z-dependent solver for n_sessions sessions: one
 * batched append, then n_steps steps as above.  w_qkv: bf16 [3d][d]; w_o:
 * bf16 [d][d].  Errors: as fmd_denoise_unit. */
int fmd_denoise_unit_qkv(fmd_unit_qkv_io* sessions, int32_t n_sessions, int32_t n_steps,
                         const void* w_qkv, const void* w_o, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The classifier-free-guided form of the z-dependent solver, as the teacher
 * samples: the deployed few-step performer is distilled from a stronger
 * teacher that uses classifier-free guidance and more solver steps
 * [Wan-Streamer (gongshangzheng blog), training stages, Stage 3 低延迟蒸馏].
 * Each unit has two branches that differ only in the clean context their
 * attention reads: a conditional cache and an unconditional cache.  Per step
 * s, for every unit:
 *   [Q | K_u | V_u] from bf16(z) as in fmd_denoise_unit_qkv (shared by both
 *       branches);
 *   O_c, O_u = attention of those queries over [valid ring ; unit tokens] of
 *       the conditional and of the unconditional cache;
 *   v = v_u + g (v_c - v_u) with v_b = O_b W_o^T, computed as
 *       bf16((1 - g) O_u + g O_c) W_o^T (one projection; g = 1 gives the
 *       conditional branch alone, g = 0 the unconditional one);
 *   z <- z - h[s] v.
 * One unit's inputs:
 *   cond, uncond   : the two branches' rings (state before the appends;
 *                    updated); distinct caches of one shape
 *   cond_/uncond_  : bf16 [slice_tokens][n_heads][head_dim] slices appended to
 *     k/v_slice      the respective ring first; 0 tokens = no append
 *   z              : fp32 [n_q][d], eps on entry, the final latent on exit
 *   h              : HOST array [n_steps] of positive step sizes
 *   guidance       : the guidance scale g (finite; any sign)
 */
typedef struct fmd_unit_cfg_io {
  fmd_kv_cache* cond;
  fmd_kv_cache* uncond;
  const void* cond_k_slice;
  const void* cond_v_slice;
  int64_t cond_slice_tokens;
  const void* uncond_k_slice;
  const void* uncond_v_slice;
  int64_t uncond_slice_tokens;
  float* z;
  int32_t n_video;
  int32_t n_audio;
  const float* h;
  float guidance;
} fmd_unit_cfg_io;

/* Workspace bytes fmd_denoise_unit_cfg needs (pure host arithmetic). */
int fmd_unit_cfg_workspace_bytes(const fmd_unit_cfg_io* sessions, int32_t n_sessions,
                                 size_t* out_bytes);

/* One denoised unit of the guided solver for n_sessions units (1 ..
 * FMD_MAX_SESSIONS / 2): one batched append of every slice, then n_steps
 * steps as above.  w_qkv: bf16 [3d][d]; w_o: bf16 [d][d].  Errors: as
 * fmd_denoise_unit_qkv; a cache used twice or a non-finite guidance scale ->
 * FMD_E_INVAL.  Nothing is enqueued when an error is returned. */
int fmd_denoise_unit_cfg(fmd_unit_cfg_io* sessions, int32_t n_sessions, int32_t n_steps,
                         const void* w_qkv, const void* w_o, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The z-dependent solver over a stack of n_layers attention layers, each with
 * its own ring: the velocity network is a block-causal transformer evaluated
 * on the unit's noisy latents with the clean context at every solver step
 * [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal Transformer, 3.4
 * 条件流匹配]; the pages give no layer structure, so a layer here is the
 * attention block of fmd_denoise_unit_qkv on a residual stream.  Per step s:
 *   r = 0;  for l = 0 .. n_layers-1:
 *     [Q | K_u | V_u] = bf16( bf16(z + r) * W_qkv[l]^T )
 *     O = attention of Q over [layer l's valid ring ; K_u, V_u]
 *     r = r + O * W_o[l]^T                       (fp32)
 *   z <- z - h[s] * r
 * With n_layers = 1 this is fmd_denoise_unit_qkv.
 * One session's inputs:
 *   caches         : [n_layers] the session's ring of each layer (state before
 *                    the appends; updated); distinct caches of one shape
 *   k/v_slices     : [n_layers] bf16 [slice_tokens][n_heads][head_dim], one
 *                    per layer; not read when slice_tokens is 0
 *   slice_tokens   : tokens appended to every layer's ring (0 = none)
 *   z              : fp32 [n_q][d], eps on entry, the final latent on exit
 *   h              : HOST array [n_steps] of positive step sizes
 */
#define FMD_MAX_LAYERS 256
typedef struct fmd_unit_layers_io {
  fmd_kv_cache* const* caches;
  const void* const* k_slices;
  const void* const* v_slices;
  int64_t slice_tokens;
  float* z;
  int32_t n_video;
  int32_t n_audio;
  const float* h;
} fmd_unit_layers_io;

/* Workspace bytes fmd_denoise_unit_layers needs (pure host arithmetic). */
int fmd_unit_layers_workspace_bytes(const fmd_unit_layers_io* sessions, int32_t n_sessions,
                                    int32_t n_layers, size_t* out_bytes);

/* One denoised unit of the layer-stack solver for n_sessions sessions: one
 * batched append of every layer's slice, then n_steps steps as above.  w_qkv,
 * w_o: HOST arrays [n_layers] of device pointers to bf16 [3d][d] and [d][d]
 * weights.  Errors: as fmd_denoise_unit_qkv; n_layers outside
 * 1..FMD_MAX_LAYERS or a cache used twice -> FMD_E_INVAL.  Nothing is
 * enqueued when an error is returned. */
int fmd_denoise_unit_layers(fmd_unit_layers_io* sessions, int32_t n_sessions, int32_t n_layers,
                            int32_t n_steps, const void* const* w_qkv, const void* const* w_o,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* fmd_strerror(int status);

/* Detail of the last error on this host thread (empty string if none). */
const char* fmd_last_error(void);

/* Kernel classes that fmd_profile_* report on. */
enum {
  FMD_KERNEL_APPEND = 0,    /* ring append */
  FMD_KERNEL_VT = 1,        /* staging of the unit's values (and keys, if needed) in the ring layouts */
  FMD_KERNEL_ATTN = 2,      /* attention main kernel */
  FMD_KERNEL_COMBINE = 3,   /* merge of the pieces of cut (head, session) lanes */
  FMD_KERNEL_PROJ = 4,      /* projection GEMM with the Euler update */
  FMD_KERNEL_QKV = 5,       /* projection of the latent to Q, K_u, V_u */
  FMD_KERNEL_CVT = 6,       /* bf16 copy of the starting latent */
  FMD_KERNEL_MIX = 7,       /* guided mix of the two branches' outputs */
  FMD_KERNEL_COUNT = 8
};

/* Per-launch timing with HIP events recorded on the launch stream around
 * every kernel of the selected classes above (all of them unless
 * fmd_profile_select narrowed the set).  enable != 0 turns recording on (and
 * clears earlier records); fmd_profile_read waits for the recorded events and
 * returns the summed duration in ms and the launch count of one class.  The
 * events are created without a system-scope fence (timing only); each
 * recorded launch still adds a few microseconds of queue time around it, which
 * is why a caller timing a whole unit may record one class only. */
int fmd_profile_enable(int enable);
int fmd_profile_read(int kernel_class, double* total_ms, int64_t* launches);

/* Kernel classes recorded while profiling is on: bit c of class_mask selects
 * class c (default: every class).  Bits at or above FMD_KERNEL_COUNT ->
 * FMD_E_INVAL.  Takes effect for launches enqueued after the call; records
 * already taken are kept. */
int fmd_profile_select(uint32_t class_mask);

/* TEST ENTRY (not for production callers).  Later attention launches cut
 * their window sequence into n_groups ranges (at most one per window) instead
 * of the planner's count; 0 restores the planner.  Process-wide: it changes
 * the work decomposition of every later call from any thread, never the
 * result beyond fp32 summation order.  Lets tests drive the one-group path
 * (no piece to merge) and particular cuts of the lanes.
 * n_groups < 0 -> FMD_E_INVAL. */
int fmd_test_force_attn_groups(int32_t n_groups);

/* Library version, "major.minor.patch". */
const char* fmd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FMD_H */
