// Attention of the unit's noisy tokens over [valid ring || the unit's own
// tokens], bidirectional inside the unit, on bf16 MFMA (gfx950).
//
// Semantics [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal Transformer;
// 3.4 条件流匹配]: the block being denoised sees every earlier (clean) block
// and itself in full, audio and video both ways; sessions are independent.
// Scale 1/sqrt(head_dim), no mask over valid keys.
//
// Work item = (session, head, key split, 256-row query block); 8 waves per
// block (two per SIMD, so one wave's MFMAs overlap the other's softmax), 32
// query rows per wave.  Keys stream through LDS in 64-key windows
// aligned to 16-slot blocks (the first and last window of a ring segment may be
// partial; their out-of-range keys are masked and their values zeroed).
//
// Per window and wave (all on v_mfma_f32_32x32x16_bf16):
//   S^T[key][query] = K * Q^T        A = K rows from LDS, B = Q^T in registers
//   online softmax over the keys of each query; each lane owns one query
//   column, so the row reductions are in-lane plus one exchange with lane^32
//   O^T[hd][query] += V^T * P^T      A = V^T (keys contiguous) from LDS,
//                                    B = P^T straight from the S^T registers
// K is loaded into the QK product with rows permuted (bits 2 and 3 of the row
// index swapped), which makes the S^T accumulator registers of lane group g
// hold 8 consecutive keys -- exactly the B-operand layout of the PV product --
// so P never leaves the registers.  V^T rows are permuted so that each lane's
// 16 output registers hold 16 consecutive features of its query.
//
// Softmax rescaling is lazy: O and the running sum are rescaled only when a
// row maximum grows by more than 2^8 (in exp2 units), which is exact (the same
// shift multiplies numerator and denominator) and bounds p <= 256.
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegInf = -__builtin_inff();

// Row permutation of the K operand: swap bits 2 and 3.
__device__ __forceinline__ int perm_k(int r) {
  return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// XOR swizzle of the 16-byte chunks of key k's row in the K tile (the row has
// HD/8 chunks; only the low 4 bits of k matter).
template <int HD>
__device__ __forceinline__ int kswz(int k) {
  return HD == 128 ? (k & 15) : ((k >> 1) & 7);
}
// Row permutation of the V^T operand: A-operand row rho = [b0 b1 | g | a0 a1]
// (bits) loads feature sigma(rho) = [b0 b1 | a0 a1 | g], so that output
// register r of lane group g holds feature 16g + r of the 32-row block.

__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HD>
struct Tiles {
  static constexpr int KC = HD / 16;           // 16-wide k chunks of the QK product
  static constexpr int HB = HD / 32;           // 32-row feature blocks of the PV product
  static constexpr int K_BYTES = kAttnWindow * HD * 2;
  static constexpr int V_BYTES = kAttnWindow * HD * 2;
  static constexpr int K_BLOCKS = K_BYTES / 1024;        // 1 KiB operand blocks
  static constexpr int V_BLOCKS = V_BYTES / 1024;
  static constexpr int K_PER_WAVE = K_BLOCKS / kAttnWaves;
  static constexpr int V_PER_WAVE = V_BLOCKS / kAttnWaves;
  static constexpr int STAGES = 3;                       // K and V triple-buffered
  static constexpr int LDS_BYTES = STAGES * (K_BYTES + V_BYTES);
};

struct Window {
  const bf16* k;      // K of the window's first key
  const bf16* v;      // V block of the window's first key
  int start;          // first key of the window (multiple of 16)
  int lo, hi;         // valid keys [lo, hi) of its segment
  bool full;          // every key of the window is valid
};

// The keys one work item covers: windows [0, nw) of one key segment (the
// valid ring range before the wrap point, the one after it, or the unit's own
// keys), window j starting at key start0 + 64j of the segment.  In both key
// layouts key k of a segment sits at element k*HD of the segment's base
// (K: [keys][HD]; V: [keys/16][HD][16]).  Keys outside [lo, hi) are not part
// of the segment; only the first and the last window of a segment can hold
// such keys.  Every value involved is wave-uniform (scalar).
struct Span {
  const bf16* k;
  const bf16* v;
  int start0, lo, hi, nw;
};

template <int HD>
__device__ __forceinline__ Window window_of(const Span& sp, int j) {
  Window r;
  r.start = sp.start0 + j * kAttnWindow;
  r.k = sp.k + (int64_t)r.start * HD;
  r.v = sp.v + (int64_t)r.start * HD;
  r.lo = sp.lo;
  r.hi = sp.hi;
  r.full = r.start >= sp.lo && r.start + kAttnWindow <= sp.hi;
  return r;
}

// Direct-to-LDS loads of one window; the hardware puts lane i's 16 bytes at
// base + 16*i of the wave's 1 KiB destination.  K: the window's keys are kept
// row by row (key k at byte 2*HD*k), each wave instruction reading 1 KiB of
// whole rows (512/HD keys); the 16-byte chunk c of key k sits at chunk position
// c ^ kswz(k) of its row, so that the QK operand reads (16 lanes = 16 keys of
// one chunk per LDS cycle) hit 16 different bank groups.  V^T: block
// b = c*HB + hb, lane (g, e) -> feature 32hb + sigma(e), keys 16c + 8g .. +7,
// which is one contiguous 1 KiB of the [keys/16][HD][16] layout per
// instruction.  koff/voff are the lane offsets (elements, loop-invariant).
// In a partial window every lane still loads (so each wave issues the same
// number of loads), from an address clamped into the valid range; scores of
// invalid keys are masked and their values zeroed in LDS before use.
template <int HD>
__device__ __forceinline__ void load_window(const Window& w, char* kdst, char* vdst, bool do_k,
                                            bool do_v, const int (&koff)[Tiles<HD>::K_PER_WAVE],
                                            const int (&voff)[Tiles<HD>::V_PER_WAVE],
                                            int wave) {
  using T = Tiles<HD>;
  if (w.full) {
    if (do_k)
#pragma unroll
      for (int i = 0; i < T::K_PER_WAVE; ++i)
        __builtin_amdgcn_global_load_lds(w.k + koff[i], kdst + (wave + kAttnWaves * i) * 1024,
                                         16, 0, 0);
    if (do_v)
#pragma unroll
      for (int i = 0; i < T::V_PER_WAVE; ++i)
        __builtin_amdgcn_global_load_lds(w.v + voff[i], vdst + (wave + kAttnWaves * i) * 1024,
                                         16, 0, 0);
  } else {
    if (do_k)
#pragma unroll
      for (int i = 0; i < T::K_PER_WAVE; ++i) {
        const int rel = koff[i] / HD;              // key within the window
        const int col = koff[i] - rel * HD;
        const int key = min(max(w.start + rel, w.lo), w.hi - 1);
        __builtin_amdgcn_global_load_lds(w.k + (key - w.start) * HD + col,
                                         kdst + (wave + kAttnWaves * i) * 1024, 16, 0, 0);
      }
    if (do_v)
#pragma unroll
      for (int i = 0; i < T::V_PER_WAVE; ++i) {
        // voff = c*16*HD + feat*16 + 8g: chunk of 8 keys starting at 16c + 8g.
        const int c = voff[i] / (16 * HD);
        const int rem = voff[i] - c * 16 * HD;
        const int feat = rem >> 4, g8 = rem & 15;
        int key0 = w.start + c * 16 + g8;
        key0 = min(max(key0, w.lo & ~7), (w.hi - 1) & ~7);    // an in-range 8-key chunk
        const int rel = key0 - w.start;
        __builtin_amdgcn_global_load_lds(w.v + (rel & ~15) * HD + feat * 16 + (rel & 15),
                                         vdst + (wave + kAttnWaves * i) * 1024, 16, 0, 0);
      }
  }
}

// Zero, in a window's V tile in LDS, the values of keys outside [lo, hi)
// (they came from clamped loads or other ring slots, which may hold anything).
// P is 0 for those keys, but 0 * NaN would poison O.  Partial windows only.
template <int HD>
__device__ __forceinline__ void zero_invalid_v(char* vbuf, const Window& win) {
  using T = Tiles<HD>;
  for (int slot = threadIdx.x; slot < T::V_BLOCKS * 64; slot += kAttnThreads) {
    const int b = slot >> 6, l = slot & 63;
    const int c = b / T::HB, g = l >> 5;
    const int key0 = win.start + c * 16 + g * 8;
    unsigned keep = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      keep |= (key0 + t >= win.lo && key0 + t < win.hi ? 1u : 0u) << t;
    if (keep == 0xFFu) continue;
    union { u32x4 u; unsigned short hw[8]; } x;
    x.u = *reinterpret_cast<const u32x4*>(vbuf + slot * 16);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (!(keep & (1u << t))) x.hw[t] = 0;
    *reinterpret_cast<u32x4*>(vbuf + slot * 16) = x.u;
  }
}

// One wave-wide direct-to-LDS load: lane i's 16 bytes at src go to dst + 16*i.
__device__ __forceinline__ void dma16(const bf16* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Wait until at most N of this wave's loads are outstanding, then barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);   // vmcnt(N); expcnt/lgkmcnt unconstrained
  __asm__ volatile("" ::: "memory");
  __syncthreads();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Scores of keys outside the window's valid range -> -inf (partial windows).
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], const Window& win) {
  const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = win.start + kb * 32 + (r >> 3) * 16 + g * 8 + (r & 7);
      if (key < win.lo || key >= win.hi) s[kb][r] = kNegInf;
    }
}

// Row maximum of a window's scores for this lane's query, in exp2 units.
__device__ __forceinline__ float row_max(const f32x16 (&s)[2], float scale_log2) {
  float m = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) m = max3f(m, s[0][r], s[1][r]);
  return max_xor32(m) * scale_log2;
}

// Lazy rescale: only when some row's maximum grew by more than the threshold.
template <int HB>
__device__ __forceinline__ void maybe_rescale(float mx, f32x16 (&o)[HB], float& m_run,
                                              float& l_run) {
  if (__ballot(mx > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[hb][r] *= alpha;
  }
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnArgs a) {
  using T = Tiles<HD>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  // LDS: K buffers 0..2, then V buffers 0..2.
  auto kbuf = [&](int i) { return lds + i * T::K_BYTES; };
  auto vbuf = [&](int i) { return lds + T::STAGES * T::K_BYTES + i * T::V_BYTES; };

  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const AttnSess& s = a.s[si];
  const int H = a.H;
  const float scale_log2 = a.scale_log2;

  // Item order inside a session: (head, split, query block), query block fastest,
  // so the query blocks sharing one key range are adjacent (same XCD).
  int local = item - s.item0;
  const int qblk = local % s.n_qblk;
  local /= s.n_qblk;
  const int split = local % s.nsplit;
  const int h = local / s.nsplit;

  // The split's segment and window range.
  const int sg = split >= s.split0[2] ? 2 : (split >= s.split0[1] ? 1 : 0);
  const int ns_seg = s.split0[sg + 1] - s.split0[sg];
  const int ls = split - s.split0[sg];
  const int nwin_seg = s.nwin[sg];
  const int w_begin = ls * nwin_seg / ns_seg;
  const int nw = (ls + 1) * nwin_seg / ns_seg - w_begin;    // >= 1
  Span sp;
  if (sg == 2) {
    sp.k = s.kt_u + (int64_t)h * s.npad * HD;
    sp.v = s.vt_u + (int64_t)h * s.npad * HD;
    sp.lo = 0;
    sp.hi = s.n_q;
  } else {
    sp.k = s.ring_k + (int64_t)h * s.cap * HD;
    sp.v = s.ring_v + (int64_t)h * s.cap * HD;
    sp.lo = sg == 0 ? s.seg_lo[0] : s.seg_lo[1];
    sp.hi = sg == 0 ? s.seg_hi[0] : s.seg_hi[1];
  }
  sp.start0 = (sp.lo & ~15) + w_begin * kAttnWindow;
  sp.nw = nw;
  auto win = [&](int j) { return window_of<HD>(sp, j); };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j32 = lane & 31, g = lane >> 5;
  const int row0 = qblk * kAttnBlockM + wave * kAttnRowsPerWave;
  const bool active = row0 < s.n_q;                   // wave-uniform
  const int qrow = row0 + j32;

  // Loop-invariant lane offsets of the window loads.
  int koff[T::K_PER_WAVE], voff[T::V_PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::K_PER_WAVE; ++i) {
    constexpr int CPR = HD / 8;                   // 16-byte chunks per key row
    const int key = (wave + kAttnWaves * i) * (1024 / (2 * HD)) + lane / CPR;
    koff[i] = key * HD + ((lane % CPR) ^ kswz<HD>(key)) * 8;
  }
  const int sigma = (j32 & 3) | (((j32 >> 3) & 3) << 2) | (((j32 >> 2) & 1) << 4);
#pragma unroll
  for (int i = 0; i < T::V_PER_WAVE; ++i) {
    const int b = wave + kAttnWaves * i;
    voff[i] = (b / T::HB) * 16 * HD + ((b % T::HB) * 32 + sigma) * 16 + g * 8;
  }
  // QK operand reads: lane (g, rho) wants key 32kb + perm_k(rho), chunk 2kc+g;
  // byte offsets within the K tile for kb = 0 (kb adds 64*HD).
  int kroff[T::KC];
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc)
    kroff[kc] = perm_k(j32) * 2 * HD + ((2 * kc + g) ^ kswz<HD>(perm_k(j32))) * 16;
  auto kread = [&](const char* kt, int kb, int kc) {
    return *reinterpret_cast<const bf16x8*>(kt + kb * 64 * HD + kroff[kc]);
  };

  // Prologue: K(0), V(0), K(1), V(1), K(2).
  const Window w0 = win(0);
  load_window<HD>(w0, kbuf(0), vbuf(0), true, true, koff, voff, wave);
  if (nw > 1) load_window<HD>(win(1), kbuf(1), vbuf(1), true, true, koff, voff, wave);
  if (nw > 2) load_window<HD>(win(2), kbuf(2), vbuf(2), true, false, koff, voff, wave);

  // Q^T operand: lane (j, g) holds query row0+j, features 16kc+8g..+7.
  bf16x8 qr[T::KC];
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc)
    qr[kc] = qrow < s.n_q ? *reinterpret_cast<const bf16x8*>(
                                s.q + ((int64_t)qrow * H + h) * HD + kc * 16 + g * 8)
                          : bf16x8{};

  f32x16 o[T::HB];
#pragma unroll
  for (int hb = 0; hb < T::HB; ++hb) o[hb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  f32x16 s_cur[2];

  wait_loads_and_sync<0>();
  // Window 0's invalid values are zeroed here; step 0's barrier publishes it.
  if (!w0.full) zero_invalid_v<HD>(vbuf(0), w0);
  if (active) {
    s_cur[0] = s_cur[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s_cur[kb] = mfma32x32x16(kread(kbuf(0), kb, kc), qr[kc], s_cur[kb]);
    if (!w0.full) mask_scores(s_cur, w0);
    maybe_rescale<T::HB>(row_max(s_cur, scale_log2), o, m_run, l_run);
  }

  // Step j: softmax and P*V of window j, scores of window j+1, with the loads
  // of K(j+3) and V(j+2) in flight.  On entry s_cur holds window j's (masked)
  // scores with m_run already updated for them; K(j+1) and V(j) were issued
  // in step j-2 (or the prologue), K(j+2) and V(j+1) in step j-1.
  // Steady steps (j + 5 <= nw) touch only full windows, issue every load and
  // wait for a constant count: no branch but the rare rescale.  The last
  // steps (TAIL) handle partial windows and the end of the pipeline.
  // `stage` = j % 3 (a literal in the steady loop, folded after inlining).
  auto step = [&](const int j, const int stage, const bool TAIL) __attribute__((always_inline)) {
    const int st1 = stage == 2 ? 0 : stage + 1;   // (j+1) % 3
    const int st2 = st1 == 2 ? 0 : st1 + 1;       // (j+2) % 3
    if (!TAIL) {
      wait_loads_and_sync<T::K_PER_WAVE + T::V_PER_WAVE>();
      // K(j+3) -> the buffer of K(j) (read by QK(j) in step j-1);
      // V(j+2) -> the buffer of V(j-1) (read by P*V(j-1)).
      const bf16* kp = sp.k + (int64_t)(sp.start0 + (j + 3) * kAttnWindow) * HD;
      const bf16* vp = sp.v + (int64_t)(sp.start0 + (j + 2) * kAttnWindow) * HD;
#pragma unroll
      for (int i = 0; i < T::K_PER_WAVE; ++i)
        dma16(kp + koff[i], kbuf(stage) + (wave + kAttnWaves * i) * 1024);
#pragma unroll
      for (int i = 0; i < T::V_PER_WAVE; ++i)
        dma16(vp + voff[i], vbuf(st2) + (wave + kAttnWaves * i) * 1024);
    } else {
      if (j + 2 < nw)
        wait_loads_and_sync<T::K_PER_WAVE + T::V_PER_WAVE>();
      else if (j + 1 < nw)
        wait_loads_and_sync<T::V_PER_WAVE>();
      else
        wait_loads_and_sync<0>();
      if (j > 0) {
        const Window wj = win(j);
        if (!wj.full) {
          zero_invalid_v<HD>(vbuf(stage), wj);
          __syncthreads();
        }
      }
      if (j + 3 < nw) load_window<HD>(win(j + 3), kbuf(stage), vbuf(st2), true, false, koff, voff, wave);
      if (j + 2 < nw) load_window<HD>(win(j + 2), kbuf(stage), vbuf(st2), false, true, koff, voff, wave);
    }
    if (active) {
      // (A) For each half kb of the window (32 keys): the shifted scores
      //     (FMA) are read out of s[kb], then the scores of window j+1 are
      //     accumulated into the same registers while the exponentials, the
      //     bf16 packing and the row sums of window j proceed.  In the last
      //     step the new scores read a stale in-bounds K buffer and are
      //     discarded.
      const char* kl = kbuf(st1);
      uint32_t pw[4][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // All K operands of this half are read up front so their LDS latency
        // overlaps (one wait instead of one per MFMA).
        bf16x8 ka[T::KC];
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) ka[kc] = kread(kl, kb, kc);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s_cur[kb][r], scale_log2, -m_run);
        __builtin_amdgcn_sched_barrier(0);   // keep the reads issued ahead of the MFMAs
        s_cur[kb] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) s_cur[kb] = mfma32x32x16(ka[kc], qr[kc], s_cur[kb]);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float e0 = __builtin_amdgcn_exp2f(x[c2 * 8 + 2 * t]);
            const float e1 = __builtin_amdgcn_exp2f(x[c2 * 8 + 2 * t + 1]);
            const uint32_t w2 = pack_bf16(e0, e1);
            pw[kb * 2 + c2][t] = w2;
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2),
                                                    __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                                    l_run, false);
          }
        }
        // Each MFMA followed by VALU work (exp/pack/row sum).
#pragma unroll
        for (int t = 0; t < T::KC; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      // (B) P*V of window j, and the row maximum of window j+1.  The V
      //     operands of chunk c+1 are read while chunk c's MFMAs run.
      const bf16x8* vl = reinterpret_cast<const bf16x8*>(vbuf(stage));
      bf16x8 va[2][T::HB];
#pragma unroll
      for (int hb = 0; hb < T::HB; ++hb) va[0][hb] = vl[hb * 64 + lane];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c + 1 < 4)
#pragma unroll
          for (int hb = 0; hb < T::HB; ++hb)
            va[(c + 1) & 1][hb] = vl[((c + 1) * T::HB + hb) * 64 + lane];
        __builtin_amdgcn_sched_barrier(0);   // chunk c+1's reads go out before chunk c's MFMAs
        const u32x4 pv4 = {pw[c][0], pw[c][1], pw[c][2], pw[c][3]};
        const bf16x8 pc = __builtin_bit_cast(bf16x8, pv4);
#pragma unroll
        for (int hb = 0; hb < T::HB; ++hb) o[hb] = mfma32x32x16(va[c & 1][hb], pc, o[hb]);
      }
      float mx = row_max(s_cur, scale_log2);
      // Keep the row-sum updates inside this block (they would otherwise be
      // sunk past it).
      __asm__ volatile("" ::"v"(l_run));
      // (C) window j+1: mask a partial window, then the lazy rescale (which
      //     applies to O accumulated through window j).
      if (!TAIL) {
        maybe_rescale<T::HB>(mx, o, m_run, l_run);
      } else if (j + 1 < nw) {
        const Window w1 = win(j + 1);
        if (!w1.full) {
          mask_scores(s_cur, w1);
          mx = row_max(s_cur, scale_log2);
        }
        maybe_rescale<T::HB>(mx, o, m_run, l_run);
      }
    }
  };

  int j = 0;
  for (; j + 7 <= nw; j += 3) {        // steps j, j+1, j+2 are all steady
    step(j, 0, false);
    step(j + 1, 1, false);
    step(j + 2, 2, false);
  }
  for (; j < nw; ++j) step(j, j % 3, true);

  if (!active) return;
  const float l_tot = sum_xor32(l_run);
  if (qrow >= s.n_q) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (s.nsplit == 1) {
#pragma unroll
    for (int hb = 0; hb < T::HB; ++hb) {
      union { bf16x8 v[2]; bf16 b[16]; } u;
#pragma unroll
      for (int r = 0; r < 16; ++r) u.b[r] = (bf16)(o[hb][r] * inv);
      bf16* dst = s.o + ((int64_t)qrow * H + h) * HD + hb * 32 + g * 16;
      reinterpret_cast<bf16x8*>(dst)[0] = u.v[0];
      reinterpret_cast<bf16x8*>(dst)[1] = u.v[1];
    }
  } else {
    const int64_t rowh = ((int64_t)split * s.n_q + qrow) * H + h;
#pragma unroll
    for (int hb = 0; hb < T::HB; ++hb) {
      float* dst = s.opart + rowh * HD + hb * 32 + g * 16;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v = {o[hb][r4 * 4 + 0] * inv, o[hb][r4 * 4 + 1] * inv,
                   o[hb][r4 * 4 + 2] * inv, o[hb][r4 * 4 + 3] * inv};
        reinterpret_cast<f32x4*>(dst)[r4] = v;
      }
    }
    if (g == 0) s.lse[rowh] = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
  }
}

// Merge key-split partials: O = sum_s w_s o_s / sum_s w_s, w_s = 2^(lse_s - max).
// One thread per (row, head, 8 features).
template <int HD>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int TPR = HD / 8;              // threads per (row, head)
  constexpr int GPB = 256 / TPR;           // (row, head) groups per block
  const int grp = blockIdx.x * GPB + threadIdx.x / TPR;
  if (grp >= a.items) return;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && grp >= a.s[i].item0) si = i;
  const CombineSess& s = a.s[si];
  const int64_t rh = grp - s.item0;                 // row * H + head
  const int64_t stride = (int64_t)s.n_q * a.H;      // between splits
  const int e0 = (threadIdx.x % TPR) * 8;
  float mx = kNegInf;
  for (int k = 0; k < s.nsplit; ++k) mx = fmaxf(mx, s.lse[k * stride + rh]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int k = 0; k < s.nsplit; ++k) {
    const float w = __builtin_amdgcn_exp2f(s.lse[k * stride + rh] - mx);
    wsum += w;
    const f32x4* src = reinterpret_cast<const f32x4*>(s.opart + (k * stride + rh) * HD + e0);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] += w * x0[t];
      acc[4 + t] += w * x1[t];
    }
  }
  const float inv = 1.0f / wsum;
  bf16x8 out;
#pragma unroll
  for (int t = 0; t < 8; ++t) out[t] = (bf16)(acc[t] * inv);
  *reinterpret_cast<bf16x8*>(s.o + rh * HD + e0) = out;
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int head_dim, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  // The pipeline uses more than the default 64 KiB of LDS (gfx950 has 160 KiB
  // per CU); raise the kernels' dynamic-LDS limit once.
  static const hipError_t attr_err = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<128>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Tiles<128>::LDS_BYTES);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, Tiles<64>::LDS_BYTES);
    return e;
  }();
  if (attr_err != hipSuccess) return attr_err;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, dim3(a.items), dim3(kAttnThreads), Tiles<128>::LDS_BYTES,
                       st, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(a.items), dim3(kAttnThreads), Tiles<64>::LDS_BYTES,
                       st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  const int gpb = 256 / (head_dim / 8);
  const int blocks = (a.items + gpb - 1) / gpb;
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmd
