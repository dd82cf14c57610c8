// Attention of the unit's noisy tokens over [valid ring || the unit's own
// tokens], bidirectional inside the unit, on bf16 MFMA (gfx950).
//
// Semantics [Wan-Streamer (gongshangzheng blog), 3.3 Block-Causal Transformer;
// 3.4 条件流匹配]: the block being denoised sees every earlier (clean) block
// and itself in full, audio and video both ways; sessions are independent.
// Scale 1/sqrt(head_dim), no mask over valid keys.
//
// Work decomposition: the 64-key windows of a launch form one sequence
// (head-major, then session, then the session's key segments), cut into equal
// contiguous ranges, one per group of work-groups.  A group has one work-group
// per 256-row query block; its work-groups walk the range together on one XCD
// and share the keys in its L2.  One work-group per CU, all resident at once,
// so the launch has no dispatch tail.  A work-group walks its range as spans:
// a span is the part of one lane's (head, session) key segment in the range.
// A lane that is one span is written whole; the spans of a lane cut by group
// or segment boundaries are its pieces, each written normalised with its
// log-sum-exp and merged by the combine kernel.
//
// Per work-group: 8 waves (two per SIMD, so one wave's MFMAs overlap the
// other's softmax), 32 query rows per wave.  Keys stream through LDS in
// 64-key windows aligned to 16-slot blocks (the first and last window of a
// ring segment may be partial; their out-of-range keys are masked and their
// values zeroed).
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
// Q^T is multiplied by scale * log2(e) (and rounded to bf16) once per span,
// and every QK product after the first window starts its accumulation
// from -m (m: the row's running maximum), so the MFMA returns the shifted
// score in exp2 units and exp2 takes it as it is: no per-score FMA.  Softmax
// rescaling is lazy: m, O and the running sum move only when a row maximum
// grows by more than 2^8, which is exact (the same shift multiplies numerator
// and denominator) and bounds p <= 256.
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
  static constexpr int STAGES = 4;                       // K and V quadruple-buffered
  static constexpr int LDS_BYTES = STAGES * (K_BYTES + V_BYTES);
};

struct Window {
  int start;          // first key of the window (multiple of 16)
  int lo, hi;         // valid keys [lo, hi) of its segment
  bool full;          // every key of the window is valid
};

// The keys one work item covers: windows [0, nw) of one key segment (the
// valid ring range before the wrap point, the one after it, or the unit's own
// keys), window j starting at key start0 + 64j of the segment.  Keys outside
// [lo, hi) are not part of the segment; only the first and the last window of
// a segment can hold such keys.  Every value involved is wave-uniform.
struct Span {
  int start0, lo, hi, nw;
};

__device__ __forceinline__ Window window_of(const Span& sp, int j) {
  Window r;
  r.start = sp.start0 + j * kAttnWindow;
  r.lo = sp.lo;
  r.hi = sp.hi;
  r.full = r.start >= sp.lo && r.start + kAttnWindow <= sp.hi;
  return r;
}

// Window loads go global -> LDS through buffer resources (MUBUF loads with
// the lds bit): one resource per head and key segment, whose size is the
// segment's storage (cap or npad keys, or up to the last unit key), so that a
// lane whose range-checked offset falls past it reads zeros instead of
// faulting.  Key k of a segment sits at byte 2*HD*k of the ring layouts (K:
// [keys][HD]; V: [keys/16][HD][16]) and at byte 2*H*HD*k of unit keys read
// where the caller keeps them ([n][H][HD]); `row_bytes` is that key stride.
// The hardware puts lane i's 16 bytes at M0 + 16*i.
//
// The load is issued from inline assembly on purpose: it has no register
// outputs, and the compiler, which cannot tell one LDS stage buffer from
// another, would otherwise wait for every LDS load in flight before each LDS
// read.  The kernel orders these loads itself: s_waitcnt vmcnt(N) and a
// barrier before any wave reads a tile (wait_loads_and_sync), and a barrier
// between the last read of a buffer and the next load into it.
// Direct-to-LDS loads of one window.  K: the window's keys are kept row by
// row (key k at byte 2*HD*k), each wave instruction reading 1 KiB of whole
// rows (512/HD keys); the 16-byte chunk c of key k sits at chunk position
// c ^ kswz(k) of its row, so that the QK operand reads (16 lanes = 16 keys of
// one chunk per LDS cycle) hit 16 different bank groups.  V^T: block
// b = c*HB + hb, lane (g, e) -> feature 32hb + sigma(e), keys 16c + 8g .. +7,
// which is one contiguous 1 KiB of the [keys/16][HD][16] layout per
// instruction.  koff/voff are those lane offsets in bytes (loop-invariant).
// CHECKED loads put the window offset into the range-checked lane offset
// (first and last windows of a segment, which may reach past its storage);
// the others pass it as the scalar offset.  Scores of keys outside [lo, hi)
// are masked and their values zeroed in LDS before use.
// Offsets are 32-bit unsigned byte counts: a window that starts below the
// segment's end (start * row_bytes < 2^31) can reach up to 64 keys past it,
// which the range check turns into zeros.
template <int HD, bool CHECKED, int N>
__device__ __forceinline__ void load_tile(const i32x4& rs, int start, int row_bytes, char* dst,
                                          const int (&off)[N], int wave) {
  const uint32_t woff = (uint32_t)start * (uint32_t)row_bytes;
  // LDS destination: one wave-uniform base (the tile plus this wave's first
  // 1 KiB block) and a constant offset per instruction.
  const uint32_t base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst + wave * 1024;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (CHECKED)
      dma16_at(rs, (int)((uint32_t)off[i] + woff), 0, base, kAttnWaves * i * 1024);
    else
      dma16_at(rs, off[i], (int)woff, base, kAttnWaves * i * 1024);
  }
}

// Zero, in a window's V tile in LDS, the values of keys outside [lo, hi)
// (ring slots outside the valid range may hold anything).
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

// vmcnt(N), then a bare s_barrier: no release fence, so the LDS reads still
// in flight (the next window's first operands, from a buffer that no load
// issued after this barrier touches) need not complete first.  Used where no
// wave has written LDS since the previous barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N, 15));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
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

// Row maximum of a window's scores for this lane's query.
__device__ __forceinline__ float row_max(const f32x16 (&s)[2]) {
  float m = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) m = max3f(m, s[0][r], s[1][r]);
  return max_xor32(m);
}

// Lazy rescale on shifted scores (score minus the running maximum m, which
// the QK product starts from); mx is a window's shifted row maximum.  When
// some row grew past the threshold, every row's m moves up by max(mx, 0), and
// O, the row sum, the window's shifted scores and the QK start value (negm,
// -m in every register) follow.
template <int HB>
__device__ __forceinline__ void maybe_rescale(float mx, f32x16 (&o)[HB], f32x16 (&s)[2],
                                              f32x16& negm, float& m_run, float& l_run) {
  if (__ballot(mx > kRescaleThreshold)) {
    const float dm = fmaxf(mx, 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-dm);
    m_run += dm;
    l_run *= alpha;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[hb][r] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] -= dm;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_run;
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

  // Work-group -> (group, query block).  The work-groups of one group are
  // consecutive logical ids, which xcd_remap places on one XCD: they walk the
  // same keys at about the same time and share them in that XCD's L2.
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = logical / a.qb;
  const int qblk = logical - grp * a.qb;
  const int64_t g_begin = (int64_t)grp * a.total / a.groups;
  const int64_t g_end = (int64_t)(grp + 1) * a.total / a.groups;
  const int H = a.H;
  const float scale_log2 = a.scale_log2;
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // The group's windows [g_begin, g_end) of the launch's window sequence
  // (head-major, then session, then the session's segments), walked as spans:
  // each span is the part of one lane's key segment in the range, and is one
  // piece of its lane.  Only the span position crosses from one span to the
  // next.
  int h = 0, si = 0, wa = 0;
  if (g_begin < g_end) {
    h = (int)(g_begin / a.per_head);
    const int r = (int)(g_begin - (int64_t)h * a.per_head);
#pragma unroll
    for (int i = 1; i < kMaxSessPerLaunch; ++i)
      if (i < a.n_sess && r >= a.s[i].lane0) si = i;
    wa = r - a.s[si].lane0;
  }
#pragma nounroll
  for (int64_t left = g_end - g_begin; left > 0;) {
    const AttnSess& s = a.s[si];
    const int sg = wa < s.nwin[0] ? 0 : (wa < s.nwin[0] + s.nwin[1] ? 1 : 2);
    const int seg_first = sg == 0 ? 0 : (sg == 1 ? s.nwin[0] : s.nwin[0] + s.nwin[1]);
    const int nw = (int)min((int64_t)(seg_first + s.nwin[sg] - wa), left);
    if (qblk < s.n_qblk) {                       // uniform over the work-group
    const int w_begin = wa - seg_first;
    Span sp;
    i32x4 rk, rv;
    if (sg == 2) {
      rk = make_rsrc(s.kt_u + h * s.ku_head, s.ku_bytes);
      rv = make_rsrc(s.vt_u + (int64_t)h * s.npad * HD, s.npad * HD * 2);
      sp.lo = 0;
      sp.hi = s.n_q;
    } else {
      rk = make_rsrc(s.ring_k + (int64_t)h * s.cap * HD, (int)s.cap * HD * 2);
      rv = make_rsrc(s.ring_v + (int64_t)h * s.cap * HD, (int)s.cap * HD * 2);
      sp.lo = sg == 0 ? s.seg_lo[0] : s.seg_lo[1];
      sp.hi = sg == 0 ? s.seg_hi[0] : s.seg_hi[1];
    }
    sp.start0 = (sp.lo & ~15) + w_begin * kAttnWindow;
    sp.nw = nw;
    auto win = [&](int j) { return window_of(sp, j); };
    // Every wave is done with the previous span's tiles before the prologue
    // reloads them.
    __syncthreads();

    // Opaque copies of the wave and lane index: the load offsets and operand
    // addresses the span derives from them are recomputed per span instead of
    // being hoisted out of the span loop and kept live through every span.
    // (The lane index comes from mbcnt, so the work-item id register need
    // not stay live across spans.)
    int wave = wave0, lane;
    __asm__ volatile("" : "+s"(wave));
    __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0"
                     : "=v"(lane));
    const int j32 = lane & 31, g = lane >> 5;
    const int row0 = qblk * kAttnBlockM + wave * kAttnRowsPerWave;
    const bool active = __builtin_amdgcn_readfirstlane(row0 < s.n_q ? 1 : 0) != 0;   // wave-uniform

    // Loop-invariant lane offsets (bytes) of the window loads; krow: the
    // segment's elements from one key to the next.
    const int krow = sg == 2 ? s.ku_stride : HD;
    int koff[T::K_PER_WAVE], voff[T::V_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::K_PER_WAVE; ++i) {
      constexpr int CPR = HD / 8;                   // 16-byte chunks per key row
      const int key = (wave + kAttnWaves * i) * (1024 / (2 * HD)) + lane / CPR;
      koff[i] = (key * krow + ((lane % CPR) ^ kswz<HD>(key)) * 8) * 2;
    }
    const int sigma = (j32 & 3) | (((j32 >> 3) & 3) << 2) | (((j32 >> 2) & 1) << 4);
#pragma unroll
    for (int i = 0; i < T::V_PER_WAVE; ++i) {
      const int b = wave + kAttnWaves * i;
      voff[i] = ((b / T::HB) * 16 * HD + ((b % T::HB) * 32 + sigma) * 16 + g * 8) * 2;
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

    // Prologue: K(0), V(0), K(1), V(1), K(2), V(2), K(3).
    const Window w0 = win(0);
    load_tile<HD, true>(rk, w0.start, krow * 2, kbuf(0), koff, wave);
    load_tile<HD, true>(rv, w0.start, HD * 2, vbuf(0), voff, wave);
#pragma unroll
    for (int t = 1; t < 3; ++t) {
      if (t < nw) {
        load_tile<HD, true>(rk, w0.start + t * kAttnWindow, krow * 2, kbuf(t), koff, wave);
        load_tile<HD, true>(rv, w0.start + t * kAttnWindow, HD * 2, vbuf(t), voff, wave);
      }
    }
    if (nw > 3)
      load_tile<HD, true>(rk, w0.start + 3 * kAttnWindow, krow * 2, kbuf(3), koff, wave);

    // Q^T operand: lane (j, g) holds query row0+j, features 16kc+8g..+7.  The
    // address comes from an opaque copy of the lane index, so that nothing
    // derived from it stays live from one span to the next.
    int lane_q = lane;
    __asm__ volatile("" : "+v"(lane_q));
    const int qrow_q = row0 + (lane_q & 31), g_q = lane_q >> 5;
    bf16x8 qr[T::KC];
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc)
      qr[kc] = qrow_q < s.n_q ? *reinterpret_cast<const bf16x8*>(
                                    s.q + ((int64_t)qrow_q * H + h) * HD + kc * 16 + g_q * 8)
                              : bf16x8{};
    // Q^T pre-scaled by scale * log2(e): scores leave the MFMA in exp2 units.
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[kc][e] = (bf16)((float)qr[kc][e] * scale_log2);

    f32x16 o[T::HB];
#pragma unroll
    for (int hb = 0; hb < T::HB; ++hb) o[hb] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;
    f32x16 sA[2], sB[2];   // shifted scores of two windows (alternate steps)
    f32x16 negm;           // -m_run in every register: the QK product's start value
    // Per step: NQK + NPV MFMA slots; operand reads run D slots ahead in a ring
    // of R registers, and the first D reads of a step are issued at the end of
    // the step before (across its barrier).
    constexpr int NQK = 2 * T::KC;
    constexpr int NPV = 4 * T::HB;
    constexpr int N = NQK + NPV;
    constexpr int D = 3;                  // operand read distance (slots)
    constexpr int R = D + 1;              // operand ring size
    static_assert(N % R == 0, "the ring position of slot 0 repeats every step");
    bf16x8 opr[R];

    wait_loads_and_sync<0>();
    // Window 0's invalid values are zeroed here and published by a barrier of
    // their own (step 0's barrier may be a bare one).
    if (!w0.full) {
      zero_invalid_v<HD>(vbuf(0), w0);
      __syncthreads();
    }
    if (active) {
      sA[0] = sA[1] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sA[kb] = mfma32x32x16(kread(kbuf(0), kb, kc), qr[kc], sA[kb]);
      if (!w0.full) mask_scores(sA, w0);
      m_run = row_max(sA);   // finite: window 0 holds a valid key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[kb][r] -= m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_run;
#pragma unroll
      for (int i = 0; i < D; ++i) opr[i] = kread(kbuf(1), 0, i);
    }

    // Step j: softmax and P*V of window j, scores of window j+1, with the loads
    // of K(j+3), K(j+4) and V(j+2), V(j+3) in flight (four LDS stages each).
    // On entry window j's shifted (and masked) scores are in sA (j even) or sB
    // (j odd), with m_run already updated for them, and the first D operands of
    // QK(j+1) are in the ring.  Steady steps (j + 6 <= nw) touch only full
    // windows, issue every load and wait for a constant count: no branch but the
    // rare rescale.  The last steps (TAIL) handle partial windows and the end
    // of the pipeline.  `stage` = j % 4 and PAR = j % 2 are literals after
    // inlining.
    auto step = [&](const int j, const int stage, const bool TAIL, const bool PAR)
                    __attribute__((always_inline)) {
      f32x16 (&sc)[2] = PAR ? sB : sA;   // window j (its P*V this step)
      f32x16 (&sn)[2] = PAR ? sA : sB;   // window j+1 (its QK this step)
      const int st1 = (stage + 1) & 3, st2 = (stage + 2) & 3, st3 = (stage + 3) & 3;
      // On entry K(j+2) and V(j) must have landed (K(j+2) for the reads that
      // end this step); loads are issued K before V, so the ones that may still
      // be in flight are V(j+1) (step j-2), K(j+3) and V(j+2) (step j-1).
      if (!TAIL) {
        wait_loads_and_barrier<2 * T::V_PER_WAVE + T::K_PER_WAVE>();
        // K(j+4) -> the buffer of K(j) (read by QK(j) in step j-1);
        // V(j+3) -> the buffer of V(j-1) (read by P*V(j-1)).
        load_tile<HD, false>(rk, sp.start0 + (j + 4) * kAttnWindow, krow * 2, kbuf(stage), koff,
                             wave);
        load_tile<HD, false>(rv, sp.start0 + (j + 3) * kAttnWindow, HD * 2, vbuf(st3), voff,
                             wave);
      } else {
        if (j + 3 < nw)
          wait_loads_and_sync<2 * T::V_PER_WAVE + T::K_PER_WAVE>();
        else if (j + 2 < nw)
          wait_loads_and_sync<2 * T::V_PER_WAVE>();
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
        if (j + 4 < nw)
          load_tile<HD, true>(rk, sp.start0 + (j + 4) * kAttnWindow, krow * 2, kbuf(stage), koff,
                              wave);
        if (j + 3 < nw)
          load_tile<HD, true>(rv, sp.start0 + (j + 3) * kAttnWindow, HD * 2, vbuf(st3), voff,
                              wave);
      }
      if (active) {
        // One step is NQK + NPV MFMA slots, issued in this order: the QK
        // product of window j+1 (half kb = 0, then 1; C starts at -m), then
        // the P*V product of window j (16-key chunks c = 0..3).  Each slot
        // issues the LDS read of the operand D slots ahead (a ring of D+1
        // registers), its MFMA, and a share of the softmax VALU work of window
        // j, so that the matrix core and the VALU stay busy together instead of
        // alternating phases:
        //   E(g)    two exp2, one bf16 pack and one row-sum dot2 (group g =
        //           8 kb + 4 c2 + t -> P chunk 2kb + c2, keys 8t'..), each done
        //           before the P*V chunk that needs it;
        //   max     the row maximum of window j+1's scores, after their MFMAs.
        // sched_barrier(0) after each slot keeps this order.
        const char* kl = kbuf(st1);
        const bf16x8* vl = reinterpret_cast<const bf16x8*>(vbuf(stage));
        auto operand = [&](int i) {
          return i < NQK ? kread(kl, i / T::KC, i % T::KC)
                         : vl[((i - NQK) / T::HB * T::HB + (i - NQK) % T::HB) * 64 + lane];
        };
        uint32_t pw[4][4];
        float mxa = kNegInf, mxb = kNegInf;
        // Slot of E group g and of the k-th max op of half kb.
        auto e_slot = [](int g) {
          return T::KC == 8 ? (g < 8 ? 2 * g : 9 + 2 * (g - 8)) : (g < 8 ? g : 5 + (g - 8));
        };
        auto max_slot = [](int kb, int k) {
          return (kb == 0 ? T::KC : NQK) + 3 + (T::KC == 8 ? k : k / 2);
        };
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          // The first wave of a SIMD wins the matrix pipe and runs ahead; it
          // drops its priority for the second half of the step so that the
          // other wave, which sets the step's length, issues first.
          if (i == 0) __builtin_amdgcn_s_setprio(1);
          if (i == N / 2) __builtin_amdgcn_s_setprio(0);
          if (i + D < N) opr[(i + D) % R] = operand(i + D);
          if (i < NQK) {
            const int kb = i / T::KC, kc = i % T::KC;
            sn[kb] = mfma32x32x16(opr[i % R], qr[kc], kc == 0 ? negm : sn[kb]);
          } else {
            const int c = (i - NQK) / T::HB, hb = (i - NQK) % T::HB;
            const u32x4 pv4 = {pw[c][0], pw[c][1], pw[c][2], pw[c][3]};
            o[hb] = mfma32x32x16(opr[i % R], __builtin_bit_cast(bf16x8, pv4), o[hb]);
          }
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            if (e_slot(g) != i) continue;
            const int kb = g >> 3, c2 = (g >> 2) & 1, t = g & 3;
            const float e0 = __builtin_amdgcn_exp2f(sc[kb][c2 * 8 + 2 * t]);
            const float e1 = __builtin_amdgcn_exp2f(sc[kb][c2 * 8 + 2 * t + 1]);
            const uint32_t w2 = pack_bf16(e0, e1);
            pw[kb * 2 + c2][t] = w2;
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2),
                                                    __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                                    l_run, false);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (max_slot(0, k) == i) mxa = max3f(mxa, sn[0][2 * k], sn[0][2 * k + 1]);
            if (max_slot(1, k) == i) mxb = max3f(mxb, sn[1][2 * k], sn[1][2 * k + 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        float mx = max_xor32(fmaxf(mxa, mxb));
        // (C) window j+1: mask a partial window, then the lazy rescale (which
        //     applies to O accumulated through window j).
        if (!TAIL) {
          maybe_rescale<T::HB>(mx, o, sn, negm, m_run, l_run);
        } else if (j + 1 < nw) {
          const Window w1 = win(j + 1);
          if (!w1.full) {
            mask_scores(sn, w1);
            mx = row_max(sn);
          }
          maybe_rescale<T::HB>(mx, o, sn, negm, m_run, l_run);
        }
        // The next step's first D operands, read before its barrier: QK(j+2)
        // reads K(j+2), which landed before this step's barrier and is not
        // reloaded before the next one.
#pragma unroll
        for (int i = 0; i < D; ++i) opr[i] = kread(kbuf(st2), 0, i);
      }
    };

    int j = 0;
    for (; j + 9 <= nw; j += 4) {        // steps j .. j+3 are all steady
      step(j, 0, false, false);
      step(j + 1, 1, false, true);
      step(j + 2, 2, false, false);
      step(j + 3, 3, false, true);
    }
    // j is even here: window j's scores are in sA.
    for (; j + 1 < nw; j += 2) {
      step(j, j & 3, true, false);
      step(j + 1, (j + 1) & 3, true, true);
    }
    if (j < nw) step(j, j & 3, true, false);

    if (active) {
      // The session's output fields are read again here (through an opaque
      // copy of its index) rather than kept in registers through the key
      // loop, and the piece index is computed here.
      int s_e = si;
      __asm__ volatile("" : "+s"(s_e));
      const AttnSess& se = a.s[s_e];
      // (Opaque copies of the divisor keep the division's set-up from being
      // hoisted out of the span loop.)
      int64_t total = a.total;
      int groups = a.groups;
      __asm__ volatile("" : "+s"(total), "+s"(groups));
      const int64_t lane_first = (int64_t)h * a.per_head + se.lane0;
      const int piece =
          piece_of(lane_first, lane_first + wa, se.nwin[0], se.nwin[1], total, groups);
      const bool whole = piece_of(lane_first, lane_first + se.nwin_total - 1, se.nwin[0],
                                  se.nwin[1], total, groups) == 0;
      const float l_tot = sum_xor32(l_run);
      // The output row is recomputed here from an opaque copy of the lane
      // index, so that no address derived from it stays live through the key
      // loop.
      int lane_o = lane;
      __asm__ volatile("" : "+v"(lane_o));
      const int qrow_o = row0 + (lane_o & 31), g_o = lane_o >> 5;
      if (qrow_o < se.n_q) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        // A whole lane: the final O; else this piece's normalised partial
        // (bf16) and its log-sum-exp, merged by the combine kernel.
        bf16* const dst_row =
            whole ? se.o + ((int64_t)qrow_o * H + h) * HD
                  : se.opart + (((int64_t)piece * se.n_q + qrow_o) * H + h) * HD;
#pragma unroll
        for (int hb = 0; hb < T::HB; ++hb) {
          union { bf16x8 v[2]; bf16 b[16]; } u;
#pragma unroll
          for (int r = 0; r < 16; ++r) u.b[r] = (bf16)(o[hb][r] * inv);
          bf16* dst = dst_row + hb * 32 + g_o * 16;
          reinterpret_cast<bf16x8*>(dst)[0] = u.v[0];
          reinterpret_cast<bf16x8*>(dst)[1] = u.v[1];
        }
        if (!whole && g_o == 0)
          se.lse[((int64_t)piece * se.n_q + qrow_o) * H + h] =
              l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
      }
    }
    }  // qblk < n_qblk
    // The next span.
    left -= nw;
    wa += nw;
    if (wa == a.s[si].nwin_total) {
      wa = 0;
      if (++si == a.n_sess) {
        si = 0;
        ++h;
      }
    }
  }
}

// Merge the pieces of the lanes cut into several: O = sum_j w_j o_j /
// sum_j w_j, w_j = 2^(lse_j - max) (o_j: bf16 pieces, each normalised by its
// own row sum).  A lane lying in one piece was written whole by the attention
// kernel and is skipped.  One block per (session, head, 16-row chunk): the
// lane's piece count is computed once per block; one thread per (row, 8
// features), the loads of all pieces of a row in flight together.
template <int HD>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int TPR = HD / 8;              // threads per row
  constexpr int RPP = 256 / TPR;           // rows per pass
  const int item = blockIdx.x;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const CombineSess& s = a.s[si];
  const int chunks = (s.n_q + kCombineRowsPerBlock - 1) / kCombineRowsPerBlock;
  const int local = item - s.item0;
  const int h = local / chunks;
  const int chunk = local - h * chunks;
  const int64_t lane_first = (int64_t)h * a.per_head + s.lane0;
  const int ns = piece_of(lane_first, lane_first + s.nwin_total - 1, s.n0, s.n1, a.total,
                          a.groups) + 1;
  if (ns == 1) return;
  const int64_t stride = (int64_t)s.n_q * a.H;      // (row, head) pairs between pieces
  const int e0 = (threadIdx.x % TPR) * 8;
  const int r_end = min(s.n_q, (chunk + 1) * kCombineRowsPerBlock);
#pragma unroll 1
  for (int r0 = chunk * kCombineRowsPerBlock; r0 < r_end; r0 += RPP) {
    const int row = r0 + threadIdx.x / TPR;
    if (row >= s.n_q) break;
    const int64_t rh = (int64_t)row * a.H + h;
    const float* lse = s.lse + rh;
    const bf16* part = s.opart + rh * HD + e0;
    // One pass in batches of 4 pieces, every load of a batch issued before
    // any is used; the running maximum rescales what is accumulated so far.
    constexpr int B = 4;
    float m = kNegInf, wsum = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ns; k0 += B) {
      float l[B];
      bf16x8 x[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const bool in = k0 + u < ns;
        l[u] = in ? lse[(k0 + u) * stride] : kNegInf;
        x[u] = in ? *reinterpret_cast<const bf16x8*>(part + (k0 + u) * stride * HD) : bf16x8{};
      }
      float bm = l[0];
#pragma unroll
      for (int u = 1; u < B; ++u) bm = fmaxf(bm, l[u]);
      const float m_new = fmaxf(m, bm);
      if (m_new == kNegInf) continue;          // no key so far
      const float c = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m is -inf
      wsum *= c;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= c;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const float w = __builtin_amdgcn_exp2f(l[u] - m_new);
        wsum += w;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] += w * (float)x[u][t];
      }
      m = m_new;
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    bf16x8 out;
#pragma unroll
    for (int t = 0; t < 8; ++t) out[t] = (bf16)(acc[t] * inv);
    *reinterpret_cast<bf16x8*>(s.o + rh * HD + e0) = out;
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int head_dim, hipStream_t st) {
  const int blocks = a.groups * a.qb;
  if (blocks <= 0 || a.total <= 0) return hipSuccess;
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
    hipLaunchKernelGGL(attn_kernel<128>, dim3(blocks), dim3(kAttnThreads), Tiles<128>::LDS_BYTES,
                       st, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(blocks), dim3(kAttnThreads), Tiles<64>::LDS_BYTES,
                       st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(a.items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(a.items), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmd
