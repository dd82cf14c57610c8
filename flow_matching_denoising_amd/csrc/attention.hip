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
// Row permutation of the V^T operand: row rho = [b0 b1 | g | a0 a1] loads
// feature [b0 b1 | a0 a1 | g]; sigma_inv maps a feature back to its row.
__device__ __forceinline__ int sigma_inv(int x) {
  return (x & 3) | (((x >> 4) & 1) << 2) | (((x >> 2) & 3) << 3);
}

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
  static constexpr int PARTS = HD / 8;         // 16-byte parts of one key row
  static constexpr int K_BYTES = kAttnWindow * HD * 2;
  static constexpr int V_BYTES = kAttnWindow * HD * 2;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_CHUNKS = K_BYTES / 16 / kAttnThreads;   // per thread
  static constexpr int V_CHUNKS = V_BYTES / 16 / kAttnThreads;
};

struct Window {
  const bf16* kbase;   // address of key 0 of the window's key space, this head
  int64_t kstride;     // elements between consecutive keys
  const bf16* vbase;   // address of 16-key block 0 of the window's key space
  int start;           // first key index of the window (multiple of 16)
  int lo, hi;          // valid keys [lo, hi)
  bool full;           // every key of the window is valid
};

__device__ __forceinline__ Window make_window(const AttnSess& s, int H, int h, int HD, int w) {
  Window win;
  int seg;
  if (w < s.nwin[0]) {
    seg = 0;
  } else if (w < s.nwin[0] + s.nwin[1]) {
    seg = 1;
    w -= s.nwin[0];
  } else {
    seg = 2;
    w -= s.nwin[0] + s.nwin[1];
  }
  if (seg < 2) {
    const int lo = s.seg_lo[seg];
    win.kbase = s.ring_k + (int64_t)h * s.cap * HD;
    win.kstride = HD;
    win.vbase = s.ring_v + (int64_t)h * (s.cap / 16) * HD * 16;
    win.start = (lo & ~15) + w * kAttnWindow;
    win.lo = lo;
    win.hi = s.seg_hi[seg];
  } else {
    win.kbase = s.k_u + (int64_t)h * HD;
    win.kstride = (int64_t)H * HD;
    win.vbase = s.vt_u + (int64_t)h * (s.npad / 16) * HD * 16;
    win.start = w * kAttnWindow;
    win.lo = 0;
    win.hi = s.n_q;
  }
  win.full = win.start >= win.lo && win.start + kAttnWindow <= win.hi;
  return win;
}

// Global -> registers for one window.
template <int HD>
__device__ __forceinline__ void stage_load(const Window& win, u32x4 (&kr)[Tiles<HD>::K_CHUNKS],
                                           u32x4 (&vr)[Tiles<HD>::V_CHUNKS]) {
  using T = Tiles<HD>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    const int c = tid + kAttnThreads * i;
    const int rho = (c & 7) | (((c >> 6) & 3) << 3);
    const int part = ((c >> 3) & 7) | (HD == 128 ? ((c >> 8) & 1) << 3 : 0);
    const int kb = HD == 128 ? (c >> 9) : (c >> 8);
    const int key = win.start + kb * 32 + perm_k(rho);
    if (win.full || (key >= win.lo && key < win.hi))
      kr[i] = ld16(win.kbase + (int64_t)key * win.kstride + part * 8);
    else
      kr[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < T::V_CHUNKS; ++i) {
    const int c = tid + kAttnThreads * i;
    const int hd_lo = c & 31;
    const int g = (c >> 5) & 1;
    const int hd_hi = HD == 128 ? ((c >> 6) & 3) : ((c >> 6) & 1);
    const int blk = HD == 128 ? (c >> 8) : (c >> 7);
    const int hd = hd_hi * 32 + hd_lo;
    const int key0 = win.start + blk * 16 + g * 8;
    const bf16* src = win.vbase + ((int64_t)(win.start / 16 + blk) * HD + hd) * 16 + g * 8;
    if (win.full || (key0 >= win.lo && key0 + 8 <= win.hi)) {
      vr[i] = ld16(src);
    } else if (key0 + 8 <= win.lo || key0 >= win.hi) {
      vr[i] = u32x4{0u, 0u, 0u, 0u};
    } else {
      union { u32x4 v; unsigned short u[8]; } x;
      x.v = ld16(src);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (key0 + j < win.lo || key0 + j >= win.hi) x.u[j] = 0;
      vr[i] = x.v;
    }
  }
}

// Registers -> LDS, in the MFMA operand order (each 1 KiB block is read by one
// ds_read_b128 of a whole wave, lane (g, row) at (g*32 + row)*16).
template <int HD>
__device__ __forceinline__ void stage_store(char* lds, const u32x4 (&kr)[Tiles<HD>::K_CHUNKS],
                                            const u32x4 (&vr)[Tiles<HD>::V_CHUNKS]) {
  using T = Tiles<HD>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    const int c = tid + kAttnThreads * i;
    const int rho = (c & 7) | (((c >> 6) & 3) << 3);
    const int part = ((c >> 3) & 7) | (HD == 128 ? ((c >> 8) & 1) << 3 : 0);
    const int kb = HD == 128 ? (c >> 9) : (c >> 8);
    const int kc = part >> 1, g = part & 1;
    st16(lds + (((kb * T::KC + kc) * 64 + g * 32 + rho) << 4), kr[i]);
  }
  char* vl = lds + T::K_BYTES;
#pragma unroll
  for (int i = 0; i < T::V_CHUNKS; ++i) {
    const int c = tid + kAttnThreads * i;
    const int hd_lo = c & 31;
    const int g = (c >> 5) & 1;
    const int hb = HD == 128 ? ((c >> 6) & 3) : ((c >> 6) & 1);
    const int blk = HD == 128 ? (c >> 8) : (c >> 7);
    st16(vl + (((blk * T::HB + hb) * 64 + g * 32 + sigma_inv(hd_lo)) << 4), vr[i]);
  }
}

// One 64-key window for one wave (32 query rows).
template <int HD>
__device__ __forceinline__ void window_compute(const char* lds, const Window& win,
                                               const bf16x8 (&qr)[Tiles<HD>::KC],
                                               f32x16 (&o)[Tiles<HD>::HB], float& m_run,
                                               float& l_run, float scale_log2) {
  using T = Tiles<HD>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const bf16x8* kl = reinterpret_cast<const bf16x8*>(lds);
  const bf16x8* vl = reinterpret_cast<const bf16x8*>(lds + T::K_BYTES);

  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      s[kb] = mfma32x32x16(kl[(kb * T::KC + kc) * 64 + lane], qr[kc], s[kb]);
  }

  if (!win.full) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = win.start + kb * 32 + (r >> 3) * 16 + g * 8 + (r & 7);
        if (key < win.lo || key >= win.hi) s[kb][r] = kNegInf;
      }
  }

  // Row maximum of this window (scaled after the max: the scale is positive).
  float m = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, fmaxf(s[0][r], s[1][r]));
  const float mx = max_xor32(m) * scale_log2;
  if (__ballot(mx > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int hb = 0; hb < T::HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[hb][r] *= alpha;
  }

  // p = exp2(s * scale_log2 - m).  S^T registers 8c'..8c'+7 of kb hold keys
  // 32kb + 16c' + 8g .. +7, i.e. the B operand of PV chunk c = 2kb + c'.
  bf16x8 p[4];
  float lsum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = __builtin_amdgcn_exp2f(
          __builtin_fmaf(s[c >> 1][(c & 1) * 8 + j], scale_log2, -m_run));
      lsum += e;
      p[c][j] = (bf16)e;
    }
  }
  l_run += lsum;

#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int hb = 0; hb < T::HB; ++hb)
      o[hb] = mfma32x32x16(vl[(c * T::HB + hb) * 64 + lane], p[c], o[hb]);
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnArgs a) {
  using T = Tiles<HD>;
  __shared__ __attribute__((aligned(16))) char lds[2 * T::BUF_BYTES];

  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const AttnSess& s = a.s[si];
  const int H = a.H;

  // Item order inside a session: (head, split, query block), query block fastest,
  // so the query blocks sharing one key range are adjacent (same XCD).
  int local = item - s.item0;
  const int qblk = local % s.n_qblk;
  local /= s.n_qblk;
  const int split = local % s.nsplit;
  const int h = local / s.nsplit;
  const int w_begin = (int)((int64_t)split * s.nwin_total / s.nsplit);
  const int w_end = (int)((int64_t)(split + 1) * s.nwin_total / s.nsplit);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  const int row0 = qblk * kAttnBlockM + wave * kAttnRowsPerWave;
  const bool active = row0 < s.n_q;
  const int qrow = row0 + j;

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

  u32x4 kr[T::K_CHUNKS], vr[T::V_CHUNKS];
  if (w_begin < w_end) stage_load<HD>(make_window(s, H, h, HD, w_begin), kr, vr);
  for (int w = w_begin; w < w_end; ++w) {
    char* buf = lds + ((w - w_begin) & 1) * T::BUF_BYTES;
    stage_store<HD>(buf, kr, vr);
    __syncthreads();
    const Window win = make_window(s, H, h, HD, w);
    if (w + 1 < w_end) stage_load<HD>(make_window(s, H, h, HD, w + 1), kr, vr);
    if (active) window_compute<HD>(buf, win, qr, o, m_run, l_run, a.scale_log2);
  }

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
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, dim3(a.items), dim3(kAttnThreads), 0, st, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3(a.items), dim3(kAttnThreads), 0, st, a);
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
