// Projection of the latent to the unit's Q, K_u and V_u on bf16 MFMA, with
// large tiles: [Q | K_u | V_u] = bf16(z) * W_qkv^T, rounded to bf16.
//
// The velocity network is evaluated on the noisy latents of the unit at every
// solver step [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配], so every
// step starts with this projection (n_q x 3d x d: 146 GFLOP for the
// 640x368-class unit).
//
// Tile 256 rows x 256 output features, k step 64, 8 waves (two per SIMD) in a
// 2 x 4 layout: wave (wm, wn) owns rows 128wm..+127 and features 64wn..+63 of
// the tile (4 x 2 MFMA 32x32 accumulators).  Per 16-k sub-step a wave reads 4
// A and 2 B operand fragments (1 KiB each) from LDS for 8 MFMAs.  A 928-row
// unit is 4 row tiles and the 15,360-wide projection 60 feature tiles: 240
// work-groups, one round on 256 CUs; consecutive work-groups (one XCD) take
// the row tiles of one feature tile, so each weight tile is fetched once into
// that XCD's L2 and the small bf16 latent is what every XCD re-reads.
//
// Operands go global -> LDS with MUBUF loads (lds bit), issued by the first
// wave of each SIMD, one 1 KiB block (8 rows x 64 k) per wave instruction, 16-byte chunk c of row r stored at chunk
// position c ^ ((r >> 1) & 7) (bank-conflict-free operand reads).  Two LDS
// stages of 64 KiB: the loads of k step t+1 are in flight while k step t is
// multiplied, one barrier per k step, taken before the step's last 16-k
// sub-step so that the matrix pipe keeps working through it.  Rows past n_q (or past n_out for W)
// read as zeros through the buffer resources' ranges.
//
// The MFMAs take the weight fragment as their first operand, so a lane's
// accumulator registers hold one latent row and runs of 4 consecutive output
// features.  The epilogue stages the bf16 tile in LDS and writes each output
// in the layout its consumer reads, in whole 128-byte lines:
//   Q    [n_q][H][hd]                 (row-major, as the attention reads Q);
//   K_u  [H][npad][hd]                (the K ring's layout);
//   V_u  [H][npad/16][hd][16]         (the V ring's 16-key blocks),
// with npad = n_q rounded up to 16 and the rows n_q..npad-1 of K_u and V_u
// zero (the latent rows past n_q read as zeros, so their products are 0).
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr int WBM = 256, WBN = 256, WBK = 64;
constexpr int WWAVES = 8;
constexpr int WM_WAVES = 2, WN_WAVES = WWAVES / WM_WAVES;      // wave grid over the tile
constexpr int WTM = WBM / WM_WAVES, WTN = WBN / WN_WAVES;       // 128 x 64 per wave
constexpr int WMI = WTM / 32, WNJ = WTN / 32;                   // 4 x 2 accumulators
constexpr int WROWS = 1024 / (WBK * 2);                         // 8 rows per 1 KiB block
constexpr int WA_BLOCKS = WBM / WROWS;                          // 32
constexpr int WB_BLOCKS = WBN / WROWS;                          // 32
constexpr int WSTAGE_BYTES = (WA_BLOCKS + WB_BLOCKS) * 1024;    // 64 KiB
constexpr int WSTAGES = 2;
constexpr int WLOAD_WAVES = 4;                                  // one per SIMD
constexpr int WLOADS = (WA_BLOCKS + WB_BLOCKS) / WLOAD_WAVES;   // 16 per loading wave per stage
constexpr int WLDS_BYTES = WSTAGES * WSTAGE_BYTES;              // 128 KiB
constexpr int WTILE_ROW_BYTES = WBN * 2;                        // epilogue tile row: 512 B
static_assert(WA_BLOCKS % WLOAD_WAVES == 0, "A blocks split evenly over the loading waves");
static_assert(WBM * WTILE_ROW_BYTES <= WLDS_BYTES, "the bf16 tile fits in the stages");

__device__ __forceinline__ int operand_swz(int row) { return (row >> 1) & 7; }

// Epilogue tile: row R holds 512 bytes; the 16-byte chunk of features
// 8c..8c+7 sits at chunk position c ^ (R & 31), and its two 8-byte halves are
// swapped when bit 4 of R is set.  Both make the accumulator writes (32 rows x
// one half per instruction) and the reads below bank-conflict-free.
__device__ __forceinline__ int chunk_off(int row, int chunk) {
  return row * WTILE_ROW_BYTES + ((chunk ^ (row & 31)) << 4);
}
__device__ __forceinline__ int tile_off(int row, int chunk, int half) {
  return chunk_off(row, chunk) + ((half ^ ((row >> 4) & 1)) << 3);
}

}  // namespace

__global__ __launch_bounds__(WWAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qkv_wide_kernel(QkvArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const QkvSess& s = a.s[si];
  const int n_q = s.n_q;
  const int d = a.d, n_out = 3 * a.d;
  const int local = item - s.item0;
  const int m0 = (local % s.n_mtiles) * WBM;
  const int n0 = (local / s.n_mtiles) * WBN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;
  const int wm = wave / WN_WAVES, wn = wave % WN_WAVES;

  const i32x4 ra = make_rsrc(s.zb + (int64_t)m0 * d, min(WBM, n_q - m0) * d * 2);
  const i32x4 rb = make_rsrc(a.w + (int64_t)n0 * d, min(WBN, n_out - n0) * d * 2);

  // The loads come from the first wave of each SIMD (waves 0..3): wave w
  // fills 1 KiB blocks w + 4i of a stage (i < 8 -> A blocks, else B), and the
  // SIMD's other wave only multiplies, so a stall at a load's issue holds up
  // one of the SIMD's two MFMA streams, not both (138 -> 127 us per
  // 640x368-class launch; with the second wave of each SIMD as the loader,
  // 137 against 132 on a slower box).
  // Lane i of a block: row i/8, k chunk (i%8) ^ swizzle(row).
  const int lw = wave & (WLOAD_WAVES - 1);
  int voff[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int b = lw + WLOAD_WAVES * i;
    const int rt = (b % WA_BLOCKS) * WROWS + (lane >> 3);
    const int chunk = (lane & 7) ^ operand_swz(rt);
    voff[i] = rt * d * 2 + chunk * 16;
  }
  auto load_stage = [&](int kt, int st) __attribute__((always_inline)) {
    char* base = lds + st * WSTAGE_BYTES;
    if (wave < WLOAD_WAVES) {
#pragma unroll
      for (int i = 0; i < WLOADS; ++i)
        dma16(i < WA_BLOCKS / WLOAD_WAVES ? ra : rb, voff[i], kt * WBK * 2,
              base + (lw + WLOAD_WAVES * i) * 1024);
    }
  };
  // Operand read of row `row` (of the A or B region), 16-k sub-step ks: lane
  // (g, r) wants k chunk 2ks + g.
  auto rd = [&](const char* region, int row, int ks) {
    return *reinterpret_cast<const bf16x8*>(region + row * (WBK * 2) +
                                            (((2 * ks + g) ^ operand_swz(row)) * 16));
  };

  f32x16 acc[WMI][WNJ];
#pragma unroll
  for (int i = 0; i < WMI; ++i)
#pragma unroll
    for (int j = 0; j < WNJ; ++j) acc[i][j] = f32x16{};

  const int nk = d / WBK;
  auto read_frags = [&](int kt, int ks, bf16x8 (&fa)[WMI], bf16x8 (&fb)[WNJ])
                        __attribute__((always_inline)) {
    const char* al = lds + (kt & 1) * WSTAGE_BYTES;
    const char* bl = al + WA_BLOCKS * 1024;
#pragma unroll
    for (int i = 0; i < WMI; ++i) fa[i] = rd(al, wm * WTM + i * 32 + r, ks);
#pragma unroll
    for (int j = 0; j < WNJ; ++j) fb[j] = rd(bl, wn * WTN + j * 32 + r, ks);
  };
  auto mma = [&](const bf16x8 (&fa)[WMI], const bf16x8 (&fb)[WNJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WMI; ++i)
#pragma unroll
      for (int j = 0; j < WNJ; ++j) acc[i][j] = mfma32x32x16(fb[j], fa[i], acc[i][j]);
  };
  bf16x8 fa[2][WMI], fb[2][WNJ];
  // The four 16-k sub-steps of k step kt; sub-step 3 is preceded by `before_last`.
  auto k_step = [&](int kt, auto&& before_last) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3)
        read_frags(kt, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      else
        before_last();
      mma(fa[ks & 1], fb[ks & 1]);
    }
  };
  load_stage(0, 0);
  wait_loads_and_sync<0>();
  if (nk > 1) load_stage(1, 1);
  read_frags(0, 0, fa[0], fb[0]);
  // Between sub-steps 2 and 3 of k step kt, while their MFMAs run: wait for
  // k step kt+1's loads and the barrier (after which every wave is done with
  // stage kt), refill stage kt with k step kt+2, and read the first fragments
  // of k step kt+1.  (The last k step is peeled off, so the loop body is one
  // straight path.)
  for (int kt = 0; kt + 1 < nk; ++kt)
    k_step(kt, [&] {
      wait_loads_and_sync<0>();
      if (kt + 2 < nk) load_stage(kt + 2, kt & 1);
      read_frags(kt + 1, 0, fa[0], fb[0]);
    });
  k_step(nk - 1, [] {});

  // Epilogue.  Accumulator (i, j), register q of lane (r, g): tile row
  // WTM wm + 32i + r, feature WTN wn + 32j + 8(q/4) + 4g + q%4.
  __syncthreads();   // every wave is done reading the stages
#pragma unroll
  for (int i = 0; i < WMI; ++i)
#pragma unroll
    for (int j = 0; j < WNJ; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row = wm * WTM + i * 32 + r;
        const int chunk = (wn * WTN + j * 32) / 8 + q4;
        union { bf16 b[4]; uint2 u; } w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w.b[e] = (bf16)acc[i][j][q4 * 4 + e];
        *reinterpret_cast<uint2*>(lds + tile_off(row, chunk, g)) = w.u;
      }
  __syncthreads();

  const int hd = a.hd;
  const int npad = s.npad;
  const int nblk = npad / 16;
  // Q and K_u: one thread per (row, 16-byte chunk); a wave writes two rows.
  if (n0 < 2 * d) {
#pragma unroll 4
    for (int idx = threadIdx.x; idx < WBM * (WBN / 8); idx += WWAVES * 64) {
      const int row = idx >> 5, chunk = idx & 31;
      const int n = n0 + chunk * 8;
      const int m = m0 + row;
      if (n >= 2 * d || m >= npad) continue;
      const u32x4 x = ld16(lds + chunk_off(row, chunk));
      const bool flip = (row >> 4) & 1;
      const u32x4 v = flip ? u32x4{x[2], x[3], x[0], x[1]} : x;
      if (n < d) {
        if (m < n_q) st16(s.q + (int64_t)m * d + n, v);
      } else {
        const int f = n - d, h = f / hd, e = f - h * hd;
        st16(s.kt + ((int64_t)h * npad + m) * hd + e, v);
      }
    }
  }
  // V_u: one thread per (16-row block, feature, half of the block's keys);
  // consecutive threads write consecutive 16-byte pieces of a [hd][16] block.
  if (n0 + WBN > 2 * d) {
#pragma unroll 4
    for (int idx = threadIdx.x; idx < (WBM / 16) * WBN * 2; idx += WWAVES * 64) {
      const int half = idx & 1, f = (idx >> 1) & (WBN - 1), b = idx >> 9;
      const int n = n0 + f;
      if (n < 2 * d || n >= n_out || m0 + b * 16 >= npad) continue;
      union { bf16 e[8]; u32x4 v; } u;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = b * 16 + half * 8 + t;
        u.e[t] = *reinterpret_cast<const bf16*>(lds + tile_off(row, f >> 3, (f >> 2) & 1) +
                                                (f & 3) * 2);
      }
      const int fv = n - 2 * d, h = fv / hd, e = fv - h * hd;
      st16(s.vt + (((int64_t)h * nblk + (m0 >> 4) + b) * hd + e) * 16 + half * 8, u.v);
    }
  }
}

hipError_t launch_qkv_wide(const QkvArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  static const hipError_t attr_err =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&qkv_wide_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, WLDS_BYTES);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(qkv_wide_kernel, dim3(a.items), dim3(WWAVES * 64), WLDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace fmd
