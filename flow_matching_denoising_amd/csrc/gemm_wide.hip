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
// A and 2 B operand fragments (1 KiB each) from LDS for 8 MFMAs, 0.75 reads per
// MFMA (the 160 x 128 tile of the W_o projection, one wave per 32 features,
// needs 1.2).  A 928-row unit is 4 row tiles and the 15,360-wide projection 60
// feature tiles: 240 work-groups, one round on 256 CUs.  Operands go global ->
// LDS with MUBUF loads (lds bit), one 1 KiB block (8 rows x 64 k) per wave
// instruction, chunk c of row r stored at chunk position c ^ ((r >> 1) & 7)
// (bank-conflict-free operand reads).  Two LDS stages of 64 KiB: the loads of
// k step t+1 are in flight while k step t is multiplied.  Rows past n_q (or
// past n_out for W) read as zeros through the buffer resources' ranges.
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr int WBM = 256, WBN = 256, WBK = 64;
constexpr int WWAVES = 8;
constexpr int WA_BLOCKS = WBM / 8;                      // 32 blocks of 8 rows x 64 k
constexpr int WB_BLOCKS = WBN / 8;                      // 32
constexpr int WSTAGE_BYTES = (WA_BLOCKS + WB_BLOCKS) * 1024;   // 64 KiB
constexpr int WLOADS = (WA_BLOCKS + WB_BLOCKS) / WWAVES;       // 8 per wave per stage
constexpr int WLDS_BYTES = 2 * WSTAGE_BYTES;                   // 128 KiB
static_assert(WA_BLOCKS % WWAVES == 0, "A blocks split evenly over waves");

__device__ __forceinline__ void wait_all_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0, 15));
  __asm__ volatile("" ::: "memory");
  __syncthreads();
  __asm__ volatile("" ::: "memory");
}

}  // namespace

__global__ __launch_bounds__(WWAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qkv_wide_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const ProjSess& s = a.s[si];
  const int n_q = s.n_q;
  const int d = a.d, n_out = a.n_out;
  const int local = item - s.item0;
  const int m0 = (local % s.n_mtiles) * WBM;
  const int n0 = (local / s.n_mtiles) * WBN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;

  const i32x4 ra = make_rsrc(s.a + (int64_t)m0 * d, min(WBM, n_q - m0) * d * 2);
  const i32x4 rb = make_rsrc(a.w + (int64_t)n0 * d, min(WBN, n_out - n0) * d * 2);

  // Wave w fills 1 KiB blocks w + 8i of a stage: i < 4 -> A blocks, else B.
  // Lane i of a block: row i/8, k chunk (i%8) ^ swizzle(row).
  int voff[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int b = wave + WWAVES * i;
    const int rt = (b % WA_BLOCKS) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rt >> 1) & 7);
    voff[i] = rt * d * 2 + chunk * 16;
  }
  auto load_stage = [&](int kt, int st) __attribute__((always_inline)) {
    char* base = lds + st * WSTAGE_BYTES;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i)
      dma16(i < WA_BLOCKS / WWAVES ? ra : rb, voff[i], kt * WBK * 2,
            base + (wave + WWAVES * i) * 1024);
  };
  // Operand read of row `row` (of the A or B region), 16-k sub-step ks: lane
  // (g, r) wants k chunk 2ks + g.
  auto rd = [&](const char* region, int row, int ks) {
    return *reinterpret_cast<const bf16x8*>(
        region + (row >> 3) * 1024 + (row & 7) * 128 + (((2 * ks + g) ^ ((row >> 1) & 7)) * 16));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = d / WBK;
  load_stage(0, 0);
  wait_all_loads_and_sync();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    // Every wave has finished reading the other stage (barrier at the end of
    // the previous k step): refill it with k step kt+1.
    if (kt + 1 < nk) load_stage(kt + 1, st ^ 1);
    const char* al = lds + st * WSTAGE_BYTES;
    const char* bl = al + WA_BLOCKS * 1024;
    bf16x8 fa[2][4], fb[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = rd(al, wm * 128 + i * 32 + r, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[0][j] = rd(bl, wn * 64 + j * 32 + r, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[cur ^ 1][i] = rd(al, wm * 128 + i * 32 + r, ks + 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[cur ^ 1][j] = rd(bl, wn * 64 + j * 32 + r, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
    }
    // This wave's loads of k step kt+1 have landed; after the barrier every
    // wave's have, and nobody reads stage st any more.
    wait_all_loads_and_sync();
  }

  // Epilogue: column n of the product is column n % d of Q, K_u or V_u.
  // C layout: lane (col r, group g), register q -> row 8*(q/4) + 4*g + q%4.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + r;
    if (n >= n_out) continue;
    const int t = n >= 2 * d ? 2 : (n >= d ? 1 : 0);
    bf16* const oc = s.out[t] + (n - t * d);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * 128 + i * 32 + (q >> 2) * 8 + g * 4 + (q & 3);
        if (m < n_q) oc[(int64_t)m * d] = (bf16)acc[i][j][q];
      }
  }
}

hipError_t launch_qkv_wide(const ProjArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  static const hipError_t attr_err =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&qkv_wide_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, WLDS_BYTES);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(qkv_wide_kernel, dim3(a.items), dim3(WWAVES * 64), WLDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace fmd
