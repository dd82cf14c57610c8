// Velocity projection v = O * W^T on bf16 MFMA, with the rectified-flow Euler
// update z <- z - h * v fused into the epilogue.
//
// One network predicts the velocity of both modalities, and along the linear
// interpolation path that velocity is constant, so an ODE solver integrates
// it in few steps [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配].  The
// velocity network is reduced here to one dense output projection of the
// attention output; sampling runs tau from 1 to 0 with positive step sizes h.
//
// Tile 256 rows x 128 output features, k step 64, 8 waves as 4 x 2, each wave
// 64 x 64 = 2 x 2 MFMA 32x32 tiles, fp32 accumulators.  Large tiles keep the
// L2->CU traffic near 47 B/clk per CU at full MFMA rate.  O and W rows are both
// k-contiguous ([n_q][d] and [d_out][d_in]).  Operands go global -> LDS with
// global_load_lds_dwordx4, one 1 KiB block (8 rows x 64 k) per wave
// instruction, each row read whole (128 contiguous bytes): gathering the MFMA
// operand order directly (32 rows x 32 bytes per instruction) runs at about a
// third of the L2 bandwidth.  Inside a block, the 16-byte chunk c of row r is
// stored at chunk position c ^ ((r >> 1) & 7), which keeps the ds_read_b128
// operand reads (16 lanes = 16 rows of one chunk per LDS cycle) free of bank
// conflicts; the per-lane read offsets are loop-invariant.  Three LDS stages
// (144 KiB) keep two k steps of loads in flight.  Item order inside a session:
// output-feature tile major, row tile minor, so the row tiles that share one
// slab of W are adjacent and run on the same XCD.
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr int BM = kProjTile;                       // 256 rows
constexpr int BN = kProjTileN;                      // 128 output features
constexpr int BK = 64;
constexpr int WAVES = 8;
constexpr int STAGES = 3;
constexpr int A_BLOCKS = (BM / 32) * (BK / 16);     // 32 operand blocks of 1 KiB
constexpr int B_BLOCKS = (BN / 32) * (BK / 16);     // 16
constexpr int STAGE_BYTES = (A_BLOCKS + B_BLOCKS) * 1024;
constexpr int LOADS_PER_WAVE = (A_BLOCKS + B_BLOCKS) / WAVES;   // 6
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;     // 144 KiB

template <int N>
__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);   // vmcnt(N); expcnt/lgkmcnt unconstrained
  __asm__ volatile("" ::: "memory");
  __syncthreads();
  __asm__ volatile("" ::: "memory");
}

}  // namespace

__global__ __launch_bounds__(WAVES * 64) void proj_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const ProjSess& s = a.s[si];
  const int d = a.d;
  const int local = item - s.item0;
  const int mt = local % s.n_mtiles;
  const int nt = local / s.n_mtiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;        // 4 x 2 waves of 64 x 64
  const int r = lane & 31, g = lane >> 5;

  // Loop-invariant load sources: wave w fills 1 KiB blocks w, w+8, ... (blocks
  // 0..31: A = O rows, 32..47: B = W rows; block b holds 8 consecutive rows of
  // its operand, lane i -> row i/8, k chunk (i%8) ^ swizzle(row)).  Rows past
  // n_q (O) or d (W) are clamped to the last row: computed, never stored.
  const bf16* src[LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) {
    const int b = wave + WAVES * i;
    const int rib = lane >> 3;                       // row within the block
    if (b < A_BLOCKS) {
      const int rt = b * 8 + rib;                    // row within the A tile
      const int chunk = (lane & 7) ^ ((rt >> 1) & 7);
      const int row = min(m0 + rt, s.n_q - 1);
      src[i] = s.o + (int64_t)row * d + chunk * 8;
    } else {
      const int rt = (b - A_BLOCKS) * 8 + rib;       // row within the B tile
      const int chunk = (lane & 7) ^ ((rt >> 1) & 7);
      const int row = min(n0 + rt, d - 1);           // d may be an odd multiple of 64
      src[i] = a.w + (int64_t)row * d + chunk * 8;
    }
  }
  auto load_stage = [&](int kt, int st) {
    char* base = lds + st * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i)
      __builtin_amdgcn_global_load_lds(src[i] + kt * BK, base + (wave + WAVES * i) * 1024, 16, 0,
                                       0);
  };
  // Operand reads: lane (g, r) of a 32-row tile wants row r, k chunk 2kc+g;
  // byte offset within the tile (tile bases are compile-time immediates).
  int roff[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    roff[kc] = (r >> 3) * 1024 + ((r & 7) * 8 + ((2 * kc + g) ^ ((r >> 1) & 7))) * 16;

  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  const int nk = d / BK;
  load_stage(0, 0);
  if (nk > 1) load_stage(1, 1);
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk)
      wait_loads_and_sync<LOADS_PER_WAVE>();    // k step kt landed; kt+1 may be in flight
    else
      wait_loads_and_sync<0>();
    const int st2 = st == 0 ? 2 : st - 1;       // (kt+2) % 3: the buffer of k step kt-1
    if (kt + 2 < nk) load_stage(kt + 2, st2);
    const char* al = lds + st * STAGE_BYTES;
    const char* bl = al + A_BLOCKS * 1024;
    bf16x8 av[4][2], bv[4][2];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[kc][i] = *reinterpret_cast<const bf16x8*>(al + (2 * wm + i) * 4096 + roff[kc]);
        bv[kc][i] = *reinterpret_cast<const bf16x8*>(bl + (2 * wn + i) * 4096 + roff[kc]);
      }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = mfma32x32x16(av[kc][i], bv[kc][jn], acc[i][jn]);
    st = st == 2 ? 0 : st + 1;
  }

  // Epilogue: z[m][n] -= h * v[m][n].  C layout: lane (col r, group g),
  // register q -> row 8*(q/4) + 4*g + q%4 of the 32x32 tile.
  const float hstep = s.h;
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
    const int n = n0 + (2 * wn + jn) * 32 + r;
    if (n >= d) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + (2 * wm + i) * 32 + (q >> 2) * 8 + g * 4 + (q & 3);
        if (m < s.n_q) {
          float* zp = s.z + (int64_t)m * d + n;
          *zp = *zp - hstep * acc[i][jn][q];
        }
      }
    }
  }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&proj_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      LDS_BYTES);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(proj_kernel, dim3(a.items), dim3(WAVES * 64), LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace fmd
