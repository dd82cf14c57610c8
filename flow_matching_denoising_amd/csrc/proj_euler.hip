// Velocity projection v = O * W^T on bf16 MFMA, with the rectified-flow Euler
// update z <- z - h * v fused into the epilogue.
//
// One network predicts the velocity of both modalities, and along the linear
// interpolation path that velocity is constant, so an ODE solver integrates
// it in few steps [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配].  The
// velocity network is reduced here to one dense output projection of the
// attention output; sampling runs tau from 1 to 0 with positive step sizes h.
//
// Tile 128 x 128 (rows x output features), k step 64, 4 waves as 2 x 2, each
// wave 64 x 64 = 2 x 2 MFMA 32x32 tiles, fp32 accumulators.  O and W rows are
// both k-contiguous ([n_q][d] and [d_out][d_in]), so both operands are loaded
// with 16-byte lanes.  LDS holds each operand in MFMA operand order (one
// contiguous 1 KiB block per ds_read_b128 of a wave).  Item order inside a
// session: output-feature tile major, row tile minor, so the row tiles that
// share one slab of W are adjacent and run on the same XCD.
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr int BK = 64;
constexpr int OP_BYTES = kProjTile * BK * 2;        // 16 KiB per operand tile
constexpr int BUF_BYTES = 2 * OP_BYTES;
constexpr int CHUNKS = OP_BYTES / 16 / 256;         // 4 per thread per operand

__device__ __forceinline__ void chunk_coords(int c, int& row, int& part) {
  const int rho = (c & 7) | (((c >> 6) & 3) << 3);
  part = (c >> 3) & 7;
  row = (c >> 8) * 32 + rho;
}
__device__ __forceinline__ int lds_offset(int row, int part) {
  return ((((row >> 5) * 4 + (part >> 1)) * 64 + (part & 1) * 32 + (row & 31)) << 4);
}

}  // namespace

__global__ __launch_bounds__(256) void proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF_BYTES];
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
  const int m0 = mt * kProjTile, n0 = nt * kProjTile;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  u32x4 ar[CHUNKS], br[CHUNKS];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      int row, part;
      chunk_coords(tid + 256 * i, row, part);
      const int m = m0 + row, n = n0 + row;
      ar[i] = m < s.n_q ? ld16(s.o + (int64_t)m * d + k0 + part * 8) : u32x4{0u, 0u, 0u, 0u};
      br[i] = n < d ? ld16(a.w + (int64_t)n * d + k0 + part * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](char* buf) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      int row, part;
      chunk_coords(tid + 256 * i, row, part);
      const int off = lds_offset(row, part);
      st16(buf + off, ar[i]);
      st16(buf + OP_BYTES + off, br[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};

  const int nk = d / BK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    char* buf = lds + (kt & 1) * BUF_BYTES;
    store(buf);
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * BK);
    const bf16x8* al = reinterpret_cast<const bf16x8*>(buf);
    const bf16x8* bl = reinterpret_cast<const bf16x8*>(buf + OP_BYTES);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = al[((2 * wm + i) * 4 + kc) * 64 + lane];
        bv[i] = bl[((2 * wn + i) * 4 + kc) * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) acc[i][jn] = mfma32x32x16(av[i], bv[jn], acc[i][jn]);
    }
  }

  // Epilogue: z[m][n] -= h * v[m][n].  C layout: lane (col j, group g),
  // register r -> row 8*(r/4) + 4*g + r%4 of the 32x32 tile.
  const int j = lane & 31, g = lane >> 5;
  const float hstep = s.h;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int n = n0 + (2 * wn + jn) * 32 + j;
      if (n >= d) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (2 * wm + i) * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        if (m < s.n_q) {
          float* zp = s.z + (int64_t)m * d + n;
          *zp = *zp - hstep * acc[i][jn][r];
        }
      }
    }
  }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  hipLaunchKernelGGL(proj_kernel, dim3(a.items), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmd
