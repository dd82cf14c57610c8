// Velocity projection v = O * W^T on bf16 MFMA, with the rectified-flow Euler
// update z <- z - h * v fused into the epilogue (or, in a layer stack, the
// residual update of one layer).
//
// One network predicts the velocity of both modalities, and along the linear
// interpolation path that velocity is constant, so an ODE solver integrates
// it in few steps [Wan-Streamer (gongshangzheng blog), 3.4 条件流匹配].  The
// velocity network is reduced here to one dense output projection of the
// attention output; sampling runs tau from 1 to 0 with positive step sizes h.
//
// Tile 160 rows x 128 output features, k step 64, 4 waves (one per SIMD);
// wave w owns output features 32w..32w+31 of the tile for all 160 rows (five
// MFMA 32x32 accumulators).  160-row tiles split a 928-row unit into 6 row
// tiles, so a 5120-wide projection is 240 work-groups: one balanced round on
// 256 CUs (256-row tiles would leave 96 CUs idle).  O and W rows are both
// k-contiguous ([n_q][d] and [d_out][d_in]).  Operands go global -> LDS with
// MUBUF loads (lds bit), one 1 KiB block (8 rows x 64 k) per wave
// instruction, each row read whole (128 contiguous bytes).  Inside a block,
// the 16-byte chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7),
// which keeps the ds_read_b128 operand reads (16 lanes = 16 rows of one
// chunk per LDS cycle) free of bank conflicts.  The buffer resources cover
// exactly the tile's valid rows, so rows past n_q (or past d for W) read as
// zeros.  Four LDS stages (144 KiB) keep three k steps of loads in flight:
// the operands come mostly from other work-groups' misses in L2 and the
// Infinity Cache, so the bytes a CU has in flight, not the L2 bandwidth,
// set its load rate.
// Item order inside a session: k part major, then output-feature tile, then
// row tile, so the row tiles that share one slab of W are adjacent and run on
// the same XCD.  With k parts (small units), each work-group multiplies one
// part of the k range and stores its fp32 partial tile; proj_reduce_kernel
// sums the parts in a fixed order and applies the epilogue.
#include "fmd_internal.h"

namespace fmd {

namespace {

constexpr int BM = kProjTile;                       // 160 rows
constexpr int BN = kProjTileN;                      // 128 output features
constexpr int BK = kProjBK;
constexpr int WAVES = 4;
constexpr int MT = BM / 32;                         // 5 row tiles of 32
constexpr int STAGES = 4;
constexpr int A_BLOCKS = BM / 8;                    // 20 blocks of 8 rows x 64 k
constexpr int B_BLOCKS = BN / 8;                    // 16
constexpr int STAGE_BYTES = (A_BLOCKS + B_BLOCKS) * 1024;
constexpr int LOADS_PER_WAVE = (A_BLOCKS + B_BLOCKS) / WAVES;   // 9
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;     // 144 KiB
static_assert(A_BLOCKS % WAVES == 0 && B_BLOCKS % WAVES == 0, "loads must split evenly over waves");
static_assert(BN == 32 * WAVES, "one 32-feature column tile per wave");
static_assert((STAGES & (STAGES - 1)) == 0, "the stage index wraps with a mask");

}  // namespace

constexpr int kProjPartial = -1;   // epilogue: store the fp32 partial tile

template <int MODE>
__global__ __launch_bounds__(WAVES * 64) void proj_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int item = xcd_remap(blockIdx.x, a.items);
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const ProjSess& s = a.s[si];
  // Session fields are read once (stores to z could otherwise force reloads).
  float* const z = s.z;
  const int n_q = s.n_q;
  const float hstep = s.h;
  const int d = a.d;
  const int ntn = (a.n_out + BN - 1) / BN;
  const int tiles = s.n_mtiles * ntn;
  const int local = item - s.item0;
  const int part = local / tiles;
  const int tl = local - part * tiles;
  const int mt = tl % s.n_mtiles;
  const int nt = tl / s.n_mtiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;

  // The tile's rows of O and W; rows past n_q (past d) read as zeros.
  const int n_out = a.n_out;
  const i32x4 ra = make_rsrc(s.a + (int64_t)m0 * d, min(BM, n_q - m0) * d * 2);
  const i32x4 rb = make_rsrc(a.w + (int64_t)n0 * d, min(BN, n_out - n0) * d * 2);

  // Loop-invariant lane offsets (bytes): wave w fills 1 KiB blocks w, w+4, ...
  // (blocks 0..19: A, 20..35: B); block b holds 8 consecutive rows of its
  // operand, lane i -> row i/8, k chunk (i%8) ^ swizzle(row).
  int voff[LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) {
    const int b = wave + WAVES * i;
    const int rt = (i < A_BLOCKS / WAVES ? b : b - A_BLOCKS) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((rt >> 1) & 7);
    voff[i] = rt * d * 2 + chunk * 16;
  }
  const int nk_all = d / BK;
  const int kb = part * nk_all / a.splits;
  const int nk = (part + 1) * nk_all / a.splits - kb;      // this work-group's k steps
  auto load_stage = [&](int kt, int st) __attribute__((always_inline)) {
    kt += kb;
    char* base = lds + st * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      // Blocks wave + 4i: i < 5 are A blocks for every wave.
      dma16(i < A_BLOCKS / WAVES ? ra : rb, voff[i], kt * BK * 2,
            base + (wave + WAVES * i) * 1024);
    }
  };
  // Operand reads: lane (g, r) of a 32-row tile wants row r, k chunk 2kc+g;
  // byte offset within the tile (tile bases are compile-time immediates).
  int roff[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    roff[kc] = (r >> 3) * 1024 + ((r & 7) * 8 + ((2 * kc + g) ^ ((r >> 1) & 7))) * 16;

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16{};
  // Pipeline: four LDS stages, k step t in buffer t % 4.  The barrier that
  // publishes k step t+1 sits DA slots before the end of k step t, right
  // after every wave has issued its last read of buffer t: the reads of
  // k step t+1's first operands then overlap the last MFMAs of k step t, and
  // the DMA of k step t+4 (into buffer t % 4) is issued after that barrier.
  // MFMA slot sl = kc*MT + i multiplies A fragment (kc, i) by B fragment kc;
  // every slot issues the read of the A fragment DA slots ahead (and the B
  // fragment of a k chunk that starts there), continuing into the next k step.
  constexpr int NS = 4 * MT;            // slots per k step
  constexpr int DA = 3, RA = 4;         // A read distance and ring size
  static_assert(NS % RA == 0 && NS / MT % 2 == 0 && DA < MT, "operand rings");
  auto aread = [&](const char* al, int sl) {
    return *reinterpret_cast<const bf16x8*>(al + (sl % MT) * 4096 + roff[sl / MT]);
  };
  auto bread = [&](const char* al, int kc) {
    return *reinterpret_cast<const bf16x8*>(al + A_BLOCKS * 1024 + wave * 4096 + roff[kc]);
  };
  load_stage(0, 0);
  if (nk > 1) load_stage(1, 1);
  if (nk > 2) load_stage(2, 2);
  if (nk > 3) load_stage(3, 3);
  if (nk > 3)
    wait_loads_and_sync<3 * LOADS_PER_WAVE>();
  else if (nk > 2)
    wait_loads_and_sync<2 * LOADS_PER_WAVE>();
  else if (nk > 1)
    wait_loads_and_sync<LOADS_PER_WAVE>();
  else
    wait_loads_and_sync<0>();
  bf16x8 ar[RA], br[2];
  br[0] = bread(lds, 0);
#pragma unroll
  for (int sl = 0; sl < DA; ++sl) ar[sl % RA] = aread(lds, sl);
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int stn = (st + 1) & (STAGES - 1);    // buffer of k step kt+1
    const char* al = lds + st * STAGE_BYTES;
    const char* aln = lds + stn * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      if (sl == NS - DA && more) {
        // This wave's reads of buffer st are all issued; wait for them and
        // for k step kt+1's DMA (k steps kt+2 and kt+3 may stay in flight),
        // then barrier.
        if (kt + 3 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS_PER_WAVE, 0));
        else if (kt + 2 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS_PER_WAVE, 0));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0, 0));
        __asm__ volatile("" ::: "memory");
        __syncthreads();
        __asm__ volatile("" ::: "memory");
        if (kt + 4 < nk) load_stage(kt + 4, st);
      }
      const int nx = sl + DA;
      if (nx < NS) {
        ar[nx % RA] = aread(al, nx);
        if (nx % MT == 0) br[(nx / MT) & 1] = bread(al, nx / MT);
      } else if (more) {
        ar[nx % RA] = aread(aln, nx - NS);
        if ((nx - NS) % MT == 0) br[((nx - NS) / MT) & 1] = bread(aln, (nx - NS) / MT);
      }
      acc[sl % MT] = mfma32x32x16(ar[sl % RA], br[(sl / MT) & 1], acc[sl % MT]);
      __builtin_amdgcn_sched_barrier(0);
    }
    st = stn;
  }

  // Epilogue.  C layout: lane (col r, group g), register q -> row
  // 8*(q/4) + 4*g + q%4 of the 32x32 tile.
  const int n = n0 + wave * 32 + r;
  if (n >= n_out) return;
  const bool full = m0 + BM <= n_q;                // uniform
  // Every z (and r) value of the lane's 160 rows is loaded before the first
  // store: the stores to z could alias later loads as far as the compiler
  // knows, so loads issued per row tile would wait out the memory latency
  // once per tile.
  auto row = [&](int i, int q) { return m0 + i * 32 + (q >> 2) * 8 + g * 4 + (q & 3); };
  if constexpr (MODE == kProjPartial) {
    float* const pc = s.part + (int64_t)part * n_q * d + n;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (full || row(i, q) < n_q) pc[(int64_t)row(i, q) * d] = acc[i][q];
  } else if constexpr (MODE == kProjEuler) {
    // z[m][n] -= h * y[m][n] (and zb = bf16(z)).
    float* const zc = z + n;
    bf16* const zbc = s.zb ? s.zb + n : nullptr;
    float zv[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        zv[i][q] = (full || row(i, q) < n_q) ? zc[(int64_t)row(i, q) * d] : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = row(i, q);
        if (full || m < n_q) {
          const float zn = zv[i][q] - hstep * acc[i][q];
          zc[(int64_t)m * d] = zn;
          if (zbc) zbc[(int64_t)m * d] = (bf16)zn;
        }
      }
  } else if constexpr (MODE == kProjLayer || MODE == kProjLayerLast) {
    // Residual stream of a layer stack (see kProjLayer / kProjLayerLast).
    float* const zc = z + n;
    float* const rc = s.r + n;
    bf16* const zbc = s.zb ? s.zb + n : nullptr;
    float zv[MT][16], rv[MT][16];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const bool in = full || row(i, q) < n_q;
        zv[i][q] = in ? zc[(int64_t)row(i, q) * d] : 0.f;
        rv[i][q] = in ? rc[(int64_t)row(i, q) * d] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = row(i, q);
        if (full || m < n_q) {
          const float rn = rv[i][q] + acc[i][q];
          if constexpr (MODE == kProjLayer) {
            rc[(int64_t)m * d] = rn;
            if (zbc) zbc[(int64_t)m * d] = (bf16)(zv[i][q] + rn);
          } else {
            const float zn = zv[i][q] - hstep * rn;
            zc[(int64_t)m * d] = zn;
            rc[(int64_t)m * d] = 0.f;
            if (zbc) zbc[(int64_t)m * d] = (bf16)zn;
          }
        }
      }
  }
}

// zb = bf16(z) (round to nearest even), 8 elements per thread.
__global__ __launch_bounds__(256) void cvt_kernel(CvtArgs a) {
  const int64_t grp = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (grp >= a.items) return;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && grp >= a.s[i].item0) si = i;
  const CvtSess& s = a.s[si];
  const int64_t e = (grp - s.item0) * 8;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(s.z + e);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(s.z + e + 4);
  bf16x8 y;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    y[t] = (bf16)x0[t];
    y[4 + t] = (bf16)x1[t];
  }
  *reinterpret_cast<bf16x8*>(s.zb + e) = y;
  if (s.r) {
    *reinterpret_cast<f32x4*>(s.r + e) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(s.r + e + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The guided velocity v_u + g (v_c - v_u) of two branches that share W_o is
// ((1 - g) O_u + g O_c) W_o^T, so the branches are mixed before the one
// projection.  (1 - g) ou + g oc keeps g = 1 and g = 0 exact.
__global__ __launch_bounds__(256) void mix_kernel(MixArgs a) {
  const int64_t grp = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (grp >= a.items) return;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && grp >= a.s[i].item0) si = i;
  const MixSess& s = a.s[si];
  const int64_t e = (grp - s.item0) * 8;
  const bf16x8 c = *reinterpret_cast<const bf16x8*>(s.oc + e);
  const bf16x8 u = *reinterpret_cast<const bf16x8*>(s.ou + e);
  const float g = s.g, g1 = 1.f - s.g;
  bf16x8 y;
#pragma unroll
  for (int t = 0; t < 8; ++t) y[t] = (bf16)fmaf(g, (float)c[t], g1 * (float)u[t]);
  *reinterpret_cast<bf16x8*>(s.oc + e) = y;
}

// The split projection's second half: y = part[0] + part[1] + ... (in that
// order), then the epilogue of MODE on 4 consecutive elements per thread.
template <int MODE>
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjArgs a) {
  // Element E of the launch: sessions' [n_q][d] outputs back to back.
  const int64_t E = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int d = a.d;
  int si = -1;
  int64_t base = 0, e = 0;
#pragma unroll
  for (int i = 0; i < kMaxSessPerLaunch; ++i) {
    if (i < a.n_sess) {
      const int64_t ne_i = (int64_t)a.s[i].n_q * d;
      if (si < 0 && E < base + ne_i) {
        si = i;
        e = E - base;       // row * d + feature within session i
      }
      base += ne_i;
    }
  }
  if (si < 0) return;
  const ProjSess& s = a.s[si];
  const int64_t ne = (int64_t)s.n_q * d;
  const float* const pp = s.part + e;
  f32x4 y = *reinterpret_cast<const f32x4*>(pp);
  // Parts 1, 2, ... added in order, their loads issued four at a time.
  for (int j0 = 1; j0 < a.splits; j0 += 4) {
    f32x4 p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      p[u] = j0 + u < a.splits ? *reinterpret_cast<const f32x4*>(pp + (j0 + u) * ne)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + u < a.splits)
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] += p[u][t];
  }
  f32x4 zv = *reinterpret_cast<const f32x4*>(s.z + e);
  if constexpr (MODE == kProjEuler) {
#pragma unroll
    for (int t = 0; t < 4; ++t) zv[t] = zv[t] - s.h * y[t];
    *reinterpret_cast<f32x4*>(s.z + e) = zv;
  } else {
    f32x4 rv = *reinterpret_cast<const f32x4*>(s.r + e);
#pragma unroll
    for (int t = 0; t < 4; ++t) rv[t] += y[t];
    if constexpr (MODE == kProjLayer) {
      *reinterpret_cast<f32x4*>(s.r + e) = rv;
#pragma unroll
      for (int t = 0; t < 4; ++t) zv[t] += rv[t];   // the next layer's input z + r
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) zv[t] = zv[t] - s.h * rv[t];
      *reinterpret_cast<f32x4*>(s.z + e) = zv;
      *reinterpret_cast<f32x4*>(s.r + e) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (s.zb) {
    union { bf16 b[4]; uint2 u; } o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o.b[t] = (bf16)zv[t];
    *reinterpret_cast<uint2*>(s.zb + e) = o.u;
  }
}

hipError_t launch_proj(const ProjArgs& a, int mode, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  static const hipError_t attr_err = [] {
    const void* fns[] = {reinterpret_cast<const void*>(&proj_kernel<kProjEuler>),
                         reinterpret_cast<const void*>(&proj_kernel<kProjLayer>),
                         reinterpret_cast<const void*>(&proj_kernel<kProjLayerLast>),
                         reinterpret_cast<const void*>(&proj_kernel<kProjPartial>)};
    hipError_t e = hipSuccess;
    for (const void* f : fns)
      if (e == hipSuccess)
        e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    return e;
  }();
  if (attr_err != hipSuccess) return attr_err;
  const dim3 grid(a.items), block(WAVES * 64);
  if (a.splits > 1) mode = kProjPartial;
  switch (mode) {
    case kProjPartial:
      hipLaunchKernelGGL(proj_kernel<kProjPartial>, grid, block, LDS_BYTES, st, a);
      break;
    case kProjEuler: hipLaunchKernelGGL(proj_kernel<kProjEuler>, grid, block, LDS_BYTES, st, a); break;
    case kProjLayer: hipLaunchKernelGGL(proj_kernel<kProjLayer>, grid, block, LDS_BYTES, st, a); break;
    case kProjLayerLast:
      hipLaunchKernelGGL(proj_kernel<kProjLayerLast>, grid, block, LDS_BYTES, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_proj_reduce(const ProjArgs& a, int mode, hipStream_t st) {
  if (a.items <= 0 || a.splits <= 1) return hipSuccess;
  int64_t rows = 0;   // one thread per 4 elements of the sessions' outputs
  for (int i = 0; i < a.n_sess; ++i) rows += a.s[i].n_q;
  const int64_t threads = rows * a.d / 4;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  switch (mode) {
    case kProjEuler: hipLaunchKernelGGL(proj_reduce_kernel<kProjEuler>, grid, block, 0, st, a); break;
    case kProjLayer: hipLaunchKernelGGL(proj_reduce_kernel<kProjLayer>, grid, block, 0, st, a); break;
    case kProjLayerLast:
      hipLaunchKernelGGL(proj_reduce_kernel<kProjLayerLast>, grid, block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cvt(const CvtArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  hipLaunchKernelGGL(cvt_kernel, dim3((unsigned)((a.items + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_mix(const MixArgs& a, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  hipLaunchKernelGGL(mix_kernel, dim3((unsigned)((a.items + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmd
