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
// Tile 160 rows x 128 output features, k step 64, eight waves in two roles.
// Four MFMA waves (one per SIMD): wave w owns output features 32w..32w+31 of
// the tile for all 160 rows (five MFMA 32x32 accumulators) and only reads
// its operands from LDS.  Four DMA waves (one per SIMD) issue every global
// load and finish the epilogue: with one MFMA wave per SIMD, a wave that also
// issued the operand loads would stall its MFMA stream at each load issue,
// with nothing else on the SIMD to fill the gap.  160-row tiles split a
// 928-row unit into 6 row tiles, so a 5120-wide projection is 240
// work-groups: one balanced round on 256 CUs (256-row tiles would leave 96
// CUs idle).  O and W rows are both k-contiguous ([n_q][d] and
// [d_out][d_in]).  Operands go global -> LDS with MUBUF loads (lds bit), one
// 1 KiB block (8 rows x 64 k) per wave instruction, each row read whole (128
// contiguous bytes).  Inside a block, the 16-byte chunk c of row r is stored
// at chunk position c ^ ((r >> 1) & 7), which keeps the ds_read_b128 operand
// reads (16 lanes = 16 rows of one chunk per LDS cycle) free of bank
// conflicts.  The buffer resources cover exactly the tile's valid rows, so
// rows past n_q (or past d for W) read as zeros.  Four LDS stages (144 KiB)
// keep three k steps of loads in flight.
// Epilogue: the z (and residual) values of the tile are loaded by the DMA
// waves in chunks spread over the k loop, into registers laid out like the
// MFMA waves' accumulators, so that neither their latency nor a burst of
// every work-group reading them at once falls at the end; after the loop the
// MFMA waves hand their accumulators over through LDS and the DMA waves apply
// the update and store.
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
constexpr int WAVES = 4;                            // MFMA waves, one per SIMD
constexpr int DWAVES = 4;                           // DMA waves, one per SIMD
constexpr int THREADS = (WAVES + DWAVES) * 64;
constexpr int MT = BM / 32;                         // 5 row tiles of 32
constexpr int STAGES = 4;
constexpr int A_BLOCKS = BM / 8;                    // 20 blocks of 8 rows x 64 k
constexpr int B_BLOCKS = BN / 8;                    // 16
constexpr int STAGE_BYTES = (A_BLOCKS + B_BLOCKS) * 1024;
constexpr int LOADS_PER_WAVE = (A_BLOCKS + B_BLOCKS) / DWAVES;   // 9
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;     // 144 KiB
constexpr int ACC_WAVE_BYTES = MT * 16 * 64 * 4;    // one MFMA wave's accumulators
static_assert(A_BLOCKS % DWAVES == 0 && B_BLOCKS % DWAVES == 0, "loads must split evenly over waves");
static_assert(BN == 32 * WAVES, "one 32-feature column tile per wave");
static_assert(WAVES * ACC_WAVE_BYTES <= LDS_BYTES, "the accumulator hand-over fits in LDS");
static_assert((STAGES & (STAGES - 1)) == 0, "the stage index wraps with a mask");
// Epilogue chunk c (16 values per lane: row tile c of z, then row tile c - MT
// of the residual) is loaded in k step kZ0 + kZStep * c, after that step's
// operand loads; chunks issued in the three previous k steps are still in
// flight at a k step's wait, which counts them.
constexpr int kZ0 = 4, kZStep = 6, kZLoads = 16;

}  // namespace

constexpr int kProjPartial = -1;   // epilogue: store the fp32 partial tile

template <int MODE>
__global__ __launch_bounds__(THREADS) void proj_kernel(ProjArgs a) {
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
  const int n_out = a.n_out;
  const int nk_all = d / BK;
  const int kb = part * nk_all / a.splits;
  const int nk = (part + 1) * nk_all / a.splits - kb;      // this work-group's k steps
  const bool full = m0 + BM <= n_q;                // uniform
  // C layout of a 32x32 accumulator: lane (col r, group g), register q ->
  // row 8*(q/4) + 4*g + q%4 of the tile; row tile i starts at row m0 + 32i.
  auto row = [&](int i, int q) { return m0 + i * 32 + (q >> 2) * 8 + g * 4 + (q & 3); };
  // Where MFMA wave w's accumulator registers 4j..4j+3 of row tile i go for
  // the hand-over (lane-contiguous 16-byte slots).
  auto acc_slot = [&](int w, int i, int j) {
    return lds + w * ACC_WAVE_BYTES + ((i * 4 + j) * 64 + lane) * 16;
  };
  constexpr bool kHandOver = MODE != kProjPartial;

  if (wave >= WAVES) {
    // ---- DMA wave dw: operand loads, epilogue loads and the epilogue. ----
    const int dw = wave - WAVES;
    // The tile's rows of O and W; rows past n_q (past d) read as zeros.
    const i32x4 ra = make_rsrc(s.a + (int64_t)m0 * d, min(BM, n_q - m0) * d * 2);
    const i32x4 rb = make_rsrc(a.w + (int64_t)n0 * d, min(BN, n_out - n0) * d * 2);
    // Loop-invariant lane offsets (bytes): wave dw fills 1 KiB blocks dw,
    // dw+4, ... (blocks 0..19: A, 20..35: B); block b holds 8 consecutive
    // rows of its operand, lane i -> row i/8, k chunk (i%8) ^ swizzle(row).
    int voff[LOADS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int b = dw + DWAVES * i;
      const int rt = (i < A_BLOCKS / DWAVES ? b : b - A_BLOCKS) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ ((rt >> 1) & 7);
      voff[i] = rt * d * 2 + chunk * 16;
    }
    auto load_stage = [&](int kt, int st) __attribute__((always_inline)) {
      kt += kb;
      char* base = lds + st * STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < LOADS_PER_WAVE; ++i)
        dma16(i < A_BLOCKS / DWAVES ? ra : rb, voff[i], kt * BK * 2,
              base + (dw + DWAVES * i) * 1024);
    };
    // Epilogue inputs of column n (MFMA wave dw's lane layout): z, and for a
    // layer the residual.  Buffer loads over the tile's valid rows: every
    // chunk issues exactly kZLoads loads whatever the row and column bounds,
    // which the k loop's wait counts rely on (out-of-range lanes read zeros
    // or values that are never stored).
    constexpr int NZ = MODE == kProjEuler ? MT : (kHandOver ? 2 * MT : 0);
    const int n = n0 + dw * 32 + r;
    const int rows_here = min(BM, n_q - m0);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc(z + (int64_t)m0 * d, 0, rows_here * d * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (MODE == kProjLayer || MODE == kProjLayerLast) ? s.r + (int64_t)m0 * d : z, 0,
        rows_here * d * 4, kRsrcWord3);
    float ev[NZ > 0 ? NZ : 1][16];
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
      const int i = c < MT ? c : c - MT;
#pragma unroll
      for (int q = 0; q < kZLoads; ++q)
        ev[c][q] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(c < MT ? rz : rr,
                                                        ((row(i, q) - m0) * d + n) * 4, 0, 0));
    };
    const bool spread = NZ > 0 && kZ0 + kZStep * (NZ - 1) + 8 <= nk;

    load_stage(0, 0);
    if (nk > 1) load_stage(1, 1);
    if (nk > 2) load_stage(2, 2);
    if (nk > 3) load_stage(3, 3);
    if (nk > 3)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LOADS_PER_WAVE, 15));
    else if (nk > 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS_PER_WAVE, 15));
    else if (nk > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS_PER_WAVE, 15));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0, 15));
    bare_barrier();                                // k step 0 has landed
    for (int kt = 0; kt + 1 < nk; ++kt) {
      // k step kt+1 must have landed before the MFMA waves pass the barrier
      // that ends their reads of k step kt's buffer; that buffer then takes
      // k step kt+4.  Loads issued after k step kt+1's: k steps kt+2 and
      // kt+3, and an epilogue chunk if one went out in k steps kt-3..kt-1
      // (never in the last three waits: the last chunk goes out at least
      // eight k steps before the end).
      const int t = kt - kZ0;
      const bool recent = spread && t >= 1 && t <= kZStep * (NZ - 1) + 3 && t % kZStep >= 1 &&
                          t % kZStep <= 3;
      if (kt + 3 < nk) {
        if (recent)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS_PER_WAVE + kZLoads, 15));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS_PER_WAVE, 15));
      } else if (kt + 2 < nk) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS_PER_WAVE, 15));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0, 15));
      }
      bare_barrier();
      if (kt + 4 < nk) load_stage(kt + 4, kt & (STAGES - 1));
      if (spread) {
#pragma unroll
        for (int c = 0; c < NZ; ++c)
          if (kt == kZ0 + kZStep * c) load_chunk(c);
      }
    }
    if constexpr (kHandOver) {
      if (!spread) {
#pragma unroll
        for (int c = 0; c < NZ; ++c) load_chunk(c);
      }
      bare_barrier();                              // the MFMA waves are done with the operands
      bare_barrier();                              // their accumulators are in LDS
      float* const zc = z + n;
      bf16* const zbc = s.zb ? s.zb + n : nullptr;
      float* const rc = (MODE == kProjLayer || MODE == kProjLayerLast) ? s.r + n : nullptr;
      const bool col_in = n < n_out;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        f32x4 y4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y4[j] = *reinterpret_cast<const f32x4*>(acc_slot(dw, i, j));
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = row(i, q);
          if (!(col_in && (full || m < n_q))) continue;
          const float y = y4[q >> 2][q & 3];
          if constexpr (MODE == kProjEuler) {
            // z[m][n] -= h * y[m][n] (and zb = bf16(z)).
            const float zn = ev[i][q] - hstep * y;
            zc[(int64_t)m * d] = zn;
            if (zbc) zbc[(int64_t)m * d] = (bf16)zn;
          } else if constexpr (MODE == kProjLayer) {
            // Residual stream of a layer stack (see kProjLayer).
            const float rn = ev[MT + i][q] + y;
            rc[(int64_t)m * d] = rn;
            if (zbc) zbc[(int64_t)m * d] = (bf16)(ev[i][q] + rn);
          } else {
            // The stack's last layer (see kProjLayerLast).
            const float zn = ev[i][q] - hstep * (ev[MT + i][q] + y);
            zc[(int64_t)m * d] = zn;
            rc[(int64_t)m * d] = 0.f;
            if (zbc) zbc[(int64_t)m * d] = (bf16)zn;
          }
        }
      }
    }
    return;
  }

  // ---- MFMA wave. ----
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
  // after every MFMA wave has issued its last read of buffer t: the reads of
  // k step t+1's first operands then overlap the last MFMAs of k step t, and
  // the DMA waves load k step t+4 into buffer t % 4 after that barrier.
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
  bare_barrier();                                  // k step 0 has landed
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
        // This wave's reads of buffer st are all issued; wait for them, then
        // barrier (the DMA waves have waited for k step kt+1's loads).
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(63, 0));
        bare_barrier();
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

  if constexpr (MODE == kProjPartial) {
    const int n = n0 + wave * 32 + r;
    if (n >= n_out) return;
    float* const pc = s.part + (int64_t)part * n_q * d + n;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (full || row(i, q) < n_q) pc[(int64_t)row(i, q) * d] = acc[i][q];
  } else {
    // Hand the accumulators to the DMA waves once every MFMA wave is done
    // reading operands.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63, 0));
    bare_barrier();
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(acc_slot(wave, i, j)) =
            f32x4{acc[i][4 * j], acc[i][4 * j + 1], acc[i][4 * j + 2], acc[i][4 * j + 3]};
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63, 0));
    bare_barrier();
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

// y = part[0] + part[1] + ... (in that order) at element offset e of one
// session's [splits][n_q][d] partials (ne = n_q * d).
__device__ __forceinline__ f32x4 sum_parts(const float* pp, int64_t ne, int splits) {
  f32x4 y = *reinterpret_cast<const f32x4*>(pp);
  // Parts 1, 2, ... added in order, their loads issued four at a time.
  for (int j0 = 1; j0 < splits; j0 += 4) {
    f32x4 p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      p[u] = j0 + u < splits ? *reinterpret_cast<const f32x4*>(pp + (j0 + u) * ne)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + u < splits)
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] += p[u][t];
  }
  return y;
}

// The split projection's second half: y = part[0] + part[1] + ... (in that
// order), then the epilogue of MODE on 4 consecutive elements per thread.
// With chain > 1 (Euler mode) the launch's sessions are `chain` consecutive
// solver steps of the same latents, step-major (session b * nc + i is step b
// of latent i, nc = n_sess / chain): each thread applies the steps' updates
// z <- z - h_b * y_b to its elements in step order.
template <int MODE>
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjArgs a) {
  // Element E of the launch: the first nc sessions' [n_q][d] outputs back to back.
  const int64_t E = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int d = a.d;
  const int chain = a.chain > 1 ? a.chain : 1;
  const int nc = a.n_sess / chain;
  int si = -1;
  int64_t base = 0, e = 0;
#pragma unroll
  for (int i = 0; i < kMaxSessPerLaunch; ++i) {
    if (i < nc) {
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
  f32x4 zv = *reinterpret_cast<const f32x4*>(s.z + e);
  if constexpr (MODE == kProjEuler) {
    for (int b = 0; b < chain; ++b) {
      const ProjSess& sb = a.s[b * nc + si];
      const f32x4 y = sum_parts(sb.part + e, ne, a.splits);
#pragma unroll
      for (int t = 0; t < 4; ++t) zv[t] = zv[t] - sb.h * y[t];
    }
    *reinterpret_cast<f32x4*>(s.z + e) = zv;
  } else {
    const f32x4 y = sum_parts(s.part + e, ne, a.splits);
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
  const dim3 grid(a.items), block(THREADS);
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
  if (a.chain > 1 && (mode != kProjEuler || a.n_sess % a.chain != 0)) return hipErrorInvalidValue;
  const int nc = a.chain > 1 ? a.n_sess / a.chain : a.n_sess;
  int64_t rows = 0;   // one thread per 4 elements of the (first nc) sessions' outputs
  for (int i = 0; i < nc; ++i) rows += a.s[i].n_q;
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
