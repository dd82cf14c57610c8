// Ring append of the thinker's K/V slice, and the staging of the unit's own
// keys and values in the ring's layouts.
//
// The performer writes each incoming K/V slice into its preallocated local
// cache at the slice's position, before the solver runs [Wan-Streamer v0.2:
// Higher Resolution, Same Latency (nanless digest), 方法概述和架构;
// Wan-Streamer v0.2 (zhao9797 blog), Infra].  Token t of a slice goes to ring
// slot (head + t) mod cap of every head.
//
// Layouts: K ring [H][cap][hd]; V ring in 16-slot blocks stored feature-major,
// [H][cap/16][hd][16], so that the attention kernel reads V with keys
// contiguous (the contraction axis of P*V) without transposing per step.  One
// work-group handles one (session, head, 16-slot block): it copies the K rows
// of the block's written slots directly (16-byte lanes), stages the V rows in
// LDS and writes the block back transposed with 16-byte stores.  A block that
// is only partly covered by the slice keeps its other slots (read-merge-write
// of the same 16 bytes by the same thread; blocks are never shared between
// work-groups, also when T == cap and the slice wraps onto its own first block).
// The slice is read once and the written blocks are not read again by this
// launch, so the global loads and stores carry the non-temporal hint
// (streaming cache policy); on the 8-session batch that moves 69 % of 8 TB/s
// against 60 % with the default policy.
#include "fmd_internal.h"

namespace fmd {

template <int HD>
__global__ __launch_bounds__(2 * HD) void append_kernel(AppendArgs a) {
  constexpr int PARTS = HD / 8;  // 16-byte parts of one token row
  __shared__ __attribute__((aligned(16))) bf16 tile[16][HD + 8];

  const int item = blockIdx.x;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const AppendSess& s = a.s[si];

  const int local = item - s.item0;
  const int h = local / s.nblk;
  const int bi = local % s.nblk;
  const int64_t nb_ring = s.cap / 16;
  int64_t pb = s.blk0 + bi;                          // physical block
  if (pb >= nb_ring) pb -= nb_ring;
  const int H = a.H;

  // Load phase: thread -> (slot r of the block, 16-byte part).
  {
    const int r = threadIdx.x / PARTS;
    const int part = threadIdx.x % PARTS;
    const int64_t p = pb * 16 + r;
    int64_t tt = p - s.head0;                    // token index: (p - head0) mod cap
    if (tt < 0) tt += s.cap;
    if (tt < s.T) {
      const int64_t src = (tt * H + h) * HD + part * 8;
      st16_nt(s.ck + ((int64_t)h * s.cap + p) * HD + part * 8, ld16_nt(s.ks + src));
      st16(&tile[r][part * 8], ld16_nt(s.vs + src));
    }
  }
  __syncthreads();

  // Store phase: thread -> (feature e, half hh of the block's 16 slots).
  {
    const int e = threadIdx.x >> 1;
    const int hh = threadIdx.x & 1;
    bf16* dst = s.cv + (((int64_t)h * nb_ring + pb) * HD + e) * 16 + hh * 8;
    unsigned written = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t p = pb * 16 + hh * 8 + i;
      int64_t tt = p - s.head0;
      if (tt < 0) tt += s.cap;
      written |= (tt < s.T ? 1u : 0u) << i;
    }
    if (written == 0) return;
    union { u32x4 v; bf16 b[8]; } u;
    if (written != 0xFFu) u.v = ld16(dst);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (written & (1u << i)) u.b[i] = tile[hh * 8 + i][e];
    st16_nt(dst, u.v);
  }
}

// The unit's own keys and values, staged in the ring's layouts so that the
// attention kernel streams every key segment the same way:
//   keys   [n][H][hd] -> [H][npad][hd]          (skipped when kt is null: the
//                                               attention then reads the keys
//                                               where they are)
//   values [n][H][hd] -> [H][npad/16][hd][16]
// (npad = n rounded up to 16; rows past n are zero).  One work-group per
// (session, head, kVtBlocks 16-token blocks); every load of a thread is
// issued before its first store.  The staged copies carry the non-temporal
// hint: a unit stages every step's values up front, and the attention of a
// later step reads them long after other traffic has passed through the
// caches (8.6 -> 8.0 us for one step's 928x40x128 values).
template <int HD>
__global__ __launch_bounds__(256) void vt_kernel(VtArgs a) {
  constexpr int PARTS = HD / 8;            // 16-byte parts of one token row
  constexpr int ROWS = 256 / PARTS;        // token rows per pass
  constexpr int TOK = kVtBlocks * 16;      // tokens per work-group
  constexpr int PASSES = TOK / ROWS;
  __shared__ __attribute__((aligned(16))) bf16 tile[TOK][HD + 8];

  const int item = blockIdx.x;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSessPerLaunch; ++i)
    if (i < a.n_sess && item >= a.s[i].item0) si = i;
  const VtSess& s = a.s[si];
  const int local = item - s.item0;
  const int nchunk = (s.nblk + kVtBlocks - 1) / kVtBlocks;
  const int h = local / nchunk;
  const int blk0 = (local - h * nchunk) * kVtBlocks;
  const int nb = min(kVtBlocks, s.nblk - blk0);
  const int H = a.H;
  const int part = threadIdx.x % PARTS;
  const bool keys = s.kt != nullptr;       // uniform: stage the keys as well as the values
  u32x4 kx[PASSES], vx[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int tok = blk0 * 16 + p * ROWS + threadIdx.x / PARTS;
    kx[p] = vx[p] = u32x4{0u, 0u, 0u, 0u};
    if (tok < s.n) {
      if (keys) kx[p] = ld16(s.k + ((int64_t)tok * H + h) * HD + part * 8);
      vx[p] = ld16(s.v + ((int64_t)tok * H + h) * HD + part * 8);
    }
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = p * ROWS + threadIdx.x / PARTS;
    if (r < nb * 16) {
      if (keys) st16(s.kt + ((int64_t)h * s.nblk * 16 + blk0 * 16 + r) * HD + part * 8, kx[p]);
      st16(&tile[r][part * 8], vx[p]);
    }
  }
  __syncthreads();
  // Values: 16-byte chunks (8 keys of one feature) of the nb blocks.
  for (int idx = threadIdx.x; idx < nb * HD * 2; idx += 256) {
    const int b = idx / (HD * 2), e = (idx >> 1) % HD, hh = idx & 1;
    union { u32x4 v; bf16 b[8]; } u;
#pragma unroll
    for (int i = 0; i < 8; ++i) u.b[i] = tile[b * 16 + hh * 8 + i][e];
    st16_nt(s.vt + (((int64_t)h * s.nblk + blk0 + b) * HD + e) * 16 + hh * 8, u.v);
  }
}

hipError_t launch_append(const AppendArgs& a, int head_dim, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, dim3(a.items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<64>, dim3(a.items), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_vt(const VtArgs& a, int head_dim, hipStream_t st) {
  if (a.items <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(vt_kernel<128>, dim3(a.items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(vt_kernel<64>, dim3(a.items), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmd
