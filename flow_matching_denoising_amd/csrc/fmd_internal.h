// Internal declarations shared by the HIP sources of libfmd (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/fmd.h"

namespace fmd {

// Sessions whose descriptors travel by value in one launch's kernel arguments
// (kept well under the 4 KiB kernel-argument limit).  Calls with more sessions
// are issued as several launches.
constexpr int kMaxSessPerLaunch = 16;
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs x 32 CUs, round-robin dispatch
constexpr int kTargetCUs = 256;     // split heuristics assume a full MI355X

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Map a hardware block id to a logical work id so that each XCD runs a
// contiguous range of logical ids (blocks are dispatched to XCDs round-robin).
// Work that shares data is then placed at adjacent logical ids and lands in
// the same XCD's L2 at about the same time.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = (n + kNumXcd - 1) / kNumXcd;
  const int tall = n % kNumXcd == 0 ? kNumXcd : n % kNumXcd;
  const int xcd = bid % kNumXcd;
  const int local = bid / kNumXcd;
  return xcd < tall ? xcd * per + local
                    : tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// The same with the non-temporal hint (data streamed once).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Global -> LDS loads through buffer resources (MUBUF loads with the lds bit).
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

// Buffer resource over [base, base + bytes): a lane whose range-checked offset
// falls at or past `bytes` reads zeros instead of faulting.
__device__ __forceinline__ i32x4 make_rsrc(const bf16* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));   // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);                                   // num_records
  r.w = kRsrcWord3;
  return r;
}

// One wave instruction: 16 bytes per lane from rs at voff + soff to
// dst + 16*lane (dst wave-uniform; voff range-checked, soff not).  Issued
// from inline assembly on purpose: it has no register outputs, and the
// compiler, which cannot tell one LDS stage buffer from another, would
// otherwise make every LDS read wait for every LDS load in flight.  Callers
// order these loads themselves: s_waitcnt vmcnt(N) and a barrier before any
// wave reads a tile (wait_loads_and_sync), a barrier between the last read of
// a buffer and the next load into it.  One wait state separates the M0 write
// from the load that reads it.  The compiler treats M0 as reserved and does
// not honour it in a clobber list; these kernels leave M0 to these helpers
// alone (a build check asserts that no compiler-generated instruction reads
// or writes it).
__device__ __forceinline__ void dma16(const i32x4& rs, int voff, int soff, char* dst) {
  const uint32_t m0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst;
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :
                   : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
                   : "memory", "m0");
}

// The same with the LDS destination given as a wave-uniform base plus an
// offset, added in the instruction sequence itself (s_add_u32 into M0): the
// compiler then keeps one base register instead of one per destination.
__device__ __forceinline__ void dma16_at(const i32x4& rs, int voff, int soff, uint32_t lds_base,
                                         uint32_t lds_off) {
  __asm__ volatile(
      "s_add_u32 m0, %0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
      :
      : "s"(lds_base), "s"(lds_off), "v"(voff), "s"(rs), "s"(soff)
      : "memory", "m0", "scc");
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14,
// expcnt (left at its maximum, 7) in bits 6:4, lgkmcnt in bits 11:8.
constexpr int vmcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// s_barrier with no fence of its own: the caller has already waited (with
// s_waitcnt) for whatever the other waves must see.
__device__ __forceinline__ void bare_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Wait until at most N of this wave's loads are outstanding, then barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N, 15));   // vmcnt(N); lgkmcnt unconstrained
  __asm__ volatile("" ::: "memory");
  __syncthreads();
  __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Launch descriptors (passed by value).
// ---------------------------------------------------------------------------

struct AppendSess {
  const bf16* ks;   // [T][H][hd]
  const bf16* vs;
  bf16* ck;         // [H][cap][hd]
  bf16* cv;         // [H][cap/16][hd][16]
  int64_t cap;
  int32_t T;
  int32_t head0;    // slot of the slice's first token
  int32_t blk0;     // first 16-slot block touched
  int32_t nblk;     // blocks touched (<= cap/16)
  int32_t item0;    // first work item of this session
  int32_t pad_;
};
struct AppendArgs {
  AppendSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t items;
};

constexpr int kVtBlocks = 4;   // 16-token blocks per work-group of the unit K/V staging

struct VtSess {
  const bf16* k;    // [n][H][hd]   the unit's keys
  const bf16* v;    // [n][H][hd]   the unit's values
  bf16* kt;         // [H][npad][hd]           keys, head-major, zero past n (nullptr: values only)
  bf16* vt;         // [H][npad/16][hd][16]   values, 16-key blocks, zero past n
  int32_t n;
  int32_t nblk;     // npad/16
  int32_t item0;    // first work-group: H * ceil(nblk / kVtBlocks) per session
  int32_t pad_;
};
struct VtArgs {
  VtSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t items;
};

struct AttnSess {
  const bf16* q;      // [n_q][H][hd]
  const bf16* kt_u;   // the unit's keys: [H][npad][hd] (a staged copy) or [n_q][H][hd] (as given)
  const bf16* vt_u;   // [H][npad/16][hd][16]   (workspace copy of the unit's values)
  int64_t ku_head;    // elements from one head's unit keys to the next's (npad*hd or hd)
  int32_t ku_stride;  // elements from one unit key to the next (hd or H*hd)
  int32_t ku_bytes;   // bytes of one head's unit keys from its first (its buffer range)
  const bf16* ring_k; // [H][cap][hd]
  const bf16* ring_v; // [H][cap/16][hd][16]
  bf16* o;            // [n_q][H][hd]            (lanes that lie in one group)
  bf16* opart;        // [npart][n_q][H][hd]     (pieces of lanes cut by group ends)
  float* lse;         // [npart][n_q][H]
  int64_t cap;
  int32_t n_q;
  int32_t npad;       // n_q rounded up to 16
  int32_t seg_lo[2];  // valid ring slots: [seg_lo[i], seg_hi[i])
  int32_t seg_hi[2];
  int32_t nwin[3];    // 64-key windows over ring seg 0, ring seg 1, unit keys
  int32_t nwin_total; // nwin[0] + nwin[1] + nwin[2]: the windows of one lane
  int32_t n_qblk;
  int32_t lane0;      // first window of this session among one head's windows
};
// The windows of a launch form one sequence: head-major, then session (lane =
// (head, session), windows [lane0, lane0 + nwin_total) of the head's
// per_head windows), then the session's segments in order.  The sequence is
// cut into `groups` equal contiguous ranges; group g covers
// [g*total/groups, (g+1)*total/groups) with `qb` work-groups, one per 256-row
// query block, that walk the range together as spans (piece_of).
struct AttnArgs {
  AttnSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t per_head;   // windows of one head over all sessions of the launch
  int32_t groups;
  int32_t qb;         // work-groups per group (the largest n_qblk)
  int64_t total;      // H * per_head
  float scale_log2;   // log2(e) / sqrt(head_dim)
};

// The group holding window x of a launch's window sequence (the largest g
// with g*total/groups <= x), and the first window of group g.  Host and
// device use these definitions.
__host__ __device__ __forceinline__ int group_of(int64_t x, int64_t total, int groups) {
  return (int)(((x + 1) * groups - 1) / total);
}
__host__ __device__ __forceinline__ int64_t group_start(int g, int64_t total, int groups) {
  return (int64_t)g * total / groups;
}

// A lane's pieces: its windows [first, first + nwin_total) cut at every group
// start inside it and at the starts of its second and third key segment
// (first + n0 and first + n0 + n1, when the segment before is non-empty).
// Returns the index of the piece holding window x (the number of distinct
// cuts in (first, x]); a lane with piece_of(first, last) == 0 is one piece.
__host__ __device__ inline int piece_of(int64_t first, int64_t x, int n0, int n1, int64_t total,
                                        int groups) {
  int k = group_of(x, total, groups) - group_of(first, total, groups);
  const int64_t cuts[2] = {n0 > 0 ? first + n0 : -1, n1 > 0 ? first + n0 + n1 : -1};
  for (int t = 0; t < 2; ++t) {
    const int64_t c = cuts[t];
    if (c > first && c <= x && group_start(group_of(c, total, groups), total, groups) != c) ++k;
  }
  return k;
}

constexpr int kCombineRowsPerBlock = 16;   // rows of one lane per combine block

struct CombineSess {
  const bf16* opart;
  const float* lse;
  bf16* o;
  int32_t n_q;
  int32_t nwin_total;
  int32_t lane0;
  int32_t n0, n1;     // windows of the ring segments (the lane's cuts)
  int32_t item0;      // first block of this session: H * ceil(n_q / 16) blocks
};
struct CombineArgs {
  CombineSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t per_head;
  int32_t groups;
  int64_t total;
  int32_t items;      // blocks
};

// Projection GEMM  Y = A * W^T  (A [n_q][d] bf16, W [n_out][d] bf16 =
// [d_out][d_in], fp32 accumulation, n_out = d), with one of three epilogues:
//   kProjEuler: z <- z - h * Y (fp32, in place), and, if zb is set,
//               zb <- bf16(z) (the next step's projection input);
//   kProjLayer: a layer of a stack adds its update to the fp32 residual
//               r <- r + Y and writes zb <- bf16(z + r), the next layer's input;
//   kProjLayerLast: the stack's last layer: z <- z - h * (r + Y), r <- 0,
//               and, if zb is set, zb <- bf16(z).
// With splits > 1 the k range is cut into `splits` equal parts: work-group
// (tile, split j) writes its fp32 partial product to part[j] ([splits][n_q][d]
// per session), and launch_proj_reduce sums the parts in order j = 0, 1, ...
// and applies the epilogue.  Used when the tiles alone would leave most CUs
// idle (small units).
constexpr int kProjEuler = 0;
constexpr int kProjLayer = 2;
constexpr int kProjLayerLast = 3;

struct ProjSess {
  const bf16* a;      // [n_q][d]
  float* z;           // [n_q][d]
  bf16* zb;           // [n_q][d] or nullptr
  float* r;           // kProjLayer*: [n_q][d] residual
  float* part;        // splits > 1: [splits][n_q][d] fp32 partial products
  int32_t n_q;
  int32_t n_mtiles;
  int32_t item0;      // first work-group: n_mtiles * n-tiles * splits per session
  float h;
};
struct ProjArgs {
  ProjSess s[kMaxSessPerLaunch];
  const bf16* w;      // [n_out][d], [d_out][d_in]
  int32_t n_sess;
  int32_t d;
  int32_t n_out;
  int32_t items;
  int32_t splits;     // k-range parts (1: the epilogue runs in the GEMM)
  int32_t chain;      // splits > 1, kProjEuler: the sessions are `chain`
                      // solver steps of n_sess / chain latents, step-major;
                      // the reduce applies them in step order (0, 1: none)
};

// Q/K/V projection of the latent: [Q | K_u | V_u] = bf16(zb * W_qkv^T)
// (W_qkv [3d][d]), each output written in the layout the attention reads:
// Q [n_q][H][hd], K_u [H][npad][hd], V_u [H][npad/16][hd][16] (rows n_q..npad-1
// of K_u and V_u zero).  256 x 256 tiles; n_mtiles counts 256-row tiles.
struct QkvSess {
  const bf16* zb;     // [n_q][d]
  bf16* q;
  bf16* kt;
  bf16* vt;
  int32_t n_q;
  int32_t npad;       // n_q rounded up to 16
  int32_t n_mtiles;
  int32_t item0;
};
struct QkvArgs {
  QkvSess s[kMaxSessPerLaunch];
  const bf16* w;      // [3d][d]
  int32_t n_sess;
  int32_t d;
  int32_t hd;
  int32_t items;
};

// bf16 copy of the latent: zb = bf16(z), [n_q][d] per session.
struct CvtSess {
  const float* z;
  bf16* zb;
  float* r;           // if set, cleared to 0 (a layer stack's residual)
  int64_t n;          // elements (n_q * d), a multiple of 8
  int64_t item0;      // first 8-element group of this session
};
struct CvtArgs {
  CvtSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int64_t items;      // 8-element groups in total
};

// Classifier-free-guided mix of a unit's two attention outputs, in place into
// the conditional one: oc = bf16((1 - g) ou + g oc), [n_q][d] per unit.
struct MixSess {
  bf16* oc;
  const bf16* ou;
  float g;
  int64_t n;          // elements (n_q * d), a multiple of 8
  int64_t item0;      // first 8-element group of this unit
};
struct MixArgs {
  MixSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int64_t items;
};

// Host-side launchers (defined next to their kernels).
hipError_t launch_append(const AppendArgs& a, int head_dim, hipStream_t st);
hipError_t launch_vt(const VtArgs& a, int head_dim, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, int head_dim, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t st);
hipError_t launch_proj(const ProjArgs& a, int mode, hipStream_t st);
// The sum of the split parts and the epilogue of `mode`, 4 elements per thread.
hipError_t launch_proj_reduce(const ProjArgs& a, int mode, hipStream_t st);
hipError_t launch_cvt(const CvtArgs& a, hipStream_t st);
hipError_t launch_mix(const MixArgs& a, hipStream_t st);
hipError_t launch_qkv_wide(const QkvArgs& a, hipStream_t st);

// Attention tiling shared by host planning and the kernel.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kAttnRowsPerWave = 32;
constexpr int kAttnBlockM = kAttnWaves * kAttnRowsPerWave;   // 256 query rows per block
constexpr int kAttnWindow = 64;                              // keys per window

// Projection tiling: 160 rows x 128 output features per block.
constexpr int kProjTile = 160;
constexpr int kProjTileN = 128;
constexpr int kProjBK = 64;
// k-range parts of a projection launch with `tiles` output tiles and nk k
// steps, when the tiles fill less than half of the chip: as many parts as fit
// the chip, at most kProjMaxSplits and at least two k steps each.  Every part
// writes an fp32 copy of the output for the reduce to read back, so filling
// the chip does not pay: on the 192x336-class unit (24 tiles, 24 k steps) 4
// parts take 14.4 us with the reduce, 10 parts (240 work-groups) 15.4, 3
// parts 14.7 and 2 parts 15.8.
constexpr int kProjMaxSplits = 4;
inline int proj_splits(int64_t tiles, int nk) {
  if (tiles <= 0 || tiles * 2 >= kTargetCUs) return 1;
  const int64_t want = std::min<int64_t>(kTargetCUs / tiles, kProjMaxSplits);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, nk / 2));
}
// Q/K/V projection tiling: 256 rows x 256 output features per block.
constexpr int kQkvTile = 256;

}  // namespace fmd
