// Internal declarations shared by the HIP sources of libfmd (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

struct VtSess {
  const bf16* k;    // [n][H][hd]   the unit's keys
  const bf16* v;    // [n][H][hd]   the unit's values
  bf16* kt;         // [H][npad][hd]           keys, head-major, zero past n
  bf16* vt;         // [H][npad/16][hd][16]   values, 16-key blocks, zero past n
  int32_t n;
  int32_t nblk;     // npad/16
  int32_t item0;
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
  const bf16* kt_u;   // [H][npad][hd]           (workspace copy of the unit's keys)
  const bf16* vt_u;   // [H][npad/16][hd][16]   (workspace copy of the unit's values)
  const bf16* ring_k; // [H][cap][hd]
  const bf16* ring_v; // [H][cap/16][hd][16]
  bf16* o;            // [n_q][H][hd]            (when nsplit == 1)
  bf16* opart;        // [nsplit][n_q][H][hd]    (when nsplit > 1)
  float* lse;         // [nsplit][n_q][H]
  int64_t cap;
  int32_t n_q;
  int32_t npad;       // n_q rounded up to 16
  int32_t seg_lo[2];  // valid ring slots: [seg_lo[i], seg_hi[i])
  int32_t seg_hi[2];
  int32_t nwin[3];    // 64-key windows over ring seg 0, ring seg 1, unit keys
  int32_t split0[4];  // key splits of segment t: [split0[t], split0[t+1]); split0[3] = nsplit
  int32_t n_qblk;
  int32_t nsplit;
  int32_t hoff;       // first item of this session among one head's items
};
// Items are numbered head-major over all sessions of the launch: head h's
// items are [h * per_head, (h + 1) * per_head), and inside them session i
// takes [hoff, hoff + nsplit * n_qblk) (hoff increasing with i).  Every XCD's
// contiguous range of items then holds the same mix of sessions.
struct AttnArgs {
  AttnSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t per_head;   // items per head, all sessions
  int32_t items;      // H * per_head
  float scale_log2;   // log2(e) / sqrt(head_dim)
};

struct CombineSess {
  const bf16* opart;
  const float* lse;
  bf16* o;
  int32_t n_q;
  int32_t nsplit;
  int32_t item0;      // first (row, head) group handled by this session
  int32_t pad_;
};
struct CombineArgs {
  CombineSess s[kMaxSessPerLaunch];
  int32_t n_sess;
  int32_t H;
  int32_t items;
};

// Projection GEMM  Y = A * W^T  (A [n_q][d] bf16, W [n_out][d] bf16 =
// [d_out][d_in], fp32 accumulation), with one of two epilogues:
//   kProjEuler: n_out = d; z <- z - h * Y (fp32, in place), and, if zb is set,
//               zb <- bf16(z) (the next step's projection input);
//   kProjQkv:   n_out = 3d; column c of Y goes to out[c / d], column c % d,
//               rounded to bf16 (the unit's Q, K_u, V_u; launch_qkv_wide);
//   kProjLayer: n_out = d; a layer of a stack adds its update to the fp32
//               residual r <- r + Y and writes zb <- bf16(z + r), the next
//               layer's input;
//   kProjLayerLast: the stack's last layer: z <- z - h * (r + Y), r <- 0,
//               and, if zb is set, zb <- bf16(z).
constexpr int kProjEuler = 0;
constexpr int kProjQkv = 1;
constexpr int kProjLayer = 2;
constexpr int kProjLayerLast = 3;

struct ProjSess {
  const bf16* a;      // [n_q][d]
  float* z;           // kProjEuler, kProjLayer*: [n_q][d]
  bf16* zb;           // kProjEuler, kProjLayer*: [n_q][d] or nullptr
  float* r;           // kProjLayer*: [n_q][d] residual
  bf16* out[3];       // kProjQkv: Q, K_u, V_u, each [n_q][d]
  int32_t n_q;
  int32_t n_mtiles;
  int32_t item0;
  float h;
};
struct ProjArgs {
  ProjSess s[kMaxSessPerLaunch];
  const bf16* w;      // [n_out][d], [d_out][d_in]
  int32_t n_sess;
  int32_t d;
  int32_t n_out;
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
hipError_t launch_cvt(const CvtArgs& a, hipStream_t st);
hipError_t launch_mix(const MixArgs& a, hipStream_t st);
// Q/K/V projection (kProjQkv semantics) with 256 x 256 tiles; ProjSess.n_mtiles
// counts 256-row tiles.
hipError_t launch_qkv_wide(const ProjArgs& a, hipStream_t st);

// Attention tiling shared by host planning and the kernel.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kAttnRowsPerWave = 32;
constexpr int kAttnBlockM = kAttnWaves * kAttnRowsPerWave;   // 256 query rows per block
constexpr int kAttnWindow = 64;                              // keys per window

// Projection tiling: 160 rows x 128 output features per block.
constexpr int kProjTile = 160;
constexpr int kProjTileN = 128;
// Q/K/V projection tiling: 256 rows x 256 output features per block.
constexpr int kQkvTile = 256;

}  // namespace fmd
