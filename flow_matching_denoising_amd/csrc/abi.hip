// C ABI of libfmd: argument validation, work planning, workspace layout and
// kernel launches.  Nothing is enqueued unless every argument of the call is
// valid; a failed call leaves every cache's (len, head) unchanged.
//
// One denoised unit [Wan-Streamer (gongshangzheng blog), Fig. 2 and 5.2]: the
// performer writes the thinker's K/V slice into its local cache, then runs the
// flow-matching solver: per step, attention over [valid cache || unit],
// projection to a velocity, Euler update [same page, 3.4].
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "fmd_internal.h"

using namespace fmd;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Event timing of launches (off unless enabled).
// ---------------------------------------------------------------------------
struct ProfRec {
  hipEvent_t a, b;
  int cls;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
uint32_t g_prof_mask = (1u << FMD_KERNEL_COUNT) - 1;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // Timing only: no system-scope fence (no cache writeback or invalidate).
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

template <class F>
int timed_launch(int cls, hipStream_t st, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  bool rec = false;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_on && ((g_prof_mask >> cls) & 1u)) {
      a = take_event();
      b = take_event();
      rec = a && b;
      if (!rec) {   // keep whichever was created for later
        if (a) g_event_pool.push_back(a);
        if (b) g_event_pool.push_back(b);
      }
    }
  }
  if (rec) (void)hipEventRecord(a, st);
  hipError_t err = launch();
  if (rec) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({a, b, cls});
  }
  if (err != hipSuccess)
    return fail(FMD_E_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return FMD_OK;
}

// ---------------------------------------------------------------------------
// Validation.
// ---------------------------------------------------------------------------
int check_cache(const fmd_kv_cache* c, int idx) {
  if (!c) return fail(FMD_E_INVAL, "session %d: cache is NULL", idx);
  if (!c->k || !c->v) return fail(FMD_E_INVAL, "session %d: cache k/v pointer is NULL", idx);
  if (!aligned16(c->k) || !aligned16(c->v))
    return fail(FMD_E_ALIGN, "session %d: cache k/v not 16-byte aligned", idx);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(FMD_E_SHAPE, "session %d: head_dim %d (must be 64 or 128)", idx, c->head_dim);
  if (c->n_heads < 1 || c->n_heads > 1024)
    return fail(FMD_E_SHAPE, "session %d: n_heads %d out of range", idx, c->n_heads);
  // One head's ring slice is addressed with 32-bit byte offsets.
  if (c->cap_tokens < 16 || c->cap_tokens % 16 != 0 ||
      c->cap_tokens * c->head_dim * 2 > (int64_t)INT32_MAX)
    return fail(FMD_E_SHAPE,
                "session %d: cap_tokens %lld (positive multiple of 16, cap*head_dim*2 < 2^31)",
                idx, (long long)c->cap_tokens);
  if (c->len_tokens < 0 || c->len_tokens > c->cap_tokens || c->head_tokens < 0 ||
      c->head_tokens >= c->cap_tokens)
    return fail(FMD_E_INVAL, "session %d: ring state len=%lld head=%lld out of range", idx,
                (long long)c->len_tokens, (long long)c->head_tokens);
  return FMD_OK;
}

int check_tensor(const void* p, int idx, const char* name) {
  if (!p) return fail(FMD_E_INVAL, "session %d: %s is NULL", idx, name);
  if (!aligned16(p)) return fail(FMD_E_ALIGN, "session %d: %s not 16-byte aligned", idx, name);
  return FMD_OK;
}

int check_step(const fmd_unit_step* u, int idx, bool need_z) {
  int rc;
  if ((rc = check_cache(u->cache, idx))) return rc;
  if ((rc = check_tensor(u->q, idx, "q"))) return rc;
  if ((rc = check_tensor(u->k_u, idx, "k_u"))) return rc;
  if ((rc = check_tensor(u->v_u, idx, "v_u"))) return rc;
  if (need_z && (rc = check_tensor(u->z, idx, "z"))) return rc;
  if (u->n_video < 0 || u->n_audio < 0 || (int64_t)u->n_video + u->n_audio < 1 ||
      (int64_t)u->n_video + u->n_audio > (1 << 22))
    return fail(FMD_E_INVAL, "session %d: n_video=%d n_audio=%d (need 1 <= n_q <= 2^22)", idx,
                u->n_video, u->n_audio);
  if (need_z && !(u->h > 0.f && isfinite(u->h)))
    return fail(FMD_E_INVAL, "session %d: step size h=%g must be finite and > 0", idx, u->h);
  return FMD_OK;
}

int check_same_shape(const fmd_kv_cache* c0, const fmd_kv_cache* c, int idx) {
  if (c->n_heads != c0->n_heads || c->head_dim != c0->head_dim)
    return fail(FMD_E_SHAPE, "session %d: heads %dx%d differ from session 0's %dx%d", idx,
                c->n_heads, c->head_dim, c0->n_heads, c0->head_dim);
  return FMD_OK;
}

// The sessions' latents are written in place: their fp32 [n_q][d] ranges must
// not overlap (two sessions updating the same z would race).
struct ZRange {
  uintptr_t lo, hi;
  int idx;
};
int check_disjoint_z(std::vector<ZRange> zs) {
  std::sort(zs.begin(), zs.end(), [](const ZRange& a, const ZRange& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < zs.size(); ++k)
    if (zs[k].lo < zs[k - 1].hi)
      return fail(FMD_E_INVAL, "sessions %d and %d: latents z overlap", zs[k - 1].idx, zs[k].idx);
  return FMD_OK;
}
ZRange z_range(const float* z, int64_t n_q, int d, int idx) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(z);
  return ZRange{lo, lo + (uintptr_t)n_q * d * sizeof(float), idx};
}

// ---------------------------------------------------------------------------
// Planning.
// ---------------------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Whether the attention reads a step's unit keys where the caller keeps them
// ([n][H][hd], one head's keys every H*hd elements) instead of a staged
// [H][npad][hd] copy: when they are given (not produced by the Q/K/V
// projection) and their bytes fit the kernels' 32-bit buffer offsets.
bool unit_keys_in_place(const void* k_u, int n_q, int d) {
  return k_u != nullptr && (int64_t)n_q * d * 2 < ((int64_t)1 << 31);
}

struct SessPlan {
  int n_q, npad;
  int seg_lo[2], seg_hi[2];
  int nwin[3], nwin_total;
  int n_qblk;
  // The session's launch (sessions are launched in chunks of
  // kMaxSessPerLaunch): its window sequence and groups, this session's first
  // window among one head's, and the partial slots its lanes need (0 when
  // every lane lies in one group).
  int lane0, per_head, groups, qb;
  int64_t total;
  int npart;
  int proj_splits;   // k-range parts of the launch's projection (1: none)
  int proj_chain;    // > 1: a unit projects this many steps in one launch
  size_t off_kt, off_vt, off_o, off_opart, off_lse, off_part;   // workspace offsets
  size_t kv_stride;  // bytes between copies of the staged unit keys/values
};

int nwin_of(int lo, int hi) {
  if (hi <= lo) return 0;
  const int start = lo & ~15;
  return (hi - start + kAttnWindow - 1) / kAttnWindow;
}

void plan_session(const fmd_kv_cache* c, int n_q, SessPlan& p) {
  const int64_t cap = c->cap_tokens, len = c->len_tokens, head = c->head_tokens;
  p.n_q = n_q;
  p.npad = (n_q + 15) & ~15;
  p.seg_lo[0] = p.seg_hi[0] = p.seg_lo[1] = p.seg_hi[1] = 0;
  if (len > 0) {
    const int64_t start = ((head - len) % cap + cap) % cap;
    if (start + len <= cap) {
      p.seg_lo[0] = (int)start;
      p.seg_hi[0] = (int)(start + len);
    } else {
      p.seg_lo[0] = (int)start;
      p.seg_hi[0] = (int)cap;
      p.seg_lo[1] = 0;
      p.seg_hi[1] = (int)(start + len - cap);
    }
  }
  p.nwin[0] = nwin_of(p.seg_lo[0], p.seg_hi[0]);
  p.nwin[1] = nwin_of(p.seg_lo[1], p.seg_hi[1]);
  p.nwin[2] = (n_q + kAttnWindow - 1) / kAttnWindow;
  p.nwin_total = p.nwin[0] + p.nwin[1] + p.nwin[2];
  p.n_qblk = (n_q + kAttnBlockM - 1) / kAttnBlockM;
}

// Group count forced through fmd_test_force_attn_groups (0: the planner).
std::atomic<int> g_forced_groups{0};

// Groups of a launch.  One work-group per CU, all resident at once: each
// XCD's 32 CUs take floor(32 / qb) groups, so a group never straddles two
// XCDs (its work-groups share the keys in one L2).  A group's range costs
// about two windows of pipeline fill and a piece to merge per lane it cuts,
// so short sequences get fewer groups (at least kMinGroupWindows windows
// each).  Queries beyond 32 blocks per session spread a group over XCDs.
constexpr int kCusPerXcd = kTargetCUs / kNumXcd;
constexpr int kMinGroupWindows = 8;

// When a multiple of the head count H is within 15 % of that maximum, the
// largest such multiple is taken instead: then every head's windows start at
// a group boundary, so no group runs the end of one head and the start of the
// next as separate spans (each span restarts the window pipeline).  The
// 192x336-class unit (12 heads) gets 120 groups instead of 128 (attention
// 39.7 against 47.1 us per launch), an 8-way Ulysses rank (5 heads) 60
// instead of 64; 40 heads keep 64.
int choose_groups(int qb, int64_t total, int H) {
  const int forced = g_forced_groups.load(std::memory_order_relaxed);
  if (forced > 0) return (int)std::min<int64_t>(forced, total);
  int g = qb <= kCusPerXcd ? kNumXcd * (kCusPerXcd / qb) : std::max(1, kTargetCUs / qb);
  g = (int)std::min<int64_t>(g, std::max<int64_t>(1, total / kMinGroupWindows));
  g = std::max(1, g);
  const int aligned = H > 0 ? g / H * H : 0;
  if (aligned > 0 && aligned * 20 >= g * 17) g = aligned;
  return g;
}

// Plan every launch chunk's window sequence and groups.
void plan_groups(std::vector<SessPlan>& plans, int H) {
  const int n = (int)plans.size();
  for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
    const int cn = std::min(kMaxSessPerLaunch, n - c0);
    int per_head = 0, qb = 1;
    for (int k = 0; k < cn; ++k) {
      plans[c0 + k].lane0 = per_head;
      per_head += plans[c0 + k].nwin_total;
      qb = std::max(qb, plans[c0 + k].n_qblk);
    }
    const int64_t total = (int64_t)H * per_head;
    const int groups = choose_groups(qb, total, H);
    for (int k = 0; k < cn; ++k) {
      SessPlan& p = plans[c0 + k];
      p.per_head = per_head;
      p.qb = qb;
      p.groups = groups;
      p.total = total;
      int most = 1;
      for (int h = 0; h < H; ++h) {
        const int64_t first = (int64_t)h * per_head + p.lane0;
        most = std::max(most, piece_of(first, first + p.nwin_total - 1, p.nwin[0], p.nwin[1],
                                       total, groups) + 1);
      }
      p.npart = most > 1 ? most : 0;
    }
  }
}

// Workspace layout, sessions in order.  With o_external, O goes to the
// caller's buffer and takes no workspace.  kv_copies: copies of the staged
// unit keys and values (one per solver step when a unit stages every step's
// up front); copy c sits kv_stride * c bytes after the first.
size_t layout_workspace(std::vector<SessPlan>& plans, int H, int hd, bool o_external,
                        int kv_copies) {
  size_t off = 0;
  for (auto& p : plans) {
    const size_t kvb = align256((size_t)H * p.npad * hd * 2);
    p.off_kt = off;
    p.off_vt = off + kvb;
    p.kv_stride = 2 * kvb;
    off += (size_t)kv_copies * 2 * kvb;
    p.off_o = off;
    if (!o_external) off = align256(off + (size_t)p.n_q * H * hd * 2);
    p.off_opart = p.off_lse = off;
    if (p.npart > 0) {
      off = align256(off + (size_t)p.npart * p.n_q * H * hd * 2);
      p.off_lse = off;
      off = align256(off + (size_t)p.npart * p.n_q * H * 4);
    }
    p.off_part = off;
    if (!o_external && p.proj_splits > 1)
      off = align256(off + (size_t)p.proj_splits * p.n_q * H * hd * 4);
  }
  return off;
}

// The projection's k-range parts, per launch chunk (every session of a chunk
// is counted as projected; a guided pair projects once, so this errs towards
// fewer parts there).
void plan_proj(std::vector<SessPlan>& plans, int d) {
  const int n = (int)plans.size();
  const int ntiles = (d + kProjTileN - 1) / kProjTileN;
  for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
    const int cn = std::min(kMaxSessPerLaunch, n - c0);
    int64_t tiles = 0;
    for (int k = 0; k < cn; ++k)
      tiles += (int64_t)((plans[c0 + k].n_q + kProjTile - 1) / kProjTile) * ntiles;
    const int splits = proj_splits(tiles, d / kProjBK);
    for (int k = 0; k < cn; ++k) plans[c0 + k].proj_splits = splits;
  }
}

int plan_steps(const fmd_unit_step* units, int n, bool o_external, std::vector<SessPlan>& plans,
               size_t* bytes, int kv_copies = 1) {
  const int H = units[0].cache->n_heads, hd = units[0].cache->head_dim;
  plans.resize(n);
  for (int i = 0; i < n; ++i)
    plan_session(units[i].cache, units[i].n_video + units[i].n_audio, plans[i]);
  plan_groups(plans, H);
  plan_proj(plans, H * hd);
  *bytes = layout_workspace(plans, H, hd, o_external, kv_copies);
  return FMD_OK;
}

int validate_steps(const fmd_unit_step* units, int n, bool need_z) {
  if (!units) return fail(FMD_E_INVAL, "units is NULL");
  if (n < 1 || n > FMD_MAX_SESSIONS)
    return fail(FMD_E_INVAL, "n_units=%d (must be 1..%d)", n, FMD_MAX_SESSIONS);
  int rc;
  std::vector<ZRange> zs;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_step(&units[i], i, need_z))) return rc;
    if (i && (rc = check_same_shape(units[0].cache, units[i].cache, i))) return rc;
    const int d = units[i].cache->n_heads * units[i].cache->head_dim;
    if (need_z) zs.push_back(z_range(units[i].z, units[i].n_video + units[i].n_audio, d, i));
  }
  return check_disjoint_z(zs);
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return FMD_OK;
  if (!ws) return fail(FMD_E_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(FMD_E_ALIGN, "workspace not 256-byte aligned");
  if (have < need)
    return fail(FMD_E_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return FMD_OK;
}

// Enqueue the step kernels (validation already done).  o_out != nullptr:
// attention only, O to the caller's buffer.
// zb_out (optional, one per projected unit): where the projection epilogue
// also writes bf16(z) after the update (the next step's input to the Q/K/V
// projection).
// guidance != nullptr: the units come in pairs (2i conditional, 2i+1
// unconditional) that share q, k_u, v_u, z and h; pair i is guided with scale
// guidance[i].  The pair's unit keys and values are transposed once, both
// branches attend, their outputs are mixed (in place into the conditional
// one) and one projection updates z.
// proj_mode: kProjEuler, or kProjLayer / kProjLayerLast for a layer of a
// stack, with r_out (one fp32 residual per projected unit).
// kv_staged: the unit keys and values already sit in each session's (each
// pair's first branch's) kt/vt workspace slots, copy kv_copy (written there by
// the Q/K/V projection, or by a unit's staging of every step up front); no
// staging launch.
// phases: kPhaseAttn enqueues the staging, attention, merge and mix launches,
// kPhaseProj the projection; a unit whose steps' attention runs as one launch
// calls the two phases separately (each session's O stays in its workspace
// slot, plans[...].off_o, in between).
constexpr int kPhaseAttn = 1, kPhaseProj = 2, kPhaseAll = 3;

int enqueue_steps(const fmd_unit_step* units, int n, const std::vector<SessPlan>& plans,
                  const void* w_o, char* ws, bf16* o_out, hipStream_t st,
                  bf16* const* zb_out = nullptr, const float* guidance = nullptr,
                  int proj_mode = kProjEuler, float* const* r_out = nullptr,
                  bool kv_staged = false, int kv_copy = 0, int phases = kPhaseAll) {
  const int H = units[0].cache->n_heads, hd = units[0].cache->head_dim;
  const int d = H * hd;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  const int per_proj = guidance ? 2 : 1;
  int64_t o_row = 0;
  for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
    const int cn = std::min(kMaxSessPerLaunch, n - c0);
    VtArgs va = {};
    AttnArgs aa = {};
    CombineArgs ca = {};
    MixArgs ma = {};
    ProjArgs pa = {};
    va.n_sess = aa.n_sess = ca.n_sess = cn;
    pa.n_sess = cn / per_proj;
    ma.n_sess = guidance ? cn / 2 : 0;
    va.H = aa.H = ca.H = H;
    aa.scale_log2 = scale_log2;
    pa.d = d;
    pa.n_out = d;
    pa.w = static_cast<const bf16*>(w_o);
    pa.splits = plans[c0].proj_splits;
    bool any_split = false;
    bf16* o_prev = nullptr;
    for (int k = 0; k < cn; ++k) {
      const fmd_unit_step& u = units[c0 + k];
      const SessPlan& p = plans[c0 + k];
      const fmd_kv_cache* c = u.cache;
      const bool second = guidance && (k & 1);
      const SessPlan& pk = second ? plans[c0 + k - 1] : p;   // a pair shares the first's
      bf16* kt = reinterpret_cast<bf16*>(ws + pk.off_kt + kv_copy * pk.kv_stride);
      bf16* vt = reinterpret_cast<bf16*>(ws + pk.off_vt + kv_copy * pk.kv_stride);
      bf16* o = o_out ? o_out + o_row * d : reinterpret_cast<bf16*>(ws + p.off_o);
      o_row += p.n_q;

      const bool k_in_place = unit_keys_in_place(u.k_u, p.n_q, d);
      // A session without transpose work gets an empty range at the current end.
      va.s[k] = VtSess{static_cast<const bf16*>(u.k_u), static_cast<const bf16*>(u.v_u),
                       k_in_place ? nullptr : kt, vt, p.n_q, p.npad / 16, va.items, 0};
      if (!second && !kv_staged) va.items += H * ((p.npad / 16 + kVtBlocks - 1) / kVtBlocks);

      AttnSess& as = aa.s[k];
      as.q = static_cast<const bf16*>(u.q);
      if (k_in_place) {
        as.kt_u = static_cast<const bf16*>(u.k_u);
        as.ku_head = hd;
        as.ku_stride = d;
        as.ku_bytes = (int32_t)(((int64_t)(p.n_q - 1) * d + hd) * 2);
      } else {
        as.kt_u = kt;
        as.ku_head = (int64_t)p.npad * hd;
        as.ku_stride = hd;
        as.ku_bytes = p.npad * hd * 2;
      }
      as.vt_u = vt;
      as.ring_k = static_cast<const bf16*>(c->k);
      as.ring_v = static_cast<const bf16*>(c->v);
      as.o = o;
      as.opart = reinterpret_cast<bf16*>(ws + p.off_opart);
      as.lse = reinterpret_cast<float*>(ws + p.off_lse);
      as.cap = c->cap_tokens;
      as.n_q = p.n_q;
      as.npad = p.npad;
      for (int t = 0; t < 2; ++t) {
        as.seg_lo[t] = p.seg_lo[t];
        as.seg_hi[t] = p.seg_hi[t];
      }
      for (int t = 0; t < 3; ++t) as.nwin[t] = p.nwin[t];
      as.nwin_total = p.nwin_total;
      as.n_qblk = p.n_qblk;
      as.lane0 = p.lane0;
      aa.per_head = ca.per_head = p.per_head;
      aa.groups = ca.groups = p.groups;
      aa.qb = p.qb;
      aa.total = ca.total = p.total;

      ca.s[k] = CombineSess{as.opart, as.lse, o,         p.n_q,       p.nwin_total,
                            p.lane0,  p.nwin[0], p.nwin[1], ca.items};
      if (p.npart > 0) {
        ca.items += H * ((p.n_q + kCombineRowsPerBlock - 1) / kCombineRowsPerBlock);
        any_split = true;
      }

      if (second) {
        const int64_t ne = (int64_t)p.n_q * d;
        ma.s[k / 2] = MixSess{o_prev, o, guidance[(c0 + k) / 2], ne, ma.items};
        ma.items += ne / 8;
        continue;
      }
      o_prev = o;
      const int j = k / per_proj, unit = (c0 + k) / per_proj;
      const int mtiles = (p.n_q + kProjTile - 1) / kProjTile;
      const int ntiles = (d + kProjTileN - 1) / kProjTileN;
      pa.s[j] = ProjSess{o,        u.z,     zb_out ? zb_out[unit] : nullptr,
                         r_out ? r_out[unit] : nullptr,
                         reinterpret_cast<float*>(ws + p.off_part),
                         p.n_q,    mtiles,  pa.items, u.h};
      pa.items += mtiles * ntiles * pa.splits;
    }
    // Sessions whose lanes all lie in one group take no combine items; the
    // combine kernel finds its session by item0, so they get an empty range
    // at the current end.
    int rc;
    if (phases & kPhaseAttn) {
      if (va.items > 0 &&
          (rc = timed_launch(FMD_KERNEL_VT, st, [&] { return launch_vt(va, hd, st); })))
        return rc;
      if ((rc = timed_launch(FMD_KERNEL_ATTN, st, [&] { return launch_attn(aa, hd, st); })))
        return rc;
      if (any_split &&
          (rc = timed_launch(FMD_KERNEL_COMBINE, st, [&] { return launch_combine(ca, hd, st); })))
        return rc;
      if (guidance &&
          (rc = timed_launch(FMD_KERNEL_MIX, st, [&] { return launch_mix(ma, st); })))
        return rc;
    }
    if ((phases & kPhaseProj) && !o_out && (rc = timed_launch(FMD_KERNEL_PROJ, st, [&] {
                     hipError_t e = launch_proj(pa, proj_mode, st);
                     return e == hipSuccess ? launch_proj_reduce(pa, proj_mode, st) : e;
                   })))
      return rc;
  }
  return FMD_OK;
}

// ---------------------------------------------------------------------------
// Append.
// ---------------------------------------------------------------------------
int check_append(const fmd_kv_cache* c, const void* ks, const void* vs, int64_t T, int idx) {
  int rc;
  if ((rc = check_cache(c, idx))) return rc;
  if ((rc = check_tensor(ks, idx, "k_slice"))) return rc;
  if ((rc = check_tensor(vs, idx, "v_slice"))) return rc;
  if (T < 1) return fail(FMD_E_INVAL, "session %d: slice of %lld tokens", idx, (long long)T);
  if (T > c->cap_tokens)
    return fail(FMD_E_CAPACITY, "session %d: slice of %lld tokens exceeds capacity %lld", idx,
                (long long)T, (long long)c->cap_tokens);
  return FMD_OK;
}

// Enqueue appends (validated) and advance each cache's host state.
int enqueue_appends(fmd_kv_cache* const* caches, const void* const* ks, const void* const* vs,
                    const int64_t* T, int n, hipStream_t st) {
  const int H = caches[0]->n_heads, hd = caches[0]->head_dim;
  for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
    const int cn = std::min(kMaxSessPerLaunch, n - c0);
    AppendArgs a = {};
    a.n_sess = cn;
    a.H = H;
    for (int k = 0; k < cn; ++k) {
      const fmd_kv_cache* c = caches[c0 + k];
      const int64_t cap = c->cap_tokens, head = c->head_tokens, t = T[c0 + k];
      const int64_t nb_ring = cap / 16;
      const int64_t blk0 = head / 16;
      const int64_t blk_last = (head + t - 1) / 16;            // linear (unwrapped)
      const int64_t nblk = std::min(blk_last - blk0 + 1, nb_ring);
      a.s[k] = AppendSess{static_cast<const bf16*>(ks[c0 + k]), static_cast<const bf16*>(vs[c0 + k]),
                          static_cast<bf16*>(c->k), static_cast<bf16*>(c->v), cap, (int32_t)t,
                          (int32_t)head, (int32_t)blk0, (int32_t)nblk, a.items, 0};
      a.items += H * (int)nblk;
    }
    int rc = timed_launch(FMD_KERNEL_APPEND, st, [&] { return launch_append(a, hd, st); });
    if (rc) return rc;
    for (int k = 0; k < cn; ++k) {
      fmd_kv_cache* c = caches[c0 + k];
      const int64_t t = T[c0 + k];
      c->head_tokens = (c->head_tokens + t) % c->cap_tokens;
      c->len_tokens = std::min(c->len_tokens + t, c->cap_tokens);
    }
  }
  return FMD_OK;
}

}  // namespace

// Scratch of fmd_denoise_unit_noalloc: one copy per GPU the library runs on,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel or a copy (in host code the name is a host-side stand-in, not a
// device address): it uses the address hipGetSymbolAddress returns for the
// current device, looked up once per device.
static __device__ __align__(256) char scratch[FMD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;   // per device ordinal; nullptr until looked up

// The device address of this GPU's scratch.  `st` must belong to the current
// device (the address is per device).
int device_scratch(hipStream_t st, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FMD_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (st) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return fail(FMD_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(FMD_E_INVAL, "stream belongs to device %d, the current device is %d", sdev, dev);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FMD_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FMD_OK;
}

}  // namespace

extern "C" {

const char* fmd_version(void) { return "0.2.0"; }

int fmd_test_force_attn_groups(int32_t n_groups) {
  g_last_error.clear();
  if (n_groups < 0) return fail(FMD_E_INVAL, "n_groups=%d (must be >= 0)", n_groups);
  g_forced_groups.store(n_groups, std::memory_order_relaxed);
  return FMD_OK;
}

const char* fmd_strerror(int status) {
  switch (status) {
    case FMD_OK: return "ok";
    case FMD_E_INVAL: return "invalid argument";
    case FMD_E_SHAPE: return "unsupported or mismatched shape";
    case FMD_E_CAPACITY: return "slice longer than the ring capacity";
    case FMD_E_ALIGN: return "pointer not aligned";
    case FMD_E_WORKSPACE: return "workspace missing or too small";
    case FMD_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fmd_last_error(void) { return g_last_error.c_str(); }

int fmd_kv_append(fmd_kv_cache* cache, const void* k_slice, const void* v_slice,
                  int64_t n_tokens, void* stream) {
  g_last_error.clear();
  int rc = check_append(cache, k_slice, v_slice, n_tokens, 0);
  if (rc) return rc;
  fmd_kv_cache* cs[1] = {cache};
  const void* ks[1] = {k_slice};
  const void* vs[1] = {v_slice};
  int64_t ts[1] = {n_tokens};
  return enqueue_appends(cs, ks, vs, ts, 1, static_cast<hipStream_t>(stream));
}

int fmd_kv_append_batched(fmd_kv_cache* const* caches, const void* const* k_slices,
                          const void* const* v_slices, const int64_t* n_tokens,
                          int32_t n_sessions, void* stream) {
  g_last_error.clear();
  if (!caches || !k_slices || !v_slices || !n_tokens)
    return fail(FMD_E_INVAL, "NULL array argument");
  if (n_sessions < 1 || n_sessions > FMD_MAX_SESSIONS)
    return fail(FMD_E_INVAL, "n_sessions=%d (must be 1..%d)", n_sessions, FMD_MAX_SESSIONS);
  int rc;
  for (int i = 0; i < n_sessions; ++i) {
    if ((rc = check_append(caches[i], k_slices[i], v_slices[i], n_tokens[i], i))) return rc;
    if (i && (rc = check_same_shape(caches[0], caches[i], i))) return rc;
    for (int j = 0; j < i; ++j)
      if (caches[j] == caches[i])
        return fail(FMD_E_INVAL, "session %d: same cache as session %d", i, j);
  }
  return enqueue_appends(caches, k_slices, v_slices, n_tokens, n_sessions,
                         static_cast<hipStream_t>(stream));
}

int fmd_workspace_bytes(const fmd_unit_step* units, int32_t n_units, size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(FMD_E_INVAL, "out_bytes is NULL");
  int rc = validate_steps(units, n_units, false);
  if (rc) return rc;
  std::vector<SessPlan> plans;
  return plan_steps(units, n_units, false, plans, out_bytes);
}

int fmd_denoise_step(const fmd_unit_step* units, int32_t n_units, const void* w_o,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_steps(units, n_units, true);
  if (rc) return rc;
  if ((rc = check_tensor(w_o, 0, "w_o"))) return rc;
  std::vector<SessPlan> plans;
  size_t need = 0;
  plan_steps(units, n_units, false, plans, &need);
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  return enqueue_steps(units, n_units, plans, w_o, static_cast<char*>(workspace), nullptr,
                       static_cast<hipStream_t>(stream));
}

int fmd_attention(const fmd_unit_step* units, int32_t n_units, void* o_out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_steps(units, n_units, false);
  if (rc) return rc;
  if ((rc = check_tensor(o_out, 0, "o_out"))) return rc;
  std::vector<SessPlan> plans;
  size_t need = 0;
  plan_steps(units, n_units, true, plans, &need);
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  return enqueue_steps(units, n_units, plans, nullptr, static_cast<char*>(workspace),
                       static_cast<bf16*>(o_out), static_cast<hipStream_t>(stream));
}

static int validate_unit_io(const fmd_unit_io* ss, int n, int n_steps) {
  if (!ss) return fail(FMD_E_INVAL, "sessions is NULL");
  if (n < 1 || n > FMD_MAX_SESSIONS)
    return fail(FMD_E_INVAL, "n_sessions=%d (must be 1..%d)", n, FMD_MAX_SESSIONS);
  if (n_steps < 1) return fail(FMD_E_INVAL, "n_steps=%d (must be >= 1)", n_steps);
  int rc;
  for (int i = 0; i < n; ++i) {
    const fmd_unit_io& s = ss[i];
    if ((rc = check_cache(s.cache, i))) return rc;
    if (i && (rc = check_same_shape(ss[0].cache, s.cache, i))) return rc;
    for (int j = 0; j < i; ++j)
      if (ss[j].cache == s.cache) return fail(FMD_E_INVAL, "session %d: same cache as %d", i, j);
    if (s.slice_tokens < 0)
      return fail(FMD_E_INVAL, "session %d: slice_tokens %lld", i, (long long)s.slice_tokens);
    if (s.slice_tokens > 0 &&
        (rc = check_append(s.cache, s.k_slice, s.v_slice, s.slice_tokens, i)))
      return rc;
    if (s.step_stride_elems < 0 || (s.step_stride_elems * 2) % 16 != 0)
      return fail(FMD_E_ALIGN, "session %d: step stride %lld elements (>= 0, multiple of 8)", i,
                  (long long)s.step_stride_elems);
    if (!s.h) return fail(FMD_E_INVAL, "session %d: h is NULL", i);
    for (int k = 0; k < n_steps; ++k)
      if (!(s.h[k] > 0.f && isfinite(s.h[k])))
        return fail(FMD_E_INVAL, "session %d: h[%d]=%g must be finite and > 0", i, k, s.h[k]);
    fmd_unit_step u = {s.cache, s.q, s.k_u, s.v_u, s.z, s.n_video, s.n_audio, s.h[0]};
    if ((rc = check_step(&u, i, true))) return rc;
  }
  std::vector<ZRange> zs;
  for (int i = 0; i < n; ++i)
    zs.push_back(z_range(ss[i].z, ss[i].n_video + ss[i].n_audio,
                         ss[i].cache->n_heads * ss[i].cache->head_dim, i));
  return check_disjoint_z(zs);
}

// The post-append ring states of a unit's sessions (for planning).
static void post_append_steps(const fmd_unit_io* ss, int n, std::vector<fmd_kv_cache>& after,
                              std::vector<fmd_unit_step>& steps) {
  after.resize(n);
  steps.resize(n);
  for (int i = 0; i < n; ++i) {
    after[i] = *ss[i].cache;
    if (ss[i].slice_tokens > 0) {
      after[i].head_tokens = (after[i].head_tokens + ss[i].slice_tokens) % after[i].cap_tokens;
      after[i].len_tokens = std::min(after[i].len_tokens + ss[i].slice_tokens, after[i].cap_tokens);
    }
    steps[i] = fmd_unit_step{&after[i], ss[i].q, ss[i].k_u, ss[i].v_u, ss[i].z,
                             ss[i].n_video, ss[i].n_audio, ss[i].h[0]};
  }
}

// Copies of the staged unit keys and values a unit needs: every step's are
// staged up front, once when every session reuses one set for all steps.
static int unit_kv_copies(const fmd_unit_io* ss, int n, int n_steps) {
  for (int i = 0; i < n; ++i)
    if (ss[i].step_stride_elems != 0) return n_steps;
  return 1;
}

// Solver steps whose attention one launch covers in fmd_denoise_unit.  There
// the steps' Q, K_u and V_u are inputs (no step's attention reads the latent),
// so the attention of several steps is one launch whose sessions are the
// (step, session) pairs, and the projections then update z step by step, in
// order.  The batch is the largest divisor of n_steps whose pairs fit one
// launch, so every batch of a unit has the same plan.
static int unit_step_batch(int n_sessions, int n_steps) {
  const int most = std::max(1, kMaxSessPerLaunch / n_sessions);
  for (int b = std::min(n_steps, most); b > 1; --b)
    if (n_steps % b == 0) return b;
  return 1;
}

// Plan a validated unit: the post-append ring states, the plans of one batch
// of steps (entry b * n + i: step b of the batch, session i) and the workspace
// bytes.  Workspace: per session, the staged unit values (and keys, when they
// are not read in place) of every step (one copy when every session reuses
// one set) and the projection's fp32 partials (shared by the steps, which
// project one after another); per (step of the batch, session), O, the pieces
// of the lanes cut by group ends and, when the batch's split projections
// share one launch, that step's partials.
static void plan_unit(const fmd_unit_io* sessions, int n, int n_steps,
                      std::vector<fmd_kv_cache>& after, std::vector<fmd_unit_step>& steps,
                      std::vector<SessPlan>& plans, size_t* need) {
  post_append_steps(sessions, n, after, steps);
  const int B = unit_step_batch(n, n_steps);
  const int H = after[0].n_heads, hd = after[0].head_dim, d = H * hd;
  const int copies = unit_kv_copies(sessions, n, n_steps);
  plans.assign((size_t)B * n, SessPlan{});
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
      plan_session(&after[i], steps[i].n_video + steps[i].n_audio, plans[(size_t)b * n + i]);
  plan_groups(plans, H);
  // Each step projects its n sessions (launch chunks as in enqueue_steps),
  // unless the batch's projections split over the k range: then the B steps'
  // partial products are one launch (B * n <= kMaxSessPerLaunch) and one
  // reduce applies the steps' updates in order (proj_chain = B).
  std::vector<SessPlan> one(plans.begin(), plans.begin() + n);
  plan_proj(one, d);
  int chain_splits = 1;
  if (B > 1) {
    int64_t tiles = 0;
    for (const auto& p : plans)
      tiles += (int64_t)((p.n_q + kProjTile - 1) / kProjTile) * ((d + kProjTileN - 1) / kProjTileN);
    chain_splits = proj_splits(tiles, d / kProjBK);
  }
  const bool chain = chain_splits > 1;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    // Keys the attention reads in place take no staging room.
    const size_t kvb = align256((size_t)H * one[i].npad * hd * 2);
    const int kv_regions = unit_keys_in_place(sessions[i].k_u, one[i].n_q, d) ? 1 : 2;
    const size_t kv_off = off;
    off += (size_t)copies * kv_regions * kvb;
    const size_t part_off = off;
    if (!chain && one[i].proj_splits > 1)
      off = align256(off + (size_t)one[i].proj_splits * one[i].n_q * d * 4);
    for (int b = 0; b < B; ++b) {
      SessPlan& p = plans[(size_t)b * n + i];
      p.proj_splits = chain ? chain_splits : one[i].proj_splits;
      p.proj_chain = chain ? B : 1;
      p.off_kt = kv_off;
      p.off_vt = kv_off + (kv_regions - 1) * kvb;
      p.kv_stride = kv_regions * kvb;
      p.off_part = part_off;
    }
  }
  for (auto& p : plans) {
    p.off_o = off;
    off = align256(off + (size_t)p.n_q * d * 2);
    p.off_opart = p.off_lse = off;
    if (p.npart > 0) {
      off = align256(off + (size_t)p.npart * p.n_q * d * 2);
      p.off_lse = off;
      off = align256(off + (size_t)p.npart * p.n_q * H * 4);
    }
    if (chain) {   // each step's own partials: the steps' products run together
      p.off_part = off;
      off = align256(off + (size_t)chain_splits * p.n_q * d * 4);
    }
  }
  *need = off;
}

// The projections of a batch of m = B * n (step, session) pairs (step-major,
// one launch chunk) whose k range is split: one launch of every pair's fp32
// partial products, then one reduce that applies the B steps' Euler updates
// to each latent in step order.
static int enqueue_proj_chain(const fmd_unit_step* units, int m, int chain,
                              const std::vector<SessPlan>& plans, const void* w_o, char* ws,
                              hipStream_t st) {
  const int d = units[0].cache->n_heads * units[0].cache->head_dim;
  const int ntiles = (d + kProjTileN - 1) / kProjTileN;
  ProjArgs pa = {};
  pa.n_sess = m;
  pa.d = d;
  pa.n_out = d;
  pa.w = static_cast<const bf16*>(w_o);
  pa.splits = plans[0].proj_splits;
  pa.chain = chain;
  for (int k = 0; k < m; ++k) {
    const SessPlan& p = plans[k];
    const int mtiles = (p.n_q + kProjTile - 1) / kProjTile;
    pa.s[k] = ProjSess{reinterpret_cast<bf16*>(ws + p.off_o), units[k].z, nullptr, nullptr,
                       reinterpret_cast<float*>(ws + p.off_part), p.n_q, mtiles, pa.items,
                       units[k].h};
    pa.items += mtiles * ntiles * pa.splits;
  }
  return timed_launch(FMD_KERNEL_PROJ, st, [&] {
    hipError_t e = launch_proj(pa, kProjEuler, st);
    return e == hipSuccess ? launch_proj_reduce(pa, kProjEuler, st) : e;
  });
}

int fmd_unit_workspace_bytes(const fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps,
                             size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(FMD_E_INVAL, "out_bytes is NULL");
  int rc = validate_unit_io(sessions, n_sessions, n_steps);
  if (rc) return rc;
  std::vector<fmd_kv_cache> after;
  std::vector<fmd_unit_step> steps;
  std::vector<SessPlan> plans;
  plan_unit(sessions, n_sessions, n_steps, after, steps, plans, out_bytes);
  return FMD_OK;
}

// One launch chunk at a time, the unit keys and values of every step of
// every session into their staging copies (copy s for step s).
static int enqueue_unit_staging(const fmd_unit_io* ss, int n, int n_steps,
                                const std::vector<SessPlan>& plans, char* ws, hipStream_t st) {
  const int H = ss[0].cache->n_heads, hd = ss[0].cache->head_dim;
  const int copies = unit_kv_copies(ss, n, n_steps);
  std::vector<VtSess> all;
  for (int s = 0; s < copies; ++s)
    for (int i = 0; i < n; ++i) {
      const SessPlan& p = plans[i];
      const int64_t off = (int64_t)s * ss[i].step_stride_elems;
      // Keys the attention reads in place (the same test as enqueue_steps')
      // are not copied.
      const bool k_in_place = unit_keys_in_place(ss[i].k_u, p.n_q, H * hd);
      all.push_back(VtSess{static_cast<const bf16*>(ss[i].k_u) + off,
                           static_cast<const bf16*>(ss[i].v_u) + off,
                           k_in_place ? nullptr
                                      : reinterpret_cast<bf16*>(ws + p.off_kt + s * p.kv_stride),
                           reinterpret_cast<bf16*>(ws + p.off_vt + s * p.kv_stride), p.n_q,
                           p.npad / 16, 0, 0});
    }
  for (size_t c0 = 0; c0 < all.size(); c0 += kMaxSessPerLaunch) {
    const int cn = (int)std::min<size_t>(kMaxSessPerLaunch, all.size() - c0);
    VtArgs va = {};
    va.n_sess = cn;
    va.H = H;
    for (int k = 0; k < cn; ++k) {
      va.s[k] = all[c0 + k];
      va.s[k].item0 = va.items;
      va.items += H * ((va.s[k].nblk + kVtBlocks - 1) / kVtBlocks);
    }
    int rc;
    if ((rc = timed_launch(FMD_KERNEL_VT, st, [&] { return launch_vt(va, hd, st); }))) return rc;
  }
  return FMD_OK;
}

// One unit (validated, planned): the batched append, the staging of every
// step's unit keys and values, then the steps on the given workspace.
static int run_unit(fmd_unit_io* sessions, int n_sessions, int n_steps, const void* w_o,
                    std::vector<fmd_unit_step>& steps, const std::vector<SessPlan>& plans,
                    char* workspace, hipStream_t st) {
  int rc;
  std::vector<fmd_kv_cache*> caches;
  std::vector<const void*> ks, vs;
  std::vector<int64_t> ts;
  for (int i = 0; i < n_sessions; ++i) {
    if (sessions[i].slice_tokens > 0) {
      caches.push_back(sessions[i].cache);
      ks.push_back(sessions[i].k_slice);
      vs.push_back(sessions[i].v_slice);
      ts.push_back(sessions[i].slice_tokens);
    }
  }
  if (!caches.empty() &&
      (rc = enqueue_appends(caches.data(), ks.data(), vs.data(), ts.data(), (int)caches.size(), st)))
    return rc;
  if ((rc = enqueue_unit_staging(sessions, n_sessions, n_steps, plans, workspace, st))) return rc;
  const int n = n_sessions, B = (int)plans.size() / n_sessions;
  const bool one_copy = unit_kv_copies(sessions, n, n_steps) == 1;
  std::vector<fmd_unit_step> att((size_t)B * n);
  std::vector<SessPlan> pb(plans);
  for (int s0 = 0; s0 < n_steps; s0 += B) {
    // The attention of steps s0 .. s0 + B - 1: one launch (per chunk of
    // kMaxSessPerLaunch pairs), each pair reading its step's staged copy.
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < n; ++i) {
        const int s = s0 + b;
        const size_t e = (size_t)b * n + i;
        const int64_t off = (int64_t)s * sessions[i].step_stride_elems;
        fmd_unit_step& u = att[e];
        u = steps[i];
        u.cache = sessions[i].cache;   // now in its post-append state
        u.q = static_cast<const bf16*>(sessions[i].q) + off;
        u.k_u = static_cast<const bf16*>(sessions[i].k_u) + off;
        u.v_u = static_cast<const bf16*>(sessions[i].v_u) + off;
        u.h = sessions[i].h[s];
        const size_t copy = one_copy ? 0 : (size_t)s;
        pb[e].off_kt = plans[e].off_kt + copy * plans[e].kv_stride;
        pb[e].off_vt = plans[e].off_vt + copy * plans[e].kv_stride;
      }
    if ((rc = enqueue_steps(att.data(), B * n, pb, w_o, workspace, nullptr, st, nullptr, nullptr,
                            kProjEuler, nullptr, true, 0, kPhaseAttn)))
      return rc;
    // Then each step's projection and Euler update, in step order.
    if (pb[0].proj_chain > 1) {
      if ((rc = enqueue_proj_chain(att.data(), B * n, B, pb, w_o, workspace, st))) return rc;
      continue;
    }
    for (int b = 0; b < B; ++b) {
      const std::vector<SessPlan> ps(pb.begin() + (size_t)b * n, pb.begin() + (size_t)(b + 1) * n);
      if ((rc = enqueue_steps(att.data() + (size_t)b * n, n, ps, w_o, workspace, nullptr, st,
                              nullptr, nullptr, kProjEuler, nullptr, true, 0, kPhaseProj)))
        return rc;
    }
  }
  return FMD_OK;
}

int fmd_denoise_unit(fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps, const void* w_o,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_unit_io(sessions, n_sessions, n_steps);
  if (rc) return rc;
  if ((rc = check_tensor(w_o, 0, "w_o"))) return rc;
  std::vector<fmd_kv_cache> after;
  std::vector<fmd_unit_step> steps;
  std::vector<SessPlan> plans;
  size_t need = 0;
  plan_unit(sessions, n_sessions, n_steps, after, steps, plans, &need);
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  return run_unit(sessions, n_sessions, n_steps, w_o, steps, plans,
                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

int fmd_denoise_unit_noalloc(fmd_unit_io* sessions, int32_t n_sessions, int32_t n_steps,
                             const void* w_o, void* stream) {
  g_last_error.clear();
  int rc = validate_unit_io(sessions, n_sessions, n_steps);
  if (rc) return rc;
  if ((rc = check_tensor(w_o, 0, "w_o"))) return rc;
  std::vector<fmd_kv_cache> after;
  std::vector<fmd_unit_step> steps;
  std::vector<SessPlan> plans;
  size_t need = 0;
  plan_unit(sessions, n_sessions, n_steps, after, steps, plans, &need);
  if (need > (size_t)FMD_NOALLOC_SCRATCH_BYTES)
    return fail(FMD_E_WORKSPACE,
                "this unit needs %zu bytes of scratch; the static scratch holds %zu "
                "(use fmd_denoise_unit with a workspace)",
                need, (size_t)FMD_NOALLOC_SCRATCH_BYTES);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  if ((rc = device_scratch(st, &ws))) return rc;
  return run_unit(sessions, n_sessions, n_steps, w_o, steps, plans, ws, st);
}

// The z-dependent solver's driver, shared by the plain, the guided and the
// layer-stack form.  One solver unit has one latent z and its caches:
//   plain:   nb = 1, L = 1: cache[0];
//   guided:  nb = 2, L = 1: cache[0] conditional, cache[1] unconditional; its
//            attention sessions are numbered unit * 2 + branch;
//   layers:  nb = 1, L >= 1: cache[l] is layer l's ring.
struct SolverUnit {
  std::vector<fmd_kv_cache*> cache;
  std::vector<int64_t> slice_tokens;   // appended before the steps (for planning)
  float* z;
  int32_t n_video, n_audio;
  const float* h;
  float g;
};

// Workspace: per unit bf16 z (the Q/K/V projection's input) and Q ([n_q][d]
// bf16 each) and, for a layer stack, the fp32 residual; then the step
// workspace of fmd_denoise_step, sized for the largest layer (the layers of a
// step run one after another and reuse it).  The projection writes K_u and V_u
// straight into the step workspace's unit key/value slots (of the unit's
// first attention session).
struct SolverLayout {
  std::vector<std::vector<fmd_kv_cache>> after;   // per layer: per attention session
  std::vector<std::vector<fmd_unit_step>> steps;  // per layer
  std::vector<std::vector<SessPlan>> plans;       // per layer
  std::vector<size_t> off;                        // per unit: zb, q, [r]
  size_t slab_total = 0, bytes = 0;
};

static size_t unit_slab(int n_q, int d) { return align256((size_t)n_q * d * 2); }

static void layout_solver(const std::vector<SolverUnit>& us, int nb, int n_layers,
                          SolverLayout& L) {
  const int n = (int)us.size();
  const int d = us[0].cache[0]->n_heads * us[0].cache[0]->head_dim;
  L.after.assign(n_layers, std::vector<fmd_kv_cache>((size_t)n * nb));
  L.steps.assign(n_layers, std::vector<fmd_unit_step>((size_t)n * nb));
  L.plans.assign(n_layers, {});
  L.off.resize(n);
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const int n_q = us[i].n_video + us[i].n_audio;
    L.off[i] = off;
    off += 2 * unit_slab(n_q, d);
    if (n_layers > 1) off += 2 * unit_slab(n_q, d);   // fp32 residual
  }
  L.slab_total = off;
  size_t step_bytes = 0;
  for (int l = 0; l < n_layers; ++l) {
    for (int i = 0; i < n; ++i) {
      const SolverUnit& u = us[i];
      for (int b = 0; b < nb; ++b) {
        const int c = n_layers > 1 ? l : b;
        fmd_kv_cache& a = L.after[l][(size_t)i * nb + b];
        a = *u.cache[c];
        if (u.slice_tokens[c] > 0) {
          a.head_tokens = (a.head_tokens + u.slice_tokens[c]) % a.cap_tokens;
          a.len_tokens = std::min(a.len_tokens + u.slice_tokens[c], a.cap_tokens);
        }
        // q/k_u/v_u are placeholders here (set per step); planning needs shapes only.
        L.steps[l][(size_t)i * nb + b] =
            fmd_unit_step{&a, u.z, u.z, u.z, u.z, u.n_video, u.n_audio, u.h[0]};
      }
    }
    size_t bytes = 0;
    plan_steps(L.steps[l].data(), n * nb, false, L.plans[l], &bytes);
    step_bytes = std::max(step_bytes, bytes);
  }
  L.bytes = L.slab_total + step_bytes;
}

// Enqueue the solver (validated, appends already enqueued): a bf16 copy of
// each starting latent (and a cleared residual for a layer stack), then per
// step and layer the Q/K/V projection of every unit and the attention +
// projection step over all attention sessions.  w_qkv / w_o: one per layer.
static int run_solver(const std::vector<SolverUnit>& us, int nb, int n_layers, int n_steps,
                      const void* const* w_qkv, const void* const* w_o, char* ws,
                      SolverLayout& L, hipStream_t st) {
  const int n = (int)us.size();
  const int H = us[0].cache[0]->n_heads, hd = us[0].cache[0]->head_dim;
  const int d = H * hd;
  std::vector<bf16*> zb(n), q(n);
  std::vector<float*> r(n, nullptr);
  for (int i = 0; i < n; ++i) {
    const size_t slab = unit_slab(us[i].n_video + us[i].n_audio, d);
    zb[i] = reinterpret_cast<bf16*>(ws + L.off[i]);
    q[i] = reinterpret_cast<bf16*>(ws + L.off[i] + slab);
    if (n_layers > 1) r[i] = reinterpret_cast<float*>(ws + L.off[i] + 2 * slab);
  }
  int rc;
  for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
    const int cn = std::min(kMaxSessPerLaunch, n - c0);
    CvtArgs ca = {};
    ca.n_sess = cn;
    for (int j = 0; j < cn; ++j) {
      const int i = c0 + j;
      const int64_t ne = (int64_t)(us[i].n_video + us[i].n_audio) * d;
      ca.s[j] = CvtSess{us[i].z, zb[i], r[i], ne, ca.items};
      ca.items += ne / 8;
    }
    if ((rc = timed_launch(FMD_KERNEL_CVT, st, [&] { return launch_cvt(ca, st); }))) return rc;
  }

  std::vector<float> g(n);
  for (int i = 0; i < n; ++i) g[i] = us[i].g;
  char* step_ws = ws + L.slab_total;
  for (int s = 0; s < n_steps; ++s) {
    for (int l = 0; l < n_layers; ++l) {
      for (int c0 = 0; c0 < n; c0 += kMaxSessPerLaunch) {
        const int cn = std::min(kMaxSessPerLaunch, n - c0);
        QkvArgs pa = {};
        pa.n_sess = cn;
        pa.d = d;
        pa.hd = hd;
        pa.w = static_cast<const bf16*>(w_qkv[l]);
        const int ntiles = (3 * d + kQkvTile - 1) / kQkvTile;
        for (int j = 0; j < cn; ++j) {
          const int i = c0 + j;
          const int n_q = us[i].n_video + us[i].n_audio;
          const int mtiles = (n_q + kQkvTile - 1) / kQkvTile;
          const SessPlan& p = L.plans[l][(size_t)i * nb];
          pa.s[j] = QkvSess{zb[i], q[i], reinterpret_cast<bf16*>(step_ws + p.off_kt),
                            reinterpret_cast<bf16*>(step_ws + p.off_vt), n_q, p.npad, mtiles,
                            pa.items};
          pa.items += mtiles * ntiles;
        }
        if ((rc = timed_launch(FMD_KERNEL_QKV, st, [&] { return launch_qkv_wide(pa, st); })))
          return rc;
      }
      std::vector<fmd_unit_step>& steps = L.steps[l];
      for (int i = 0; i < n; ++i) {
        for (int b = 0; b < nb; ++b) {
          fmd_unit_step& u = steps[(size_t)i * nb + b];
          u.cache = us[i].cache[n_layers > 1 ? l : b];   // now in its post-append state
          u.q = q[i];
          u.k_u = nullptr;   // staged by the projection
          u.v_u = nullptr;
          u.z = us[i].z;
          u.h = us[i].h[s];
        }
      }
      const bool last_layer = l + 1 == n_layers;
      const int mode = n_layers == 1 ? kProjEuler : (last_layer ? kProjLayerLast : kProjLayer);
      // The last layer of the last step needs no bf16 copy of its result.
      const bool need_zb = !(last_layer && s + 1 == n_steps);
      if ((rc = enqueue_steps(steps.data(), n * nb, L.plans[l], w_o[l], step_ws, nullptr, st,
                              need_zb ? zb.data() : nullptr, nb == 2 ? g.data() : nullptr, mode,
                              n_layers > 1 ? r.data() : nullptr, true)))
        return rc;
    }
  }
  return FMD_OK;
}

static int check_unit_latent(const float* z, int32_t n_video, int32_t n_audio, const float* h,
                             int n_steps, int i) {
  int rc;
  if ((rc = check_tensor(z, i, "z"))) return rc;
  if (n_video < 0 || n_audio < 0 || (int64_t)n_video + n_audio < 1 ||
      (int64_t)n_video + n_audio > (1 << 22))
    return fail(FMD_E_INVAL, "session %d: n_video=%d n_audio=%d (need 1 <= n_q <= 2^22)", i,
                n_video, n_audio);
  if (!h) return fail(FMD_E_INVAL, "session %d: h is NULL", i);
  for (int k = 0; k < n_steps; ++k)
    if (!(h[k] > 0.f && isfinite(h[k])))
      return fail(FMD_E_INVAL, "session %d: h[%d]=%g must be finite and > 0", i, k, h[k]);
  return FMD_OK;
}

static int check_unit_slice(const fmd_kv_cache* c, const void* ks, const void* vs, int64_t T,
                            int i) {
  if (T < 0) return fail(FMD_E_INVAL, "session %d: slice_tokens %lld", i, (long long)T);
  return T > 0 ? check_append(c, ks, vs, T, i) : FMD_OK;
}

// One batched append of every non-empty slice.
static int enqueue_unit_appends(const std::vector<fmd_kv_cache*>& caches,
                                const std::vector<const void*>& ks,
                                const std::vector<const void*>& vs,
                                const std::vector<int64_t>& ts, hipStream_t st) {
  std::vector<fmd_kv_cache*> c;
  std::vector<const void*> k, v;
  std::vector<int64_t> t;
  for (size_t i = 0; i < caches.size(); ++i) {
    if (ts[i] > 0) {
      c.push_back(caches[i]);
      k.push_back(ks[i]);
      v.push_back(vs[i]);
      t.push_back(ts[i]);
    }
  }
  if (c.empty()) return FMD_OK;
  return enqueue_appends(c.data(), k.data(), v.data(), t.data(), (int)c.size(), st);
}

// ---------------------------------------------------------------------------
// The z-dependent solver: Q, K_u, V_u projected from the latent every step.
// ---------------------------------------------------------------------------
static int validate_unit_qkv(const fmd_unit_qkv_io* ss, int n, int n_steps) {
  if (!ss) return fail(FMD_E_INVAL, "sessions is NULL");
  if (n < 1 || n > FMD_MAX_SESSIONS)
    return fail(FMD_E_INVAL, "n_sessions=%d (must be 1..%d)", n, FMD_MAX_SESSIONS);
  if (n_steps < 1) return fail(FMD_E_INVAL, "n_steps=%d (must be >= 1)", n_steps);
  int rc;
  for (int i = 0; i < n; ++i) {
    const fmd_unit_qkv_io& s = ss[i];
    if ((rc = check_cache(s.cache, i))) return rc;
    if (i && (rc = check_same_shape(ss[0].cache, s.cache, i))) return rc;
    for (int j = 0; j < i; ++j)
      if (ss[j].cache == s.cache) return fail(FMD_E_INVAL, "session %d: same cache as %d", i, j);
    if ((rc = check_unit_slice(s.cache, s.k_slice, s.v_slice, s.slice_tokens, i))) return rc;
    if ((rc = check_unit_latent(s.z, s.n_video, s.n_audio, s.h, n_steps, i))) return rc;
  }
  std::vector<ZRange> zs;
  for (int i = 0; i < n; ++i)
    zs.push_back(z_range(ss[i].z, ss[i].n_video + ss[i].n_audio,
                         ss[i].cache->n_heads * ss[i].cache->head_dim, i));
  return check_disjoint_z(zs);
}

static std::vector<SolverUnit> qkv_units(const fmd_unit_qkv_io* ss, int n) {
  std::vector<SolverUnit> us(n);
  for (int i = 0; i < n; ++i)
    us[i] = SolverUnit{{ss[i].cache}, {ss[i].slice_tokens}, ss[i].z, ss[i].n_video,
                       ss[i].n_audio, ss[i].h, 1.f};
  return us;
}

int fmd_unit_qkv_workspace_bytes(const fmd_unit_qkv_io* sessions, int32_t n_sessions,
                                 size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(FMD_E_INVAL, "out_bytes is NULL");
  int rc = validate_unit_qkv(sessions, n_sessions, 1);
  if (rc) return rc;
  SolverLayout L;
  layout_solver(qkv_units(sessions, n_sessions), 1, 1, L);
  *out_bytes = L.bytes;
  return FMD_OK;
}

int fmd_denoise_unit_qkv(fmd_unit_qkv_io* sessions, int32_t n_sessions, int32_t n_steps,
                         const void* w_qkv, const void* w_o, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_unit_qkv(sessions, n_sessions, n_steps);
  if (rc) return rc;
  if ((rc = check_tensor(w_qkv, 0, "w_qkv"))) return rc;
  if ((rc = check_tensor(w_o, 0, "w_o"))) return rc;
  const std::vector<SolverUnit> us = qkv_units(sessions, n_sessions);
  SolverLayout L;
  layout_solver(us, 1, 1, L);
  if ((rc = check_workspace(workspace, workspace_bytes, L.bytes))) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<fmd_kv_cache*> caches;
  std::vector<const void*> ks, vs;
  std::vector<int64_t> ts;
  for (int i = 0; i < n_sessions; ++i) {
    caches.push_back(sessions[i].cache);
    ks.push_back(sessions[i].k_slice);
    vs.push_back(sessions[i].v_slice);
    ts.push_back(sessions[i].slice_tokens);
  }
  if ((rc = enqueue_unit_appends(caches, ks, vs, ts, st))) return rc;
  return run_solver(us, 1, 1, n_steps, &w_qkv, &w_o, static_cast<char*>(workspace), L, st);
}

// ---------------------------------------------------------------------------
// The classifier-free-guided solver: two branches per unit.
// ---------------------------------------------------------------------------
static int validate_unit_cfg(const fmd_unit_cfg_io* ss, int n, int n_steps) {
  if (!ss) return fail(FMD_E_INVAL, "sessions is NULL");
  if (n < 1 || n > FMD_MAX_SESSIONS / 2)
    return fail(FMD_E_INVAL, "n_sessions=%d (must be 1..%d)", n, FMD_MAX_SESSIONS / 2);
  if (n_steps < 1) return fail(FMD_E_INVAL, "n_steps=%d (must be >= 1)", n_steps);
  int rc;
  for (int i = 0; i < n; ++i) {
    const fmd_unit_cfg_io& s = ss[i];
    const fmd_kv_cache* cs[2] = {s.cond, s.uncond};
    for (int b = 0; b < 2; ++b) {
      if ((rc = check_cache(cs[b], i))) return rc;
      if ((rc = check_same_shape(ss[0].cond, cs[b], i))) return rc;
      for (int j = 0; j <= i; ++j)
        for (int c = 0; c < 2; ++c)
          if ((j < i || c < b) && (c ? ss[j].uncond : ss[j].cond) == cs[b])
            return fail(FMD_E_INVAL, "session %d: a cache appears twice", i);
    }
    if ((rc = check_unit_slice(s.cond, s.cond_k_slice, s.cond_v_slice, s.cond_slice_tokens, i)))
      return rc;
    if ((rc = check_unit_slice(s.uncond, s.uncond_k_slice, s.uncond_v_slice,
                               s.uncond_slice_tokens, i)))
      return rc;
    if ((rc = check_unit_latent(s.z, s.n_video, s.n_audio, s.h, n_steps, i))) return rc;
    if (!isfinite(s.guidance))
      return fail(FMD_E_INVAL, "session %d: guidance %g is not finite", i, s.guidance);
  }
  std::vector<ZRange> zs;
  for (int i = 0; i < n; ++i)
    zs.push_back(z_range(ss[i].z, ss[i].n_video + ss[i].n_audio,
                         ss[i].cond->n_heads * ss[i].cond->head_dim, i));
  return check_disjoint_z(zs);
}

static std::vector<SolverUnit> cfg_units(const fmd_unit_cfg_io* ss, int n) {
  std::vector<SolverUnit> us(n);
  for (int i = 0; i < n; ++i)
    us[i] = SolverUnit{{ss[i].cond, ss[i].uncond},
                       {ss[i].cond_slice_tokens, ss[i].uncond_slice_tokens},
                       ss[i].z, ss[i].n_video, ss[i].n_audio, ss[i].h, ss[i].guidance};
  return us;
}

int fmd_unit_cfg_workspace_bytes(const fmd_unit_cfg_io* sessions, int32_t n_sessions,
                                 size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(FMD_E_INVAL, "out_bytes is NULL");
  int rc = validate_unit_cfg(sessions, n_sessions, 1);
  if (rc) return rc;
  SolverLayout L;
  layout_solver(cfg_units(sessions, n_sessions), 2, 1, L);
  *out_bytes = L.bytes;
  return FMD_OK;
}

int fmd_denoise_unit_cfg(fmd_unit_cfg_io* sessions, int32_t n_sessions, int32_t n_steps,
                         const void* w_qkv, const void* w_o, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_unit_cfg(sessions, n_sessions, n_steps);
  if (rc) return rc;
  if ((rc = check_tensor(w_qkv, 0, "w_qkv"))) return rc;
  if ((rc = check_tensor(w_o, 0, "w_o"))) return rc;
  const std::vector<SolverUnit> us = cfg_units(sessions, n_sessions);
  SolverLayout L;
  layout_solver(us, 2, 1, L);
  if ((rc = check_workspace(workspace, workspace_bytes, L.bytes))) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<fmd_kv_cache*> caches;
  std::vector<const void*> ks, vs;
  std::vector<int64_t> ts;
  for (int i = 0; i < n_sessions; ++i) {
    const fmd_unit_cfg_io& s = sessions[i];
    caches.insert(caches.end(), {s.cond, s.uncond});
    ks.insert(ks.end(), {s.cond_k_slice, s.uncond_k_slice});
    vs.insert(vs.end(), {s.cond_v_slice, s.uncond_v_slice});
    ts.insert(ts.end(), {s.cond_slice_tokens, s.uncond_slice_tokens});
  }
  if ((rc = enqueue_unit_appends(caches, ks, vs, ts, st))) return rc;
  return run_solver(us, 2, 1, n_steps, &w_qkv, &w_o, static_cast<char*>(workspace), L, st);
}

// ---------------------------------------------------------------------------
// The layer-stack solver: one ring and one pair of weights per layer.
// ---------------------------------------------------------------------------
static int validate_unit_layers(const fmd_unit_layers_io* ss, int n, int n_layers,
                                int n_steps) {
  if (!ss) return fail(FMD_E_INVAL, "sessions is NULL");
  if (n < 1 || n > FMD_MAX_SESSIONS)
    return fail(FMD_E_INVAL, "n_sessions=%d (must be 1..%d)", n, FMD_MAX_SESSIONS);
  if (n_layers < 1 || n_layers > FMD_MAX_LAYERS)
    return fail(FMD_E_INVAL, "n_layers=%d (must be 1..%d)", n_layers, FMD_MAX_LAYERS);
  if (n_steps < 1) return fail(FMD_E_INVAL, "n_steps=%d (must be >= 1)", n_steps);
  int rc;
  std::vector<const fmd_kv_cache*> seen;
  for (int i = 0; i < n; ++i) {
    const fmd_unit_layers_io& s = ss[i];
    if (!s.caches) return fail(FMD_E_INVAL, "session %d: caches is NULL", i);
    if (s.slice_tokens < 0)
      return fail(FMD_E_INVAL, "session %d: slice_tokens %lld", i, (long long)s.slice_tokens);
    if (s.slice_tokens > 0 && (!s.k_slices || !s.v_slices))
      return fail(FMD_E_INVAL, "session %d: slice arrays are NULL", i);
    for (int l = 0; l < n_layers; ++l) {
      if ((rc = check_cache(s.caches[l], i))) return rc;
      if ((rc = check_same_shape(ss[0].caches[0], s.caches[l], i))) return rc;
      if (s.slice_tokens > 0 &&
          (rc = check_append(s.caches[l], s.k_slices[l], s.v_slices[l], s.slice_tokens, i)))
        return rc;
      seen.push_back(s.caches[l]);
    }
    if ((rc = check_unit_latent(s.z, s.n_video, s.n_audio, s.h, n_steps, i))) return rc;
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(FMD_E_INVAL, "a cache appears twice among the sessions' layers");
  std::vector<ZRange> zs;
  for (int i = 0; i < n; ++i)
    zs.push_back(z_range(ss[i].z, ss[i].n_video + ss[i].n_audio,
                         ss[i].caches[0]->n_heads * ss[i].caches[0]->head_dim, i));
  return check_disjoint_z(zs);
}

static std::vector<SolverUnit> layer_units(const fmd_unit_layers_io* ss, int n, int n_layers) {
  std::vector<SolverUnit> us(n);
  for (int i = 0; i < n; ++i)
    us[i] = SolverUnit{std::vector<fmd_kv_cache*>(ss[i].caches, ss[i].caches + n_layers),
                       std::vector<int64_t>(n_layers, ss[i].slice_tokens), ss[i].z,
                       ss[i].n_video, ss[i].n_audio, ss[i].h, 1.f};
  return us;
}

int fmd_unit_layers_workspace_bytes(const fmd_unit_layers_io* sessions, int32_t n_sessions,
                                    int32_t n_layers, size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(FMD_E_INVAL, "out_bytes is NULL");
  int rc = validate_unit_layers(sessions, n_sessions, n_layers, 1);
  if (rc) return rc;
  SolverLayout L;
  layout_solver(layer_units(sessions, n_sessions, n_layers), 1, n_layers, L);
  *out_bytes = L.bytes;
  return FMD_OK;
}

int fmd_denoise_unit_layers(fmd_unit_layers_io* sessions, int32_t n_sessions, int32_t n_layers,
                            int32_t n_steps, const void* const* w_qkv, const void* const* w_o,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_unit_layers(sessions, n_sessions, n_layers, n_steps);
  if (rc) return rc;
  if (!w_qkv || !w_o) return fail(FMD_E_INVAL, "weight arrays are NULL");
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_tensor(w_qkv[l], l, "w_qkv"))) return rc;
    if ((rc = check_tensor(w_o[l], l, "w_o"))) return rc;
  }
  const std::vector<SolverUnit> us = layer_units(sessions, n_sessions, n_layers);
  SolverLayout L;
  layout_solver(us, 1, n_layers, L);
  if ((rc = check_workspace(workspace, workspace_bytes, L.bytes))) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<fmd_kv_cache*> caches;
  std::vector<const void*> ks, vs;
  std::vector<int64_t> ts;
  for (int i = 0; i < n_sessions; ++i) {
    const fmd_unit_layers_io& s = sessions[i];
    for (int l = 0; l < n_layers; ++l) {
      caches.push_back(s.caches[l]);
      ks.push_back(s.slice_tokens > 0 ? s.k_slices[l] : nullptr);
      vs.push_back(s.slice_tokens > 0 ? s.v_slices[l] : nullptr);
      ts.push_back(s.slice_tokens);
    }
  }
  if ((rc = enqueue_unit_appends(caches, ks, vs, ts, st))) return rc;
  return run_solver(us, 1, n_layers, n_steps, w_qkv, w_o, static_cast<char*>(workspace), L, st);
}

int fmd_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof.clear();
  g_prof_on = enable != 0;
  return FMD_OK;
}

int fmd_profile_select(uint32_t class_mask) {
  if (class_mask >> FMD_KERNEL_COUNT)
    return fail(FMD_E_INVAL, "class mask 0x%x has bits at or above %d", class_mask,
                FMD_KERNEL_COUNT);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = class_mask;
  return FMD_OK;
}

int fmd_profile_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(FMD_E_INVAL, "NULL output");
  if (kernel_class < 0 || kernel_class >= FMD_KERNEL_COUNT)
    return fail(FMD_E_INVAL, "kernel class %d", kernel_class);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0;
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (r.cls != kernel_class) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return fail(FMD_E_HIP, "event wait: %s", hipGetErrorString(e));
    float ms = 0;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(FMD_E_HIP, "event time: %s", hipGetErrorString(e));
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return FMD_OK;
}

}  // extern "C"
