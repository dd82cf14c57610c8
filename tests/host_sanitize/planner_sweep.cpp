// Seeded sweep of libfmd's host code through its C ABI, for a build whose host
// code runs under AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing
// here touches a GPU: only the workspace planners (ring segments, key-split
// choice, the per-XCD dispatch simulation, workspace layout) and the argument
// validation run, on fake 256-byte-aligned device addresses that are never
// dereferenced.
//
// Checks beside the sanitizers:
//  - every planner call on a valid description succeeds and is deterministic
//    (the same bytes twice);
//  - the unit planner agrees with the step planner on the post-append state
//    (one step; the unit keys read in place take no staging room);
//  - the z-dependent planner needs at least the plain one's bytes (the same
//    plan plus its slabs), the guided one at least its four slabs per unit;
//  - invalid descriptions are rejected with the documented status and leave
//    the caches' (len, head) untouched.
// Prints one summary line; exit status 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "../../include/fmd.h"

namespace {

uintptr_t g_next = 0x100000000ull;   // fake device addresses, 256-byte aligned
void* fake(size_t bytes) {
  void* p = reinterpret_cast<void*>(g_next);
  g_next += (bytes + 4095) & ~size_t(4095);
  return p;
}

int g_fail = 0;
#define CHECK(cond, ...)                                     \
  do {                                                       \
    if (!(cond)) {                                           \
      fprintf(stderr, "check failed: %s: ", #cond);          \
      fprintf(stderr, __VA_ARGS__);                          \
      fprintf(stderr, " (%s)\n", fmd_last_error());          \
      ++g_fail;                                              \
    }                                                        \
  } while (0)

struct Session {
  fmd_kv_cache cache;
  fmd_kv_cache cache_u;   // unconditional branch (guided planner)
  int64_t slice;
  int32_t n_video, n_audio;
};

Session random_session(std::mt19937_64& rng, int H, int hd) {
  Session s{};
  auto U = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  const int64_t max_cap = (int64_t)((1u << 31) - 1) / (hd * 2);
  int64_t cap = 16 * U(1, 4096);
  if (U(0, 15) == 0) cap = (max_cap / 16) * 16;           // largest ring
  s.cache = {fake(1), fake(1), H, hd, cap, 0, 0};
  const int kind = (int)U(0, 3);
  s.cache.len_tokens = kind == 0 ? 0 : (kind == 1 ? cap : U(0, cap));
  s.cache.head_tokens = U(0, cap - 1);
  s.cache_u = s.cache;
  s.cache_u.k = fake(1);
  s.cache_u.v = fake(1);
  s.slice = U(0, 2) == 0 ? 0 : U(1, cap < 4096 ? cap : 4096);
  s.n_video = (int32_t)U(0, 3000);
  s.n_audio = (int32_t)U(s.n_video == 0 ? 1 : 0, 16);
  return s;
}

void post_append(const Session& s, fmd_kv_cache* out) {
  *out = s.cache;
  if (s.slice > 0) {
    out->head_tokens = (s.cache.head_tokens + s.slice) % s.cache.cap_tokens;
    out->len_tokens = s.cache.len_tokens + s.slice < s.cache.cap_tokens
                          ? s.cache.len_tokens + s.slice
                          : s.cache.cap_tokens;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 300;
  std::mt19937_64 rng(20261203);
  float h[8] = {0.25f, 0.25f, 0.25f, 0.25f, 0.1f, 0.1f, 0.1f, 0.1f};
  int64_t planned = 0, rejected = 0;
  for (int c = 0; c < cases; ++c) {
    const int hds[2] = {64, 128};
    const int hd = hds[rng() % 2];
    const int Hs[6] = {1, 2, 5, 12, 40, 64};
    const int H = Hs[rng() % 6];
    const int n = 1 + (int)(rng() % (c % 7 == 0 ? 64 : 8));   // sometimes the maximum batch
    std::vector<Session> ss;
    for (int i = 0; i < n; ++i) ss.push_back(random_session(rng, H, hd));
    const int64_t d = (int64_t)H * hd;

    // Unit planner vs step planner on the post-append state.
    std::vector<fmd_unit_io> io(n);
    std::vector<fmd_kv_cache> after(n);
    std::vector<fmd_unit_step> st(n);
    for (int i = 0; i < n; ++i) {
      const Session& s = ss[i];
      const int64_t nq = (int64_t)s.n_video + s.n_audio;
      io[i] = {&ss[i].cache, fake(1), fake(1), s.slice, fake(1), fake(1), fake(1), 0,
               static_cast<float*>(fake((size_t)(nq * d * 4))), s.n_video, s.n_audio, h};
      post_append(s, &after[i]);
      st[i] = {&after[i], io[i].q, io[i].k_u, io[i].v_u, io[i].z, s.n_video, s.n_audio, 0.5f};
    }
    size_t a = 0, b = 0, a2 = 0;
    int rc = fmd_unit_workspace_bytes(io.data(), n, 1, &a);
    CHECK(rc == FMD_OK, "case %d: unit planner rc=%d", c, rc);
    rc = fmd_workspace_bytes(st.data(), n, &b);
    CHECK(rc == FMD_OK, "case %d: step planner rc=%d", c, rc);
    // One step: the step planner's regions, less the staging room of unit
    // keys that the attention reads in place (n_q * d * 2 bytes below 2^31).
    size_t keys_in_place = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t nq = (int64_t)ss[i].n_video + ss[i].n_audio;
      if (nq * d * 2 < ((int64_t)1 << 31))
        keys_in_place += ((size_t)H * ((nq + 15) & ~15) * hd * 2 + 255) & ~(size_t)255;
    }
    CHECK(a + keys_in_place == b, "case %d: unit %zu + keys %zu vs step %zu bytes", c, a,
          keys_in_place, b);
    rc = fmd_unit_workspace_bytes(io.data(), n, 1, &a2);
    CHECK(rc == FMD_OK && a2 == a, "case %d: planner not deterministic", c);
    int64_t min_bytes = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t nq = (int64_t)ss[i].n_video + ss[i].n_audio;
      min_bytes += (nq * d * 2 < ((int64_t)1 << 31) ? 2 : 3) * nq * d * 2;   // [unit K,] unit V, O
    }
    CHECK((int64_t)a >= min_bytes, "case %d: %zu bytes < %lld", c, a, (long long)min_bytes);
    // Four steps with their own inputs: every step's values (and keys not
    // read in place) are staged, and the attention of B steps (the largest
    // divisor of 4 with B * n <= 16) runs as one launch, each with its own O.
    {
      std::vector<fmd_unit_io> io4(io);
      for (int i = 0; i < n; ++i)
        io4[i].step_stride_elems = ((int64_t)ss[i].n_video + ss[i].n_audio) * d;
      size_t a4 = 0, a4b = 0;
      rc = fmd_unit_workspace_bytes(io4.data(), n, 4, &a4);
      CHECK(rc == FMD_OK, "case %d: 4-step unit planner rc=%d", c, rc);
      rc = fmd_unit_workspace_bytes(io4.data(), n, 4, &a4b);
      CHECK(rc == FMD_OK && a4b == a4, "case %d: 4-step planner not deterministic", c);
      const int B = n <= 4 ? 4 : (n <= 8 ? 2 : 1);
      int64_t min4 = 0;
      for (int i = 0; i < n; ++i) {
        const int64_t nq = (int64_t)ss[i].n_video + ss[i].n_audio;
        min4 += (4 * (nq * d * 2 < ((int64_t)1 << 31) ? 1 : 2) + B) * nq * d * 2;
      }
      CHECK((int64_t)a4 >= min4, "case %d: 4-step %zu bytes < %lld", c, a4, (long long)min4);
    }
    ++planned;

    // The z-dependent and layer-stack planners.
    std::vector<fmd_unit_qkv_io> qio(n);
    for (int i = 0; i < n; ++i)
      qio[i] = {&ss[i].cache, io[i].k_slice, io[i].v_slice, ss[i].slice, io[i].z,
                ss[i].n_video, ss[i].n_audio, h};
    size_t q = 0;
    rc = fmd_unit_qkv_workspace_bytes(qio.data(), n, &q);
    CHECK(rc == FMD_OK && q >= a, "case %d: qkv planner rc=%d %zu < %zu", c, rc, q, a);
    if (n <= FMD_MAX_SESSIONS / 2) {
      std::vector<fmd_unit_cfg_io> cio(n);
      for (int i = 0; i < n; ++i)
        cio[i] = {&ss[i].cache, &ss[i].cache_u, io[i].k_slice, io[i].v_slice, ss[i].slice,
                  fake(1), fake(1), ss[i].slice, io[i].z, ss[i].n_video, ss[i].n_audio, h,
                  3.0f};
      size_t g = 0;
      rc = fmd_unit_cfg_workspace_bytes(cio.data(), n, &g);
      // Its own key-split choice may differ from the single-branch one; it
      // holds at least each unit's four bf16 [n_q][d] slabs.
      int64_t slabs = 0;
      for (int i = 0; i < n; ++i) slabs += 4 * ((int64_t)ss[i].n_video + ss[i].n_audio) * d * 2;
      CHECK(rc == FMD_OK && (int64_t)g >= slabs, "case %d: guided planner rc=%d %zu < %lld", c,
            rc, g, (long long)slabs);
    }
    {
      const int L = 1 + (int)(rng() % 3);
      std::vector<std::vector<fmd_kv_cache>> rings(n, std::vector<fmd_kv_cache>(L));
      std::vector<std::vector<fmd_kv_cache*>> rp(n, std::vector<fmd_kv_cache*>(L));
      std::vector<std::vector<const void*>> sk(n, std::vector<const void*>(L));
      std::vector<fmd_unit_layers_io> lio(n);
      for (int i = 0; i < n; ++i) {
        for (int l = 0; l < L; ++l) {
          rings[i][l] = ss[i].cache;
          rings[i][l].k = fake(1);
          rings[i][l].v = fake(1);
          rp[i][l] = &rings[i][l];
          sk[i][l] = fake(1);
        }
        lio[i] = {rp[i].data(), sk[i].data(), sk[i].data(), ss[i].slice, io[i].z,
                  ss[i].n_video, ss[i].n_audio, h};
      }
      size_t lb = 0;
      rc = fmd_unit_layers_workspace_bytes(lio.data(), n, L, &lb);
      CHECK(rc == FMD_OK, "case %d: layer planner rc=%d", c, rc);
    }

    // Rejections leave every cache's state as it was.
    std::vector<fmd_kv_cache> before(n);
    for (int i = 0; i < n; ++i) before[i] = ss[i].cache;
    const int victim = (int)(rng() % n);
    const int what = (int)(rng() % 5);
    fmd_unit_io saved = io[victim];
    int want = FMD_E_INVAL;
    switch (what) {
      case 0: io[victim].z = nullptr; break;
      case 1: io[victim].q = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(io[victim].q) + 8);
              want = FMD_E_ALIGN; break;
      case 2: io[victim].slice_tokens = ss[victim].cache.cap_tokens + 1; want = FMD_E_CAPACITY; break;
      case 3: io[victim].n_video = -1; break;
      default: io[victim].h = nullptr; break;
    }
    rc = fmd_denoise_unit(io.data(), n, 4, fake(1), fake(1), (size_t)1 << 40, nullptr);
    CHECK(rc == want, "case %d: rejection %d gave %d, want %d", c, what, rc, want);
    rc = fmd_denoise_unit_noalloc(io.data(), n, 4, fake(1), nullptr);
    CHECK(rc == want, "case %d: no-alloc rejection %d gave %d, want %d", c, what, rc, want);
    for (int i = 0; i < n; ++i)
      CHECK(memcmp(&before[i], &ss[i].cache, sizeof(fmd_kv_cache)) == 0,
            "case %d: session %d state changed by a rejected call", c, i);
    io[victim] = saved;
    ++rejected;
  }
  printf("planner sweep: %lld planned, %lld rejected, %d failed checks\n", (long long)planned,
         (long long)rejected, g_fail);
  return g_fail ? 1 : 0;
}
