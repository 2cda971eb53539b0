// Host-only driver of the wvd C ABI in dry-run mode, built with the address
// and undefined-behaviour sanitizers on the host code (tests/test_sanitizers.py).
// It walks the full launch schedule of every workload (and the argument
// checks of every entry point) without a GPU: no device pointer is ever
// dereferenced in dry-run mode, so the placeholders below are never touched.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "wvd.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
    ++g_failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* fake(uintptr_t k) { return reinterpret_cast<void*>(k << 20); }

struct Case {
  int c, h, w, n_weights;
  std::vector<int> Ts;
};

void run_case(const Case& k) {
  size_t nprep = 0;
  EXPECT(wvd_prepared_bytes_n(k.c, k.h, k.w, k.n_weights, &nprep) == WVD_OK && nprep > 0);
  std::vector<const void*> ws(k.n_weights, fake(1));
  wvd_plan* plan = nullptr;
  EXPECT(wvd_prepare(k.c, k.h, k.w, ws.data(), k.n_weights, WVD_DTYPE_BF16, fake(2), nprep, nullptr, &plan) ==
         WVD_OK);
  if (!plan) return;
  EXPECT(wvd_prepare(k.c, k.h, k.w, ws.data(), k.n_weights, WVD_DTYPE_BF16, fake(2), nprep - 1, nullptr, &plan) ==
         WVD_ENOSPACE);
  size_t nstate = 0;
  EXPECT(wvd_state_bytes(plan, &nstate) == WVD_OK && nstate > 0);
  for (int T : k.Ts) {
    for (int P : {1, 2, 3, 4, 8, 16, 64}) {
      size_t nws = 0;
      EXPECT(wvd_workspace_bytes(plan, T, P, &nws) == WVD_OK && nws > 0);
      EXPECT(wvd_decode(plan, fake(3), WVD_DTYPE_BF16, T, P, fake(4), fake(5), nws, nullptr) == WVD_OK);
      EXPECT(wvd_last_launch_count(plan) > 0);
      EXPECT(wvd_decode(plan, fake(3), WVD_DTYPE_F32, T, P, fake(4), fake(5), nws - 1, nullptr) == WVD_ENOSPACE);
      const int st = wvd_decode_static(plan, fake(3), WVD_DTYPE_BF16, T, P, fake(4), nullptr);
      EXPECT(st == (nws <= WVD_STATIC_WORKSPACE_BYTES ? WVD_OK : WVD_ENOSPACE));
      // the clip in two chunks
      if (T >= 2) {
        const int a = T / 2;
        size_t nc = 0;
        EXPECT(wvd_chunk_workspace_bytes(plan, a, P, &nc) == WVD_OK);
        EXPECT(wvd_decode_chunk(plan, fake(3), WVD_DTYPE_BF16, a, 0, P, fake(6), nstate, fake(4), fake(5), nc,
                                nullptr) == WVD_OK);
        EXPECT(wvd_chunk_workspace_bytes(plan, T - a, P, &nc) == WVD_OK);
        EXPECT(wvd_decode_chunk(plan, fake(3), WVD_DTYPE_BF16, T - a, a, P, fake(6), nstate, fake(4), fake(5), nc,
                                nullptr) == WVD_OK);
        EXPECT(wvd_decode_chunk(plan, fake(3), WVD_DTYPE_BF16, T - a, a, P, fake(6), nstate - 1, fake(4), fake(5),
                                nc, nullptr) == WVD_ENOSPACE);
      }
    }
  }
  // argument checks
  size_t n = 0;
  EXPECT(wvd_workspace_bytes(plan, 0, 1, &n) == WVD_EINVAL);
  EXPECT(wvd_workspace_bytes(plan, 1, 0, &n) == WVD_EINVAL);
  EXPECT(wvd_decode(plan, nullptr, 0, 1, 1, fake(4), fake(5), 1, nullptr) == WVD_EINVAL);
  EXPECT(wvd_decode(plan, fake(3), 7, 1, 1, fake(4), fake(5), 1, nullptr) == WVD_EINVAL);
  EXPECT(wvd_decode(plan, fake(3), 0, 1, 1, fake(4), reinterpret_cast<void*>(uintptr_t(8)), 1 << 30, nullptr) ==
         WVD_EINVAL);
  EXPECT(wvd_decode_chunk(plan, fake(3), 0, 1, -1, 1, fake(6), nstate, fake(4), fake(5), 1, nullptr) == WVD_EINVAL);
  double ms[6], fl[6];
  long long cnt[6];
  EXPECT(wvd_profile_enable(plan, 0) == WVD_OK);
  EXPECT(wvd_profile_read(plan, ms, fl, cnt, 6) == WVD_OK);
  unsigned flags = 7;
  EXPECT(wvd_range_flags(nullptr, 1, &flags) == WVD_OK && flags == 0);
  wvd_destroy(plan);
}

}  // namespace

int main() {
  wvd_set_dry_run(1);
  const std::vector<Case> cases = {
      {16, 4, 6, WVD_NUM_WEIGHTS, {1, 2, 5}},
      {16, 4, 6, WVD_NUM_WEIGHTS_DEEP, {1, 2, 5}},
      {64, 22, 39, WVD_NUM_WEIGHTS, {1, 3}},
      {64, 22, 39, WVD_NUM_WEIGHTS_DEEP, {3}},
      {256, 2, 3, WVD_NUM_WEIGHTS, {1, 3}},
      {256, 44, 78, WVD_NUM_WEIGHTS, {1, 2, 13, 49, 121}},
      {256, 44, 78, WVD_NUM_WEIGHTS_DEEP, {2, 49}},
  };
  for (const Case& k : cases) run_case(k);
  // entry points that must reject without a plan
  size_t n = 0;
  EXPECT(wvd_prepared_bytes(24, 4, 6, &n) == WVD_EUNSUPPORTED);
  EXPECT(wvd_prepared_bytes(16, 4, 6, nullptr) == WVD_EINVAL);
  EXPECT(wvd_workspace_bytes(nullptr, 1, 1, &n) == WVD_EINVAL);
  EXPECT(wvd_decode_static(nullptr, fake(3), 0, 1, 1, fake(4), nullptr) == WVD_EINVAL);
  EXPECT(wvd_last_launch_count(nullptr) == -1);
  wvd_destroy(nullptr);
  EXPECT(wvd_status_string(-5)[0] != 0 && wvd_last_error() != nullptr);
  if (g_failures) {
    std::fprintf(stderr, "%d failure(s)\n", g_failures);
    return 1;
  }
  std::printf("dry-run schedule of %zu workloads clean\n", cases.size());
  return 0;
}
