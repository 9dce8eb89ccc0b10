// abi_driver.cpp -- drives every entry point of la_api.cpp's host path (argument
// validation, workspace sizes, launch plans) under the host sanitizers, with
// the stand-in launchers of stub_launchers.cpp: no GPU, no device memory.
// Device pointers are fake aligned addresses that the host code never reads.
// Exits non-zero on the first failed expectation; the sanitizers abort on
// any memory error or undefined behaviour.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "linattn.h"

namespace la {
extern int g_launches;
}

static int g_fail = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,    \
                   __LINE__, #cond);                                       \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static void* P(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x10000000 + 0x100000 * i); }
static float* F(uintptr_t i) { return static_cast<float*>(P(i)); }

static la_shape shape(int64_t B, int64_t H, int64_t L, int d, int nseg, int dtype, int split) {
  la_shape s;
  std::memset(&s, 0, sizeof(s));
  s.B = B;
  s.H = H;
  s.L = L;
  s.dk = s.dv = d;
  s.nseg = nseg;
  s.dtype = dtype;
  s.split = split;
  return s;
}

// An invalid call must fail with `want`, set la_last_error and launch nothing.
static void expect_reject(la_status got, la_status want, int launches_before, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                 la_last_error());
    ++g_fail;
  }
  EXPECT(la::g_launches == launches_before);
  EXPECT(std::strncmp(la_last_error(), la_status_str(want), std::strlen(la_status_str(want))) == 0);
}

// Every entry point on one valid shape with workspaces of the queried sizes.
static void run_all(const la_shape& s, bool expect_ok) {
  const size_t wf = la_fwd_workspace_bytes(&s), wb = la_bwd_workspace_bytes(&s);
  const size_t wg = la_fwd_gated_workspace_bytes(&s), wgb = la_bwd_gated_workspace_bytes(&s);
  const size_t wt = la_decay_grad_workspace_bytes(&s);
  la_status r[8];
  r[0] = la_chunk_fwd(&s, P(1), P(2), P(3), F(4), F(5), P(6), F(7), wf ? P(8) : nullptr, wf, nullptr);
  r[1] = la_chunk_fwd(&s, P(1), P(2), P(3), F(4), nullptr, nullptr, F(7), wf ? P(8) : nullptr, wf,
                      nullptr);
  r[2] = la_chunk_bwd(&s, P(1), P(2), P(3), F(4), F(5), P(9), F(10), P(11), P(12), P(13), F(14),
                      wb ? P(15) : nullptr, wb, nullptr);
  r[3] = la_chunk_bwd_from_fwd(&s, P(1), P(2), P(3), F(4), nullptr, P(9), nullptr,
                               wf ? P(8) : nullptr, P(11), P(12), P(13), nullptr,
                               wb ? P(15) : nullptr, wb, nullptr);
  r[4] = la_chunk_fwd_gated(&s, P(1), P(2), P(3), F(16), F(5), P(6), F(7), wg ? P(8) : nullptr, wg,
                            nullptr);
  r[5] = la_chunk_bwd_gated(&s, P(1), P(2), P(3), F(16), F(5), P(9), F(10), P(11), P(12), P(13),
                            F(14), F(17), wgb ? P(15) : nullptr, wgb, nullptr);
  r[6] = la_decay_grad(&s, P(1), P(2), P(3), F(4), F(5), P(9), F(10), F(18), wt ? P(15) : nullptr, wt,
                       nullptr);
  r[7] = la_step(s.B, s.H, s.dk, s.dv, s.dtype, P(1), P(2), P(3), F(4), F(5), F(19), P(6), nullptr);
  for (int i = 0; i < 8; ++i) {
    if (expect_ok && r[i] != LA_OK) {
      std::fprintf(stderr, "entry %d rejected B=%lld H=%lld L=%lld d=%d nseg=%d dtype=%d split=%d: %s\n",
                   i, (long long)s.B, (long long)s.H, (long long)s.L, s.dk, s.nseg, s.dtype, s.split,
                   la_last_error());
      ++g_fail;
    }
  }
}

int main() {
  // ---- valid shapes: every entry point accepts them and plans launches
  const int64_t Ls[] = {0, 1, 63, 64, 65, 1000, 4096, 16384, 65536};
  const int ds[] = {64, 128};
  const int splits[] = {0, 1, 2, 3, 7, 64};
  for (int64_t L : Ls)
    for (int d : ds)
      for (int split : splits)
        for (int dtype = 0; dtype < 2; ++dtype) {
          const int before = la::g_launches;
          run_all(shape(2, 3, L, d, 1, dtype, split), true);
          if (L > 0) EXPECT(la::g_launches > before);
        }
  run_all(shape(1, 32, 65536, 128, 1, 0, 0), true);
  run_all(shape(1, 16, 1 << 20, 128, 64, 0, 0), true);
  run_all(shape(1, 16, 262144, 128, 1, 0, 0), true);
  run_all(shape(3, 2, 64 * 12, 64, 4, 1, 2), true);

  // ---- invalid shapes and arguments: rejected, nothing launched
  int b = la::g_launches;
  la_shape s = shape(1, 2, 128, 64, 1, 0, 0);
  expect_reject(la_chunk_fwd(nullptr, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, nullptr, 0,
                             nullptr),
                LA_ERR_INVALID_ARG, b, "null shape");
  la_shape bad = s;
  bad.B = -1;
  expect_reject(la_chunk_fwd(&bad, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, nullptr, 0, nullptr),
                LA_ERR_INVALID_ARG, b, "negative B");
  bad = s;
  bad.reserved = 1;
  expect_reject(la_chunk_bwd(&bad, P(1), P(2), P(3), F(4), nullptr, P(9), nullptr, P(11), P(12), P(13),
                             nullptr, nullptr, 0, nullptr),
                LA_ERR_INVALID_ARG, b, "reserved");
  bad = s;
  bad.dk = 96;
  bad.dv = 96;
  expect_reject(la_chunk_fwd_gated(&bad, P(1), P(2), P(3), F(16), nullptr, P(6), nullptr, nullptr, 0,
                                   nullptr),
                LA_ERR_UNSUPPORTED, b, "d = 96");
  bad = s;
  bad.L = 100;
  bad.nseg = 3;
  expect_reject(la_decay_grad(&bad, P(1), P(2), P(3), F(4), nullptr, P(9), nullptr, F(18), nullptr, 0,
                              nullptr),
                LA_ERR_INVALID_ARG, b, "L % nseg");
  expect_reject(la_chunk_fwd(&s, P(1), nullptr, P(3), F(4), nullptr, P(6), nullptr, nullptr, 0, nullptr),
                LA_ERR_INVALID_ARG, b, "K null");
  expect_reject(la_chunk_fwd(&s, P(1), P(2), (char*)P(3) + 4, F(4), nullptr, P(6), nullptr, nullptr, 0,
                             nullptr),
                LA_ERR_INVALID_ARG, b, "V misaligned");
  la_shape s3 = shape(1, 2, 640, 64, 1, 0, 3);
  expect_reject(la_chunk_fwd(&s3, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, nullptr, 0, nullptr),
                LA_ERR_WORKSPACE, b, "workspace missing");
  expect_reject(la_chunk_fwd(&s3, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, P(8),
                             la_fwd_workspace_bytes(&s3) - 1, nullptr),
                LA_ERR_WORKSPACE, b, "workspace short");
  expect_reject(la_chunk_bwd_gated(&s3, P(1), P(2), P(3), F(16), nullptr, P(9), nullptr, P(11), P(12),
                                   P(13), nullptr, nullptr, P(15), la_bwd_gated_workspace_bytes(&s3) - 256,
                                   nullptr),
                LA_ERR_WORKSPACE, b, "gated workspace short");
  expect_reject(la_state_scan(1, 2, 3, 64, 64, nullptr, F(4), 64, nullptr, F(2), nullptr, 0, nullptr),
                LA_ERR_INVALID_ARG, b, "scan dS null");
  expect_reject(la_state_scan_gated(1, 2, -1, 64, 64, F(1), F(2), nullptr, F(3), nullptr, 0, nullptr),
                LA_ERR_INVALID_ARG, b, "scan P < 0");
  expect_reject(la_step(2, 3, 64, 64, 0, P(1), P(2), P(3), F(4), F(5), F(5) + 16, P(6), nullptr),
                LA_ERR_INVALID_ARG, b, "step S overlaps S_out");
  // huge shapes: rejected by the size checks, no overflow on the way
  const int64_t big[] = {(int64_t)1 << 30, (int64_t)1 << 40, INT64_MAX / 2, INT64_MAX};
  for (int64_t x : big) {
    la_shape h = shape(x, 3, 1 << 16, 128, 1, 0, 0);
    EXPECT(la_fwd_workspace_bytes(&h) == 0);
    EXPECT(la_bwd_gated_workspace_bytes(&h) == 0);
    EXPECT(la_chunk_fwd(&h, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, nullptr, 0, nullptr) !=
           LA_OK);
    h = shape(1, 1, x, 128, 1, 0, 0);
    EXPECT(la_chunk_fwd(&h, P(1), P(2), P(3), F(4), nullptr, P(6), nullptr, nullptr, 0, nullptr) !=
           LA_OK);
    EXPECT(la_state_scan(x, 7, 3, 128, 128, F(1), F(2), 64, nullptr, F(3), nullptr, 0, nullptr) != LA_OK);
    EXPECT(la_step(x, 5, 128, 128, 0, P(1), P(2), P(3), F(4), nullptr, F(5), nullptr, nullptr) != LA_OK);
  }
  EXPECT(la::g_launches == b);

  // ---- a deterministic sweep of random shapes: every call either plans
  // launches or is rejected by a check; the sanitizers watch the arithmetic
  uint64_t st = 0x9E3779B97F4A7C15ull;
  auto rnd = [&](uint64_t n) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (st >> 33) % n;
  };
  int accepted = 0;
  for (int i = 0; i < 3000; ++i) {
    const int64_t B = (int64_t)rnd(5), H = (int64_t)rnd(40);
    const int nseg = 1 + (int)rnd(4);
    const int64_t L = (int64_t)rnd(3) == 0 ? (int64_t)rnd(200000) * nseg : (int64_t)rnd(5000) * nseg;
    const int d = rnd(5) == 0 ? 96 : (rnd(2) ? 64 : 128);
    la_shape r = shape(B, H, L, d, nseg, (int)rnd(3) == 2 ? 7 : (int)rnd(2), (int)rnd(10));
    const la_status st0 = la_chunk_fwd(&r, P(1), P(2), P(3), F(4), F(5), P(6), F(7), P(8),
                                       la_fwd_workspace_bytes(&r), nullptr);
    run_all(r, false);
    if (st0 == LA_OK) ++accepted;
  }
  EXPECT(accepted > 500);
  std::printf("abi_driver: %d launches planned, %d random shapes accepted, %d failures\n",
              la::g_launches, accepted, g_fail);
  return g_fail ? 1 : 0;
}
