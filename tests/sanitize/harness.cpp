// Drives every C-ABI entry point of libflashbev's host layer through valid and
// invalid arguments, built with AddressSanitizer and UndefinedBehaviorSanitizer
// against host-only launcher stand-ins (launch_stubs.cpp).  Pointers are fake
// addresses that the host layer only compares with NULL or checks for alignment.
// Prints "ok" and returns 0 when every expectation holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <thread>

#include <hip/hip_runtime.h>

#include "../../include/flashbev.h"

extern int stub_launches;
extern hipError_t stub_status;

static int failures = 0;

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, fbev_last_error()); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static void* const P = reinterpret_cast<void*>(0x10000);
static float* const FP = reinterpret_cast<float*>(0x10000);
static const fbev_range RNG = {-50.f, 50.f, -50.f, 50.f, -5.f, 3.f};

// The status of `call`, and whether it reached a launcher.
template <class F>
static fbev_status run(F call, bool* launched) {
  const int before = stub_launches;
  const fbev_status s = call();
  *launched = stub_launches != before;
  return s;
}

static void expect_rejected_impl(fbev_status s, bool launched, fbev_status want) {
  EXPECT(s == want);
  EXPECT(!launched);
  EXPECT(std::strlen(fbev_last_error()) > 0);
}

// the call runs (and sets `l`) before `l` is read
#define expect_rejected(call, l, want)            \
  do {                                            \
    const fbev_status s_ = (call);                \
    expect_rejected_impl(s_, (l), (want));        \
  } while (0)

int main() {
  bool l = false;
  const int32_t big = std::numeric_limits<int32_t>::max(), neg = std::numeric_limits<int32_t>::min();
  const float nan = std::nanf(""), inf = std::numeric_limits<float>::infinity();

  // ---- fbev_forward / fbev_backward
  fbev_feat_desc fd = {1, 6, 64, 16, 44};
  auto fwd = [&](fbev_feat_desc d, fbev_range r, int X, int Y, int Z, const void* feat, float* out, int dt) {
    return run([&] { return fbev_forward(feat, (fbev_dtype)dt, d, FP, FP, FP, r, X, Y, Z, out, nullptr, nullptr); },
               &l);
  };
  EXPECT(fwd(fd, RNG, 200, 200, 8, P, FP, 0) == FBEV_OK && l);
  EXPECT(fwd(fd, RNG, 200, 200, 8, P, FP, 1) == FBEV_OK && l);
  const fbev_feat_desc bad_fd[] = {{-1, 6, 64, 16, 44}, {1, 65, 64, 16, 44}, {1, 6, 64, neg, 44},
                                   {big, big, big, big, big}, {1, 6, -64, 16, 44}};
  for (const auto& d : bad_fd) {
    const fbev_status s = fwd(d, RNG, 200, 200, 8, P, FP, 0);
    EXPECT(s != FBEV_OK && !l);
  }
  for (int X : {-1, neg, big, 65537}) expect_rejected(fwd(fd, RNG, X, 200, 8, P, FP, 0), l, FBEV_ERR_INVALID_ARGUMENT);
  const fbev_range bad_r[] = {{nan, 50.f, -50.f, 50.f, -5.f, 3.f}, {-50.f, inf, -50.f, 50.f, -5.f, 3.f},
                              {10.f, -10.f, -50.f, 50.f, -5.f, 3.f}, {-50.f, 50.f, -50.f, 50.f, 3.f, 3.f}};
  for (const auto& r : bad_r) expect_rejected(fwd(fd, r, 200, 200, 8, P, FP, 0), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fwd(fd, RNG, 200, 200, 8, nullptr, FP, 0), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fwd(fd, RNG, 200, 200, 8, P, nullptr, 0), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fwd(fd, RNG, 200, 200, 8, P, FP, 9), l, FBEV_ERR_UNSUPPORTED);
  expect_rejected(fwd({1, 6, 63, 16, 44}, RNG, 200, 200, 8, P, FP, 1), l, FBEV_ERR_UNSUPPORTED);
  expect_rejected(fwd(fd, RNG, 200, 200, 8, reinterpret_cast<char*>(P) + 2, FP, 0), l, FBEV_ERR_UNSUPPORTED);
  expect_rejected(fwd({1, 64, 4096, 128, 128}, RNG, 8, 8, 4, P, FP, 0), l, FBEV_ERR_UNSUPPORTED);
  // empty problems: OK, nothing launched
  EXPECT(fwd({0, 6, 64, 16, 44}, RNG, 200, 200, 8, nullptr, nullptr, 0) == FBEV_OK && !l);
  EXPECT(fwd(fd, RNG, 0, 200, 8, P, nullptr, 0) == FBEV_OK && !l);

  auto bwd = [&](fbev_feat_desc d, int X, int Y, int Z, const float* g, float* gF) {
    return run([&] { return fbev_backward(g, d, FP, FP, FP, RNG, X, Y, Z, gF, nullptr); }, &l);
  };
  EXPECT(bwd(fd, 200, 200, 8, FP, FP) == FBEV_OK && l);
  expect_rejected(bwd(fd, 200, 200, 8, nullptr, FP), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(bwd(fd, 200, 200, 8, FP, nullptr), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(bwd(fd, 200, -200, 8, FP, FP), l, FBEV_ERR_INVALID_ARGUMENT);
  EXPECT(bwd({big, 1, 1, 1, 1}, 1, 1, 1, FP, FP) == FBEV_OK && l);   // many samples, each one small

  // a launcher's failure comes back as FBEV_ERR_DEVICE with HIP's text
  stub_status = hipErrorLaunchFailure;
  EXPECT(fwd(fd, RNG, 200, 200, 8, P, FP, 0) == FBEV_ERR_DEVICE && l);
  EXPECT(std::strstr(fbev_last_error(), "fbev_forward launch") != nullptr);
  EXPECT(std::strstr(fbev_last_error(), "stub launch failure") != nullptr);
  EXPECT(bwd(fd, 200, 200, 8, FP, FP) == FBEV_ERR_DEVICE && l);
  stub_status = hipSuccess;

  // ---- multi-level
  const int32_t ratios[4] = {1, 2, 4, 8}, bad_ratios[3] = {1, 3, 4};
  auto fl = [&](int L, const int32_t* r, fbev_feat_desc d) {
    return run([&] { return fbev_forward_levels(P, FBEV_DTYPE_F32, d, L, r, FP, FP, FP, RNG, 100, 100, 8, FP,
                                                 nullptr, nullptr); }, &l);
  };
  EXPECT(fl(3, ratios, fd) == FBEV_OK && l);
  expect_rejected(fl(5, ratios, fd), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fl(0, ratios, fd), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fl(3, nullptr, fd), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(fl(3, bad_ratios, fd), l, FBEV_ERR_INVALID_ARGUMENT);
  EXPECT(run([&] { return fbev_backward_levels(FP, fd, 3, ratios, FP, FP, FP, RNG, 100, 100, 8, FP, nullptr); }, &l)
             == FBEV_OK && l);

  // ---- temporal
  auto tf = [&](int Cp, const float* prev, const float* ego, int X, int Y) {
    return run([&] { return fbev_forward_temporal(P, FBEV_DTYPE_F32, fd, FP, FP, FP, RNG, X, Y, 8, prev, Cp, ego, FP,
                                                   nullptr, nullptr); }, &l);
  };
  EXPECT(tf(64, FP, FP, 200, 200) == FBEV_OK && l);
  expect_rejected(tf(-1, FP, FP, 200, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(tf(64, nullptr, FP, 200, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(tf(64, FP, nullptr, 200, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(tf(64, FP, FP, 65536, 65536), l, FBEV_ERR_UNSUPPORTED);
  auto tb = [&](int Cp, int X, int Y) {
    return run([&] { return fbev_backward_temporal(FP, fd, FP, FP, FP, RNG, X, Y, 8, Cp, FP, FP, FP, nullptr); }, &l);
  };
  EXPECT(tb(64, 200, 200) == FBEV_OK && l);
  expect_rejected(tb(64, 200, 10), l, FBEV_ERR_UNSUPPORTED);     // 0.5 m x 10 m cells
  EXPECT(tb(0, 200, 10) == FBEV_OK && l);                         // no previous map: the aspect does not matter
  expect_rejected(tb(big, 200, 200), l, FBEV_ERR_UNSUPPORTED);

  // ---- camera gradients
  size_t bytes = 0;
  EXPECT(fbev_backward_cameras_workspace(fd, 200, 200, 8, &bytes) == FBEV_OK && bytes > 0);
  EXPECT(fbev_backward_cameras_workspace(fd, 200, 200, 8, nullptr) == FBEV_ERR_INVALID_ARGUMENT);
  EXPECT(fbev_backward_cameras_workspace({-1, 6, 64, 16, 44}, 200, 200, 8, &bytes) == FBEV_ERR_INVALID_ARGUMENT);
  auto cg = [&](void* ws, size_t n) {
    return run([&] { return fbev_backward_cameras(FP, FP, fd, FP, FP, FP, RNG, 200, 200, 8, FP, FP, FP, ws, n,
                                                   nullptr); }, &l);
  };
  EXPECT(fbev_backward_cameras_workspace(fd, 200, 200, 8, &bytes) == FBEV_OK);
  EXPECT(cg(P, bytes) == FBEV_OK && l);
  expect_rejected(cg(P, bytes - 1), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(cg(nullptr, bytes), l, FBEV_ERR_INVALID_ARGUMENT);

  // the allocation-free variant: no workspace argument; an oversize problem is refused before any launch
  EXPECT(run([&] { return fbev_backward_cameras_noalloc(FP, FP, fd, FP, FP, FP, RNG, 200, 200, 8, FP, FP, FP,
                                                        nullptr); }, &l) == FBEV_OK && l);
  expect_rejected(run([&] { return fbev_backward_cameras_noalloc(FP, FP, {1, 30, 4, 8, 22}, FP, FP, FP, RNG, 200, 200,
                                                                 8, FP, FP, FP, nullptr); }, &l),
                  l, FBEV_ERR_UNSUPPORTED);
  EXPECT(std::strstr(fbev_last_error(), "allocation-free variant holds") != nullptr);

  // ---- Lift-Splat
  auto lf = [&](int D, float dmin, float dstep, int X) {
    return run([&] { return fbev_lss_forward(FP, FP, fd, D, dmin, dstep, FP, FP, FP, RNG, X, 200, FP, nullptr); },
               &l);
  };
  EXPECT(lf(41, 4.f, 1.f, 200) == FBEV_OK && l);
  expect_rejected(lf(41, 4.f, 0.f, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(lf(41, 4.f, nan, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(lf(-1, 4.f, 1.f, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(lf(big, 4.f, 1.f, 200), l, FBEV_ERR_INVALID_ARGUMENT);
  EXPECT(run([&] { return fbev_lss_backward(FP, FP, FP, fd, 41, 4.f, 1.f, FP, FP, FP, RNG, 200, 200, FP, FP,
                                            nullptr); }, &l) == FBEV_OK && l);

  // ---- Deformable Aggregation
  auto df = [&](int Q, int Kp) {
    return run([&] { return fbev_deform_forward(FP, fd, FP, FP, FP, FP, FP, FP, Q, Kp, FP, nullptr); }, &l);
  };
  EXPECT(df(900, 13) == FBEV_OK && l);
  expect_rejected(df(900, 257), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(df(-1, 13), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(df(big, 13), l, FBEV_ERR_UNSUPPORTED);
  EXPECT(fbev_deform_backward_workspace(fd, 900, 13, &bytes) == FBEV_OK);
  auto db = [&](void* ws, size_t n) {
    return run([&] { return fbev_deform_backward(FP, FP, fd, FP, FP, FP, FP, FP, FP, 900, 13, FP, FP, FP, FP, ws, n,
                                                  nullptr); }, &l);
  };
  EXPECT(db(P, bytes) == FBEV_OK && l);
  expect_rejected(db(P, bytes - 1), l, FBEV_ERR_INVALID_ARGUMENT);
  expect_rejected(db(reinterpret_cast<char*>(P) + 8, bytes), l, FBEV_ERR_INVALID_ARGUMENT);

  // ---- status strings, version, and the last-error text is per thread
  EXPECT(std::strcmp(fbev_status_string(FBEV_OK), "ok") == 0);
  EXPECT(std::strlen(fbev_status_string((fbev_status)12345)) > 0);
  EXPECT(fbev_abi_version() == FBEV_ABI_VERSION);
  expect_rejected(fwd(fd, RNG, -1, 200, 8, P, FP, 0), l, FBEV_ERR_INVALID_ARGUMENT);
  std::thread th([] { EXPECT(std::strlen(fbev_last_error()) == 0); });
  th.join();
  EXPECT(std::strstr(fbev_last_error(), "negative grid size") != nullptr);

  if (failures == 0) std::printf("ok\n");
  return failures == 0 ? 0 : 1;
}
