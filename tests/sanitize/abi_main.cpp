// Sanitizer driver for the library's host code (test infrastructure): the C
// ABI's validation and planning, which run on the host before anything is
// launched.  Built host-only (no device code) with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  It queries the
// workspace sizes of every path over a grid of shapes, dtypes and configs
// (every plan the library can form, and the rejected ones), and calls every
// entry point with null or rejected arguments, which must return an error
// before any HIP call.
#include <cstdint>
#include <cstdio>

#include "gla.h"

static int bad = 0;
static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "line %d: %s\n", line, what);
    bad = 1;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

int main() {
  EXPECT(gla_abi_version() == GLA_ABI_VERSION);
  for (int s = -1; s <= 8; ++s) EXPECT(gla_status_string(s) != nullptr);

  const int Ls[] = {0, 1, 15, 63, 64, 65, 200, 2048, 16384};
  const int ds[] = {8, 16, 32, 48, 64, 96, 128, 256, 512, 1024};
  const int Cs[] = {8, 16, 32, 64, 128};
  long plans = 0;
  for (int dt = -1; dt <= 2; ++dt)
    for (int L : Ls)
      for (int dk : ds)
        for (int dv : ds)
          for (int C : Cs)
            for (int B : {0, 1, 3})
              for (int H : {1, 4}) {
                const gla_dims d{B, H, L, dk, dv, C, 16};
                size_t w = 0;
                const gla_status s = gla_fwd_workspace_size(&d, dt, &w);
                EXPECT(s >= GLA_OK && s <= GLA_ERR_HIP);
                plans += s == GLA_OK;
                gla_bwd_workspace_size(&d, dt, &w);
                ggla_fwd_workspace_size(&d, dt, &w);
                ggla_bwd_workspace_size(&d, dt, &w);
                for (int algo = -1; algo <= 4; ++algo)
                  for (int wv : {0, 1, 2, 3, 4, 8})
                    for (int sg : {-1, 0, 1, 2, 16}) {
                      const gla_fwd_config f{algo, wv, sg};
                      gla_fwd_ex_workspace_size(&d, dt, &f, &w);
                    }
                for (int algo = -1; algo <= 3; ++algo) {
                  const gla_bwd_config b{algo};
                  gla_bwd_ex_workspace_size(&d, dt, &b, &w);
                }
              }
  EXPECT(plans > 0);

  // rejected calls return before anything reaches the GPU
  const gla_dims d{2, 4, 256, 64, 128, 64, 16};
  size_t w = 0;
  EXPECT(gla_fwd_workspace_size(nullptr, GLA_BF16, &w) == GLA_ERR_NULL);
  EXPECT(gla_fwd_workspace_size(&d, GLA_BF16, nullptr) == GLA_ERR_NULL);
  EXPECT(gla_fwd(&d, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, 0, nullptr) == GLA_ERR_NULL);
  EXPECT(gla_fwd(&d, 7, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, 0, nullptr) == GLA_ERR_DTYPE);
  const gla_dims bad_shape{2, 4, 256, 40, 128, 64, 16};
  EXPECT(gla_fwd(&bad_shape, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, nullptr, 0, nullptr) == GLA_ERR_SHAPE);
  EXPECT(gla_bwd(&d, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
         GLA_ERR_NULL);
  EXPECT(gla_decode(&d, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr) == GLA_ERR_NULL);
  EXPECT(ggla_fwd(&d, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, 0, nullptr) == GLA_ERR_NULL);
  const gla_fwd_config two{GLA_FWD_TWO_PASS, 0, 0};
  EXPECT(gla_fwd_ex(&d, GLA_BF16, &two, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, 0, nullptr) == GLA_ERR_NULL);
  EXPECT(gla_fwd_noalloc(&bad_shape, GLA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr) != GLA_OK);
  const gla_dims huge{64, 64, 16384, 256, 512, 64, 16};
  static char dummy[64] __attribute__((aligned(256)));
  void* p = dummy;
  EXPECT(gla_fwd_noalloc(&huge, GLA_BF16, p, p, p, (const float*)p, nullptr, p, nullptr,
                         nullptr) == GLA_ERR_WORKSPACE);
  // the profiler's records without a GPU: empty
  EXPECT(gla_profile_count() == 0);
  const char* name = nullptr;
  float ms = 0.f;
  EXPECT(gla_profile_get(0, &name, &ms) != GLA_OK);

  std::printf(bad ? "host sanitizer run FAILED\n" : "host sanitizer run clean (%ld plans)\n", plans);
  return bad;
}
