// Drives every entry point of the C ABI (include/moe.h) through its host-side checks, built
// with AddressSanitizer and UBSan against the stand-in launchers of launch_stubs.cpp: each
// case states the status it must return and whether it may reach a launcher.  Pointers are
// fake 16-byte-aligned addresses that the checks never dereference; the outputs the checks
// do write (workspace sizes) are real host memory.  Prints "ok <n> cases" and exits 0.
#include <cstdio>
#include <cstring>

#include "moe.h"

namespace moe_stub {
extern int launches;
}

namespace {
int failures = 0, cases = 0;

void expect(const char* what, int line, int32_t got, int32_t want, bool launch_wanted, int before) {
  ++cases;
  const bool launched = moe_stub::launches != before;
  if (got != want || launched != launch_wanted) {
    std::printf("FAIL line %d %s: status %d (want %d), launched %d (want %d)\n", line, what, got, want, launched,
                launch_wanted);
    ++failures;
  }
}

#define EXPECT(call, want, launch)                         \
  do {                                                     \
    const int before_ = moe_stub::launches;                \
    const int32_t got_ = (call);                           \
    expect(#call, __LINE__, got_, want, launch, before_);  \
  } while (0)

char* const P = reinterpret_cast<char*>(uintptr_t(1) << 20);
float* const PF = reinterpret_cast<float*>(P);
int32_t* const PI = reinterpret_cast<int32_t*>(P);
uint8_t* const PU = reinterpret_cast<uint8_t*>(P);
}  // namespace

int main() {
  // version, status strings (every code, and unknown ones), never NULL
  EXPECT(moe_abi_version() == MOE_ABI_VERSION ? 0 : 1, 0, false);
  for (int s = -3; s < 8; ++s) {
    const char* str = moe_status_str(s);
    EXPECT(str != nullptr && std::strlen(str) > 0 ? 0 : 1, 0, false);
  }

  size_t n = 0;
  EXPECT(moe_route_workspace_size(100, 8, &n), MOE_OK, false);
  EXPECT(moe_route_workspace_size(100, 8, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_route_workspace_size(-1, 8, &n), MOE_INVALID_ARG, false);
  EXPECT(moe_route_workspace_size(10, 257, &n), MOE_INVALID_ARG, false);
  EXPECT(moe_router_route_workspace_size(1000, 8, &n), MOE_OK, false);
  EXPECT(moe_router_route_workspace_size(10, 0, &n), MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_workspace_size(&n), MOE_OK, false);
  EXPECT(moe_grouped_gemm_workspace_size(nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_router_backward_workspace_size(100, 64, 8, MOE_BF16, &n), MOE_OK, false);
  EXPECT(moe_router_backward_workspace_size(100, 20, 8, MOE_BF16, &n), MOE_INVALID_ARG, false);
  EXPECT(moe_router_backward_workspace_size(100, 64, 8, 4, &n), MOE_UNSUPPORTED, false);

  // router logits
  EXPECT(moe_router_logits(P, P, 10, 16, 8, MOE_BF16, PF, nullptr), MOE_OK, true);
  EXPECT(moe_router_logits(P, P, 10, 16, 0, MOE_BF16, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_router_logits(P, P, 10, 20, 8, MOE_BF16, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_router_logits(P, P, 10, 16, 8, 3, PF, nullptr), MOE_UNSUPPORTED, false);
  EXPECT(moe_router_logits(P + 8, P, 10, 16, 8, MOE_BF16, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_router_logits(nullptr, nullptr, 0, 16, 8, MOE_BF16, nullptr, nullptr), MOE_OK, false);

  // routing
  const size_t ws = 4096;
  EXPECT(moe_route(PF, nullptr, 100, 8, 2, 0, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr), MOE_OK, true);
  EXPECT(moe_route(PF, nullptr, 100, 8, 9, 0, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_route(PF, nullptr, 100, 64, 33, 0, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_route(PF, nullptr, 100, 8, 2, 2, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr), MOE_UNSUPPORTED, false);
  EXPECT(moe_route(nullptr, nullptr, 100, 8, 2, 0, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr), MOE_INVALID_ARG,
         false);
  EXPECT(moe_route(PF, nullptr, 100, 8, 2, 0, 1, PI, PF, PI, PI, PI, PI, P, 16, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_route(PF, nullptr, int64_t(1) << 28, 8, 8, 0, 1, PI, PF, PI, PI, PI, PI, P, ws, nullptr),
         MOE_INVALID_ARG, false);

  // fused router, with a workspace and without one
  EXPECT(moe_router_route(P, P, nullptr, 100, 64, 8, 2, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI, PI, P, ws,
                          nullptr),
         MOE_OK, true);
  EXPECT(moe_router_route(P, P, nullptr, 100, 64, 8, 2, MOE_F32, 0, 1, nullptr, PI, PF, PI, PI, PI, PI, P, ws,
                          nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_router_route(P, P, nullptr, 100, 64, 8, 2, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI, PI, P, 0,
                          nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_router_route_noalloc(P, P, nullptr, 100, 64, 8, 2, MOE_BF16, 1, 1, PF, PI, PF, PI, PI, PI, PI, nullptr),
         MOE_OK, true);
  EXPECT(moe_router_route_noalloc(P, P, nullptr, 131072, 64, 256, 8, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI, PI,
                                  nullptr),
         MOE_OK, true);
  EXPECT(moe_router_route_noalloc(P, P, nullptr, 131104, 64, 256, 8, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI,
                                  PI, nullptr),
         MOE_SCRATCH_LIMIT, false);
  EXPECT(moe_router_route_noalloc(P, P, PF + 1, 100, 64, 8, 2, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI, PI,
                                  nullptr),
         MOE_OK, true);
  EXPECT(moe_router_route_noalloc(P, P, reinterpret_cast<float*>(P + 2), 100, 64, 8, 2, MOE_BF16, 0, 1, nullptr, PI,
                                  PF, PI, PI, PI, PI, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_router_route_noalloc(P, P, nullptr, 100, 64, 8, 9, MOE_BF16, 0, 1, nullptr, PI, PF, PI, PI, PI, PI,
                                  nullptr),
         MOE_INVALID_ARG, false);

  // permute and combine
  EXPECT(moe_permute(P, 10, 16, 2, MOE_BF16, PI, nullptr, nullptr, nullptr, P, nullptr), MOE_OK, true);
  EXPECT(moe_permute(P, 10, 16, 2, MOE_BF16, PI, PF, P, PF, P, nullptr), MOE_OK, true);
  EXPECT(moe_permute(P, 10, 12, 2, MOE_BF16, PI, nullptr, nullptr, nullptr, P, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_permute(P, 10, 16, 2, MOE_BF16, PI, nullptr, P, nullptr, P, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_permute(P, 10, 16, 33, MOE_BF16, PI, nullptr, nullptr, nullptr, P, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_permute(nullptr, 0, 16, 2, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), MOE_OK,
         false);
  EXPECT(moe_unpermute_combine(P, PI, PF, 10, 16, 2, MOE_BF16, P, nullptr), MOE_OK, true);
  EXPECT(moe_unpermute_combine(P, PI, nullptr, 10, 16, 0, MOE_BF16, P, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_unpermute_combine(P, nullptr, nullptr, 10, 16, 2, MOE_BF16, P, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_unpermute_combine(P + 4, PI, nullptr, 10, 16, 2, MOE_BF16, P, nullptr), MOE_INVALID_ARG, false);

  // grouped GEMM
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_NK, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, nullptr, P,
                          nullptr, 0, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_NK, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_SWIGLU, nullptr, P, P, P,
                          ws, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_KN, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_DSWIGLU, P, nullptr, P,
                          nullptr, 0, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_NK, PI, 512, 12, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, nullptr, P,
                          nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_NK, PI, 512, 256, 128, MOE_MAX_GROUPS + 1, MOE_BF16, MOE_EPI_NONE,
                          nullptr, nullptr, P, nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm(P, P, 2, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, nullptr, P, nullptr, 0,
                          nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_KN, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_SWIGLU, nullptr, nullptr, P,
                          nullptr, 0, nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_KN, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_DSWIGLU, nullptr, nullptr,
                          P, nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm(P, P, MOE_LAYOUT_NK, PI, 512, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, nullptr, P,
                          P + 8, ws, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm(nullptr, P, MOE_LAYOUT_NK, PI, 0, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, nullptr,
                          nullptr, nullptr, 0, nullptr),
         MOE_OK, false);

  // gate/up GEMM on gathered token rows
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 2, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_SWIGLU, P, P, P, ws, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 2, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, P, nullptr, 0,
                                 nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 2, P, PI, 256, 96, 4, MOE_BF16, MOE_EPI_NONE, nullptr, P, nullptr, 0,
                                 nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 2, P, PI, 256, 128, 4, MOE_F32, MOE_EPI_NONE, nullptr, P, nullptr, 0,
                                 nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 2, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_DSWIGLU, nullptr, P, nullptr,
                                 0, nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm_gather(P, nullptr, 256, 2, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, P,
                                 nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_gather(P, PI, 256, 0, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr, P, nullptr, 0,
                                 nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_gather(nullptr, nullptr, 0, 2, P, PI, 256, 128, 4, MOE_BF16, MOE_EPI_NONE, nullptr,
                                 nullptr, nullptr, 0, nullptr),
         MOE_OK, false);

  // weight gradient
  EXPECT(moe_grouped_gemm_wgrad(P, P, PI, 64, 16, 16, 2, MOE_BF16, 0, PF, nullptr), MOE_OK, true);
  EXPECT(moe_grouped_gemm_wgrad(P, P, PI, 64, 12, 16, 2, MOE_BF16, 0, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_wgrad(P, P, nullptr, 64, 16, 16, 2, MOE_BF16, 0, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_wgrad(P, P, PI, 64, 16, 16, 2, 5, 0, PF, nullptr), MOE_UNSUPPORTED, false);

  // router backward
  EXPECT(moe_route_backward(PF, nullptr, PI, PF, 10, 8, 2, 0, 1, PF, nullptr), MOE_OK, true);
  EXPECT(moe_route_backward(PF, nullptr, PI, PF, 10, 8, 9, 0, 1, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_route_backward(PF, nullptr, PI, PF, 10, 8, 2, 2, 1, PF, nullptr), MOE_UNSUPPORTED, false);
  EXPECT(moe_route_backward(PF, nullptr, nullptr, PF, 10, 8, 2, 0, 1, PF, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_router_logits_backward(PF, P, P, 100, 64, 8, MOE_BF16, PF, P, 0, P, ws, nullptr), MOE_OK, true);
  EXPECT(moe_router_logits_backward(PF, P, P, 100, 64, 8, MOE_BF16, PF, P, 0, P, ws - 1, nullptr), MOE_INVALID_ARG,
         false);
  EXPECT(moe_router_logits_backward(PF, nullptr, P, 100, 64, 8, MOE_BF16, PF, nullptr, 0, P, ws, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_router_logits_backward(PF, P, P, 100, 64, 8, MOE_BF16, nullptr, nullptr, 0, nullptr, 0, nullptr),
         MOE_OK, false);

  // MXFP8
  EXPECT(moe_mx_quantize(P, 10, 64, MOE_BF16, PU, PU, nullptr), MOE_OK, true);
  EXPECT(moe_mx_quantize(P, 10, 48, MOE_BF16, PU, PU, nullptr), MOE_INVALID_ARG, false);
  EXPECT(moe_mx_quantize(P, 10, 64, MOE_F32, PU, PU, nullptr), MOE_UNSUPPORTED, false);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 256, 4, MOE_EPI_SWIGLU, P, nullptr, nullptr, 0, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 256, 4, MOE_EPI_NONE, P, nullptr, P, 1 << 20, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 256, 4, MOE_EPI_SWIGLU_MX, P, PU, nullptr, 0, nullptr),
         MOE_OK, true);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 256, 4, MOE_EPI_SWIGLU_MX, P, nullptr, nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 192, 4, MOE_EPI_NONE, P, nullptr, nullptr, 0, nullptr),
         MOE_INVALID_ARG, false);
  EXPECT(moe_grouped_gemm_mx(PU, PU, PU, PU, PI, 512, 256, 256, 4, MOE_EPI_DSWIGLU, P, nullptr, nullptr, 0, nullptr),
         MOE_UNSUPPORTED, false);
  EXPECT(moe_permute_mx(PU, PU, 10, 512, 2, PI, PU, PU, nullptr), MOE_OK, true);
  EXPECT(moe_permute_mx(PU, PU, 10, 256, 2, PI, PU, PU, nullptr), MOE_INVALID_ARG, false);

  if (failures) {
    std::printf("%d of %d cases failed\n", failures, cases);
    return 1;
  }
  std::printf("ok %d cases\n", cases);
  return 0;
}
