// Host-only stand-ins for the kernel launchers and workspace sizes that the C ABI layer
// (moe_abi.cpp) calls after its argument checks, so that the checks can be built and run
// on a machine without a GPU under AddressSanitizer and UBSan.  Every launcher records
// that it was reached and succeeds; the sizes are fixed values the driver knows.
#include "internal.h"

namespace moe_stub {
int launches = 0;
constexpr size_t kWorkspace = 4096;
}  // namespace moe_stub

namespace moe {
namespace {
hipError_t hit() {
  ++moe_stub::launches;
  return hipSuccess;
}
}  // namespace

size_t route_workspace_bytes(int64_t T, int E) { return T > 0 && E > 0 ? moe_stub::kWorkspace : 0; }
size_t router_route_workspace_bytes(int64_t T, int E) {
  // the real formula: ceil(T / 32) E int32 counts, rounded up to 256 bytes (the noalloc limit reads it)
  return (size_t)((((T + 31) / 32) * E * 4 + 255) / 256 * 256);
}
size_t grouped_gemm_workspace_bytes() { return moe_stub::kWorkspace; }
size_t router_backward_workspace_bytes(int64_t T, int64_t, int, int dtype) {
  return dtype == 1 && T > 0 ? moe_stub::kWorkspace : 0;
}

hipError_t launch_router_logits(const void*, const void*, int64_t, int64_t, int, int, float*, hipStream_t) {
  return hit();
}
hipError_t launch_router_route(const void*, const void*, const float*, int64_t, int64_t, int, int, int, int, float*,
                               int32_t*, float*, int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t) {
  return hit();
}
hipError_t launch_router_route_noalloc(const void*, const void*, const float*, int64_t, int64_t, int, int, int, int,
                                       float*, int32_t*, float*, int32_t*, int32_t*, int32_t*, int32_t*,
                                       hipStream_t) {
  return hit();
}
hipError_t launch_route(const float*, const float*, int64_t, int, int, int, int, int32_t*, float*, int32_t*, int32_t*,
                        int32_t*, int32_t*, void*, hipStream_t) {
  return hit();
}
hipError_t launch_route_scan_finalize(int32_t*, int, int, int64_t, int, int, const int32_t*, int32_t*, int32_t*,
                                      int32_t*, int32_t*, hipStream_t) {
  return hit();
}
hipError_t launch_permute(const void*, int64_t, int64_t, int, int, const int32_t*, const float*, const void*, float*,
                          void*, hipStream_t) {
  return hit();
}
hipError_t launch_combine(const void*, const int32_t*, const float*, int64_t, int64_t, int, int, void*, hipStream_t) {
  return hit();
}
hipError_t launch_grouped_gemm(const void*, const void*, int, const int32_t*, int64_t, int64_t, int64_t, int, int, int,
                               const void*, void*, void*, void*, size_t, hipStream_t) {
  return hit();
}
hipError_t launch_grouped_gemm_gather(const void*, int64_t, const int32_t*, int, const void*, const int32_t*, int64_t,
                                      int64_t, int64_t, int, int, void*, void*, void*, size_t, hipStream_t) {
  return hit();
}
hipError_t launch_grouped_wgrad(const void*, const void*, const int32_t*, int64_t, int64_t, int64_t, int, int, int,
                                float*, hipStream_t) {
  return hit();
}
hipError_t launch_route_backward(const float*, const float*, const int32_t*, const float*, int64_t, int, int, int,
                                 int, float*, hipStream_t) {
  return hit();
}
hipError_t launch_router_logits_backward(const float*, const void*, const void*, int64_t, int64_t, int, int, float*,
                                         void*, int, void*, hipStream_t) {
  return hit();
}
hipError_t launch_permute_rows(const void*, int64_t, int64_t, int, const int32_t*, void*, hipStream_t) {
  return hit();
}
hipError_t launch_mx_quantize(const void*, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { return hit(); }
hipError_t launch_grouped_gemm_mx(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*,
                                  int64_t, int64_t, int64_t, int, int, void*, uint8_t*, void*, size_t, hipStream_t) {
  return hit();
}
}  // namespace moe
