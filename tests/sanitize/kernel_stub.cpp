// Host-only stand-ins for the kernel side of the library (wkv6_internal.h),
// for the sanitizer build of the C ABI layer: they enqueue nothing, report no
// workspace, and count how often a call got past the argument checks.
#include "wkv6_internal.h"

int g_enqueued = 0;

namespace wkv6 {

size_t workspace_bytes(const FwdArgs&) { return 0; }
hipError_t enqueue_fwd(const FwdArgs&, void*, hipStream_t) {
  ++g_enqueued;
  return hipSuccess;
}
hipError_t enqueue_fwd_noalloc(const FwdArgs&, hipStream_t) {
  ++g_enqueued;
  return hipSuccess;
}
size_t bwd_workspace_bytes(const BwdArgs&) { return 0; }
hipError_t enqueue_bwd(const BwdArgs&, void*, hipStream_t) {
  ++g_enqueued;
  return hipSuccess;
}
hipError_t enqueue_gn_gate(const GnArgs&, hipStream_t) {
  ++g_enqueued;
  return hipSuccess;
}
size_t wkv4_workspace_bytes(const Wkv4Args&) { return 0; }
hipError_t enqueue_wkv4(const Wkv4Args&, void*, hipStream_t) {
  ++g_enqueued;
  return hipSuccess;
}

}  // namespace wkv6
