// Host-only stand-ins for the kernel launchers of libmoe.so, for the sanitized
// build of the C ABI's host logic (argument checks, exact capacity, workspace
// layout).  Test infrastructure: every launcher reports hipErrorNotSupported, so
// a call that gets past validation returns MOE_ERR_HIP and nothing is computed.
#include "moe_internal.h"

namespace moe {

namespace {
hipError_t no_device() { return hipErrorNotSupported; }
}  // namespace

hipError_t launch_router_split(const Plan&, const float*, void*, hipStream_t) { return no_device(); }
hipError_t launch_router_topk(const Plan&, const void*, const float*, const float*, int32_t*, float*, void*,
                              hipStream_t, bool, float*) { return no_device(); }
hipError_t launch_router_aux(const Plan&, double, float*, void*, hipStream_t) { return no_device(); }
hipError_t launch_router_rre(const Plan&, const int32_t*, int32_t*, float*, void*, hipStream_t) {
  return no_device();
}
hipError_t launch_dispatch_hist(const Plan&, const int32_t*, void*, hipStream_t) { return no_device(); }
hipError_t launch_dispatch_scan(const Plan&, int32_t*, int32_t*, void*, hipStream_t) { return no_device(); }
hipError_t launch_dispatch_slot_gather(const Plan&, const void*, const int32_t*, int32_t*, int32_t*, void*,
                                       void*, hipStream_t) { return no_device(); }
hipError_t launch_gather_slots(const Plan&, const void*, const int32_t*, const int32_t*, void*, hipStream_t) {
  return no_device();
}
hipError_t launch_expert_ffn(const Plan&, const void*, const int32_t*, const void*, const void*, void*,
                             void*, hipStream_t) { return no_device(); }
bool up_reads_token_rows(const Plan&) { return false; }
hipError_t launch_expert_ffn_rows(const Plan&, const void*, const int32_t*, const int32_t*, const void*,
                                  const void*, void*, void*, hipStream_t) { return no_device(); }
hipError_t launch_expert_up(const Plan&, const void*, const int32_t*, const void*, void*, hipStream_t) {
  return no_device();
}
hipError_t launch_expert_ffn_fused(const Plan&, int, const void*, const int32_t*, const void*, const void*,
                                   void*, hipStream_t) { return no_device(); }
hipError_t launch_expert_down(const Plan&, const void*, const int32_t*, const void*, void*, hipStream_t) {
  return no_device();
}
hipError_t launch_backward(const Plan&, const BwdArgs&, hipStream_t) { return no_device(); }
hipError_t launch_sparse_clip(const Plan&, float*, float*, void*, void*, double, float*, void*, hipStream_t) {
  return no_device();
}
hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  return no_device();
}
hipError_t launch_combine(const Plan&, const void*, const int32_t*, const int32_t*, const float*, void*,
                          hipStream_t) { return no_device(); }

}  // namespace moe
