// moe_bounded_forward_static: the layer's forward pass on a library-owned
// scratch array instead of a caller workspace, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).
//
// The scratch array lives in the code object (a file-scope __device__
// array): each GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never uses the array's name as
// a device address (on the host it is only a stand-in symbol); the entry
// point asks the runtime for the current device's address once, keeps it per
// device, and passes that address to the same launch sequence the workspace
// variant runs.  The forward pass needs no part of its workspace cleared on
// entry, so nothing is filled here.
#include <mutex>

#include "moe_internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; guarded by g_scratch_mu

// The current device's address of `scratch`, looked up on its first use on
// that device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr || (uintptr_t)p % 256) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API int moe_bounded_forward_static(const moe_plan_t* plan, const void* X, const void* W_r,
                                       const float* router_bias, const void* W_gate,
                                       const void* W_up, const void* W_down, void* Y,
                                       int32_t* topk_idx, float* gates, float* logits,
                                       void* stream, moe_stats_t* stats) {
  if (int s = check_forward_args(plan, X, W_r, W_gate, W_up, W_down, Y, topk_idx, gates))
    return s;
  const moe_plan_t& P = *plan;
  if (P.N > 0) {
    // the workspace this call's layout needs (logits live there unless the
    // caller passes them) must fit the scratch array; nothing is enqueued
    // otherwise
    const size_t need = make_layout(P, Pass::Forward, logits == nullptr, false).total;
    if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  }
  void* ws = nullptr;
  if (P.N > 0 && scratch_address(&ws) != hipSuccess) return MOE_EHIP;
  return forward_impl(P, X, W_r, router_bias, W_gate, W_up, W_down, Y, topk_idx, gates, logits,
                      ws, (hipStream_t)stream, stats);
}
