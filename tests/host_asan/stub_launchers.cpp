// Test double for the kernel launchers of the C-ABI library: each records the
// argument block the host code built and returns success, so that the host
// code (argument checks, derived sizes, debug pre-pass) can be built with the
// address and undefined-behaviour sanitizers and run without a GPU. Nothing
// here runs on a device.
#include "stub_launchers.hpp"

namespace la {

StubLog g_stub;

hipError_t launch_rope_pair(const RopeArgs& q, const RopeArgs& k, const RopeAngles& ang, int D, int dt,
                            hipStream_t) {
  ++g_stub.rope;
  g_stub.rope_q = q;
  g_stub.rope_k = k;
  g_stub.angles = ang;
  g_stub.D = D;
  g_stub.dt = dt;
  return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs& a, int D, int G, int dt, hipStream_t) {
  ++g_stub.prefill;
  g_stub.pre = a;
  g_stub.D = D;
  g_stub.G = G;
  g_stub.dt = dt;
  return hipSuccess;
}
hipError_t launch_ring_finalize(const PrefillArgs& a, int D, int dt, hipStream_t st) {
  return launch_prefill_merge(a, D, dt, st);   // counted as a merge
}
hipError_t launch_prefill_merge(const PrefillArgs& a, int D, int dt, hipStream_t) {
  ++g_stub.merge;
  g_stub.pre_merge = a;
  g_stub.D = D;
  g_stub.dt = dt;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, int D, int G, hipStream_t) {
  ++g_stub.decode;
  g_stub.dec = a;
  g_stub.D = D;
  g_stub.G = G;
  return hipSuccess;
}
hipError_t launch_combine(const CombineArgs& a, int D, int dt, hipStream_t) {
  ++g_stub.combine;
  g_stub.comb = a;
  g_stub.D = D;
  g_stub.dt = dt;
  return hipSuccess;
}
hipError_t launch_backward(const BwdArgs& a, int D, int G, hipStream_t) {
  ++g_stub.backward;
  g_stub.bwd = a;
  g_stub.D = D;
  g_stub.G = G;
  return hipSuccess;
}

}  // namespace la

namespace la {

// no device: the scratch lookup fails like a runtime without a GPU would
hipError_t prefill_sched(hipStream_t, unsigned** sched) {
  *sched = nullptr;   // no queue counters: one workgroup per item
  return hipSuccess;
}
hipError_t decode_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  return hipErrorNoDevice;
}

}  // namespace la
