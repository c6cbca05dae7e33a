// Host-only stand-ins for the kernel launchers of csa_kernels.hip, so that
// csa_api.cpp (argument validation, planning, the C ABI) can be built by a
// host compiler with sanitizers for the CPU tests.  The CPU tests never reach
// a launch: every call they make is rejected or answered before it.
#include "../../gated_pooling_amd/csrc/csa_launch.h"

namespace csa {
bool launch_fwd(int, int, const FwdParams&, const LaunchShape&, hipStream_t) { return false; }
bool launch_bwd(int, int, const BwdParams&, const LaunchShape&, hipStream_t) { return false; }
void launch_dape_reduce(const ReduceParams&, hipStream_t) {}
bool launch_seg_scan(int, const SegParams&, int32_t*, int32_t*, hipStream_t) { return false; }
bool launch_fwd128(int, const Fwd128Params&, uint32_t, size_t, hipStream_t) { return false; }
bool launch_bwd128(int, const Bwd128Params&, uint32_t, size_t, hipStream_t) { return false; }
hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}
}  // namespace csa
