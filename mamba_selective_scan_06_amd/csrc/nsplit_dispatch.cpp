// Host-side selection of the NSPLIT instantiation for (dtype, N).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_internal.hpp"

namespace ssm {
namespace nsplit_detail {
// Defined once per (S, K) in nsplit_inst.hip.
template <typename S, int K>
hipError_t launch_nsplit_t(const Problem& p, hipStream_t stream);
}  // namespace nsplit_detail

namespace {
template <typename S>
hipError_t launch_nsplit_s(const Problem& p, hipStream_t stream) {
  using nsplit_detail::launch_nsplit_t;
  switch (p.dstate) {
    case 4: return launch_nsplit_t<S, 1>(p, stream);
    case 8: return launch_nsplit_t<S, 2>(p, stream);
    case 16: return launch_nsplit_t<S, 4>(p, stream);
    case 32: return launch_nsplit_t<S, 8>(p, stream);
    case 64: return launch_nsplit_t<S, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_nsplit(const Problem& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_nsplit_s<float>(p, stream) : launch_nsplit_s<uint16_t>(p, stream);
}

}  // namespace ssm
