// Host-side selection of the NSPLIT instantiation for (dtype, N).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_internal.hpp"

namespace ssm {
namespace nsplit_detail {
// Defined once per (S, K, WIN) in nsplit_inst.hip.
template <typename S, int K, bool WIN>
hipError_t launch_nsplit_t(const Problem& p, hipStream_t stream);
}  // namespace nsplit_detail

namespace {
template <typename S, bool WIN>
hipError_t launch_nsplit_w(const Problem& p, hipStream_t stream) {
  using nsplit_detail::launch_nsplit_t;
  switch (p.dstate) {
    case 4: return launch_nsplit_t<S, 1, WIN>(p, stream);
    case 8: return launch_nsplit_t<S, 2, WIN>(p, stream);
    case 16: return launch_nsplit_t<S, 4, WIN>(p, stream);
    case 32: return launch_nsplit_t<S, 8, WIN>(p, stream);
    case 64: return launch_nsplit_t<S, 16, WIN>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename S>
hipError_t launch_nsplit_s(const Problem& p, hipStream_t stream) {
  return p.windowed ? launch_nsplit_w<S, true>(p, stream) : launch_nsplit_w<S, false>(p, stream);
}
}  // namespace

hipError_t launch_nsplit(const Problem& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_nsplit_s<float>(p, stream) : launch_nsplit_s<uint16_t>(p, stream);
}

}  // namespace ssm
