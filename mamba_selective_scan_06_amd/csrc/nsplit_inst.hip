// One instantiation of the NSPLIT forward scan: storage type NSPLIT_S and
// K = NSPLIT_K states per wave (N = 4K).  The build compiles this file once
// per (type, K) pair so the kernels build in parallel.
#include "scan_nsplit_impl.hpp"

#if !defined(NSPLIT_S) || !defined(NSPLIT_K)
#error "compile with -DNSPLIT_S=<float|uint16_t> -DNSPLIT_K=<1|2|4|8|16>"
#endif

namespace ssm {
namespace nsplit_detail {
template hipError_t launch_nsplit_t<NSPLIT_S, NSPLIT_K>(const Problem& p, hipStream_t stream);
}  // namespace nsplit_detail
}  // namespace ssm
