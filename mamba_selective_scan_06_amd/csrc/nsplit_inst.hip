// One instantiation of the NSPLIT forward scan: storage type NSPLIT_S,
// K = NSPLIT_K states per wave (N = 4K), and row addressing NSPLIT_WIN (1:
// windows moved along rows of 2 GiB or more).  The build compiles this file
// once per (type, K, addressing) so the kernels build in parallel.
#include "scan_nsplit_impl.hpp"

#if !defined(NSPLIT_S) || !defined(NSPLIT_K) || !defined(NSPLIT_WIN)
#error "compile with -DNSPLIT_S=<float|uint16_t> -DNSPLIT_K=<1|2|4|8|16> -DNSPLIT_WIN=<0|1>"
#endif

namespace ssm {
namespace nsplit_detail {
template hipError_t launch_nsplit_t<NSPLIT_S, NSPLIT_K, NSPLIT_WIN != 0>(const Problem& p, hipStream_t stream);
}  // namespace nsplit_detail
}  // namespace ssm
