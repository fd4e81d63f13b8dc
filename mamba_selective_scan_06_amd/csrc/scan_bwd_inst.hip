// The backward kernels of one storage type: compiled with -DBWD_S=float or
// -DBWD_S=uint16_t (bf16 bits), so the two instantiations build in parallel.
#include "scan_bwd_impl.hpp"

#ifndef BWD_S
#error "compile with -DBWD_S=float or -DBWD_S=uint16_t"
#endif

template hipError_t ssm::bwd::launch_typed<BWD_S>(const ssm::BwdProblem& p, hipStream_t stream);
