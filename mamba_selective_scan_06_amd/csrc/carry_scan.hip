// Carry combine of a time-split forward scan: a wave-level associative scan
// over the segments' (a, b) pairs.
//
// Segment j of a chain (b, d, n) is the affine map h -> a_j h + b_j with
// a_j = exp(A[d,n] sum_{t in j} delta_t) (the product of its decays, one exp
// of the summed step size) and b_j = the state it reaches from zero (written
// by the state-only pass).  Applying segments in order composes the maps with
// the operator (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2), which is
// associative but not commutative (the explainer page's parallel associative
// scan; the page does not write the operator out).  The state entering
// segment s is the composition of segments 0..s-1 applied to h0.
//
// One row of P lanes (P = 16, 32 or 64, the smallest power of two >= the
// segments that have a summary) holds one chain, lane j = segment j; the
// inclusive scan runs in log2(P) steps of DPP data movement inside the wave
// (row_shr by 1, 2, 4, 8 within 16-lane rows, then row_bcast:15 and
// row_bcast:31 across rows), each step one multiply and one fused
// multiply-add.  Lane j then holds the maps of segments 0..j and writes the
// state entering segment j+1 over its own summary in the workspace.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

// (a, b) <- (a_src a, a b_src + b) with (a_src, b_src) the pair of the lane the
// DPP control names; lanes without a source take the identity (1, 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void combine_step(float& a, float& b) {
  const float as = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f),
                                                                          __builtin_bit_cast(int, a), CTRL, ROW_MASK,
                                                                          0xf, false));
  const float bs = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 0.0f),
                                                                          __builtin_bit_cast(int, b), CTRL, ROW_MASK,
                                                                          0xf, false));
  b = __builtin_fmaf(a, bs, b);
  a = as * a;
}

// P lanes per chain; grid covers chains = batch * dim * dstate.
template <int P>
__global__ __launch_bounds__(256) void carry_scan_kernel(float* __restrict__ ws_state, const float* __restrict__ ws_dsum,
                                                         const float* __restrict__ A, const float* __restrict__ h0,
                                                         int64_t batch, int64_t dim, int64_t dstate, int splits) {
  constexpr int CPW = 64 / P;  // chains per wave
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t chain = wave * CPW + lane / P;
  const int j = lane % P;  // segment
  const int64_t chains = batch * dim * dstate;
  const bool live = chain < chains && j < splits - 1;  // segments with a summary
  const int64_t cc = chain < chains ? chain : chains - 1;
  const int64_t n = cc % dstate, d = (cc / dstate) % dim, b = cc / (dstate * dim);
  const int64_t seg = b * splits + j;
  float a = 1.0f, v = 0.0f;
  if (live) {
    a = fast_exp2(A[d * dstate + n] * kLog2e * ws_dsum[seg * dim + d]);
    v = ws_state[(seg * dim + d) * dstate + n];
  }
  combine_step<0x111, 0xf>(a, v);  // row_shr:1
  combine_step<0x112, 0xf>(a, v);  // row_shr:2
  combine_step<0x114, 0xf>(a, v);  // row_shr:4
  combine_step<0x118, 0xf>(a, v);  // row_shr:8
  if constexpr (P >= 32) combine_step<0x142, 0xa>(a, v);  // row_bcast:15 into rows 1 and 3
  if constexpr (P >= 64) combine_step<0x143, 0xc>(a, v);  // row_bcast:31 into rows 2 and 3
  if (live) {
    const float hin = h0 ? h0[(b * dim + d) * dstate + n] : 0.0f;
    ws_state[(seg * dim + d) * dstate + n] = __builtin_fmaf(a, hin, v);  // state entering segment j + 1
  }
}

template <int P>
hipError_t launch_p(const Problem& p, hipStream_t stream) {
  const int64_t chains = p.batch * p.dim * p.dstate;
  const int64_t waves = (chains + (64 / P) - 1) / (64 / P);
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(carry_scan_kernel<P>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p.ws_state,
                     p.ws_dsum, p.A, p.h0, p.batch, p.dim, p.dstate, p.splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_carry_scan(const Problem& p, hipStream_t stream) {
  const int nsum = p.splits - 1;  // segments with a summary
  if (nsum <= 16) return launch_p<16>(p, stream);
  if (nsum <= 32) return launch_p<32>(p, stream);
  return launch_p<64>(p, stream);
}

}  // namespace ssm
