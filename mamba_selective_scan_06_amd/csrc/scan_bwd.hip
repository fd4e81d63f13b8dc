// Backward scan: the launches shared by both storage types (segment combine,
// fixed-order sums over batch rows and segments, problems with nothing to
// scan) and the dispatch on the storage type.  The per-type kernels are in
// scan_bwd_impl.hpp, compiled once per type by scan_bwd_inst.hip.
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

// ---- 2. combine the segment summaries ------------------------------------------------
// states: combine the forward summaries too (no checkpoints from the forward).
__global__ __launch_bounds__(256) void bwd_combine_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                                                          const float* __restrict__ dhT, float* __restrict__ segh,
                                                          float* __restrict__ segc, const float* __restrict__ segds,
                                                          int64_t Bsz, int64_t D, int N, int64_t nseg, bool states) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (b, d, n)
  if (i >= Bsz * D * N) return;
  const int64_t dn = i % (D * N), b = i / (D * N), d = dn / N, n = dn % N;
  const float a2 = A[dn] * kLog2e;
  if (states) {
    float h = h0 ? h0[i] : 0.0f;
    for (int64_t s = 0; s < nseg; ++s) {
      const int64_t si = (b * nseg + s) * D + d;
      const float e = segh[si * N + n];
      segh[si * N + n] = h;
      h = __builtin_fmaf(fast_exp2(a2 * segds[si]), h, e);
    }
  }
  // the adjoint leaving each segment's end; segment 0's own decay is not needed
  float g = dhT ? dhT[i] : 0.0f;
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t si = (b * nseg + s) * D + d;
    const float e = s > 0 ? segc[si * N + n] : 0.0f;  // the segment's adjoint from zero
    segc[si * N + n] = g;
    if (s > 0) g = __builtin_fmaf(fast_exp2(a2 * segds[si]), g, e);
  }
}

__global__ __launch_bounds__(256) void bwd_reduce_d_kernel(const float* __restrict__ pA, const float* __restrict__ pD,
                                                           const float* __restrict__ pbias, float* __restrict__ gA,
                                                           float* __restrict__ gD, float* __restrict__ gbias,
                                                           int64_t rows, int64_t D, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (d, n)
  if (i >= D * N) return;
  const int64_t d = i / N;
  float sa = 0.0f;
#pragma unroll 8
  for (int64_t r = 0; r < rows; ++r) sa += pA[r * D * N + i];  // r = (b, s), loads in flight eight at a time
  if (gA) gA[i] = sa;
  if (i % N == 0) {
    float sd = 0.0f, sbias = 0.0f;
#pragma unroll 8
    for (int64_t r = 0; r < rows; ++r) {
      sd += pD[r * D + d];
      sbias += pbias[r * D + d];
    }
    if (gD) gD[d] = sd;
    if (gbias) gbias[d] = sbias;
  }
}

// ---- problems without a token or without a chain ---------------------------------------------
__global__ __launch_bounds__(256) void fill_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                           int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

unsigned blocks256(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

hipError_t zero_bytes(void* p, int64_t bytes, hipStream_t stream) {
  if (!p || bytes <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u16_kernel, dim3(blocks256(bytes / 2)), dim3(256), 0, stream, static_cast<uint16_t*>(p),
                     bytes / 2);
  return hipGetLastError();
}

}  // namespace

namespace bwd {

hipError_t launch_combine(const BwdProblem& p, hipStream_t stream) {
  const int64_t bdn = p.batch * p.dim * p.dstate;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(blocks256(bdn)), dim3(256), 0, stream, p.A, p.h0, p.dhT, p.segh,
                     p.segc, p.segds, p.batch, p.dim, static_cast<int>(p.dstate), static_cast<int64_t>(p.splits),
                     p.ck_in == nullptr);
  return hipGetLastError();
}

hipError_t launch_reduce_d(const BwdProblem& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_reduce_d_kernel, dim3(blocks256(p.dim * p.dstate)), dim3(256), 0, stream, p.pA, p.pD,
                     p.pbias, p.dA, p.dD, p.ddelta_bias, p.batch * p.splits, p.dim, static_cast<int>(p.dstate));
  return hipGetLastError();
}

}  // namespace bwd

hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream) {
  return p.dtype == 0 ? bwd::launch_typed<float>(p, stream) : bwd::launch_typed<uint16_t>(p, stream);
}

// With no token the state passes through unchanged (hT = h0), so dh0 = dhT and
// every other gradient is an empty sum; with no chain the sums over d or b are
// empty.  Every non-empty output is written.
hipError_t launch_bwd_empty(const BwdProblem& p, hipStream_t stream) {
  const int64_t es = p.dtype == 0 ? 4 : 2;
  const int64_t bdn = p.batch * p.dim * p.dstate;
  hipError_t e = hipSuccess;
  if (p.dh0 && bdn > 0) {
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks256(bdn)), dim3(256), 0, stream, p.dh0, p.dhT, bdn);
    e = hipGetLastError();
  }
  const int64_t bln = p.batch * p.seqlen * p.dstate;
  if (e == hipSuccess) e = zero_bytes(p.dA, p.dim * p.dstate * 4, stream);
  if (e == hipSuccess) e = zero_bytes(p.dD, p.dim * 4, stream);
  if (e == hipSuccess) e = zero_bytes(p.ddelta_bias, p.dim * 4, stream);
  if (e == hipSuccess) e = zero_bytes(p.dB, bln * es, stream);
  if (e == hipSuccess) e = zero_bytes(p.dC, bln * es, stream);
  return e;
}

}  // namespace ssm
