// DECODE family (seqlen == 1): one recurrent step per (b, d), the O(1)-per-token
// inference update of the fixed-size state (page youngju.dev "Mamba 논문 리뷰",
// section 6 comparison table; recurrence of section 2.2).
//
// The step is bound by the state traffic (read h0, write hT: 8 bytes per
// state against ~0.3 bytes of token input), so the layout is chosen for
// perfectly coalesced 16-byte state accesses: Q = N/4 consecutive lanes share
// one channel and each owns 4 consecutive states (one float4 of h0/hT/A).  The
// per-channel scalars (softplus, gate) are recomputed by the Q lanes of a
// channel; the readout sum over n is reduced across them with lane shuffles.
// h0 and hT may be the same buffer: every lane reads its own states before
// writing them (each state float4 belongs to exactly one lane and one row).
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

template <typename S>
__device__ __forceinline__ void load4(const S* p, float out[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float out[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float out[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xffff0000u);
}

#ifndef SSM_DECODE_ROWS
#define SSM_DECODE_ROWS 1
#endif
// Batch rows per thread (R): with R > 1 every thread keeps R independent state
// loads in flight.  With the state's non-temporal loads, one row per thread
// (more threads) measured fastest: 34.2-34.4 us per step against 35.4-35.6
// for two rows and 36.6 for four.
constexpr int kDecodeRows = SSM_DECODE_ROWS;

// The state is streamed: read once and written once per step, so its accesses
// carry the non-temporal hint (loads with it measured 5% faster per step; the
// stores alone made no difference).
typedef float f4v __attribute__((ext_vector_type(4)));

template <typename S, int Q, bool ZOH>
__global__ __launch_bounds__(256) void scan_decode_kernel(
    const S* __restrict__ x, const S* __restrict__ dl, const float* __restrict__ A,
    const S* __restrict__ Bm, const S* __restrict__ Cm, const float* __restrict__ Dsk,
    const S* __restrict__ z, const float* __restrict__ bias, const float* h0, float* hT,
    S* __restrict__ y, int64_t Bsz, int64_t D) {
  constexpr int N = 4 * Q;
  constexpr int CH = 256 / Q;  // channels per block
  constexpr int R = kDecodeRows;
  const int q = threadIdx.x % Q;
  const int64_t dq = static_cast<int64_t>(blockIdx.x) * CH + threadIdx.x / Q;
  const bool dact = dq < D;
  const int64_t d = dact ? dq : D - 1;  // inactive lanes read a valid channel, write nothing
  float a[4], an[4], ia[4];
  {
    const float4 av = *reinterpret_cast<const float4*>(A + d * N + 4 * q);
    an[0] = av.x; an[1] = av.y; an[2] = av.z; an[3] = av.w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = an[k] * kLog2e;
      ia[k] = ZOH ? 1.0f / an[k] : 0.0f;
    }
  }
  const float bias_d = bias ? bias[d] : 0.0f;
  const float D_d = Dsk ? Dsk[d] : 0.0f;

  float hv[R][4], xv[R], rawd[R];
  bool act[R];
  int64_t idx[R], brow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t bq = static_cast<int64_t>(blockIdx.y) * R + r;
    act[r] = dact && bq < Bsz;
    brow[r] = bq < Bsz ? bq : Bsz - 1;
    idx[r] = brow[r] * D + d;  // (b, t=0, d) and (b, d) share this index
    if (h0) {
      const f4v hv4 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(h0 + idx[r] * N + 4 * q));
      hv[r][0] = hv4.x; hv[r][1] = hv4.y; hv[r][2] = hv4.z; hv[r][3] = hv4.w;
    } else {
      hv[r][0] = hv[r][1] = hv[r][2] = hv[r][3] = 0.0f;
    }
    xv[r] = to_f32(x[idx[r]]);
    rawd[r] = to_f32(dl[idx[r]]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = brow[r];
    float Bv[4], Cv[4];
    load4<S>(Bm + b * N + 4 * q, Bv);
    load4<S>(Cm + b * N + 4 * q, Cv);
    const float dt = softplus_f32(rawd[r] + bias_d);
    const float u = dt * xv[r];
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float ab = fast_exp2(dt * a[k]);
      if constexpr (ZOH)  // zero-order-hold input term: (exp(dt A) - 1) / A * B x
        hv[r][k] = __builtin_fmaf(ab, hv[r][k], (zoh_coef(dt, an[k], ia[k], ab) * xv[r]) * Bv[k]);
      else
        hv[r][k] = __builtin_fmaf(ab, hv[r][k], u * Bv[k]);
      acc = __builtin_fmaf(Cv[k], hv[r][k], acc);
    }
    // Sum the Q partial readouts of this channel (lanes q = 0..Q-1 are adjacent).
#pragma unroll
    for (int off = 1; off < Q; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (act[r]) {
      if (hT)
        __builtin_nontemporal_store((f4v){hv[r][0], hv[r][1], hv[r][2], hv[r][3]},
                                    reinterpret_cast<f4v*>(hT + idx[r] * N + 4 * q));
      if (q == 0) {
        acc = __builtin_fmaf(D_d, xv[r], acc);
        if (z) acc *= silu_f32(to_f32(z[idx[r]]));
        store_elem(y + idx[r], acc);
      }
    }
  }
}

template <typename S, int Q, bool ZOH>
hipError_t launch_decode_z(const Problem& p, hipStream_t stream) {
  constexpr int CH = 256 / Q;
  dim3 grid(static_cast<unsigned>((p.dim + CH - 1) / CH),
            static_cast<unsigned>((p.batch + kDecodeRows - 1) / kDecodeRows));
  hipLaunchKernelGGL((scan_decode_kernel<S, Q, ZOH>), grid, dim3(256), 0, stream,
                     static_cast<const S*>(p.x), static_cast<const S*>(p.delta), p.A,
                     static_cast<const S*>(p.B), static_cast<const S*>(p.C), p.D,
                     static_cast<const S*>(p.z), p.delta_bias, p.h0, p.hT, static_cast<S*>(p.y), p.batch,
                     p.dim);
  return hipGetLastError();
}

template <typename S, int Q>
hipError_t launch_decode_t(const Problem& p, hipStream_t stream) {
  return (p.flags & kFlagZoh) ? launch_decode_z<S, Q, true>(p, stream) : launch_decode_z<S, Q, false>(p, stream);
}

template <typename S>
hipError_t launch_decode_s(const Problem& p, hipStream_t stream) {
  switch (p.dstate) {
    case 4: return launch_decode_t<S, 1>(p, stream);
    case 8: return launch_decode_t<S, 2>(p, stream);
    case 16: return launch_decode_t<S, 4>(p, stream);
    case 32: return launch_decode_t<S, 8>(p, stream);
    case 64: return launch_decode_t<S, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const Problem& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_decode_s<float>(p, stream) : launch_decode_s<uint16_t>(p, stream);
}

}  // namespace ssm
