// The block's prologue on x before the scan: a depthwise causal convolution
// followed by SiLU (page youngju.dev "Mamba 논문 리뷰", section 3.4 listing:
// Conv1d over channels with groups = channels and padding = width - 1, output
// cut to the first L positions, then SiLU):
//   u[b,t,d] = SiLU(bias[d] + sum_{k<W} w[d,k] x[b, t-(W-1)+k, d]),
// where x at a negative token index is zero or, with a carried state, row
// W-1+i of state (the previous call's last W-1 input rows).
//
// One pass over x, bound by HBM: every thread owns CG consecutive channels
// (16 bytes of a token row: 8 bf16 or 4 fp32) and a run of TT = 128 tokens, keeping
// the W-1 previous inputs of its channels in registers as a sliding window.
// Consecutive threads hold consecutive channel groups, so a wave reads and
// writes 1 KiB contiguous per token.  The window is seeded from the W-1 rows
// before the run (from x, or the carried state before token 0), an overlap of
// (W-1)/TT extra reads that the L2 mostly serves.  Tokens are processed in
// batches of 8 whose rows' loads are issued first; u is written with
// non-temporal stores.  (Measured at B4 L8192 D4096 bf16: runs of 64/128/256
// tokens and batches of 4/8/16 move the time by under 10% except 256-token
// runs, which leave too few waves; non-temporal stores gain 6%.)
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

// CG channels of one token row as fp32 (CG * sizeof(S) == 16 bytes, aligned).
// Each input row is read once (the window of earlier rows stays in
// registers), so the loads carry the non-temporal hint (about 2% faster).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
template <typename S, int CG>
__device__ __forceinline__ void load_row(const S* p, float (&o)[CG]) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  if constexpr (sizeof(S) == 2) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    o[0] = __uint_as_float(v.x), o[1] = __uint_as_float(v.y), o[2] = __uint_as_float(v.z), o[3] = __uint_as_float(v.w);
  }
}

template <typename S, int CG>
__device__ __forceinline__ void store_row(S* p, const float (&v)[CG]) {
  uint32_t w[4];
  if constexpr (sizeof(S) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __bfloat16_as_ushort(__float2bfloat16(v[2 * i]));
      const uint32_t hi = __bfloat16_as_ushort(__float2bfloat16(v[2 * i + 1]));
      w[i] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
  }
  // u is not read again by this kernel: stream it past the caches (nt)
  uint4* q = reinterpret_cast<uint4*>(p);
  __builtin_nontemporal_store(w[0], &q->x);
  __builtin_nontemporal_store(w[1], &q->y);
  __builtin_nontemporal_store(w[2], &q->z);
  __builtin_nontemporal_store(w[3], &q->w);
}

// Single-channel access for the path where D is not a multiple of CG.
template <typename S>
__device__ __forceinline__ void load_row(const S* p, float (&o)[1]) {
  o[0] = to_f32(*p);
}
template <typename S>
__device__ __forceinline__ void store_row(S* p, const float (&v)[1]) {
  store_elem(p, v[0]);
}

#ifndef SSM_CONV_TT
#define SSM_CONV_TT 128
#endif
#ifndef SSM_CONV_UNROLL
#define SSM_CONV_UNROLL 8
#endif
// Tokens per thread (a run) and tokens whose loads are issued together.
constexpr int kConvRun = SSM_CONV_TT;
constexpr int kConvBatch = SSM_CONV_UNROLL;

template <typename S, int W, int CG>
__global__ __launch_bounds__(256) void conv_silu_kernel(const S* __restrict__ x, const float* __restrict__ w,
                                                        const float* __restrict__ bias, const S* __restrict__ state,
                                                        S* __restrict__ u, int64_t L, int64_t D, int64_t ngroups,
                                                        int64_t TT) {
  constexpr int H = W - 1;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  const int64_t b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * TT;
  const int64_t t1 = t0 + TT < L ? t0 + TT : L;
  const int64_t d0 = gi * CG;
  float wk[W][CG], bs[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k][c] = w[(d0 + c) * W + k];
    bs[c] = bias ? bias[d0 + c] : 0.0f;
  }
  const S* xb = x + b * L * D + d0;
  S* ub = u + b * L * D + d0;
  // the W-1 inputs before token t0
  float win[H > 0 ? H : 1][CG];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t i = t0 - H + j;
    if (i >= 0) {
      load_row<S>(xb + i * D, win[j]);
    } else if (state) {
      load_row<S>(state + (b * H + H + i) * D + d0, win[j]);
    } else {
#pragma unroll
      for (int c = 0; c < CG; ++c) win[j][c] = 0.0f;
    }
  }
  auto step = [&](const float (&xr)[CG], int64_t t) {
    float out[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      float acc = bs[c];
#pragma unroll
      for (int k = 0; k < H; ++k) acc = __builtin_fmaf(wk[k][c], win[k][c], acc);
      acc = __builtin_fmaf(wk[H][c], xr[c], acc);
      out[c] = silu_f32(acc);
    }
    store_row<S>(ub + t * D, out);
#pragma unroll
    for (int j = 0; j + 1 < H; ++j)
#pragma unroll
      for (int c = 0; c < CG; ++c) win[j][c] = win[j + 1][c];
    if constexpr (H > 0) {
#pragma unroll
      for (int c = 0; c < CG; ++c) win[H - 1][c] = xr[c];
    }
  };
  int64_t t = t0;
  for (; t + kConvBatch <= t1; t += kConvBatch) {
    float xr[kConvBatch][CG];
#pragma unroll
    for (int q = 0; q < kConvBatch; ++q) load_row<S>(xb + (t + q) * D, xr[q]);
#pragma unroll
    for (int q = 0; q < kConvBatch; ++q) step(xr[q], t + q);
  }
  for (; t < t1; ++t) {
    float xr[CG];
    load_row<S>(xb + t * D, xr);
    step(xr, t);
  }
}

// state_out[b, j, d] = input row L-(W-1)+j: from x, or from the carried state
// when that row precedes token 0 (calls shorter than W-1), or zero.
template <typename S>
__global__ __launch_bounds__(256) void conv_state_out_kernel(const S* __restrict__ x, const S* __restrict__ state,
                                                             S* __restrict__ state_out, int64_t Bsz, int64_t L,
                                                             int64_t D, int H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (b, j, d)
  if (i >= Bsz * H * D) return;
  const int64_t d = i % D, j = (i / D) % H, b = i / (D * H);
  const int64_t src = L - H + j;
  S v{};
  if (src >= 0)
    v = x[(b * L + src) * D + d];
  else if (state)
    v = state[(b * H + H + src) * D + d];
  state_out[i] = v;
}

template <typename S, int W>
hipError_t launch_conv_w(const ConvProblem& p, hipStream_t stream) {
  constexpr int CGV = 16 / static_cast<int>(sizeof(S));
  const auto* x = static_cast<const S*>(p.x);
  const auto* st = static_cast<const S*>(p.state);
  auto* u = static_cast<S*>(p.u);
  // tokens per thread: kConvRun, more when the sequence would need over 65535 runs
  int64_t TT = kConvRun;
  while ((p.seqlen + TT - 1) / TT > 65535) TT *= 2;
  const unsigned nt = static_cast<unsigned>((p.seqlen + TT - 1) / TT);
  if (p.dim % CGV == 0) {
    const int64_t ng = p.dim / CGV;
    hipLaunchKernelGGL((conv_silu_kernel<S, W, CGV>), dim3(static_cast<unsigned>((ng + 255) / 256), nt,
                       static_cast<unsigned>(p.batch)), dim3(256), 0, stream, x, p.weight, p.bias, st, u, p.seqlen,
                       p.dim, ng, TT);
  } else {
    hipLaunchKernelGGL((conv_silu_kernel<S, W, 1>), dim3(static_cast<unsigned>((p.dim + 255) / 256), nt,
                       static_cast<unsigned>(p.batch)), dim3(256), 0, stream, x, p.weight, p.bias, st, u, p.seqlen,
                       p.dim, p.dim, TT);
  }
  return hipGetLastError();
}

template <typename S>
hipError_t launch_conv_s(const ConvProblem& p, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.seqlen > 0) {
    switch (p.width) {
      case 1: e = launch_conv_w<S, 1>(p, stream); break;
      case 2: e = launch_conv_w<S, 2>(p, stream); break;
      case 3: e = launch_conv_w<S, 3>(p, stream); break;
      default: e = launch_conv_w<S, 4>(p, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  const int H = p.width - 1;
  const int64_t n = p.batch * H * p.dim;
  if (p.state_out && n > 0) {
    hipLaunchKernelGGL((conv_state_out_kernel<S>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const S*>(p.x), static_cast<const S*>(p.state), static_cast<S*>(p.state_out),
                       p.batch, p.seqlen, p.dim, H);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_conv(const ConvProblem& p, hipStream_t stream) {
  return p.dtype == 0 ? launch_conv_s<float>(p, stream) : launch_conv_s<uint16_t>(p, stream);
}

}  // namespace ssm
