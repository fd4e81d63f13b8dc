// Backward pass of the selective scan: gradients of a scalar loss with
// respect to every input, given dL/dy and optionally dL/dhT.
//
// Per chain (b, d) the forward is (page youngju.dev "Mamba 논문 리뷰",
// sections 2.2, 3.1, 3.3, 3.4)
//   v = raw + bias, delta = softplus(v), a_n = exp(delta A_n), u = delta x,
//   h_t = a h_{t-1} + u B_t,  y0 = C_t . h_t + D x,  y = y0 SiLU(z),
// and its reverse-mode derivative, walked from t = L-1 down to 0 with the
// adjoint g_n = dL/dhT_n at the start, is
//   gy0 = dy SiLU(z),  dz = dy y0 SiLU'(z),  dD += gy0 x,
//   lam_n = gy0 C_t,n + g_n,  ga_n = lam_n h_{t-1,n},
//   dA_n += ga_n a_n delta,  dB_t,n += lam_n u,  dC_t,n += gy0 h_t,n,
//   gdelta = sum_n ga_n a_n A_n + x sum_n lam_n B_t,n,
//   dx = gy0 D + delta sum_n lam_n B_t,n,  draw = gdelta sigmoid(v),
//   dbias += draw,  g_n = a_n lam_n;  dh0 = g after t = 0.
// Under the zero-order hold (section 2.2) the input term is c_n B_t,n x with
// c_n = (a_n - 1) / A_n in place of u B_t,n, which changes four lines:
//   dB_t,n += lam_n c_n x,  dx = gy0 D + sum_n lam_n c_n B_t,n,
//   gdelta = sum_n ga_n a_n A_n + x sum_n lam_n B_t,n a_n   (dc_n/ddelta = a_n),
//   dA_n += ga_n a_n delta + lam_n B_t,n x dc_n/dA_n;
// the decays, the adjoint's recurrence and the segment fix-ups are the same.
//
// Parallel layout.  G = ceil(N / 8) adjacent lanes share one channel (b, d),
// each owning K = 8 consecutive states (K = 4 when N <= 4), so one wave holds
// 64 / G channels; sums over n are finished across the G lanes with lane
// shuffles.  B_t and C_t reach every lane as one vector load of its K values.
// To fill the chip the sequence is cut into S segments, and both recurrences
// are linear, so a segment can be run from a zero start and fixed up
// afterwards: with P = exp(A * sum of delta over the span), the true state is
// the zero-start state + P o (state entering the span), and the same holds for
// the adjoint walked backwards.
//
//   1. local:   per segment, the forward from zero storing the state entering
//               every chunk of T tokens (a checkpoint) and the running delta
//               sum there; then (S > 1) the adjoint from zero backwards.
//   2. combine: per (b, d, n), walk the S segment summaries forwards (true
//               state entering each segment) and backwards (true adjoint
//               leaving each segment's end).
//   3. main:    per segment, walk its chunks backwards: rebuild the chunk's
//               T states in registers from the fixed-up checkpoint, then run
//               the adjoint through them and write dx, ddelta, dz.
//   4. reduce:  dB, dC sum over channels and dA, dD, dbias over batch rows and
//               segments.  Kernel 3 writes per-wave and per-segment partials
//               and kernel 4 adds them in a fixed order, so every result is
//               independent of scheduling.
// Given the forward's checkpoints (true states after every chunk), pass 1
// runs only the adjoint, pass 2 only combines the adjoint, and pass 3 starts
// each chunk from its checkpoint as it is.
#pragma once

#include "buffer_io.hpp"
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

__device__ __forceinline__ float sigmoid_f32(float v) { return fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }

// d/dA_n of the hold's input coefficient c = (a - 1) / A_n, a = exp(z),
// z = delta A_n: (delta a - c) / A_n.  That difference cancels as z -> 0, so
// for |z| < 1/2 the series delta^2 sum_{k>=1} k z^(k-1) / (k+1)! is taken
// through z^7 (truncation below 3e-8 relative).  One v_cmp + v_cndmask picks
// the branch after both are computed (A_n = 0: z = 0, the series; the closed
// form's 0 * inf is discarded).
__device__ __forceinline__ float zoh_coef_dA(float dt, float inv_An, float a, float c, float z) {
  float p = __builtin_fmaf(z, 1.0f / 45360.0f, 1.0f / 5760.0f);
  p = __builtin_fmaf(z, p, 1.0f / 840.0f);
  p = __builtin_fmaf(z, p, 1.0f / 144.0f);
  p = __builtin_fmaf(z, p, 1.0f / 30.0f);
  p = __builtin_fmaf(z, p, 1.0f / 8.0f);
  p = __builtin_fmaf(z, p, 1.0f / 3.0f);
  p = __builtin_fmaf(z, p, 0.5f);
  const float series = dt * dt * p;
  const float closed = __builtin_fmaf(dt, a, -c) * inv_An;
  float r;
  asm("v_cmp_gt_f32_e64 vcc, %4, |%1|\n\tv_cndmask_b32_e32 %0, %3, %2, vcc"
      : "=v"(r)
      : "v"(z), "v"(series), "v"(closed), "s"(0.5f)
      : "vcc");
  return r;
}

template <bool B>
struct Tag {
  static constexpr bool value = B;
};

template <int V>
constexpr int log2i() {
  return V <= 1 ? 0 : 1 + log2i<V / 2>();
}

// ---- cross-lane sums ---------------------------------------------------------------
// Value held by lane l ^ M.  M = 1, 2: DPP quad permutations; M = 4: two DPP
// row shifts by 4 and a select; M = 8: DPP rotation of each 16-lane row by 8,
// which is l ^ 8; otherwise ds_bpermute.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (M == 1)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  else if constexpr (M == 2)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  else if constexpr (M == 8)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));
  else if constexpr (M == 4) {
    // lanes with bit 2 clear read lane + 4 (row_shl:4), the others lane - 4 (row_shr:4)
    const float up = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xF, 0xF, true));
    const float dn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
    return (__lane_id() & 4) ? dn : up;
  } else
    return __shfl_xor(v, M, 64);
}

// Sum over the G lanes of a channel (adjacent lanes); every lane gets the total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += xor_lane<1>(v);
  if constexpr (G >= 4) v += xor_lane<2>(v);
  if constexpr (G >= 8) v += xor_lane<4>(v);
  return v;
}

// One halving exchange between lanes l and l ^ M.  Lanes with bit M clear
// return lo + partner's lo, lanes with bit M set hi + partner's hi.  For
// M = 32 and 16 one v_permlane32_swap / v_permlane16_swap does it: it trades
// the upper half (odd rows) of its first operand with the lower half (even
// rows) of its second, after which the two registers' sum is the answer in
// every lane.
template <int M>
__device__ __forceinline__ float halve(float lo, float hi, bool upper) {
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const float send = upper ? lo : hi;
    const float keep = upper ? hi : lo;
    return keep + xor_lane<M>(send);
  }
}

template <int M, int G, int CNT, int V>
__device__ __forceinline__ void channel_sum_stage(float (&v)[V], int lane) {
  if constexpr (M >= G && M >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool upper = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) v[i] = halve<M>(v[i], v[i + H], upper);
      channel_sum_stage<M / 2, G, H, V>(v, lane);
    } else {
      v[0] += xor_lane<M>(v[0]);
      channel_sum_stage<M / 2, G, 1, V>(v, lane);
    }
  }
}

// Sum V values per lane over the 64 / G channels of the wave (lanes l and
// l ^ m for m >= G hold the same states of different channels).  On return
// lane l holds, in v[0], the total of its value index l >> (6 - log2 V).
// The first log2 V stages each halve the values a lane carries.
template <int V, int G>
__device__ __forceinline__ void channel_sum(float (&v)[V], int lane) {
  static_assert(V * G <= 64, "one wave holds at most 64 / G channels");
  channel_sum_stage<32, G, V, V>(v, lane);
}

// ---- loads and stores of a lane's K states -----------------------------------------------
// K consecutive values of one B or C row starting at state n0.  FULL (every
// lane's K states exist, N == G K) takes one aligned vector load; otherwise
// every value is loaded from a clamped index and missing states become 0 by a
// select, so no lane-dependent branch is taken.
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}

template <bool FULL, int K>
__device__ __forceinline__ void load_vec(const uint16_t* row, int n0, int N, float (&o)[K]) {
  if constexpr (FULL) {
    if constexpr (K == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + n0);
      unpack_bf16x2(v.x, o[0], o[1]);
      unpack_bf16x2(v.y, o[2], o[3]);
      unpack_bf16x2(v.z, o[4], o[5]);
      unpack_bf16x2(v.w, o[6], o[7]);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(row + n0);
      unpack_bf16x2(v.x, o[0], o[1]);
      unpack_bf16x2(v.y, o[2], o[3]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float v = to_f32(row[min(n0 + k, N - 1)]);
      o[k] = n0 + k < N ? v : 0.0f;
    }
  }
}

template <bool FULL, int K>
__device__ __forceinline__ void load_vec(const float* row, int n0, int N, float (&o)[K]) {
  if constexpr (FULL) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + n0 + k);
      o[k] = v.x;
      o[k + 1] = v.y;
      o[k + 2] = v.z;
      o[k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float v = row[min(n0 + k, N - 1)];
      o[k] = n0 + k < N ? v : 0.0f;
    }
  }
}

// The lane's K states n0 .. n0 + K - 1 of channel d from one checkpoint entry
// laid out in quarters (4, D, M), M = ceil(N / 4): state n at [n / M][d][n % M].
// Runs of 4 states that stay inside a quarter (M a multiple of 4, n0 too)
// are one 16-byte load; otherwise state by state, missing states 0.
template <bool FULL, int K>
__device__ __forceinline__ void load_ckpt(const float* entry, int64_t d, int64_t D, int n0, int N, float (&o)[K]) {
  const int M = ckpt_quarter(N);
  if (FULL && (M & 3) == 0) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const int n = n0 + k;
      const float4 v = *reinterpret_cast<const float4*>(entry + ((n / M) * D + d) * M + n % M);
      o[k] = v.x, o[k + 1] = v.y, o[k + 2] = v.z, o[k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int n = min(n0 + k, N - 1);
      const float v = entry[((n / M) * D + d) * M + n % M];
      o[k] = n0 + k < N ? v : 0.0f;
    }
  }
}

// Checkpoints and gradients are written once and not read again by the
// writing kernel: their stores carry the non-temporal hint (0.6% faster).
template <bool FULL, int K>
__device__ __forceinline__ void store_states(float* row, int n0, int N, const float (&v)[K]) {
  if constexpr (FULL) {
#pragma unroll
    for (int k = 0; k < K; k += 4)
      __builtin_nontemporal_store((float __attribute__((ext_vector_type(4)))){v[k], v[k + 1], v[k + 2], v[k + 3]},
                                  reinterpret_cast<float __attribute__((ext_vector_type(4)))*>(row + n0 + k));
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (n0 + k < N) row[n0 + k] = v[k];
  }
}

// ---- buffer access relative to a segment --------------------------------------------------
// Token tensors are addressed through a buffer descriptor based at the
// segment's first token: a per-lane byte offset (channel or state) in the VGPR
// operand and a per-token byte offset in the scalar operand.  The planner cuts
// segments so that every such span stays below 2 GiB.
using Rsrc = __amdgpu_buffer_rsrc_t;

template <typename S>
__device__ __forceinline__ float ld1(Rsrc r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(S) == 4)
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0));
  else
    return __uint_as_float(
        static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0))
        << 16);
}

// Raw bits of one element (bf16 zero-extended): loads whose values are
// widened only where they are used stay independent of each other.
template <typename S>
__device__ __forceinline__ uint32_t ld1raw(Rsrc r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(S) == 4)
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

template <typename S>
__device__ __forceinline__ void st1(Rsrc r, uint32_t voff, uint32_t soff, float v) {
  if constexpr (sizeof(S) == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voff), static_cast<int>(soff), kStreamPolicy);
  } else {
    const __hip_bfloat16 hb = __float2bfloat16(v);
    __builtin_amdgcn_raw_buffer_store_b16(__bfloat16_as_ushort(hb), r, static_cast<int>(voff), static_cast<int>(soff), kStreamPolicy);
  }
}

// K values of a B or C row: the lane's states n0 .. n0 + K - 1 (voff = n0 * sizeof(S)).
template <typename S, bool FULL, int K>
__device__ __forceinline__ void ldk(Rsrc r, uint32_t voff, uint32_t soff, int n0, int N, float (&o)[K]) {
  const int vo = static_cast<int>(voff), so = static_cast<int>(soff);
  if constexpr (FULL && sizeof(S) == 2 && K == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
    unpack_bf16x2(v[0], o[0], o[1]);
    unpack_bf16x2(v[1], o[2], o[3]);
    unpack_bf16x2(v[2], o[4], o[5]);
    unpack_bf16x2(v[3], o[6], o[7]);
  } else if constexpr (FULL && sizeof(S) == 2 && K == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
    unpack_bf16x2(v[0], o[0], o[1]);
    unpack_bf16x2(v[1], o[2], o[3]);
  } else if constexpr (FULL) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 4 * k, so, 0);
      o[k] = __uint_as_float(v[0]);
      o[k + 1] = __uint_as_float(v[1]);
      o[k + 2] = __uint_as_float(v[2]);
      o[k + 3] = __uint_as_float(v[3]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int n = min(n0 + k, N - 1);
      const float v = ld1<S>(r, static_cast<uint32_t>(n) * sizeof(S), soff);
      o[k] = n0 + k < N ? v : 0.0f;
    }
  }
}

// The raw words of a lane's K values of one B or C row, loaded now and widened
// later, so that a whole chunk's loads can be issued before the first use.
template <typename S, bool FULL, int K>
struct RawK {
  static constexpr bool kPacked = FULL && sizeof(S) == 2;
  static constexpr int W = kPacked ? K / 2 : K;
  uint32_t w[W];

  __device__ __forceinline__ void load(Rsrc r, uint32_t voff, uint32_t soff, int n0, int N) {
    const int vo = static_cast<int>(voff), so = static_cast<int>(soff);
    if constexpr (kPacked && K == 8) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
      w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = v[3];
    } else if constexpr (kPacked) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
      w[0] = v[0], w[1] = v[1];
    } else if constexpr (FULL) {
#pragma unroll
      for (int k = 0; k < K; k += 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 4 * k, so, 0);
        w[k] = v[0], w[k + 1] = v[1], w[k + 2] = v[2], w[k + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int n = min(n0 + k, N - 1);
        w[k] = __float_as_uint(ld1<S>(r, static_cast<uint32_t>(n) * sizeof(S), soff));
      }
    }
  }

  __device__ __forceinline__ void unpack(float (&o)[K], int n0, int N) const {
    if constexpr (kPacked) {
#pragma unroll
      for (int i = 0; i < W; ++i) unpack_bf16x2(w[i], o[2 * i], o[2 * i + 1]);
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) o[k] = (FULL || n0 + k < N) ? __uint_as_float(w[k]) : 0.0f;
    }
  }
};

template <int G>
struct Chain {
  int64_t b, s, blk, d;
  int lane, q, n0;    // q: lane's place among its channel's G lanes; n0 = q K
  bool active;        // the lane's channel exists (inactive lanes mirror channel D - 1)
  int64_t t_begin, t_end;
};

template <int K, int G>
__device__ __forceinline__ Chain<G> chain_of(int64_t D, int64_t L, int64_t seg_len) {
  constexpr int CH = 64 / G;
  Chain<G> c;
  c.b = blockIdx.y;
  c.s = blockIdx.z;
  // A workgroup of G waves covers 64 consecutive channels, so the waves that
  // read the two halves of a 128-byte line of a bf16 (B, L, D) row share a CU
  // (and its L2) rather than landing on different XCDs.  c.blk numbers the
  // waves, which is also the row of the wave's partial dB / dC sums.
  c.blk = static_cast<int64_t>(blockIdx.x) * G + (threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.q = c.lane % G;
  c.n0 = c.q * K;
  const int64_t dd = c.blk * CH + c.lane / G;
  c.active = dd < D;
  c.d = c.active ? dd : D - 1;
  c.t_begin = c.s * seg_len;
  c.t_end = c.t_begin + seg_len < L ? c.t_begin + seg_len : L;
  return c;
}

// Buffer descriptors of one segment's token tensors, and the lane's offsets.
template <typename S>
struct Seg {
  Rsrc x, dl, B, C, z, dy;
  uint32_t tok, nrow;  // bytes per token of a (B, L, D) / (B, L, N) tensor
  uint32_t vd, vn;     // the lane's channel / first-state byte offset within a token
  uint32_t span;       // bytes of the segment in a (B, L, D) tensor
  int64_t e0;          // element index of the segment's first token in a (B, L, D) tensor
  template <int G>
  __device__ __forceinline__ Seg(const Chain<G>& c, const S* xp, const S* dlp, const S* Bp, const S* Cp,
                                 const S* zp, const S* dyp, int64_t L, int64_t D, int N) {
    const int64_t rows = c.t_end - c.t_begin;
    e0 = (c.b * L + c.t_begin) * D;
    const int64_t n0 = (c.b * L + c.t_begin) * N;
    tok = static_cast<uint32_t>(D * sizeof(S));
    nrow = static_cast<uint32_t>(N * sizeof(S));
    span = static_cast<uint32_t>(rows * D * sizeof(S));
    const uint32_t nspan = static_cast<uint32_t>(rows * N * sizeof(S));
    x = make_buf(xp + e0, span);
    dl = make_buf(dlp + e0, span);
    dy = make_buf(dyp + e0, span);
    z = make_buf((zp ? zp : xp) + e0, span);
    B = make_buf(Bp + n0, nspan);
    C = make_buf(Cp + n0, nspan);
    vd = static_cast<uint32_t>(c.d * sizeof(S));
    vn = static_cast<uint32_t>(c.n0 * sizeof(S));
  }
};

// Structured decays: when A[d, n] == (n+1) A[d, 0] holds exactly for every
// state of every channel of the wave (the S4D-real diagonal, A = -(1..N)),
// decay n is r^(n+1) with r = exp(delta A[d, 0]), so a lane takes two exps
// (r and its first decay) and K - 1 multiplies instead of K exps.
template <bool FULL, int K, int G>
__device__ __forceinline__ bool structured_decay(const float* A, const Chain<G>& c, int N, int flags) {
  bool ok = !(flags & kFlagGenericA);
  const float a0 = A[c.d * N];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int n = c.n0 + k;
    const float an = A[c.d * N + min(n, N - 1)];
    ok = ok && ((!FULL && n >= N) || an == static_cast<float>(n + 1) * a0);
  }
  return __all(ok ? 1 : 0) != 0;
}

// The lane's K decays exp(dt A[d, n0 + k]) (A2 = A log2 e, A2r = A[d, 0] log2 e).
template <bool STRUCT, int K>
__device__ __forceinline__ void decays(float dt, const float (&A2)[K], float A2r, float (&an)[K]) {
  if constexpr (STRUCT) {
    const float r = fast_exp2(dt * A2r);
    an[0] = fast_exp2(dt * A2[0]);
#pragma unroll
    for (int k = 1; k < K; ++k) an[k] = an[k - 1] * r;
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) an[k] = fast_exp2(dt * A2[k]);
  }
}

// Runs compute(stage, t0) for the chunks t0 = first + i * step, i < n, with
// the loads of chunk i + 1 issued into the other stage before chunk i is
// computed, so that one chunk's memory latency hides behind the previous
// chunk's arithmetic.
template <typename Stage, typename Load, typename Compute>
__device__ __forceinline__ void pipelined(int64_t first, int64_t step, int64_t n, Load&& load, Compute&& compute) {
  if (n <= 0) return;
  Stage a, b;
  load(a, first);
  for (int64_t i = 0;;) {
    if (i + 1 < n) load(b, first + (i + 1) * step);
    compute(a, first + i * step);
    if (++i >= n) break;
    if (i + 1 < n) load(a, first + (i + 1) * step);
    compute(b, first + i * step);
    if (++i >= n) break;
  }
}

template <typename S, bool FULL, int K, int T>
struct FwdStage {
  uint32_t dl[T], x[T];
  RawK<S, FULL, K> b[T];
};

template <typename S, bool FULL, int K, int T>
struct RevStage {
  uint32_t dl[T], dy[T], z[T];
  RawK<S, FULL, K> c[T];
};

// ---- 1. per-segment local passes ---------------------------------------------------
// Chunks of T tokens are unrolled with all their loads issued first, so that
// they are in flight together.
template <typename S, int K, int G, bool FULL, bool GATE, bool ZOH>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2, 4))) void bwd_local_kernel(
    const S* __restrict__ x, const S* __restrict__ dl, const float* __restrict__ A, const S* __restrict__ Bm,
    const S* __restrict__ Cm, const S* __restrict__ z, const float* __restrict__ bias, const S* __restrict__ dy,
    float* __restrict__ ck, float* __restrict__ ckds, float* __restrict__ segh, float* __restrict__ segc,
    float* __restrict__ segds, const float* __restrict__ ck_in, int64_t L, int64_t D, int N, int64_t seg_len,
    int64_t nck, int64_t nseg, int flags) {
  constexpr int T = bwd_chunk_len(K);
  const Chain<G> c = chain_of<K, G>(D, L, seg_len);
  const Seg<S> sg(c, x, dl, Bm, Cm, z, dy, L, D, N);
  float A2[K], h[K], iA[ZOH ? K : 1];  // iA: 1 / A_n for the hold's coefficient
  load_vec<FULL, K>(A + c.d * N, c.n0, N, A2);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if constexpr (ZOH) iA[k] = 1.0f / A2[k];
    A2[k] *= kLog2e;
    h[k] = 0.0f;
  }
  const float A2r = A[c.d * N] * kLog2e;
  const bool structured = structured_decay<FULL, K>(A, c, N, flags);
  const float bs = bias ? bias[c.d] : 0.0f;
  float ds = 0.0f;
  auto checkpoint = [&](int64_t t0) {
    if (c.active) {
      const int64_t ci = (c.b * nck + t0 / T) * D + c.d;
      if (c.q == 0) ckds[ci] = ds;
      store_states<FULL, K>(ck + ci * N, c.n0, N, h);
    }
  };
  // The forward from zero, one chunk at a time: a chunk's loads are all issued
  // before its steps.  Whole chunks are pipelined (next chunk's loads first);
  // the segment's cut-short last chunk, if any, guards each token.
  using FS = FwdStage<S, FULL, K, T>;
  auto fwd_load = [&](FS& st, int64_t t0, auto ragged) {
    constexpr bool RAGGED = decltype(ragged)::value;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (!RAGGED || t0 + j < c.t_end) {  // wave-uniform
        const uint32_t r = static_cast<uint32_t>(t0 + j - c.t_begin);
        st.dl[j] = ld1raw<S>(sg.dl, sg.vd, r * sg.tok);
        st.x[j] = ld1raw<S>(sg.x, sg.vd, r * sg.tok);
        st.b[j].load(sg.B, sg.vn, r * sg.nrow, c.n0, N);
      }
    }
  };
  auto fwd_steps = [&](const FS& st, int64_t t0, auto ragged, auto structs) {
    constexpr bool RAGGED = decltype(ragged)::value;
    checkpoint(t0);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (!RAGGED || t0 + j < c.t_end) {
        const float dt = softplus_f32(bits_to_f32<S>(st.dl[j]) + bs);
        const float xv = bits_to_f32<S>(st.x[j]);
        const float u = dt * xv;
        ds += dt;
        float Bv[K], an[K];
        st.b[j].unpack(Bv, c.n0, N);
        decays<decltype(structs)::value>(dt, A2, A2r, an);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          if constexpr (ZOH)
            h[k] = __builtin_fmaf(an[k], h[k], (zoh_coef(dt, A2[k] * kLn2, iA[k], an[k]) * xv) * Bv[k]);
          else
            h[k] = __builtin_fmaf(an[k], h[k], u * Bv[k]);
        }
      }
    }
  };
  const int64_t t_tail = c.t_begin + (c.t_end - c.t_begin) / T * T;  // seg_len is a multiple of T
  const int64_t si = (c.b * nseg + c.s) * D + c.d;
  auto fwd_pass = [&](auto structs) {
    pipelined<FS>(
        c.t_begin, T, (t_tail - c.t_begin) / T, [&](FS& st, int64_t t0) { fwd_load(st, t0, Tag<false>{}); },
        [&](const FS& st, int64_t t0) { fwd_steps(st, t0, Tag<false>{}, structs); });
    if (t_tail < c.t_end) {
      FS st;
      fwd_load(st, t_tail, Tag<true>{});
      fwd_steps(st, t_tail, Tag<true>{}, structs);
    }
  };
  const bool own_ck = ck_in == nullptr;  // else the forward's checkpoints hold the states
  if (own_ck) {
    if (structured)
      fwd_pass(Tag<true>{});
    else
      fwd_pass(Tag<false>{});
    if (c.active) {
      if (c.q == 0) segds[si] = ds;
      store_states<FULL, K>(segh + si * N, c.n0, N, h);
    }
  }
  if (nseg == 1 || c.s == 0) return;  // the adjoint entering segment 0 from the left is never needed
  ds = 0.0f;  // the adjoint pass sums delta again (the combine's decay over the segment)
  float g[K];
#pragma unroll
  for (int k = 0; k < K; ++k) g[k] = 0.0f;
  // The adjoint from zero, walked backwards chunk by chunk (cut-short last
  // chunk first, then the whole chunks, pipelined as above).
  using RS = RevStage<S, FULL, K, T>;
  auto rev_load = [&](RS& st, int64_t t0, auto ragged) {
    constexpr bool RAGGED = decltype(ragged)::value;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (!RAGGED || t0 + j < c.t_end) {  // wave-uniform
        const uint32_t r = static_cast<uint32_t>(t0 + j - c.t_begin);
        st.dl[j] = ld1raw<S>(sg.dl, sg.vd, r * sg.tok);
        st.dy[j] = ld1raw<S>(sg.dy, sg.vd, r * sg.tok);
        if constexpr (GATE) st.z[j] = ld1raw<S>(sg.z, sg.vd, r * sg.tok);
        st.c[j].load(sg.C, sg.vn, r * sg.nrow, c.n0, N);
      }
    }
  };
  auto rev_steps = [&](const RS& st, int64_t t0, auto ragged, auto structs) {
    constexpr bool RAGGED = decltype(ragged)::value;
#pragma unroll
    for (int j = T - 1; j >= 0; --j) {
      if (!RAGGED || t0 + j < c.t_end) {
        const float dt = softplus_f32(bits_to_f32<S>(st.dl[j]) + bs);
        ds += dt;
        float gy0 = bits_to_f32<S>(st.dy[j]);
        if constexpr (GATE) gy0 *= silu_f32(bits_to_f32<S>(st.z[j]));
        float Cv[K], an[K];
        st.c[j].unpack(Cv, c.n0, N);
        decays<decltype(structs)::value>(dt, A2, A2r, an);
#pragma unroll
        for (int k = 0; k < K; ++k) g[k] = an[k] * __builtin_fmaf(gy0, Cv[k], g[k]);
      }
    }
  };
  auto rev_pass = [&](auto structs) {
    if (t_tail < c.t_end) {
      RS st;
      rev_load(st, t_tail, Tag<true>{});
      rev_steps(st, t_tail, Tag<true>{}, structs);
    }
    pipelined<RS>(
        t_tail - T, -T, (t_tail - c.t_begin) / T, [&](RS& st, int64_t t0) { rev_load(st, t0, Tag<false>{}); },
        [&](const RS& st, int64_t t0) { rev_steps(st, t0, Tag<false>{}, structs); });
  };
  if (structured)
    rev_pass(Tag<true>{});
  else
    rev_pass(Tag<false>{});
  if (c.active) {
    store_states<FULL, K>(segc + si * N, c.n0, N, g);
    if (!own_ck && c.q == 0) segds[si] = ds;
  }
}

// ---- 3. the adjoint walk ------------------------------------------------------------------
template <typename S, int K, int G, bool FULL, bool GATE, bool ZOH>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(FULL ? 2 : 1, 2))) void bwd_main_kernel(
    const S* __restrict__ x, const S* __restrict__ dl, const float* __restrict__ A, const S* __restrict__ Bm,
    const S* __restrict__ Cm, const float* __restrict__ Dsk, const S* __restrict__ z,
    const float* __restrict__ bias, const S* __restrict__ dy, const float* __restrict__ ck,
    const float* __restrict__ ckds, const float* __restrict__ segh, const float* __restrict__ segc,
    const float* __restrict__ ck_in, const float* __restrict__ h0, S* __restrict__ gx, S* __restrict__ gdl,
    S* __restrict__ gz, float* __restrict__ gh0, float* __restrict__ pB, float* __restrict__ pC,
    float* __restrict__ pA, float* __restrict__ pD, float* __restrict__ pbias, int64_t L, int64_t D, int N,
    int64_t seg_len, int64_t nck, int64_t nseg, int flags) {
  constexpr int T = bwd_chunk_len(K);
  constexpr int LGK = log2i<K>();
  const Chain<G> c = chain_of<K, G>(D, L, seg_len);
  const Seg<S> sg(c, x, dl, Bm, Cm, z, dy, L, D, N);
  const int64_t nblk = static_cast<int64_t>(gridDim.x) * G;  // waves per (batch row, segment)
  const int64_t si = (c.b * nseg + c.s) * D + c.d;
  // Outputs: the (B, L, D) gradients share the inputs' offsets.  Stores carry no
  // branch: an output that was not asked for gets an empty descriptor, and an
  // inactive lane stores at an offset outside every descriptor; both are dropped
  // by the hardware range check.  The partial dB / dC rows of the segment hold
  // nblk * N floats per token.
  const Rsrc rgx = make_buf((gx ? gx : x) + sg.e0, gx ? sg.span : 0);
  const Rsrc rgdl = make_buf((gdl ? gdl : x) + sg.e0, gdl ? sg.span : 0);
  const Rsrc rgz = make_buf((gz ? gz : x) + sg.e0, gz ? sg.span : 0);
  const uint32_t vst = c.active ? sg.vd : kOutOfRange;
  const uint32_t prow = static_cast<uint32_t>(nblk * N * 4);
  const Rsrc rpB = make_buf(pB + (c.b * L + c.t_begin) * nblk * N, static_cast<uint32_t>(c.t_end - c.t_begin) * prow);
  const Rsrc rpC = make_buf(pC + (c.b * L + c.t_begin) * nblk * N, static_cast<uint32_t>(c.t_end - c.t_begin) * prow);

  float A2[K], g[K], gA[K], hin[K];  // hin: true state entering the segment
  float iA[ZOH ? K : 1];              // 1 / A_n for the hold's coefficient
  load_vec<FULL, K>(A + c.d * N, c.n0, N, A2);
  load_vec<FULL, K>(segc + si * N, c.n0, N, g);
  if (ck_in == nullptr) load_vec<FULL, K>(segh + si * N, c.n0, N, hin);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if constexpr (ZOH) iA[k] = 1.0f / A2[k];
    A2[k] *= kLog2e;
    gA[k] = 0.0f;
  }
  const float A2r = A[c.d * N] * kLog2e;
  const bool structured = structured_decay<FULL, K>(A, c, N, flags);
  const float bs = bias ? bias[c.d] : 0.0f;
  const float Dd = Dsk ? Dsk[c.d] : 0.0f;
  float gDacc = 0.0f, gbacc = 0.0f;
  // the lane that writes a channel-summed dB / dC value, and its state index
  const int wn = c.n0 + (c.lane >> (6 - LGK));
  const bool writer = (c.lane & ((64 >> LGK) - 1) & ~(G - 1)) == 0 && wn < N;
  const uint32_t vp = writer ? static_cast<uint32_t>((c.blk * N + wn) * 4) : kOutOfRange;

  // One chunk: rebuild its states, then walk it backwards.  RAGGED (the
  // segment's last chunk when it is cut short) guards every token; whole
  // chunks run unguarded so their loads can be scheduled freely.
  auto chunk = [&](int64_t cc, auto ragged, auto st) {
    constexpr bool RAGGED = decltype(ragged)::value;
    constexpr bool STRUCT = decltype(st)::value;
    const int64_t t0 = cc * T;
    // The rebuild's loads (delta, x and the lane's B words of every token) are
    // issued here, before any is used.  The backward walk reloads B with C, dy
    // and z, kAhead tokens ahead of their use, so only a few tokens' worth of
    // them is live at a time.
    constexpr int kAhead = 2;
    uint32_t dlraw[T], xraw[T];
    RawK<S, FULL, K> rb[T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const int64_t t = t0 + j;
      if (!RAGGED || t < c.t_end) {  // wave-uniform
        const uint32_t so = static_cast<uint32_t>(t - c.t_begin) * sg.tok, sn = static_cast<uint32_t>(t - c.t_begin) * sg.nrow;
        dlraw[j] = ld1raw<S>(sg.dl, sg.vd, so);
        xraw[j] = ld1raw<S>(sg.x, sg.vd, so);
        rb[j].load(sg.B, sg.vn, sn, c.n0, N);
      }
    }
    uint32_t dyv[T], zv[T];
    RawK<S, FULL, K> rb2[T], rc[T];
    auto load_rev = [&](int j) {
      const int64_t t = t0 + j;
      if (!RAGGED || t < c.t_end) {  // wave-uniform
        const uint32_t so = static_cast<uint32_t>(t - c.t_begin) * sg.tok, sn = static_cast<uint32_t>(t - c.t_begin) * sg.nrow;
        rb2[j].load(sg.B, sg.vn, sn, c.n0, N);
        rc[j].load(sg.C, sg.vn, sn, c.n0, N);
        dyv[j] = ld1raw<S>(sg.dy, sg.vd, so);
        if constexpr (GATE) zv[j] = ld1raw<S>(sg.z, sg.vd, so);
      }
    };
    // hs[0] = state entering the chunk, hs[j + 1] = state after token t0 + j;
    // dts: softplus of the chunk's raw steps
    // dts: softplus of the chunk's raw steps; lsg: v - softplus(v); xv: x
    float hs[T + 1][K], dts[T], lsg[T], xv[T];
    if (ck_in) {  // the forward's state entering the chunk (h0 for the first)
      if (cc > 0) {
        load_ckpt<FULL, K>(ck_in + (c.b * (nck - 1) + cc - 1) * 4 * D * ckpt_quarter(N), c.d, D, c.n0, N, hs[0]);
      } else if (h0) {
        load_vec<FULL, K>(h0 + (c.b * D + c.d) * N, c.n0, N, hs[0]);
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) hs[0][k] = 0.0f;
      }
    } else {
      const int64_t ci = (c.b * nck + cc) * D + c.d;
      const float ds0 = ckds[ci];
      load_vec<FULL, K>(ck + ci * N, c.n0, N, hs[0]);
#pragma unroll
      for (int k = 0; k < K; ++k) hs[0][k] = __builtin_fmaf(fast_exp2(A2[k] * ds0), hin[k], hs[0][k]);
    }
#pragma unroll
    for (int j = 0; j < T; ++j) {
      if (!RAGGED || t0 + j < c.t_end) {  // wave-uniform
        const float v = bits_to_f32<S>(dlraw[j]) + bs;
        dts[j] = softplus_f32(v);
        lsg[j] = v - dts[j];  // log of softplus'(v) = sigmoid(v)
        xv[j] = bits_to_f32<S>(xraw[j]);
        const float u = dts[j] * xv[j];
        float Bv[K], an[K];
        rb[j].unpack(Bv, c.n0, N);
        decays<STRUCT>(dts[j], A2, A2r, an);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          if constexpr (ZOH)
            hs[j + 1][k] =
                __builtin_fmaf(an[k], hs[j][k], (zoh_coef(dts[j], A2[k] * kLn2, iA[k], an[k]) * xv[j]) * Bv[k]);
          else
            hs[j + 1][k] = __builtin_fmaf(an[k], hs[j][k], u * Bv[k]);
        }
      }
    }
#pragma unroll
    for (int j = T - 1; j >= T - kAhead; --j) load_rev(j);
#pragma unroll
    for (int j = T - 1; j >= 0; --j) {
      if (j >= kAhead) load_rev(j - kAhead);
      const int64_t t = t0 + j;
      if (RAGGED && t >= c.t_end) continue;  // wave-uniform
      const uint32_t so = static_cast<uint32_t>(t - c.t_begin) * sg.tok;
      const float x_t = xv[j];
      // the decays are recomputed rather than kept from the rebuild (64 more registers)
      float dt = dts[j];
      asm volatile("" : "+v"(dt));
      const float u = dt * x_t;
      float Bv[K], Cv[K];
      rb2[j].unpack(Bv, c.n0, N);
      rc[j].unpack(Cv, c.n0, N);
      const float dy_t = bits_to_f32<S>(dyv[j]);
      float gy0 = dy_t;
      if constexpr (GATE) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) s = __builtin_fmaf(Cv[k], hs[j + 1][k], s);
        const float y0 = __builtin_fmaf(Dd, x_t, group_sum<G>(s));
        const float z_t = bits_to_f32<S>(zv[j]);
        const float sz = sigmoid_f32(z_t);
        gy0 = dy_t * z_t * sz;
        st1<S>(rgz, vst, so, dy_t * y0 * sz * __builtin_fmaf(z_t, 1.0f - sz, 1.0f));
      }
      gDacc = __builtin_fmaf(gy0, x_t, gDacc);
      // inactive lanes add nothing to the channel sums
      const float u_act = c.active ? u : 0.0f;
      const float x_act = c.active ? x_t : 0.0f;
      const float gy_act = c.active ? gy0 : 0.0f;
      // gu: sum_n lam_n B_n dc_n/ddelta (Euler: dc/ddelta = 1; hold: a_n);
      // gx: the hold's sum_n lam_n B_n c_n for dx (Euler: delta gu)
      float gu = 0.0f, gdel = 0.0f, gx = 0.0f;
      float vb[K], vc[K], an[K];
      decays<STRUCT>(dt, A2, A2r, an);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float lam = __builtin_fmaf(gy0, Cv[k], g[k]);
        g[k] = an[k] * lam;                 // adjoint of h_{t-1}
        const float gaa = g[k] * hs[j][k];  // lam a_n h_{t-1}: the decay's share
        gA[k] = __builtin_fmaf(gaa, dt, gA[k]);
        gdel = __builtin_fmaf(gaa, A2[k], gdel);  // A scaled by log2 e; undone below
        if constexpr (ZOH) {
          const float Ak = A2[k] * kLn2;
          const float ck = zoh_coef(dt, Ak, iA[k], an[k]);
          const float lb = lam * Bv[k];
          gA[k] = __builtin_fmaf(lb * x_t, zoh_coef_dA(dt, iA[k], an[k], ck, dt * Ak), gA[k]);
          gu = __builtin_fmaf(lb, an[k], gu);
          gx = __builtin_fmaf(lb, ck, gx);
          vb[k] = lam * (ck * x_act);
        } else {
          gu = __builtin_fmaf(lam, Bv[k], gu);
          vb[k] = lam * u_act;
        }
        vc[k] = gy_act * hs[j + 1][k];
      }
      gu = group_sum<G>(gu);
      gdel = __builtin_fmaf(group_sum<G>(gdel), kLn2, gu * x_t);
      // softplus' = sigmoid, taken as exp(v - softplus(v)), exact in both tails
      const float graw = gdel * fast_exp2(lsg[j] * kLog2e);
      gbacc += graw;
      if constexpr (ZOH)
        st1<S>(rgx, vst, so, __builtin_fmaf(gy0, Dd, group_sum<G>(gx)));
      else
        st1<S>(rgx, vst, so, __builtin_fmaf(gy0, Dd, gu * dt));
      st1<S>(rgdl, vst, so, graw);
      channel_sum<K, G>(vb, c.lane);
      channel_sum<K, G>(vc, c.lane);
      const uint32_t sp = static_cast<uint32_t>(t - c.t_begin) * prow;
      st1<float>(rpB, vp, sp, vb[0]);
      st1<float>(rpC, vp, sp, vc[0]);
    }
  };
  auto run = [&](auto st) {
    const int64_t c_first = c.t_begin / T;
    int64_t cc = (c.t_end - 1) / T;
    if ((cc + 1) * T > c.t_end) chunk(cc--, Tag<true>{}, st);
    for (; cc >= c_first; --cc) chunk(cc, Tag<false>{}, st);
  };
  if (structured)
    run(Tag<true>{});
  else
    run(Tag<false>{});
  if (c.active) {
    if (gh0 && c.s == 0) store_states<FULL, K>(gh0 + (c.b * D + c.d) * N, c.n0, N, g);
    store_states<FULL, K>(pA + si * N, c.n0, N, gA);
    if (c.q == 0) {
      pD[si] = gDacc;
      pbias[si] = gbacc;
    }
  }
}

// ---- 4. fixed-order sums of the partials ---------------------------------------------------
template <typename S>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ pB,
                                                            const float* __restrict__ pC, S* __restrict__ gB,
                                                            S* __restrict__ gC, int64_t rows, int N, int64_t nblk) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (b, t, n)
  if (i >= rows * N) return;
  const int64_t r = i / N, n = i % N;
  float sb = 0.0f, sc = 0.0f;
  // (unrolled so that eight rows' loads are in flight; the adds keep their order)
#pragma unroll 8
  for (int64_t k = 0; k < nblk; ++k) {
    sb += pB[(r * nblk + k) * N + n];
    sc += pC[(r * nblk + k) * N + n];
  }
  if (gB) store_elem(gB + i, sb);
  if (gC) store_elem(gC + i, sc);
}

unsigned blocks256(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

template <typename S, int K, int G, bool FULL, bool GATE, bool ZOH>
hipError_t launch_bwd_t(const BwdProblem& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.nblk / G), static_cast<unsigned>(p.batch), static_cast<unsigned>(p.splits));
  const dim3 block(64 * G);
  const int N = static_cast<int>(p.dstate);
  const auto* x = static_cast<const S*>(p.x);
  const auto* dl = static_cast<const S*>(p.delta);
  const auto* Bm = static_cast<const S*>(p.B);
  const auto* Cm = static_cast<const S*>(p.C);
  const auto* z = static_cast<const S*>(p.z);
  const auto* dy = static_cast<const S*>(p.dy);
  hipLaunchKernelGGL((bwd_local_kernel<S, K, G, FULL, GATE, ZOH>), grid, block, 0, stream, x, dl, p.A, Bm, Cm, z, p.delta_bias,
                     dy, p.ck, p.ckds, p.segh, p.segc, p.segds, p.ck_in, p.seqlen, p.dim, N, p.seg_len, p.nck,
                     static_cast<int64_t>(p.splits), p.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = bwd::launch_combine(p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<S, K, G, FULL, GATE, ZOH>), grid, block, 0, stream, x, dl, p.A, Bm, Cm, p.D, z,
                     p.delta_bias, dy, p.ck, p.ckds, p.segh, p.segc, p.ck_in, p.h0, static_cast<S*>(p.dx),
                     static_cast<S*>(p.ddelta), static_cast<S*>(p.dz), p.dh0, p.pB, p.pC, p.pA, p.pD, p.pbias,
                     p.seqlen, p.dim, N, p.seg_len, p.nck, static_cast<int64_t>(p.splits), p.flags);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = p.batch * p.seqlen;
  if (p.dB || p.dC) {
    hipLaunchKernelGGL((bwd_reduce_bc_kernel<S>), dim3(blocks256(rows * N)), dim3(256), 0, stream, p.pB, p.pC,
                       static_cast<S*>(p.dB), static_cast<S*>(p.dC), rows, N, p.nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.dA || p.dD || p.ddelta_bias) e = bwd::launch_reduce_d(p, stream);
  return e;
}

template <typename S, int K, int G, bool FULL, bool GATE>
hipError_t launch_bwd_z(const BwdProblem& p, hipStream_t stream) {
  return (p.flags & kFlagZoh) ? launch_bwd_t<S, K, G, FULL, GATE, true>(p, stream)
                              : launch_bwd_t<S, K, G, FULL, GATE, false>(p, stream);
}

template <typename S, int K, int G, bool FULL>
hipError_t launch_bwd_f(const BwdProblem& p, hipStream_t stream) {
  return p.z ? launch_bwd_z<S, K, G, FULL, true>(p, stream) : launch_bwd_z<S, K, G, FULL, false>(p, stream);
}

template <typename S, int K, int G>
hipError_t launch_bwd_kg(const BwdProblem& p, hipStream_t stream) {
  return p.dstate == K * G ? launch_bwd_f<S, K, G, true>(p, stream) : launch_bwd_f<S, K, G, false>(p, stream);
}

template <typename S>
hipError_t launch_bwd_s(const BwdProblem& p, hipStream_t stream) {
  switch (bwd_lanes_per_channel(p.dstate)) {
    case 1: return bwd_lane_states(p.dstate) == 4 ? launch_bwd_kg<S, 4, 1>(p, stream) : launch_bwd_kg<S, 8, 1>(p, stream);
    case 2: return launch_bwd_kg<S, 8, 2>(p, stream);
    case 4: return launch_bwd_kg<S, 8, 4>(p, stream);
    default: return launch_bwd_kg<S, 8, 8>(p, stream);
  }
}

}  // namespace

namespace bwd {
template <typename S>
hipError_t launch_typed(const BwdProblem& p, hipStream_t stream) {
  return launch_bwd_s<S>(p, stream);
}
}  // namespace bwd

}  // namespace ssm
