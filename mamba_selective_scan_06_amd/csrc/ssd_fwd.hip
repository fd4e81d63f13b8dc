// Mamba-2 state-space dual (SSD) layer, forward, in chunked matrix form on
// MFMA (page youngju.dev "Mamba 논문 리뷰", section 4.1: the recurrence
// h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t is also the structured masked
// attention Y = (T o M) X).  Per batch row b and head h, with scalar decay
// rate A[h], delta_t = softplus(dt + dt_bias[h]) and the Euler input term:
//   S_t = exp(delta_t A[h]) S_{t-1} + delta_t x_t B_t^T      (S: P x N, fp32)
//   y_t = S_t C_t + D[h] x_t
// Cut into chunks of Q = 64 tokens, with cs_t the running sum of delta A
// inside the chunk (cs_end its last value) and H the state entering it:
//   G      = C B^T                               (Q x Q, contraction over N)
//   M[t,s] = G[t,s] exp(cs_t - cs_s) delta_s  for s <= t, else 0
//   y      = M X + exp(cs_t) C H^T + D x        (Q x P)
//   H'     = exp(cs_end) H + (X o w)^T B,  w_s = exp(cs_end - cs_s) delta_s
// Every product is a bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation; the state H stays fp32 in registers.  The three operands that
// are computed in fp32 (M, x o w and the state copy read by C H^T) are split
// into hi + lo bf16 halves, each product taking two MFMAs: rounding them to
// one bf16 alone costs a relative 1e-2 in y and 2e-2 in the state, the split
// leaves about 2^-16.  The other operands (x, B, C) are bf16 inputs, exact.
//
// One workgroup (4 waves) per (b, h) walks the chunks in order.  Per chunk:
//   1. one wave turns dt into delta and the prefix sums cs (LDS);
//   2. x and B are written to LDS transposed (token index contiguous), x also
//      scaled by w, for the two products that contract over tokens;
//   3. each wave computes one 32x32 tile of G (its C and B operands come
//      straight from HBM, n contiguous), masks it into M (LDS), and one 32x32
//      tile of C H^T;
//   4. each wave finishes one 32x32 tile of y (M X from LDS) and N/64 tiles
//      of the state update.
// Tokens past L are padded with delta = 0 and x = B = C = 0, which leaves the
// state unchanged, and are not stored.
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // head channels (headdim)
constexpr int kPad = 8;  // bf16 padding of every LDS row (16 bytes), against bank conflicts

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ uint16_t to_bf16_bits(float v) { return __bfloat16_as_ushort(__float2bfloat16(v)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row and column of element r of a 32x32 MFMA accumulator held by lane l.
__device__ __forceinline__ int acc_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int l) { return l & 31; }

// hi and lo bf16 halves of an fp32 value: v ~ hi + lo to about 2^-16.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16_bits(v);
  lo = to_bf16_bits(v - __uint_as_float(static_cast<uint32_t>(hi) << 16));
}

template <int N>
struct SsdSmem {
  uint16_t M[2][kQ][kQ + kPad];   // masked, decayed C B^T, hi and lo halves, rows t
  uint16_t xt[kP][kQ + kPad];     // x transposed: [p][s]
  uint16_t xw[2][kP][kQ + kPad];  // x o w transposed, hi and lo: [p][s]
  uint16_t bt[N][kQ + kPad];      // B transposed: [n][s]
  uint16_t hb[2][kP][N + kPad];   // the state entering the chunk, hi and lo: [p][n]
  float dl[kQ];                   // delta per token of the chunk (0 past L)
  float cs[kQ];                   // running sum of delta A inside the chunk
};

template <int N>
__global__ __launch_bounds__(256) void ssd_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt,
                                                      const float* __restrict__ A, const uint16_t* __restrict__ Bm,
                                                      const uint16_t* __restrict__ Cm, const float* __restrict__ Dsk,
                                                      const float* __restrict__ dt_bias, const float* __restrict__ h0,
                                                      float* __restrict__ hT, uint16_t* __restrict__ y, int64_t L,
                                                      int H, int G) {
  constexpr int NT = N / 64;  // state tiles (32 x 32) per wave
  __shared__ SsdSmem<N> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t b = blockIdx.y;
  const int h = blockIdx.x;
  const int g = h / (H / G);
  const float Ah = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = Dsk ? Dsk[h] : 0.0f;
  const int64_t xrow = static_cast<int64_t>(H) * kP;  // elements between tokens in x / y
  const int64_t brow = static_cast<int64_t>(G) * N;   // elements between tokens in B / C
  const uint16_t* xb = x + (b * L * H + h) * kP;
  uint16_t* yb = y + (b * L * H + h) * kP;
  const uint16_t* Bb = Bm + (b * L * G + g) * N;
  const uint16_t* Cb = Cm + (b * L * G + g) * N;

  // this wave's tiles: (ti, tj) of G and y; state tiles q = w + 4 i of the N x P state (rows n, cols p)
  const int ti = w >> 1, tj = w & 1;
  const int col = acc_col(lane);

  // the state, fp32, in accumulator layout: Hs[i][r] = S[p = 32 (q & 1) + col][n = 32 (q >> 1) + acc_row(r)]
  float Hs[NT][16];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int q = w + 4 * i, p = 32 * (q & 1) + col;
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const int n = 32 * (q >> 1) + acc_row(r, lane);
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (h0) v = *reinterpret_cast<const float4*>(h0 + ((b * H + h) * kP + p) * N + n);
      Hs[i][r] = v.x, Hs[i][r + 1] = v.y, Hs[i][r + 2] = v.z, Hs[i][r + 3] = v.w;
    }
  }
  auto write_hb = [&]() {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int q = w + 4 * i, p = 32 * (q & 1) + col;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int n = 32 * (q >> 1) + acc_row(r, lane);
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(Hs[i][r + e], hi[e], lo[e]);
        *reinterpret_cast<uint2*>(&sm.hb[0][p][n]) =
            make_uint2(hi[0] | (static_cast<uint32_t>(hi[1]) << 16), hi[2] | (static_cast<uint32_t>(hi[3]) << 16));
        *reinterpret_cast<uint2*>(&sm.hb[1][p][n]) =
            make_uint2(lo[0] | (static_cast<uint32_t>(lo[1]) << 16), lo[2] | (static_cast<uint32_t>(lo[3]) << 16));
      }
    }
  };
  write_hb();

  const int64_t nchunks = (L + kQ - 1) / kQ;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    // ---- 1. delta and the prefix sums of delta A (wave 0, one token per lane)
    if (w == 0) {
      const int64_t t = t0 + lane;
      float d = 0.0f;
      if (t < L) d = softplus_f32(to_f32(dt[(b * L + t) * H + h]) + bias);
      float s = d * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(s, off, 64);
        if (lane >= off) s += o;
      }
      sm.dl[lane] = d;
      sm.cs[lane] = s;
    }
    // ---- loads of this chunk's x and B rows (8 channels or states per vector)
    uint4 xv[2], bv[N / 32];
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // x: 64 tokens x 8 vectors of 8 channels
      const int t = tid & 63, pg = (tid >> 6) + 4 * i;
      xv[i] = (t0 + t < L) ? *reinterpret_cast<const uint4*>(xb + (t0 + t) * xrow + 8 * pg) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < N / 32; ++i) {  // B: 64 tokens x N/8 vectors
      const int t = tid & 63, ng = (tid >> 6) + 4 * i;
      bv[i] = (t0 + t < L) ? *reinterpret_cast<const uint4*>(Bb + (t0 + t) * brow + 8 * ng) : make_uint4(0, 0, 0, 0);
    }
    // G and C H^T operands: C rows t = 32 ti + lane % 32 (also the A operand of C H^T),
    // B rows s = 32 tj + lane % 32, n = 16 k + 8 (lane / 32) + e
    bf16x8 ca[N / 16], ba[N / 16];
    {
      const int tc = 32 * ti + (lane & 31), ts = 32 * tj + (lane & 31), nh = 8 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < N / 16; ++k) {
        ca[k] = (t0 + tc < L) ? ld_bf16x8(Cb + (t0 + tc) * brow + 16 * k + nh) : zero_bf16x8();
        ba[k] = (t0 + ts < L) ? ld_bf16x8(Bb + (t0 + ts) * brow + 16 * k + nh) : zero_bf16x8();
      }
    }
    __syncthreads();  // delta, cs visible
    const float cs_end = sm.cs[kQ - 1];
    // ---- 2. transposed x, x o w and B into LDS
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = tid & 63, pg = (tid >> 6) + 4 * i;
      const float wt = fast_exp2((cs_end - sm.cs[t]) * kLog2e) * sm.dl[t];
      const uint32_t ww[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1)));
        sm.xt[8 * pg + e][t] = bits;
        split_bf16(wt * __uint_as_float(static_cast<uint32_t>(bits) << 16), sm.xw[0][8 * pg + e][t],
                   sm.xw[1][8 * pg + e][t]);
      }
    }
#pragma unroll
    for (int i = 0; i < N / 32; ++i) {
      const int t = tid & 63, ng = (tid >> 6) + 4 * i;
      const uint32_t ww[4] = {bv[i].x, bv[i].y, bv[i].z, bv[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.bt[8 * ng + e][t] = static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1)));
    }
    // ---- 3. G tile (ti, tj) masked into M; C H^T tile (ti, tj)
    if (tj <= ti) {  // the tile above the diagonal is all masked
      f32x16 gacc = {};
#pragma unroll
      for (int k = 0; k < N / 16; ++k) gacc = mfma(ca[k], ba[k], gacc);
      const int s = 32 * tj + col;
      const float cs_s = sm.cs[s], dl_s = sm.dl[s];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * ti + acc_row(r, lane);
        const float m = s <= t ? gacc[r] * fast_exp2((sm.cs[t] - cs_s) * kLog2e) * dl_s : 0.0f;
        split_bf16(m, sm.M[0][t][s], sm.M[1][t][s]);
      }
    }
    f32x16 yoff = {};
    {
      const int p = 32 * tj + (lane & 31), nh = 8 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < N / 16; ++k) {
        yoff = mfma(ca[k], ld_bf16x8(&sm.hb[0][p][16 * k + nh]), yoff);
        yoff = mfma(ca[k], ld_bf16x8(&sm.hb[1][p][16 * k + nh]), yoff);
      }
    }
    __syncthreads();  // M, xt, xw, bt complete; every read of hb done
    // ---- 4a. y tile (ti, tj) = M X + exp(cs_t) C H^T + D x
    {
      f32x16 yacc = {};
      const int t = 32 * ti + (lane & 31), p = 32 * tj + (lane & 31), kh = 8 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < 2 * (ti + 1)) {  // M[t][s] is zero for s past the tile row's end
          const bf16x8 xk = ld_bf16x8(&sm.xt[p][16 * k + kh]);
          yacc = mfma(ld_bf16x8(&sm.M[0][t][16 * k + kh]), xk, yacc);
          yacc = mfma(ld_bf16x8(&sm.M[1][t][16 * k + kh]), xk, yacc);
        }
      }
      const int pc = 32 * tj + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 32 * ti + acc_row(r, lane);
        const float xv_tp = __uint_as_float(static_cast<uint32_t>(sm.xt[pc][tr]) << 16);
        const float v = yacc[r] + fast_exp2(sm.cs[tr] * kLog2e) * yoff[r] + Dh * xv_tp;
        if (t0 + tr < L) yb[(t0 + tr) * xrow + pc] = to_bf16_bits(v);
      }
    }
    // ---- 4b. state update: H' = exp(cs_end) H + (X o w)^T B, tiles (rows n, cols p)
    {
      const float dec = fast_exp2(cs_end * kLog2e);
      const int kh = 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int q = w + 4 * i;
        const int n = 32 * (q >> 1) + (lane & 31), p = 32 * (q & 1) + (lane & 31);
        f32x16 sacc = {};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x8 bk = ld_bf16x8(&sm.bt[n][16 * k + kh]);
          sacc = mfma(bk, ld_bf16x8(&sm.xw[0][p][16 * k + kh]), sacc);
          sacc = mfma(bk, ld_bf16x8(&sm.xw[1][p][16 * k + kh]), sacc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Hs[i][r] = __builtin_fmaf(dec, Hs[i][r], sacc[r]);
      }
    }
    write_hb();
    __syncthreads();  // LDS free for the next chunk; hb holds the new state
  }
  if (hT) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int q = w + 4 * i, p = 32 * (q & 1) + col;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int n = 32 * (q >> 1) + acc_row(r, lane);
        *reinterpret_cast<float4*>(hT + ((b * H + h) * kP + p) * N + n) =
            make_float4(Hs[i][r], Hs[i][r + 1], Hs[i][r + 2], Hs[i][r + 3]);
      }
    }
  }
}

template <int N>
hipError_t launch_ssd_n(const SsdProblem& p, hipStream_t stream) {
  hipLaunchKernelGGL((ssd_fwd_kernel<N>), dim3(static_cast<unsigned>(p.nheads), static_cast<unsigned>(p.batch)),
                     dim3(256), 0, stream, static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.dt), p.A,
                     static_cast<const uint16_t*>(p.B), static_cast<const uint16_t*>(p.C), p.D, p.dt_bias, p.h0,
                     p.hT, static_cast<uint16_t*>(p.y), p.seqlen, static_cast<int>(p.nheads),
                     static_cast<int>(p.ngroups));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd(const SsdProblem& p, hipStream_t stream) {
  switch (p.dstate) {
    case 64: return launch_ssd_n<64>(p, stream);
    case 128: return launch_ssd_n<128>(p, stream);
    default: return launch_ssd_n<256>(p, stream);
  }
}

}  // namespace ssm
