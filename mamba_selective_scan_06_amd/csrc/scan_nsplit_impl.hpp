// NSPLIT family: the main forward scan on gfx950.
//
// Work decomposition.  A workgroup is 4 waves (256 lanes) and owns 64
// consecutive channels d of one batch row b, over one time segment.  Lane l of
// every wave stands for channel d0 + l; wave w holds the K = N/4 states
// n = wK .. wK+K-1 of that channel in fp32 registers.  So the 16 states of a
// channel at N = 16 live in 4 lanes of 4 different waves, and one workgroup
// keeps 64 x N independent recurrence chains on chip for the whole segment.
// This gives 4 waves per 64 channels (one per SIMD) instead of one, which the
// channel count of a Mamba layer needs to fill 1024 SIMDs without splitting
// time.
//
// Per token and channel (page youngju.dev "Mamba 논문 리뷰"):
//   delta = softplus(raw + bias)                       section 3.1
//   Abar_n = exp(delta A[d,n])                         section 2.2
//   h_n  <- Abar_n h_n + (delta x) B_t[n]              sections 2.2, 3.3 (Euler input term)
//   y     = sum_n C_t[n] h_n + D[d] x, y *= SiLU(z)    sections 2.2, 3.4
//
// Time is walked in tiles of 16 tokens with three phases and two barriers:
//   O  "owner" phase: token t of the tile is owned by wave (t mod 4), which
//      does that token's per-(t, d) scalar work exactly once for the 64
//      channels: widening, softplus, u = delta x, the decay terms, D x and
//      SiLU(z).  It publishes (decay terms, u) to LDS.
//   S  scan phase: every wave advances its K states through the 16 tokens,
//      reading the shared per-token terms from LDS and B_t, C_t through the
//      scalar unit (wave-uniform s_load, SGPR operands), and writes its
//      partial readout sum_{n in wave} C_t[n] h_n to LDS.
//   Y  the owner wave adds the 4 partial sums, D x, applies the gate, rounds
//      once and stores y_t for its tokens.
// Inputs of the owner phase are prefetched NS_PF tiles ahead into a register
// ring (one wave per SIMD cannot hide HBM latency by switching waves).
//
// Structured decays.  When A[d, n] == (n+1) A[d, 0] holds exactly for every
// channel of the block (the S4D-real diagonal of section 3.4, A = -(1..N)),
// Abar_n = r^(n+1) with r = exp(delta A[d,0]): the owner computes r and the
// start r^(wK+1) of each wave's run, and a wave derives its other K-1 decays
// by multiplying by r, one multiply per state instead of one exp.  Otherwise
// every decay is its own exp of delta A[d, n].
//
// Time splitting (for problems with too few channels to fill the GPU): the
// sequence is cut into segments.  A first launch (STATE_ONLY) runs every
// segment but the last from a zero state and stores its end state H and the
// sum of its softplus(delta).  The second launch starts segment s from
//   h = h0, then h <- exp(A_n sum_j delta) h + H_j for j = 0..s-1
// (the associative combine (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) of the
// affine steps, with the product of a segment's decays written as one exp of
// A_n times its summed step size), and runs the full scan from there.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace nsplit_detail {

constexpr int NS_T = kNsplitTile;  // tokens per tile
constexpr int NS_OWN = NS_T / 4;   // tokens owned by each wave per tile
constexpr int NS_PF = 4;           // prefetch depth in tiles (register ring slots)

// Raw (undecoded) form of one wave's K-element slice of a B_t or C_t row:
// fp32 values, bf16 pairs packed in 32-bit words, or a single bf16.
template <typename S, int K>
struct RowSlice {
  static constexpr bool kF32 = sizeof(S) == 4;
  static constexpr int kWords = kF32 ? K : (K == 1 ? 1 : K / 2);
  uint32_t v[kWords];

  // p: wave-uniform pointer to the first element (the loads become s_load).
  __device__ __forceinline__ void load(const S* p) {
    if constexpr (kF32) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int k = 0; k < K; ++k) v[k] = q[k];
    } else if constexpr (K == 1) {
      v[0] = static_cast<uint32_t>(p[0]);
    } else {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);  // even element offset
#pragma unroll
      for (int k = 0; k < kWords; ++k) v[k] = q[k];
    }
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (kF32) return __uint_as_float(v[k]);
    else if constexpr (K == 1) return __uint_as_float(v[0] << 16);
    else return (k & 1) ? __uint_as_float(v[k >> 1] & 0xffff0000u) : __uint_as_float(v[k >> 1] << 16);
  }
};

template <typename S>
struct Ring {
  S xr[NS_PF][NS_OWN];
  S dr[NS_PF][NS_OWN];
  S zr[NS_PF][NS_OWN];
};

struct Smem {
  float E[NS_T][4][64];  // decay terms: chain start per wave (structured) or delta in slot 0
  float U[NS_T][64];     // u = delta * x
  float P[NS_T][4][64];  // partial readouts per wave
  float sd[4][64];       // per-wave partial sums of delta (STATE_ONLY)
};

// Everything a segment run needs besides the tensors.  Token indices and the
// element offsets inside one batch row are 32-bit (the planner only sends
// problems with L*D and L*N below 2^31 here), so uniform index arithmetic and
// bounds tests stay on the scalar unit.
struct SegCtx {
  int32_t t_begin, t_end;  // token range of the segment, uniform
  uint32_t D, d0;          // channels, first channel of the block, uniform
  int w, lane;
  uint32_t lo;             // lane offset used for loads (clamped for inactive lanes)
  bool active;
  float A2_0, bias_d, D_d;
};

// Tokens per B/C pipeline stage (4 stages per tile; two stages live at once).
constexpr int NS_Q = 4;

template <typename S, int K, bool STATE_ONLY, bool STRUCT, bool GATE>
__device__ __forceinline__ void run_segment(Smem& sm, const S* __restrict__ xb, const S* __restrict__ db,
                                            const S* __restrict__ Bb, const S* __restrict__ Cb,
                                            const S* __restrict__ zb, S* __restrict__ yb, float (&h)[K],
                                            const float (&A2)[K], const SegCtx& c, float& dsum) {
  constexpr int N = 4 * K;
  constexpr bool kLoadZ = !STATE_ONLY && GATE;
  using Slice = RowSlice<S, K>;
  Ring<S> rg;
  const int32_t t_last = c.t_end - 1;

  // Owner-phase loads of the tile at t0 into ring slot `slot`.  Tokens past the
  // segment end are clamped to its last token: the loads stay in bounds and
  // unconditional (so the compiler can wait on exactly the older ones), and the
  // values are never used.
  auto load_tile = [&](auto slot_c, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i) {
      int32_t t = t0 + 4 * i + c.w;
      t = t < t_last ? t : t_last;
      const uint32_t row = static_cast<uint32_t>(t) * c.D + c.d0;  // wave-uniform
      rg.xr[slot][i] = xb[row + c.lo];
      rg.dr[slot][i] = db[row + c.lo];
      if constexpr (kLoadZ) rg.zr[slot][i] = zb[row + c.lo];
    }
  };

  // B_t, C_t slices of this wave for tokens t0 .. t0+NS_Q-1 (clamped).
  auto load_stage = [&](int32_t t0, Slice (&Bs)[NS_Q], Slice (&Cs)[NS_Q]) {
#pragma unroll
    for (int j = 0; j < NS_Q; ++j) {
      int32_t t = t0 + j;
      t = t < t_last ? t : t_last;
      const uint32_t off = static_cast<uint32_t>(t) * N + c.w * K;
      Bs[j].load(Bb + off);
      if constexpr (!STATE_ONLY) Cs[j].load(Cb + off);
    }
  };

  // Stage 0 of the current tile, loaded one stage ahead of use.
  Slice Bcur[NS_Q], Ccur[NS_Q];
  load_stage(c.t_begin, Bcur, Ccur);

  // One tile of 16 tokens.  Tokens past the segment end (last tile only) are
  // given the neutral step (decay 1, input 0): the states pass through them
  // unchanged, so the scan phase needs no bounds tests; their y is not stored.
  auto process_tile = [&](auto slot_c, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
    float keep_dx[NS_OWN], keep_g[NS_OWN];
    // ---- O: per-token scalar work, once per (t, d), by the owner wave -----
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i) {
      const int j = 4 * i + c.w;
      keep_dx[i] = 0.0f;
      keep_g[i] = 0.0f;
      if (t0 + j < c.t_end) {  // wave-uniform
        const float xv = to_f32(rg.xr[slot][i]);
        const float dt = softplus_f32(to_f32(rg.dr[slot][i]) + c.bias_d);
        if constexpr (STATE_ONLY) {
          dsum += dt;
        } else {
          keep_dx[i] = c.D_d * xv;
          if constexpr (GATE) keep_g[i] = silu_f32(to_f32(rg.zr[slot][i]));
        }
        if constexpr (STRUCT) {
          const float r = fast_exp2(dt * c.A2_0);
          float rk = r;  // r^K by squaring (K is a power of two)
#pragma unroll
          for (int q = 1; q < K; q <<= 1) rk *= rk;
          float e = r;
          sm.E[j][0][c.lane] = e;
          e *= rk; sm.E[j][1][c.lane] = e;
          e *= rk; sm.E[j][2][c.lane] = e;
          e *= rk; sm.E[j][3][c.lane] = e;
        } else {
          sm.E[j][0][c.lane] = dt;
        }
        sm.U[j][c.lane] = dt * xv;
      } else {
        if constexpr (STRUCT) {
          sm.E[j][0][c.lane] = 1.0f;
          sm.E[j][1][c.lane] = 1.0f;
          sm.E[j][2][c.lane] = 1.0f;
          sm.E[j][3][c.lane] = 1.0f;
        } else {
          sm.E[j][0][c.lane] = 0.0f;  // exp(0 * A) = 1
        }
        sm.U[j][c.lane] = 0.0f;
      }
    }
    __syncthreads();
    // ---- S: every wave advances its K states through the tile -------------
#pragma unroll
    for (int q = 0; q < NS_T / NS_Q; ++q) {
      // next stage: the rest of this tile, then stage 0 of the next tile
      Slice Bnext[NS_Q], Cnext[NS_Q];
      load_stage(t0 + (q + 1) * NS_Q, Bnext, Cnext);
#pragma unroll
      for (int jj = 0; jj < NS_Q; ++jj) {
        const int j = q * NS_Q + jj;
        const float u = sm.U[j][c.lane];
        float acc = 0.0f;
        if constexpr (STRUCT) {
          float a = sm.E[j][c.w][c.lane];
          const float r = sm.E[j][0][c.lane];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            if (k > 0) a *= r;
            h[k] = __builtin_fmaf(a, h[k], u * Bcur[jj].get(k));
            if constexpr (!STATE_ONLY) acc = __builtin_fmaf(Ccur[jj].get(k), h[k], acc);
          }
        } else {
          const float dt = sm.E[j][0][c.lane];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const float a = fast_exp2(dt * A2[k]);
            h[k] = __builtin_fmaf(a, h[k], u * Bcur[jj].get(k));
            if constexpr (!STATE_ONLY) acc = __builtin_fmaf(Ccur[jj].get(k), h[k], acc);
          }
        }
        if constexpr (!STATE_ONLY) sm.P[j][c.w][c.lane] = acc;
      }
#pragma unroll
      for (int jj = 0; jj < NS_Q; ++jj) {
        Bcur[jj] = Bnext[jj];
        Ccur[jj] = Cnext[jj];
      }
    }
    __syncthreads();
    // ---- Y: the owner wave finishes and stores its tokens ------------------
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int i = 0; i < NS_OWN; ++i) {
        const int j = 4 * i + c.w;
        const int32_t t = t0 + j;
        if (t < c.t_end) {  // wave-uniform
          float yv = ((sm.P[j][0][c.lane] + sm.P[j][1][c.lane]) + sm.P[j][2][c.lane]) + sm.P[j][3][c.lane];
          yv += keep_dx[i];
          if constexpr (GATE) yv *= keep_g[i];
          if (c.active) store_elem(yb + (static_cast<uint32_t>(t) * c.D + c.d0 + c.lane), yv);
        }
      }
    }
  };

  // Prime the ring, then consume tile k from slot k % NS_PF and refill it with
  // tile k + NS_PF.  Slots are compile-time constants (unrolled by NS_PF).
  static_assert(NS_PF == 4, "the ring code below is written for 4 slots");
  load_tile(std::integral_constant<int, 0>{}, c.t_begin + 0 * NS_T);
  load_tile(std::integral_constant<int, 1>{}, c.t_begin + 1 * NS_T);
  load_tile(std::integral_constant<int, 2>{}, c.t_begin + 2 * NS_T);
  load_tile(std::integral_constant<int, 3>{}, c.t_begin + 3 * NS_T);
  for (int32_t tl = c.t_begin; tl < c.t_end; tl += NS_PF * NS_T) {
    auto step = [&](auto slot_c) {
      const int32_t t0 = tl + decltype(slot_c)::value * NS_T;
      if (t0 < c.t_end) {  // workgroup-uniform
        process_tile(slot_c, t0);
        load_tile(slot_c, t0 + NS_PF * NS_T);
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
  }
}

template <typename S, int K, bool STATE_ONLY, bool GATE>
__global__ __launch_bounds__(256, 1) void scan_nsplit_kernel(
    const S* __restrict__ x, const S* __restrict__ dl, const float* __restrict__ A,
    const S* __restrict__ Bm, const S* __restrict__ Cm, const float* __restrict__ Dsk,
    const S* __restrict__ z, const float* __restrict__ bias, const float* h0, float* hT,
    S* __restrict__ y, float* __restrict__ ws_state, float* __restrict__ ws_dsum,
    int32_t L, int32_t D, int32_t seg_len, int splits, int flags) {
  constexpr int N = 4 * K;
  __shared__ Smem sm;
  SegCtx c;
  c.w = wave_id();
  c.lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y;
  const int s = blockIdx.z;
  c.D = static_cast<uint32_t>(D);
  c.d0 = blockIdx.x * 64u;
  c.active = c.d0 + c.lane < c.D;
  c.lo = c.active ? c.lane : c.D - 1 - c.d0;
  const int64_t d = c.d0 + c.lo;  // inactive lanes shadow channel D-1 and write nothing
  c.t_begin = s * seg_len;
  c.t_end = (c.t_begin + seg_len < L) ? c.t_begin + seg_len : L;

  float A2[K];
#pragma unroll
  for (int k = 0; k < K; ++k) A2[k] = A[d * N + c.w * K + k] * kLog2e;
  const float a0 = A[d * N];
  c.A2_0 = a0 * kLog2e;

  // Structured-decay test for the whole block: A[d, n] == (n+1) A[d, 0] exactly.
  bool ok = !(flags & kFlagGenericA);
#pragma unroll
  for (int k = 0; k < K; ++k) ok = ok && (A[d * N + c.w * K + k] == static_cast<float>(c.w * K + k + 1) * a0);
  const bool structured = __syncthreads_and(ok ? 1 : 0) != 0;

  c.bias_d = bias ? bias[d] : 0.0f;
  c.D_d = Dsk ? Dsk[d] : 0.0f;

  float h[K];
  if constexpr (STATE_ONLY) {
#pragma unroll
    for (int k = 0; k < K; ++k) h[k] = 0.0f;
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) h[k] = h0 ? h0[(b * D + d) * N + c.w * K + k] : 0.0f;
    // Carry in the summaries of the segments before this one.
    for (int j = 0; j < s; ++j) {
      const int64_t seg = b * splits + j;
      const float sdl = ws_dsum[seg * D + d];
#pragma unroll
      for (int k = 0; k < K; ++k)
        h[k] = __builtin_fmaf(fast_exp2(A2[k] * sdl), h[k], ws_state[(seg * D + d) * N + c.w * K + k]);
    }
  }

  // Base pointers of this batch row; offsets inside a row are 32-bit.
  const int64_t rowD = b * static_cast<int64_t>(L) * D, rowN = b * static_cast<int64_t>(L) * N;
  const S* xb = x + rowD;
  const S* db = dl + rowD;
  const S* zb = z ? z + rowD : x + rowD;  // never read without a gate
  const S* Bb = Bm + rowN;
  const S* Cb = Cm + rowN;
  S* yb = y + rowD;

  float dsum = 0.0f;
  if (structured)
    run_segment<S, K, STATE_ONLY, true, GATE>(sm, xb, db, Bb, Cb, zb, yb, h, A2, c, dsum);
  else
    run_segment<S, K, STATE_ONLY, false, GATE>(sm, xb, db, Bb, Cb, zb, yb, h, A2, c, dsum);

  if constexpr (STATE_ONLY) {
    const int64_t seg = b * splits + s;
    if (c.active) {
#pragma unroll
      for (int k = 0; k < K; ++k) ws_state[(seg * D + d) * N + c.w * K + k] = h[k];
    }
    sm.sd[c.w][c.lane] = dsum;
    __syncthreads();
    if (c.w == 0 && c.active)
      ws_dsum[seg * D + d] = ((sm.sd[0][c.lane] + sm.sd[1][c.lane]) + sm.sd[2][c.lane]) + sm.sd[3][c.lane];
  } else {
    if (hT && c.active && s == splits - 1) {
#pragma unroll
      for (int k = 0; k < K; ++k) hT[(b * D + d) * N + c.w * K + k] = h[k];
    }
  }
}

template <typename S, int K, bool STATE_ONLY, bool GATE>
void launch_one(const Problem& p, hipStream_t stream, unsigned nseg) {
  const unsigned nb = static_cast<unsigned>((p.dim + 63) / 64);
  hipLaunchKernelGGL((scan_nsplit_kernel<S, K, STATE_ONLY, GATE>), dim3(nb, static_cast<unsigned>(p.batch), nseg),
                     dim3(256), 0, stream, static_cast<const S*>(p.x), static_cast<const S*>(p.delta), p.A,
                     static_cast<const S*>(p.B), static_cast<const S*>(p.C), p.D, static_cast<const S*>(p.z),
                     p.delta_bias, p.h0, p.hT, static_cast<S*>(p.y), p.ws_state, p.ws_dsum,
                     static_cast<int32_t>(p.seqlen), static_cast<int32_t>(p.dim), static_cast<int32_t>(p.seg_len),
                     p.splits, p.flags);
}

template <typename S, int K>
hipError_t launch_nsplit_t(const Problem& p, hipStream_t stream) {
  if (p.splits > 1) {
    launch_one<S, K, true, false>(p, stream, static_cast<unsigned>(p.splits - 1));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.z)
    launch_one<S, K, false, true>(p, stream, static_cast<unsigned>(p.splits));
  else
    launch_one<S, K, false, false>(p, stream, static_cast<unsigned>(p.splits));
  return hipGetLastError();
}

}  // namespace nsplit_detail
}  // namespace ssm
