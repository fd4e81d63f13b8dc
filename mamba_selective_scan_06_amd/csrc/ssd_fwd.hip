// Matrix-state recurrences in chunked matrix form on MFMA: the Mamba-2
// state-space dual (SSD) layer (page youngju.dev "Mamba 논문 리뷰", section
// 4.1: the recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t equals the
// structured masked attention Y = (T o M) X) and its gated-linear-attention
// relatives (the linear-attention recurrence s_t = s_{t-1} + k_t^T v_t of the
// HedgeMamba review's stage 2, and the mLSTM update of the xLSTM review: the
// matrix state scaled by a forget gate plus an input-gated outer product).
//
// Per batch row b and head h, with per-token log decay a_t and input scale i_t:
//   S_t = exp(a_t) S_{t-1} + i_t x_t B_t^T      (S: P x N, fp32)
//   y_t = S_t C_t (+ D[h] x_t for SSD)
//   SSD: i_t = softplus(dt + dt_bias[h]), a_t = i_t A[h]
//   gated linear attention: a_t = log_f (0 if absent), i_t = in_gate (1 if absent);
//   optionally the feature map elu(v) + 1 on B (keys) and C (queries).
// Cut into chunks of Q = 64 tokens, cs_t the running sum of a inside the chunk
// (cs_end its last value) and H the state entering it:
//   M[t,s] = (C_t . B_s) exp(cs_t - cs_s) i_s  for s <= t, else 0;  M[t,t] += D
//   y      = M X + exp(cs_t) C H^T               (Q x P)
//   H'     = exp(cs_end) H + (X o w)^T B,  w_s = exp(cs_end - cs_s) i_s
// Every product is v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The
// operands computed in fp32 (M, x o w and the state read by C H^T) are split
// into hi + lo bf16 halves, two MFMAs each: one bf16 rounding of them costs
// about 1e-2 relative in y and 2e-2 in the state, the split about 2^-16.
// x, B and C are bf16 inputs, exact.  D enters through M's diagonal.
//
// One workgroup per (b, h) walks the chunks in order: 8 waves for N <= 128
// (two per SIMD), 4 for N = 256 (LDS).  Wave w owns the channel slice p in
// [16 (w mod 4), +16) and, with 8 waves, one half of the n range: its part of
// the state stays in registers in MFMA accumulator layout, which is also the
// operand layout C H^T needs, so the state never goes through LDS; the two
// waves of a slice exchange their halves of C H^T through LDS.  Products are
// taken transposed (y^T = X^T M^T, G^T = B C^T) so each lane's accumulator
// holds 4 consecutive channels or tokens: y leaves as 8-byte stores and M
// enters LDS as 8-byte writes.  B and C are staged in LDS with n permuted
// inside each 32-wide group so that a lane's 8 operand values for C H^T sit in
// one 16-byte read.  Global traffic uses buffer loads and stores whose
// descriptor covers the chunk's valid tokens (past L: loads read 0, stores are
// dropped), and the next chunk's x, B, C and per-token inputs are loaded
// during the current chunk (the barriers wait on LDS only).  Per chunk:
//   A. per-token prefix sums (wave 0, DPP); x^T, B^T, B, C into LDS; prefetch;
//   B. x o w into LDS; M = masked G^T tiles (12 16x16 tiles); partial C H^T;
//   C. y^T for the wave's tiles (M X from LDS), store; state update.
// Tokens past L are padded with i = 0, a = 0 and x = B = C = 0, which leaves
// the state unchanged.
//
// Time segments (when B H workgroups leave most compute units idle): segment s
// owns the chunks [s SC, (s + 1) SC).  The state recurrence over a run of
// chunks is affine in the state entering it, S_out = exp(la) S_in + S_run,
// with la the sum of the run's log decays and S_run its end state from zero.
// A state-only launch (no M, no C H^T, no y: per chunk only the scalars, B^T,
// x o w and the state update) writes S_run and la for the sub-segments of SC
// / m chunks that cover every segment but the last; it needs about a third of
// the full kernel's LDS (its VGPRs let two of its workgroups share a compute
// unit), and the planner picks m for up to three workgroups per compute unit:
// a second, shorter round balances the units better than longer sub-segments.  The full launch starts segment s from h0 and
// folds the summaries of sub-segments 0 .. s m - 1 into it in order, then runs
// the chunks as above.
#include <type_traits>

#include "buffer_io.hpp"
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // head channels (headdim)
constexpr int kPad = 8;  // bf16 padding of LDS rows (16 bytes), against bank conflicts

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ float bits_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values rounded (nearest even) to a packed bf16 pair, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// hi and lo bf16 halves of two fp32 values, packed: v ~ hi + lo to about 2^-16.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// bf16 e (0..2W-1, a compile-time constant once unrolled) of W packed words.
template <int W>
__device__ __forceinline__ uint32_t elem(const uint32_t (&v)[W], int e) {
  return (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
}

// v of the lane the DPP control names, 0 where it names none or the row is
// not in ROW_MASK.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_from(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                                 false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each 16-lane row, then each row's total carried into the rows after
// it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).  Six
// DPP adds, no LDS round trip.
__device__ __forceinline__ float wave_prefix_sum(float s) {
  s += dpp_from<0x111, 0xf>(s);
  s += dpp_from<0x112, 0xf>(s);
  s += dpp_from<0x114, 0xf>(s);
  s += dpp_from<0x118, 0xf>(s);
  s += dpp_from<0x142, 0xa>(s);
  s += dpp_from<0x143, 0xc>(s);
  return s;
}

// elu(v) + 1 on 8 packed bf16, rounded back to bf16.
__device__ __forceinline__ void feature_map(uint32_t (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
    v[i] = pack_bf16(lo > 0.0f ? lo + 1.0f : fast_exp2(lo * kLog2e), hi > 0.0f ? hi + 1.0f : fast_exp2(hi * kLog2e));
  }
}

// Eight consecutive n (n0 = 8 q) of one row into the permuted n order: inside a
// 32-wide group, position 8 g + e holds n = 4 g + (e & 3) + 16 (e >> 2).
__device__ __forceinline__ void write_perm(uint16_t* row, int n0, const uint32_t (&v)[4]) {
  const int u = n0 & 31;
  const int pp = (n0 & ~31) + 8 * ((u & 15) >> 2) + 4 * (u >> 4);
  *reinterpret_cast<uint2*>(row + pp) = make_uint2(v[0], v[1]);
  *reinterpret_cast<uint2*>(row + pp + 8) = make_uint2(v[2], v[3]);
}

// Arrays that phase C of a chunk reads and phase A of the next one writes
// (x^T, B^T, the per-token scalars) are double-buffered by chunk parity when
// the LDS allows it (N <= 128): the barrier at the end of a chunk then goes,
// and the next chunk's staging overlaps the slower waves' last products.
template <int N>
constexpr int kSsdStageBufs = N <= 128 ? 2 : 1;

template <int N, int NW>
struct alignas(16) SsdSmem {
  static constexpr int NB = kSsdStageBufs<N>;
  // Chunk-major [k / 8][row][8] arrays: the 16 lanes that read one 16-byte
  // chunk of 16 consecutive rows read 256 contiguous bytes (no bank conflict),
  // and a lane that owns a row writes its 8 values as one 16-byte store.
  uint16_t M[2][kQ / 8][kQ][8];   // masked decayed C B^T (+ D on the diagonal), hi and lo: [s/8][t][s%8]
  uint16_t xt[NB][kQ / 8][kP][8]; // x: [s/8][p][s%8]
  uint16_t xw[2][kQ / 8][kP][8];  // x o w, hi and lo: [s/8][p][s%8]
  uint16_t bt[NB][N][kQ + kPad];  // B transposed: [n][s]
  uint16_t bn[kQ][N + kPad];      // B, n permuted: [s][n]
  uint16_t cn[kQ][N + kPad];      // C, n permuted: [t][n]
  float dl[NB][kQ];               // input scale i per token (0 past L)
  float cs[NB][kQ];               // running sum of the log decay inside the chunk
  float ww[NB][kQ];               // weight of each token in the chunk's state update: exp(cs_end - cs) i
  float4 xch[NW > 4 ? NW : 1][2][64];  // halves of C H^T handed to the slice's other wave
};

// The state-only pass's part of it (same names and layouts, but for B^T:
// unpadded rows whose 16-byte chunks are swizzled, chunk c of row n stored at
// chunk c ^ ((n / 2) mod 8), so that the 16 rows one MFMA operand read spans
// still hit 64 distinct banks).  At N = 128 that is 50688 bytes.
template <int N, int NW>
struct alignas(16) SsdSmemState {
  static constexpr int NB = kSsdStageBufs<N>;
  uint16_t xw[2][kQ / 8][kP][8];
  uint16_t bt[NB][N][kQ];
  float dl[NB][kQ];
  float cs[NB][kQ];
  float ww[NB][kQ];
};

// Element (n, s) of one B^T buffer: padded rows in the full pass, swizzled
// 16-byte chunks in the state-only pass (a run of up to 8 elements starting at
// a multiple of its length stays inside one chunk).
template <bool SWZ, int W>
__device__ __forceinline__ uint16_t* bt_at(uint16_t (*b)[W], int n, int s) {
  if constexpr (SWZ) {
    static_assert(W == kQ, "swizzled rows are unpadded");
    return &b[n][(((s >> 3) ^ ((n >> 1) & 7)) << 3) | (s & 7)];
  } else {
    return &b[n][s];
  }
}

struct KArgs {
  const uint16_t* x;
  const uint16_t* dt;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* D;
  const float* dt_bias;
  const float* log_f;
  const float* in_gate;
  const float* h0;
  float* hT;
  uint16_t* y;
  float* ws_state;   // (B, R, H, P, N) end state of each state-only sub-segment, from zero
  float* ws_la;      // (B, R, H) sum of the log decays over each of them
  int64_t L;
  int64_t seg_chunks;  // chunks per segment (all of them when S = 1)
  int64_t sub_chunks;  // chunks per state-only sub-segment (seg_chunks / m)
  int H, G, S;
  int R;               // state-only sub-segments: (S - 1) m
};

// ST: the state-only pass of a time-split call (see the top of the file).
template <int N, int MODE, int NW, bool ST>
__global__ __launch_bounds__(64 * NW) void ssd_fwd_kernel(const KArgs a) {
  constexpr int NK = NW / 4;          // parts of the n range, one per wave of a channel slice
  constexpr int XT = kQ / NW;         // x tokens per staging lane (one channel each)
  constexpr int TPT = N / (8 * NW);   // tokens per staging thread for B and C (8 n each)
  constexpr int TG = kQ / TPT;        // token groups per n group
  constexpr int NMK = N / 32 / NK;    // 32-wide k steps over the wave's n part
  constexpr int NJK = N / 16 / NK;    // 16-row state tiles per wave
  static_assert(TPT >= 1 && NMK >= 1, "unsupported state size for this wave count");
  __shared__ std::conditional_t<ST, SsdSmemState<N, NW>, SsdSmem<N, NW>> sm;
  const int tid = threadIdx.x, lane = tid & 63, wi = wave_id();
  const int w = wi & 3, k = wi >> 2;  // channel slice, n part
  const int lr = lane & 15, lg = lane >> 4;
  // XCD-aware order: the hardware deals workgroups to the 8 XCDs round-robin, so
  // every 8th workgroup takes the next head.  The heads of a batch row (and time
  // segment) then run on one XCD and share its L2 for B, C and the cache lines of
  // their per-token inputs (one line holds the values of many heads).
  const int64_t nwg = static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z;
  int64_t lin = blockIdx.x + gridDim.x * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
  if (nwg % 8 == 0) lin = (lin % 8) * (nwg / 8) + lin / 8;
  const int h = static_cast<int>(lin % a.H);
  const int64_t b = (lin / a.H) % gridDim.y, seg = lin / a.H / gridDim.y, L = a.L;
  const int g = h / (a.H / a.G);
  const int64_t xrow = static_cast<int64_t>(a.H) * kP;  // elements between tokens in x / y
  const int64_t brow = static_cast<int64_t>(a.G) * N;   // elements between tokens in B / C
  const uint16_t* xb = a.x + (b * L * a.H + h) * kP;
  uint16_t* yb = a.y + (b * L * a.H + h) * kP;
  const uint16_t* Bb = a.B + (b * L * a.G + g) * N;
  const uint16_t* Cb = a.C + (b * L * a.G + g) * N;
  float Ah = 0.0f, bias = 0.0f, Dh = 0.0f;
  if constexpr (MODE == 0) {
    Ah = a.A[h];
    bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    Dh = a.D ? a.D[h] : 0.0f;
  }
  // staging roles: x as the lane's channel over the XT tokens [XT wi, XT wi + XT);
  // B and C as TPT tokens x 8 n
  const int btq = tid % TG, bng = tid / TG;
  // buffer descriptor over the rows [t0, min(t0 + 64, L)) of a (tokens x row) tensor;
  // empty (every access out of range) past the end or for an absent input
  auto rows_buf = [&](const void* base, int64_t t0, int64_t row_bytes, int64_t used_bytes, bool present = true) {
    const int64_t rows = L - t0 < kQ ? L - t0 : kQ;
    const int64_t bytes = rows > 0 && present ? (rows - 1) * row_bytes + used_bytes : 0;
    return make_buf(present ? base : a.x, static_cast<uint32_t>(bytes));
  };

  // the wave's state part: Hs[j][r] = S[p = 16 w + lr][n = 16 (k NJK + j) + 4 lg + r]
  float Hs[NJK][4];
  const int64_t spart = (16 * w + lr) * N + 16 * k * NJK + 4 * lg;  // offset inside one (P, N) state
  const int64_t sbase = (b * a.H + h) * kP * N + spart;
  // summary j of this (b, h): state at ((b R + j) H + h) P N, log decay at (b R + j) H + h
  auto summary = [&](int64_t j) { return (b * a.R + j) * a.H + h; };
#pragma unroll
  for (int j = 0; j < NJK; ++j) {
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (!ST && a.h0) v = *reinterpret_cast<const float4*>(a.h0 + sbase + 16 * j);
    Hs[j][0] = v.x, Hs[j][1] = v.y, Hs[j][2] = v.z, Hs[j][3] = v.w;
  }
  if constexpr (!ST) {  // the state entering this segment: earlier sub-segments' summaries, in order
    const int64_t runs = a.S > 1 ? seg * (a.seg_chunks / a.sub_chunks) : 0;
    for (int64_t sj = 0; sj < runs; ++sj) {
      const float dec = fast_exp2(a.ws_la[summary(sj)] * kLog2e);
      const float* src = a.ws_state + summary(sj) * kP * N + spart;
#pragma unroll
      for (int j = 0; j < NJK; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(src + 16 * j);
        Hs[j][0] = __builtin_fmaf(dec, Hs[j][0], v.x), Hs[j][1] = __builtin_fmaf(dec, Hs[j][1], v.y);
        Hs[j][2] = __builtin_fmaf(dec, Hs[j][2], v.z), Hs[j][3] = __builtin_fmaf(dec, Hs[j][3], v.w);
      }
    }
  }
  float la_total = 0.0f;  // state-only pass: the segment's summed log decay

  // raw data of the next chunk, loaded one chunk ahead
  uint32_t xr[XT], br[TPT][4], cr[TPT][4];
  uint32_t traw = 0, tlf = 0, tig = 0;  // the lane's per-token inputs (raw bits): dt, or log_f and in_gate
  auto load_x = [&](int64_t t0) {  // 16-bit loads: a wave instruction reads one 128-byte token row
    const auto r = rows_buf(xb + t0 * xrow, t0, xrow * 2, kP * 2);
#pragma unroll
    for (int j = 0; j < XT; ++j)
      xr[j] = __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<uint32_t>((XT * wi + j) * xrow * 2 + lane * 2), 0, 0);
  };
  auto load_bc = [&](int64_t t0) {
    const auto rb = rows_buf(Bb + t0 * brow, t0, brow * 2, N * 2);
    const auto rc = rows_buf(Cb + t0 * brow, t0, brow * 2, N * 2);
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const uint32_t off = static_cast<uint32_t>((TPT * btq + j) * brow * 2 + 16 * bng);
      const u32x4 vb = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
      br[j][0] = vb.x, br[j][1] = vb.y, br[j][2] = vb.z, br[j][3] = vb.w;
      if constexpr (!ST) {  // the state-only pass reads no C
        const u32x4 vc = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
        cr[j][0] = vc.x, cr[j][1] = vc.y, cr[j][2] = vc.z, cr[j][3] = vc.w;
      }
    }
  };
  auto load_tok = [&](int64_t t0) {  // wave 0 only: it turns them into delta and the prefix sums
    if (wi != 0) return;
    const int64_t i0 = (b * L + t0) * a.H + h;
    const uint32_t off = static_cast<uint32_t>(lane * a.H);
    if constexpr (MODE == 0) {
      traw = __builtin_amdgcn_raw_buffer_load_b16(rows_buf(a.dt + i0, t0, a.H * 2, 2), off * 2, 0, 0);
    } else {
      tlf = __builtin_amdgcn_raw_buffer_load_b32(rows_buf(a.log_f + i0, t0, a.H * 4, 4, a.log_f), off * 4, 0, 0);
      tig = __builtin_amdgcn_raw_buffer_load_b32(rows_buf(a.in_gate + i0, t0, a.H * 4, 4, a.in_gate), off * 4, 0, 0);
    }
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  const int64_t run = ST ? a.sub_chunks : a.seg_chunks;  // chunks this workgroup walks
  const int64_t c_begin = seg * run;
  const int64_t c_end = c_begin + run < nchunks ? c_begin + run : nchunks;
  load_bc(c_begin * kQ);
  load_tok(c_begin * kQ);
  load_x(c_begin * kQ);
  // wait for the first chunk here, so that the wait at the top of the loop is set
  // by the loop alone: only the y stores issued after the prefetch are still in
  // flight there, and the wait lets them run (vmcnt counts stores too)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * kQ;
    const int cb = kSsdStageBufs<N> == 2 ? static_cast<int>(c & 1) : 0;  // staging buffer of this chunk
    // ---- A. per-token scalars (wave 0, one token per lane); x^T, B^T, B, C into LDS
    if (wi == 0) {
      const bool valid = t0 + lane < L;
      float d, la;
      if constexpr (MODE == 0) {
        d = valid ? softplus_f32(bits_f32(traw) + bias) : 0.0f;
        la = d * Ah;
      } else {
        d = valid ? (a.in_gate ? __uint_as_float(tig) : 1.0f) : 0.0f;
        la = valid ? __uint_as_float(tlf) : 0.0f;
      }
      const float s = wave_prefix_sum(la);
      sm.dl[cb][lane] = d;
      sm.cs[cb][lane] = s;
      const float s_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), kQ - 1));
      sm.ww[cb][lane] = fast_exp2((s_end - s) * kLog2e) * d;
    }
    if constexpr (!ST) {
#pragma unroll
      for (int q = 0; q < XT / 8; ++q)
        *reinterpret_cast<uint4*>(&sm.xt[cb][XT / 8 * wi + q][lane][0]) =
            make_uint4(xr[8 * q] | (xr[8 * q + 1] << 16), xr[8 * q + 2] | (xr[8 * q + 3] << 16),
                       xr[8 * q + 4] | (xr[8 * q + 5] << 16), xr[8 * q + 6] | (xr[8 * q + 7] << 16));
    }
    if constexpr (MODE == 2) {
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        feature_map(br[j]);
        if constexpr (!ST) feature_map(cr[j]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = bt_at<ST>(sm.bt[cb], 8 * bng + e, TPT * btq);
      if constexpr (TPT == 1) {
        *dst = static_cast<uint16_t>(elem(br[0], e));
      } else {
        uint32_t q[TPT / 2];
#pragma unroll
        for (int j = 0; j < TPT / 2; ++j) q[j] = elem(br[2 * j], e) | (elem(br[2 * j + 1], e) << 16);
        if constexpr (TPT == 2) *reinterpret_cast<uint32_t*>(dst) = q[0];
        if constexpr (TPT == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(q[0], q[1]);
        if constexpr (TPT == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
    if constexpr (!ST) {
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        write_perm(sm.bn[TPT * btq + j], 8 * bng, br[j]);
        write_perm(sm.cn[TPT * btq + j], 8 * bng, cr[j]);
      }
    }
    load_bc(t0 + kQ);  // past the last chunk these read nothing
    load_tok(t0 + kQ);
    __syncthreads();  // dl, cs, ww, xt, bt, bn, cn complete

    // ---- B. x o w; masked G^T tiles into M; the wave's part of C H^T
    const float cs_end = sm.cs[cb][kQ - 1];
#pragma unroll
    for (int q = 0; q < XT / 8; ++q) {  // x o w for the lane's channel and 8 tokens
      const int c8 = XT / 8 * wi + q;
      const float4 w0 = *reinterpret_cast<const float4*>(&sm.ww[cb][8 * c8]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sm.ww[cb][8 * c8 + 4]);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        split2(wv[e] * bits_f32(xr[8 * q + e]), wv[e + 1] * bits_f32(xr[8 * q + e + 1]), hi[e / 2], lo[e / 2]);
      *reinterpret_cast<uint4*>(&sm.xw[0][c8][lane][0]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&sm.xw[1][c8][lane][0]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    load_x(t0 + kQ);
    f32x4 yo[4] = {};  // this wave's part of C H^T, tile by tile
    if constexpr (!ST) {
#pragma unroll
      for (int tk = wi; tk < 12; tk += NW) {
        // the 12 16x16 tiles of M that y reads: tk < 10 enumerates (t tile, s tile)
        // on or below the diagonal row by row; 10 and 11 are the two above it that
        // a 32-token k step of y also covers, (0, 1) and (2, 3), all zero
        int ti, si;
        if (tk < 10) {
          ti = (tk >= 1) + (tk >= 3) + (tk >= 6);
          si = tk - ti * (ti + 1) / 2;
        } else {
          ti = tk == 10 ? 0 : 2;
          si = ti + 1;
        }
        const int t = 16 * ti + lr, s0 = 16 * si + 4 * lg;
        uint2 hw = make_uint2(0, 0), lw = make_uint2(0, 0);
        if (tk < 10) {
          f32x4 acc = {};
#pragma unroll
          for (int m = 0; m < N / 32; ++m)
            acc = mfma(lds8(&sm.bn[16 * si + lr][32 * m + 8 * lg]), lds8(&sm.cn[t][32 * m + 8 * lg]), acc);
          const float cst = sm.cs[cb][t];
          const float4 css = *reinterpret_cast<const float4*>(&sm.cs[cb][s0]);
          const float4 dls = *reinterpret_cast<const float4*>(&sm.dl[cb][s0]);
          const float csv[4] = {css.x, css.y, css.z, css.w}, dlv[4] = {dls.x, dls.y, dls.z, dls.w};
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = s0 + r;
            v[r] = acc[r] * fast_exp2((cst - csv[r]) * kLog2e) * dlv[r];
            v[r] = s <= t ? v[r] : 0.0f;
            if constexpr (MODE == 0) v[r] += s == t ? Dh : 0.0f;
          }
          split2(v[0], v[1], hw.x, lw.x);
          split2(v[2], v[3], hw.y, lw.y);
        }
        *reinterpret_cast<uint2*>(&sm.M[0][s0 / 8][t][s0 % 8]) = hw;
        *reinterpret_cast<uint2*>(&sm.M[1][s0 / 8][t][s0 % 8]) = lw;
      }
#pragma unroll
      for (int mm = 0; mm < NMK; ++mm) {
        const int m = k * NMK + mm;
        uint32_t hv[4], lv[4];
        split2(Hs[2 * mm][0], Hs[2 * mm][1], hv[0], lv[0]);
        split2(Hs[2 * mm][2], Hs[2 * mm][3], hv[1], lv[1]);
        split2(Hs[2 * mm + 1][0], Hs[2 * mm + 1][1], hv[2], lv[2]);
        split2(Hs[2 * mm + 1][2], Hs[2 * mm + 1][3], hv[3], lv[3]);
        const bf16x8 hh = __builtin_bit_cast(bf16x8, make_uint4(hv[0], hv[1], hv[2], hv[3]));
        const bf16x8 hl = __builtin_bit_cast(bf16x8, make_uint4(lv[0], lv[1], lv[2], lv[3]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 cb = lds8(&sm.cn[16 * i + lr][32 * m + 8 * lg]);
          yo[i] = mfma(hh, cb, yo[i]);
          yo[i] = mfma(hl, cb, yo[i]);
        }
      }
      if constexpr (NK == 2) {  // hand the other wave of the slice its two tiles
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4 v = k ? yo[u] : yo[2 + u];
          sm.xch[w + 4 * (1 - k)][u][lane] = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    __syncthreads();  // M, x o w and the exchanged halves complete

    // ---- C. y^T for the wave's tiles; the state update
    if constexpr (!ST) {
      const auto ybuf = rows_buf(yb + t0 * xrow, t0, xrow * 2, kP * 2);
      // y tile i (16 tokens) of the slice; KS 32-token k steps cover s <= t
      auto y_tile = [&](const int i, const f32x4& yt, auto ks, u32x2& out) {
        constexpr int KS = decltype(ks)::value;
        f32x4 acc = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8 xa = lds8(&sm.xt[cb][4 * kk + lg][16 * w + lr][0]);
          acc = mfma(xa, lds8(&sm.M[0][4 * kk + lg][16 * i + lr][0]), acc);
          acc = mfma(xa, lds8(&sm.M[1][4 * kk + lg][16 * i + lr][0]), acc);
        }
        const int t = 16 * i + lr;
        const float e = fast_exp2(sm.cs[cb][t] * kLog2e);
        out = (u32x2){pack_bf16(__builtin_fmaf(e, yt[0], acc[0]), __builtin_fmaf(e, yt[1], acc[1])),
                      pack_bf16(__builtin_fmaf(e, yt[2], acc[2]), __builtin_fmaf(e, yt[3], acc[3]))};
      };
      // the stores stay outside the branches so the wait on the prefetch at the top
      // of the loop counts them exactly
      auto y_store = [&](const int i, const u32x2& out) {
        __builtin_amdgcn_raw_buffer_store_b64(out, ybuf, static_cast<uint32_t>((16 * i + lr) * xrow * 2 + (16 * w + 4 * lg) * 2),
                                              0, 0);
      };
      using One = std::integral_constant<int, 1>;
      using Two = std::integral_constant<int, 2>;
      if constexpr (NK == 2) {  // tiles 2k and 2k + 1
        f32x4 yt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float4 o = sm.xch[wi][u][lane];
          yt[u] = k ? yo[2 + u] : yo[u];
          yt[u][0] += o.x, yt[u][1] += o.y, yt[u][2] += o.z, yt[u][3] += o.w;
        }
        u32x2 out[2];
        if (k == 0) {
          y_tile(0, yt[0], One{}, out[0]);
          y_tile(1, yt[1], One{}, out[1]);
        } else {
          y_tile(2, yt[0], Two{}, out[0]);
          y_tile(3, yt[1], Two{}, out[1]);
        }
        y_store(2 * k, out[0]);
        y_store(2 * k + 1, out[1]);
      } else {
        u32x2 out[4];
        y_tile(0, yo[0], One{}, out[0]);
        y_tile(1, yo[1], One{}, out[1]);
        y_tile(2, yo[2], Two{}, out[2]);
        y_tile(3, yo[3], Two{}, out[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) y_store(i, out[i]);
      }
    }
    {
      if constexpr (ST) la_total += cs_end;
      const float dec = fast_exp2(cs_end * kLog2e);
      bf16x8 xh[2], xl[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        xh[kk] = lds8(&sm.xw[0][4 * kk + lg][16 * w + lr][0]);
        xl[kk] = lds8(&sm.xw[1][4 * kk + lg][16 * w + lr][0]);
      }
#pragma unroll
      for (int j = 0; j < NJK; ++j) {
        f32x4 sacc = {};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 bb = lds8(bt_at<ST>(sm.bt[cb], 16 * (k * NJK + j) + lr, 32 * kk + 8 * lg));
          sacc = mfma(bb, xh[kk], sacc);
          sacc = mfma(bb, xl[kk], sacc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Hs[j][r] = __builtin_fmaf(dec, Hs[j][r], sacc[r]);
      }
    }
    // single staging buffers: LDS free for the next chunk.  Double buffers: the
    // next chunk's phase A writes the other x^T, B^T and scalars, and M, x o w
    // and the exchange are written only after its first barrier, which every
    // wave reaches after finishing this chunk.
    if constexpr (kSsdStageBufs<N> == 1) __syncthreads();
  }
  if constexpr (ST) {
    float* dst = a.ws_state + summary(seg) * kP * N + spart;
#pragma unroll
    for (int j = 0; j < NJK; ++j)
      *reinterpret_cast<float4*>(dst + 16 * j) = make_float4(Hs[j][0], Hs[j][1], Hs[j][2], Hs[j][3]);
    if (tid == 0) a.ws_la[summary(seg)] = la_total;
  } else if (a.hT && seg == a.S - 1) {
#pragma unroll
    for (int j = 0; j < NJK; ++j)
      *reinterpret_cast<float4*>(a.hT + sbase + 16 * j) = make_float4(Hs[j][0], Hs[j][1], Hs[j][2], Hs[j][3]);
  }
}

template <int N, int MODE>
hipError_t launch_ssd_n(const SsdProblem& p, hipStream_t stream) {
  constexpr int NW = N <= 128 ? 8 : 4;
  KArgs k;
  k.x = static_cast<const uint16_t*>(p.x);
  k.dt = static_cast<const uint16_t*>(p.dt);
  k.A = p.A;
  k.B = static_cast<const uint16_t*>(p.B);
  k.C = static_cast<const uint16_t*>(p.C);
  k.D = p.D;
  k.dt_bias = p.dt_bias;
  k.log_f = p.log_f;
  k.in_gate = p.in_gate;
  k.h0 = p.h0;
  k.hT = p.hT;
  k.y = static_cast<uint16_t*>(p.y);
  k.ws_state = p.ws_state;
  k.ws_la = p.ws_la;
  k.L = p.seqlen;
  k.seg_chunks = p.splits > 1 ? p.seg_chunks : (p.seqlen + kQ - 1) / kQ;
  k.sub_chunks = p.splits > 1 ? p.sub_chunks : k.seg_chunks;
  k.H = static_cast<int>(p.nheads);
  k.G = static_cast<int>(p.ngroups);
  k.S = p.splits > 1 ? p.splits : 1;
  k.R = p.splits > 1 ? static_cast<int>((p.splits - 1) * (p.seg_chunks / p.sub_chunks)) : 0;
  const unsigned gh = static_cast<unsigned>(p.nheads), gb = static_cast<unsigned>(p.batch);
  if (k.S > 1) {  // summaries of the sub-segments before the last segment, then the full pass
    hipLaunchKernelGGL((ssd_fwd_kernel<N, MODE, NW, true>), dim3(gh, gb, static_cast<unsigned>(k.R)), dim3(64 * NW),
                       0, stream, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ssd_fwd_kernel<N, MODE, NW, false>), dim3(gh, gb, static_cast<unsigned>(k.S)), dim3(64 * NW), 0,
                     stream, k);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_ssd_m(const SsdProblem& p, hipStream_t stream) {
  switch (p.dstate) {
    case 64: return launch_ssd_n<64, MODE>(p, stream);
    case 128: return launch_ssd_n<128, MODE>(p, stream);
    default: return launch_ssd_n<256, MODE>(p, stream);
  }
}

// The feature map once per call: 8 bf16 per thread, the same arithmetic and
// rounding as feature_map() in the kernel's staging.
__global__ __launch_bounds__(256) void gla_feature_map_kernel(const uint4* __restrict__ k, const uint4* __restrict__ q,
                                                               uint4* __restrict__ pk, uint4* __restrict__ pq,
                                                               int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 a = k[i], b = q[i];
  uint32_t va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {b.x, b.y, b.z, b.w};
  feature_map(va);
  feature_map(vb);
  pk[i] = make_uint4(va[0], va[1], va[2], va[3]);
  pq[i] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
}

}  // namespace

hipError_t launch_gla_feature_map(const void* k, const void* q, void* pk, void* pq, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(gla_feature_map_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(q), static_cast<uint4*>(pk),
                     static_cast<uint4*>(pq), n8);
  return hipGetLastError();
}

hipError_t launch_ssd(const SsdProblem& p, hipStream_t stream) {
  switch (p.mode) {
    case 1: return launch_ssd_m<1>(p, stream);
    case 2: return launch_ssd_m<2>(p, stream);
    default: return launch_ssd_m<0>(p, stream);
  }
}

}  // namespace ssm
