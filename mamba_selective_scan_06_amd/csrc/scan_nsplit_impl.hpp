// NSPLIT family: the main forward scan on gfx950.
//
// Work decomposition.  A workgroup is 8 waves (512 lanes) and owns 64
// consecutive channels d of one batch row b, over one time segment.  Lane l of
// every wave stands for channel d0 + l.  The waves are specialised, and wave w
// runs on SIMD w mod 4, so every SIMD holds one wave of each role:
//   scan waves 0..3: wave w holds the K = N/4 states n = wK .. wK+K-1 of its
//     channel in fp32 registers and advances them through every token (the 16
//     states of a channel at N = 16 live in 4 lanes of 4 waves);
//   owner waves 4..7: owner o does the per-(t, d) scalar work of the tokens
//     j = o (mod 4) of each tile for all 64 channels: loading and widening x,
//     delta and z, softplus, u = delta x, the decay terms, D x and SiLU(z).
//     It publishes (decay terms, u) in LDS and, a tile later, adds the scan
//     waves' partial readouts, D x and the gate, rounds once and stores y_t.
// One workgroup keeps 64 x N independent recurrence chains on chip for the
// whole segment, and 64 channels of a Mamba layer give 4 scan waves, one per
// SIMD, which the channel count needs to fill 1024 SIMDs without splitting time.
//
// Per token and channel (page youngju.dev "Mamba 논문 리뷰"):
//   delta = softplus(raw + bias)                       section 3.1
//   Abar_n = exp(delta A[d,n])                         section 2.2
//   h_n  <- Abar_n h_n + (delta x) B_t[n]              sections 2.2, 3.3 (Euler input term)
//   y     = sum_n C_t[n] h_n + D[d] x, y *= SiLU(z)    sections 2.2, 3.4
//
// Time is walked in tiles of 16 tokens with one barrier per tile and the LDS
// terms double-buffered: in iteration k the scan waves consume tile k (reading
// its per-token terms, writing their partial readouts sum_{n in wave} C_t[n] h_n)
// while the owners compute tile k+1's terms into the other buffer and finish
// tile k-1 from the partials left there.

// Memory.  All loads are raw buffer loads with the whole byte offset in the
// VGPR offset (the part the range check covers), through a descriptor over one
// batch row, so loads past the row end return 0 (prefetching past the end of
// the sequence is safe).  Stores of y go through a descriptor that starts a
// tile before the segment and ends with it, and a lane whose store must not
// happen gets an offset past it.  Offsets are 32-bit: for rows of 2 GiB or
// more (WIN) the descriptors instead cover windows that start a few tiles
// behind the accesses and move forward every NS_PF tiles, so offsets stay
// below 144 tokens of a row whatever its length.
// Every input a tile needs (x, delta, z of the owned tokens, and this wave's
// slices of B_t and C_t for all 16 tokens) is loaded NS_PF tiles ahead into a
// register ring; one wave per SIMD cannot hide HBM latency by switching waves,
// and every iteration issues the same memory operations, so each wait covers
// only the oldest tile.
//
// B_t and C_t are the same for all 64 channels of a wave.  A tile's slices
// are loaded so that every 16-lane row of the wave holds the same 16 words,
// and each value is consumed straight from its lane with a DPP row broadcast
// (row_newbcast) as the first operand of the multiply that uses it: no LDS
// traffic, no scalar registers, no extra instruction.  The compiler folds the
// broadcast into v_mul_f32 for the input term; for the readout's
// fused multiply-add it does not, so v_fmac_f32_dpp is written out (see
// readout_dpp below).
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

#include "buffer_io.hpp"
#include "device_common.hpp"
#include "scan_internal.hpp"

namespace ssm {
namespace nsplit_detail {

constexpr int NS_T = kNsplitTile;  // tokens per tile
constexpr int NS_OWN = NS_T / 4;   // tokens owned by each wave per tile
constexpr int NS_PF = 4;           // prefetch depth in tiles (register ring slots)

// Broadcast lane LANE of every 16-lane row to the whole row.
template <int LANE>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(LANE >= 0 && LANE < 16, "row lane");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + LANE, 0xf, 0xf, true));
}

// Readout terms with the C value broadcast from a lane of each 16-lane row:
// acc (+)= bcast_L0(c0) h0 + bcast_L1(c1) h1 + ...  The compiler does not fuse
// a DPP move into v_fmac, so these are written out, up to four terms per
// block.  A DPP source written by a VALU instruction needs two wait states
// before the read, and the compiler's hazard checks do not see inside inline
// asm.  The sources are the C words of the tile's register ring, widened by
// VALU once per row-load (every TPL tokens): the first block after a widening
// starts with s_nop 1 (NOP), the others read registers written at least one
// whole block earlier.  The build's hazard check of the generated code
// verifies this for every instantiation.
#define SSM_DPP_TERM(OP, A, C, H, L) OP " %" #A ", %" #C ", %" #H " row_newbcast:%c" #L " row_mask:0xf bank_mask:0xf\n\t"
// Each block is emitted with or without the leading s_nop 1.
#define SSM_READOUT_ASM(NOP, BODY, ...)   \
  do {                                    \
    if constexpr (NOP)                    \
      asm("s_nop 1\n\t" BODY __VA_ARGS__); \
    else                                  \
      asm(BODY __VA_ARGS__);              \
  } while (0)
template <bool FIRST, bool NOP, int L0>
__device__ __forceinline__ float readout1(float acc, float c0, float h0) {
  if constexpr (FIRST) {
    SSM_READOUT_ASM(NOP, SSM_DPP_TERM("v_mul_f32_dpp", 0, 1, 2, 3), : "=&v"(acc) : "v"(c0), "v"(h0), "n"(L0));
  } else {
    SSM_READOUT_ASM(NOP, SSM_DPP_TERM("v_fmac_f32_dpp", 0, 1, 2, 3), : "+v"(acc) : "v"(c0), "v"(h0), "n"(L0));
  }
  return acc;
}
template <bool FIRST, bool NOP, int L0, int L1>
__device__ __forceinline__ float readout2(float acc, float c0, float c1, float h0, float h1) {
  if constexpr (FIRST) {
    SSM_READOUT_ASM(NOP, SSM_DPP_TERM("v_mul_f32_dpp", 0, 1, 3, 5) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 2, 4, 6),
                    : "=&v"(acc) : "v"(c0), "v"(c1), "v"(h0), "v"(h1), "n"(L0), "n"(L1));
  } else {
    SSM_READOUT_ASM(NOP, SSM_DPP_TERM("v_fmac_f32_dpp", 0, 1, 3, 5) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 2, 4, 6),
                    : "+v"(acc) : "v"(c0), "v"(c1), "v"(h0), "v"(h1), "n"(L0), "n"(L1));
  }
  return acc;
}
template <bool FIRST, bool NOP, int L0, int L1, int L2, int L3>
__device__ __forceinline__ float readout4(float acc, float c0, float c1, float c2, float c3, float h0, float h1,
                                          float h2, float h3) {
  if constexpr (FIRST) {
    SSM_READOUT_ASM(NOP,
                    SSM_DPP_TERM("v_mul_f32_dpp", 0, 1, 5, 9) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 2, 6, 10)
                        SSM_DPP_TERM("v_fmac_f32_dpp", 0, 3, 7, 11) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 4, 8, 12),
                    : "=&v"(acc) : "v"(c0), "v"(c1), "v"(c2), "v"(c3), "v"(h0), "v"(h1), "v"(h2), "v"(h3),
                      "n"(L0), "n"(L1), "n"(L2), "n"(L3));
  } else {
    SSM_READOUT_ASM(NOP,
                    SSM_DPP_TERM("v_fmac_f32_dpp", 0, 1, 5, 9) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 2, 6, 10)
                        SSM_DPP_TERM("v_fmac_f32_dpp", 0, 3, 7, 11) SSM_DPP_TERM("v_fmac_f32_dpp", 0, 4, 8, 12),
                    : "+v"(acc) : "v"(c0), "v"(c1), "v"(c2), "v"(c3), "v"(h0), "v"(h1), "v"(h2), "v"(h3),
                      "n"(L0), "n"(L1), "n"(L2), "n"(L3));
  }
  return acc;
}
#undef SSM_READOUT_ASM
#undef SSM_DPP_TERM

// Where this wave's slice of one B_t or C_t row lives in the ring.  A row-load
// fills 16 lanes with TPL consecutive tokens of WB words each (the same in all
// four rows of the wave); a tile takes NLD = WB row-loads per tensor.
template <typename S, int K>
struct BCLayout {
  static constexpr bool kF32 = sizeof(S) == 4;
  static constexpr bool kPairs = !kF32 && K >= 2;   // bf16 pairs in 32-bit words
  static constexpr int WB = kF32 ? K : (K >= 2 ? K / 2 : 1);
  static constexpr int TPL = 16 / WB;
  static constexpr int NLD = NS_T / TPL;
  static_assert(WB <= 16 && 16 % WB == 0, "slice must fit one 16-lane row");
  // lane holding element k of token j (j inside the tile), and its row-load
  static constexpr int load_of(int j) { return j / TPL; }
  static constexpr int lane_of(int j, int k) { return (j % TPL) * WB + (kPairs ? k / 2 : (kF32 ? k : 0)); }
  static constexpr bool odd_half(int k) { return kPairs && (k & 1); }
};

struct Smem {
  float E[2][NS_T][4][64];  // decay terms: chain start per scan wave (structured) or delta in slot 0
  float U[2][NS_T][64];     // u = delta * x
  float P[2][NS_T][4][64];  // partial readouts per scan wave
};
constexpr int kSmemBytes = static_cast<int>(sizeof(Smem));

// Uniform facts of one segment run plus the lane's identity.  Token indices
// are 32-bit; byte offsets are 32-bit inside a descriptor window.
struct SegCtx {
  int32_t L;               // tokens of a batch row
  int32_t t_begin, t_end;  // token range of the segment
  int32_t ntiles;          // tiles in the segment, rounded up to a multiple of NS_PF
  uint32_t D, d0;          // channels, first channel of the block
  int w, lane;             // wave (0..7) and lane
  bool active;             // lane's channel < D
  float A2_0, bias_d, D_d;
  float A_0, invA_0;       // A[d, 0] and 1 / A[d, 0] (zero-order hold)
};

// A wave-uniform value the optimiser must treat as unknown.  The window start
// of a turn of the ring passes through it: were each load's offset from the
// window a visible constant, the compiler would hoist them all and reschedule
// the loops (grouping a tile's LDS reads and draining the prefetch ring at the
// top of every turn), which measured about 10% slower.
__device__ __forceinline__ int32_t opaque_sgpr(int32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// A loaded register of the prefetch ring, marked as used here: the wait for
// its load, and the widening that consumes it, stay at the tile that needs it
// instead of being hoisted to the top of the ring's turn (which drains every
// load in flight there).
__device__ __forceinline__ uint32_t ring_word(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Windows over rows of tok_bytes bytes per token, from token W to token end:
// the part shared by the tensors of one layout (byte offset of W, and the
// bytes to the end capped below 2 GiB at cap_tokens = kMaxRecords / tok_bytes
// tokens), then one descriptor per tensor.  Every offset the loops use is
// under 144 tokens from W; the planner keeps that under 2 GiB, so a capped
// window still covers it.  W may be one tile before the row start (the first
// store window): the base is formed as an integer address, and nothing before
// the row is accessed.
struct WinSpan {
  uint64_t off;
  uint32_t bytes;
};

__device__ __forceinline__ WinSpan win_span(int32_t W, int32_t end, uint32_t tok_bytes, int32_t cap_tokens) {
  const int32_t rem = end - W;
  return {static_cast<uint64_t>(static_cast<int64_t>(W) * tok_bytes),
          rem < cap_tokens ? static_cast<uint32_t>(rem) * tok_bytes : static_cast<uint32_t>(kMaxRecords)};
}

template <typename S>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const S* row, const WinSpan& w) {
  return make_buf(reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(row) + w.off), w.bytes);
}

// ---- owner waves (4..7): per-token scalars, loads of x/delta/z, y -----------
// Owner wave o handles the tokens j = 4i + o (i < NS_OWN) of every tile for all
// 64 channels.  In the iteration that the scan waves spend on tile k, it
// computes the shared terms of tile k+1 into the other LDS buffer and finishes
// tile k-1 from the partial readouts the scan waves left there.
template <typename S, int K, bool STATE_ONLY, bool STRUCT, bool GATE, bool ZOH, bool WIN>
__device__ __forceinline__ void owner_loop(Smem& sm, const S* xrow, const S* dlrow, const S* zrow, S* yrow,
                                           const SegCtx& c, float& dsum) {
  constexpr uint32_t ES = sizeof(S);
  constexpr bool kLoadZ = !STATE_ONLY && GATE;
  const int o = c.w - 4;
  const uint32_t xo = (c.d0 + c.lane) * ES;
  // lanes past D store from a base past every window (no branch on the lane)
  const uint32_t yo = c.active ? (c.d0 + c.lane) * ES : kPastWindow;

  uint32_t xr[NS_PF][NS_OWN], dr[NS_PF][NS_OWN], zr[NS_PF][NS_OWN];
  float keep_dx[NS_PF][NS_OWN], keep_g[NS_PF][NS_OWN];

  // descriptor starts: the loads' at W, the stores' at Wy, a tile before the
  // segment (that tile's stores are sent out of range).  Windowed (WIN): W
  // starts with the segment and both move at every turn of the ring (the
  // loads reach 9 tiles past W, the stores 5 past Wy).
  int32_t W = WIN ? c.t_begin : 0, Wy = c.t_begin - NS_T;
  __amdgpu_buffer_rsrc_t bx, bdl, bz, by;
  const uint32_t tok_bytes = c.D * ES;
  const int32_t cap_tokens = static_cast<int32_t>(kMaxRecords / tok_bytes);
  auto set_windows = [&]() {
    const WinSpan in = win_span(W, c.L, tok_bytes, cap_tokens);
    bx = window(xrow, in);
    bdl = window(dlrow, in);
    if constexpr (kLoadZ) bz = window(zrow, in);
    if constexpr (!STATE_ONLY) by = window(yrow, win_span(Wy, c.t_end, tok_bytes, cap_tokens));
  };
  set_windows();

  auto load_tile = [&](auto slot_c, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i) {
      // x, delta and z share one layout, so one offset serves all three
      const uint32_t off = xo + static_cast<uint32_t>(t0 + 4 * i + o - W) * c.D * ES;
      xr[slot][i] = load_bits<S>(bx, off);
      dr[slot][i] = load_bits<S>(bdl, off);
      if constexpr (kLoadZ) zr[slot][i] = load_bits<S>(bz, off);
    }
  };

  // shared terms of the tile at t0 (ring slot `slot`) into LDS buffer `buf`
  auto compute_tile = [&](auto slot_c, int buf, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i) {
      const int j = 4 * i + o;
      float e0 = 1.0f, e1 = 1.0f, e2 = 1.0f, e3 = 1.0f, u = 0.0f;  // neutral step
      if constexpr (!STRUCT || ZOH) e0 = e1 = e2 = e3 = 0.0f;     // delta = 0 / exp(0) - 1 = 0
      float dx = 0.0f, g = 0.0f;
      if (t0 + j < c.t_end) {  // wave-uniform
        const float xv = bits_to_f32<S>(xr[slot][i]);
        const float dt = softplus_f32(bits_to_f32<S>(dr[slot][i]) + c.bias_d);
        if constexpr (STATE_ONLY) {
          dsum += dt;
        } else {
          dx = c.D_d * xv;
          if constexpr (GATE) g = silu_f32(bits_to_f32<S>(zr[slot][i]));
        }
        if constexpr (STRUCT && ZOH) {
          // E_m = exp(m dt A0) - 1 for the first state of each scan wave, m = wK + 1,
          // built without cancellation: E_2m = E_m (E_m + 2), E_(a+b) = E_a r^b + E_b
          const float r = fast_exp2(dt * c.A2_0);
          const float E1 = expm1_neg(dt * c.A_0, r);
          float rk = r, EK = E1;
#pragma unroll
          for (int q = 1; q < K; q <<= 1) EK = EK * (EK + 2.0f), rk *= rk;
          e0 = E1;
          e1 = __builtin_fmaf(EK, r, E1);
          e2 = __builtin_fmaf(e1, rk, EK);
          e3 = __builtin_fmaf(e2, rk, EK);
        } else if constexpr (STRUCT) {
          const float r = fast_exp2(dt * c.A2_0);
          float rk = r;  // r^K by squaring (K is a power of two)
#pragma unroll
          for (int q = 1; q < K; q <<= 1) rk *= rk;
          e0 = r;
          e1 = e0 * rk;
          e2 = e1 * rk;
          e3 = e2 * rk;
        } else {
          e0 = dt;
        }
        // the input term's per-channel factor: dt x (Euler); under the hold, x / A0
        // (structured: the scan waves keep the state scaled by n + 1) or x
        u = ZOH ? (STRUCT ? xv * c.invA_0 : xv) : dt * xv;
      }
      sm.E[buf][j][0][c.lane] = e0;
      if constexpr (STRUCT) {
        sm.E[buf][j][1][c.lane] = e1;
        sm.E[buf][j][2][c.lane] = e2;
        sm.E[buf][j][3][c.lane] = e3;
      }
      sm.U[buf][j][c.lane] = u;
      keep_dx[slot][i] = dx;
      keep_g[slot][i] = g;
    }
  };

  // Partial readouts of the tile to finish, read at the start of the
  // iteration so their LDS latency hides behind compute_tile.
  float pr[NS_OWN][4];
  auto read_partials = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) pr[i][w] = sm.P[buf][4 * i + o][w][c.lane];
  };
  // finish the tile at t0 (its keep values in slot `slot`) from the partials in pr
  auto finish_tile = [&](auto slot_c, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < NS_OWN; ++i) {
      const int j = 4 * i + o;
      float yv = ((pr[i][0] + pr[i][1]) + pr[i][2]) + pr[i][3];
      yv += keep_dx[slot][i];
      if constexpr (GATE) yv *= keep_g[slot][i];
      // by ends with the segment: tokens before it (the tile "before the
      // first" finished in the first iteration) and lanes past D are sent out
      // of range; tokens after it fail the range check.
      const int32_t tj = t0 + j;
      const uint32_t off = (tj >= c.t_begin ? yo : kPastWindow) + static_cast<uint32_t>(tj - Wy) * c.D * ES;
      store_val<S>(by, off, yv);
    }
  };

  static_assert(NS_PF == 4, "the ring code below is written for 4 slots");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  load_tile(I0{}, c.t_begin + 0 * NS_T);
  load_tile(I1{}, c.t_begin + 1 * NS_T);
  load_tile(I2{}, c.t_begin + 2 * NS_T);
  load_tile(I3{}, c.t_begin + 3 * NS_T);
  compute_tile(I0{}, 0, c.t_begin);
  load_tile(I0{}, c.t_begin + NS_PF * NS_T);
  __syncthreads();
  // iteration k (tile k scanned meanwhile): compute tile k+1, finish tile k-1
  for (int32_t k0 = 0; k0 < c.ntiles; k0 += NS_PF) {
    if constexpr (WIN) {  // this turn loads tiles k0+5..k0+8 and stores tiles k0-1..k0+2
      W = opaque_sgpr(c.t_begin + k0 * NS_T);
      Wy = W - NS_T;
      set_windows();
    }
    auto step = [&](auto kc, auto next_c, auto prev_c) {
      constexpr int kk = decltype(kc)::value;  // k0 + kk is the tile being scanned
      const int32_t tk = c.t_begin + (k0 + kk) * NS_T;
      if constexpr (!STATE_ONLY) read_partials((kk + 1) & 1);
      compute_tile(next_c, (kk + 1) & 1, tk + NS_T);
      load_tile(next_c, tk + NS_T + NS_PF * NS_T);
      if constexpr (!STATE_ONLY) finish_tile(prev_c, tk - NS_T);
      __syncthreads();
    };
    // ring slot of tile m is m % 4; k0 is a multiple of 4
    step(I0{}, I1{}, I3{});
    step(I1{}, I2{}, I0{});
    step(I2{}, I3{}, I1{});
    step(I3{}, I0{}, I2{});
  }
  // the last scanned tile (ntiles-1 has slot 3)
  if constexpr (!STATE_ONLY) {
    read_partials((c.ntiles - 1) & 1);
    finish_tile(I3{}, c.t_begin + (c.ntiles - 1) * NS_T);
  }
}

// ---- scan waves (0..3): the recurrence ---------------------------------------
// Under the zero-order hold (ZOH) the input term of state n is
// (exp(dt A_n) - 1) / A_n * B_n x.  Structured decays keep g_n = (n + 1) h_n:
// with E_n = exp((n+1) dt A0) - 1 and u = x / A0 the update is
// g_n <- g_n + E_n (g_n + B_n u), and the readout uses C_n / (n + 1).  E_n
// follows the chain E_(n+1) = E_n r + E_1, r = 1 + E_1, without cancellation.
// Generic decays compute the factor per state (zoh_coef) with u = x.
template <typename S, int K, bool STATE_ONLY, bool STRUCT, bool ZOH, bool WIN>
__device__ __forceinline__ void scan_loop(Smem& sm, const S* Brow, const S* Crow, float (&h)[K], const float (&A2)[K], const float (&An)[K],
                                          const float (&iA)[K], const SegCtx& c) {
  constexpr int N = 4 * K;
  constexpr uint32_t ES = sizeof(S);
  using BL = BCLayout<S, K>;
  constexpr int NLD = BL::NLD;
  uint32_t bq[NS_PF][NLD], cq[NS_PF][NLD];
  const int k16 = c.lane & 15;
  const uint32_t bco =
      ((k16 / BL::WB) * N + c.w * K + (BL::kPairs ? 2 * (k16 % BL::WB) : (BL::kF32 ? k16 % BL::WB : 0))) * ES;
  // ZOH with structured decays: the C words this lane holds, scaled by 1 / (n + 1)
  const int nlo = c.w * K + (BL::kPairs ? 2 * (k16 % BL::WB) : (BL::kF32 ? k16 % BL::WB : 0));
  const float cslo = (STRUCT && ZOH) ? 1.0f / static_cast<float>(nlo + 1) : 1.0f;
  const float cshi = (STRUCT && ZOH) ? 1.0f / static_cast<float>(nlo + 2) : 1.0f;

  // descriptors of B and C from token W to the row end: the row start, or
  // windowed (WIN) the segment start, moved at every turn of the ring (the
  // loads reach 8 tiles past W)
  int32_t W = WIN ? c.t_begin : 0;
  __amdgpu_buffer_rsrc_t bB, bC;
  constexpr uint32_t tok_bytes = N * ES;
  constexpr int32_t cap_tokens = static_cast<int32_t>(kMaxRecords / tok_bytes);
  auto set_windows = [&]() {
    const WinSpan sp = win_span(W, c.L, tok_bytes, cap_tokens);
    bB = window(Brow, sp);
    if constexpr (!STATE_ONLY) bC = window(Crow, sp);
  };
  set_windows();

  auto load_tile = [&](auto slot_c, int32_t t0) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t base = bco + static_cast<uint32_t>(t0 - W) * (N * ES);
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int off = static_cast<int>(base + q * BL::TPL * N * ES);  // q part folds into the immediate
      bq[slot][q] = BL::kPairs || BL::kF32 ? __builtin_amdgcn_raw_buffer_load_b32(bB, off, 0, 0)
                                           : __builtin_amdgcn_raw_buffer_load_b16(bB, off, 0, 0);
      if constexpr (!STATE_ONLY)
        cq[slot][q] = BL::kPairs || BL::kF32 ? __builtin_amdgcn_raw_buffer_load_b32(bC, off, 0, 0)
                                             : __builtin_amdgcn_raw_buffer_load_b16(bC, off, 0, 0);
    }
  };

  auto scan_tile = [&](auto slot_c, int buf) {
    constexpr int slot = decltype(slot_c)::value;
    float Blo[NLD], Bhi[NLD], Clo[NLD], Chi[NLD];
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const uint32_t bw = STATE_ONLY ? bq[slot][q] : ring_word(bq[slot][q]);
      if constexpr (BL::kF32) {
        Blo[q] = __uint_as_float(bw);
        Bhi[q] = 0.0f;
      } else {
        Blo[q] = __uint_as_float(bw << 16);
        Bhi[q] = BL::kPairs ? __uint_as_float(bw & 0xffff0000u) : 0.0f;
      }
    }
    // (Reading a token's LDS terms earlier than its use, in bursts or a few
    // tokens ahead, measured slower on this GPU: the reads stay next to it,
    // held there by a scheduling barrier after every second token.)
    auto token = [&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      constexpr int q = BL::load_of(j);
      if constexpr (!STATE_ONLY && j % BL::TPL == 0) {
        const uint32_t cw = ring_word(cq[slot][q]);
        if constexpr (BL::kF32) {
          Clo[q] = __uint_as_float(cw);
          Chi[q] = 0.0f;
        } else {
          Clo[q] = __uint_as_float(cw << 16);
          Chi[q] = BL::kPairs ? __uint_as_float(cw & 0xffff0000u) : 0.0f;
        }
        if constexpr (STRUCT && ZOH) Clo[q] *= cslo, Chi[q] *= cshi;
      }
      const float u = sm.U[buf][j][c.lane];
      float hv[K];
      float a = STRUCT ? sm.E[buf][j][c.w][c.lane] : 0.0f;  // ZOH: E of the wave's first state
      const float r0 = STRUCT ? sm.E[buf][j][0][c.lane] : 0.0f;
      const float r = (STRUCT && ZOH) ? 1.0f + r0 : r0;    // ZOH: r0 is E_1
      const float dt = STRUCT ? 0.0f : sm.E[buf][j][0][c.lane];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if constexpr (STRUCT && ZOH) {
          if (k > 0) a = __builtin_fmaf(a, r, r0);
        } else if constexpr (STRUCT) {
          if (k > 0) a *= r;
        } else {
          a = fast_exp2(dt * A2[k]);
        }
        const float bsrc = BL::odd_half(k) ? Bhi[q] : Blo[q];
        float bk;
        switch (BL::lane_of(j, k)) {  // compile-time constant after unrolling
#define SSM_BCAST_CASE(L) case L: bk = row_bcast<L>(bsrc); break;
          SSM_BCAST_CASE(0) SSM_BCAST_CASE(1) SSM_BCAST_CASE(2) SSM_BCAST_CASE(3)
          SSM_BCAST_CASE(4) SSM_BCAST_CASE(5) SSM_BCAST_CASE(6) SSM_BCAST_CASE(7)
          SSM_BCAST_CASE(8) SSM_BCAST_CASE(9) SSM_BCAST_CASE(10) SSM_BCAST_CASE(11)
          SSM_BCAST_CASE(12) SSM_BCAST_CASE(13) SSM_BCAST_CASE(14) SSM_BCAST_CASE(15)
#undef SSM_BCAST_CASE
          default: bk = 0.0f;
        }
        if constexpr (STRUCT && ZOH) {
          h[k] = __builtin_fmaf(a, h[k] + bk * u, h[k]);
        } else if constexpr (ZOH) {
          h[k] = __builtin_fmaf(a, h[k], bk * (zoh_coef(dt, An[k], iA[k], a) * u));
        } else {
          h[k] = __builtin_fmaf(a, h[k], bk * u);
        }
        hv[k] = h[k];
      }
      if constexpr (!STATE_ONLY) {
        auto csrc = [&](int k) { return BL::odd_half(k) ? Chi[q] : Clo[q]; };
        float acc = 0.0f;
        constexpr bool kWidened = j % BL::TPL == 0;  // C words widened just before this token
        if constexpr (K == 1) {
          acc = readout1<true, kWidened, BL::lane_of(j, 0)>(acc, csrc(0), hv[0]);
        } else if constexpr (K == 2) {
          acc = readout2<true, kWidened, BL::lane_of(j, 0), BL::lane_of(j, 1)>(acc, csrc(0), csrc(1), hv[0],
                                                                               hv[1]);
        } else {
          auto chunk = [&](auto g_c) {
            constexpr int g = decltype(g_c)::value;
            acc = readout4<g == 0, kWidened && g == 0, BL::lane_of(j, 4 * g), BL::lane_of(j, 4 * g + 1),
                           BL::lane_of(j, 4 * g + 2),
                           BL::lane_of(j, 4 * g + 3)>(acc, csrc(4 * g), csrc(4 * g + 1), csrc(4 * g + 2),
                                                      csrc(4 * g + 3), hv[4 * g], hv[4 * g + 1], hv[4 * g + 2],
                                                      hv[4 * g + 3]);
          };
          chunk(std::integral_constant<int, 0>{});
          if constexpr (K >= 8) chunk(std::integral_constant<int, 1>{});
          if constexpr (K >= 12) chunk(std::integral_constant<int, 2>{});
          if constexpr (K >= 16) chunk(std::integral_constant<int, 3>{});
        }
        sm.P[buf][j][c.w][c.lane] = acc;
      }
      // keep each pair of tokens' LDS reads, arithmetic and writes together
      // (pairs share paired LDS instructions): reads grouped further ahead of
      // their tokens measured slower.  The state-only pass (no readout) is
      // left to the scheduler (no pinned ring words either), which does
      // better there.
      if constexpr (!STATE_ONLY && j % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... js>(std::integer_sequence<int, js...>) {
      (token(std::integral_constant<int, js>{}), ...);
    }(std::make_integer_sequence<int, NS_T>{});
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  load_tile(I0{}, c.t_begin + 0 * NS_T);
  load_tile(I1{}, c.t_begin + 1 * NS_T);
  load_tile(I2{}, c.t_begin + 2 * NS_T);
  load_tile(I3{}, c.t_begin + 3 * NS_T);
  __syncthreads();
  for (int32_t k0 = 0; k0 < c.ntiles; k0 += NS_PF) {
    if constexpr (WIN) {  // this turn loads tiles k0+4..k0+7
      W = opaque_sgpr(c.t_begin + k0 * NS_T);
      set_windows();
    }
    auto step = [&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      scan_tile(kc, kk & 1);
      load_tile(kc, c.t_begin + (k0 + kk + NS_PF) * NS_T);
      __syncthreads();
    };
    step(I0{});
    step(I1{});
    step(I2{});
    step(I3{});
  }
}

template <typename S, int K, bool STATE_ONLY, bool GATE, bool ZOH, bool WIN>
__global__ __launch_bounds__(512, 1) void scan_nsplit_kernel(
    const S* __restrict__ x, const S* __restrict__ dl, const float* __restrict__ A,
    const S* __restrict__ Bm, const S* __restrict__ Cm, const float* __restrict__ Dsk,
    const S* __restrict__ z, const float* __restrict__ bias, const float* h0, float* hT,
    S* __restrict__ y, float* __restrict__ ws_state, float* __restrict__ ws_dsum,
    int32_t L, int32_t D, int32_t seg_len, int splits, int flags) {
  constexpr int N = 4 * K;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  SegCtx c;
  c.w = wave_id();
  c.lane = threadIdx.x & 63;
  const int sw = c.w & 3;  // scan wave index of this lane's states (owners shadow it)
  const int64_t b = blockIdx.y;
  const int s = blockIdx.z;
  c.D = static_cast<uint32_t>(D);
  c.d0 = blockIdx.x * 64u;
  c.active = c.d0 + c.lane < c.D;
  const uint32_t lo = c.active ? c.lane : c.D - 1 - c.d0;
  const int64_t d = c.d0 + lo;  // inactive lanes shadow channel D-1 for per-channel reads
  c.L = L;
  c.t_begin = s * seg_len;
  c.t_end = (c.t_begin + seg_len < L) ? c.t_begin + seg_len : L;
  const int32_t nt = (c.t_end - c.t_begin + NS_T - 1) / NS_T;
  c.ntiles = (nt + NS_PF - 1) / NS_PF * NS_PF;

  float A2[K], An[K], iA[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    An[k] = A[d * N + sw * K + k];
    A2[k] = An[k] * kLog2e;
    iA[k] = ZOH ? 1.0f / An[k] : 0.0f;
  }
  const float a0 = A[d * N];
  c.A2_0 = a0 * kLog2e;
  c.A_0 = a0;
  c.invA_0 = ZOH ? 1.0f / a0 : 0.0f;

  // Structured-decay test for the whole block: A[d, n] == (n+1) A[d, 0] exactly
  // (and, under the hold, A[d, 0] != 0: the structured form divides by it).
  bool ok = !(flags & kFlagGenericA) && (!ZOH || a0 != 0.0f);
#pragma unroll
  for (int k = 0; k < K; ++k) ok = ok && (A[d * N + sw * K + k] == static_cast<float>(sw * K + k + 1) * a0);
  const bool structured = __syncthreads_and(ok ? 1 : 0) != 0;

  c.bias_d = bias ? bias[d] : 0.0f;
  c.D_d = Dsk ? Dsk[d] : 0.0f;

  // this batch row of the (B, L, D) and (B, L, N) tensors
  const int64_t rowD = b * static_cast<int64_t>(L) * D, rowN = b * static_cast<int64_t>(L) * N;

  float dsum = 0.0f;
  float h[K];
  if (c.w >= 4) {
    const S* zrow = z ? z + rowD : x + rowD;  // never read without a gate
    if (structured)
      owner_loop<S, K, STATE_ONLY, true, GATE, ZOH, WIN>(sm, x + rowD, dl + rowD, zrow, y + rowD, c, dsum);
    else
      owner_loop<S, K, STATE_ONLY, false, GATE, ZOH, WIN>(sm, x + rowD, dl + rowD, zrow, y + rowD, c, dsum);
  } else {
    if constexpr (STATE_ONLY) {
#pragma unroll
      for (int k = 0; k < K; ++k) h[k] = 0.0f;
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) h[k] = h0 ? h0[(b * D + d) * N + sw * K + k] : 0.0f;
      // Carry in the summaries of the segments before this one.
      for (int j = 0; j < s; ++j) {
        const int64_t seg = b * splits + j;
        const float sdl = ws_dsum[seg * D + d];
#pragma unroll
        for (int k = 0; k < K; ++k)
          h[k] = __builtin_fmaf(fast_exp2(A2[k] * sdl), h[k], ws_state[(seg * D + d) * N + sw * K + k]);
      }
    }
    if (structured) {
      if constexpr (ZOH) {  // the structured hold runs on g_n = (n + 1) h_n
#pragma unroll
        for (int k = 0; k < K; ++k) h[k] *= static_cast<float>(sw * K + k + 1);
      }
      scan_loop<S, K, STATE_ONLY, true, ZOH, WIN>(sm, Bm + rowN, Cm + rowN, h, A2, An, iA, c);
      if constexpr (ZOH) {
#pragma unroll
        for (int k = 0; k < K; ++k) h[k] *= 1.0f / static_cast<float>(sw * K + k + 1);
      }
    } else {
      scan_loop<S, K, STATE_ONLY, false, ZOH, WIN>(sm, Bm + rowN, Cm + rowN, h, A2, An, iA, c);
    }
  }

  if constexpr (STATE_ONLY) {
    // per-channel sum of delta: owner partials through LDS (reusing E)
    __syncthreads();
    float* sdv = &sm.E[0][0][0][0];
    if (c.w >= 4) sdv[(c.w - 4) * 64 + c.lane] = dsum;
    __syncthreads();
    const int64_t seg = b * splits + s;
    if (c.w < 4 && c.active) {
#pragma unroll
      for (int k = 0; k < K; ++k) ws_state[(seg * D + d) * N + sw * K + k] = h[k];
    }
    if (c.w == 0 && c.active)
      ws_dsum[seg * D + d] = ((sdv[c.lane] + sdv[64 + c.lane]) + sdv[128 + c.lane]) + sdv[192 + c.lane];
  } else {
    if (hT && c.w < 4 && c.active && s == splits - 1) {
#pragma unroll
      for (int k = 0; k < K; ++k) hT[(b * D + d) * N + sw * K + k] = h[k];
    }
  }
}

template <typename S, int K, bool STATE_ONLY, bool GATE, bool ZOH, bool WIN>
void launch_one(const Problem& p, hipStream_t stream, unsigned nseg) {
  const unsigned nb = static_cast<unsigned>((p.dim + 63) / 64);
  hipLaunchKernelGGL((scan_nsplit_kernel<S, K, STATE_ONLY, GATE, ZOH, WIN>), dim3(nb, static_cast<unsigned>(p.batch), nseg),
                     dim3(512), kSmemBytes, stream, static_cast<const S*>(p.x), static_cast<const S*>(p.delta), p.A,
                     static_cast<const S*>(p.B), static_cast<const S*>(p.C), p.D, static_cast<const S*>(p.z),
                     p.delta_bias, p.h0, p.hT, static_cast<S*>(p.y), p.ws_state, p.ws_dsum,
                     static_cast<int32_t>(p.seqlen), static_cast<int32_t>(p.dim), static_cast<int32_t>(p.seg_len),
                     p.splits, p.flags);
}

template <typename S, int K, bool ZOH, bool WIN>
hipError_t launch_nsplit_z(const Problem& p, hipStream_t stream) {
  if (p.splits > 1) {
    launch_one<S, K, true, false, ZOH, WIN>(p, stream, static_cast<unsigned>(p.splits - 1));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.z)
    launch_one<S, K, false, true, ZOH, WIN>(p, stream, static_cast<unsigned>(p.splits));
  else
    launch_one<S, K, false, false, ZOH, WIN>(p, stream, static_cast<unsigned>(p.splits));
  return hipGetLastError();
}

// WIN: the windowed addressing for rows of 2 GiB or more (p.windowed).
template <typename S, int K, bool WIN>
hipError_t launch_nsplit_t(const Problem& p, hipStream_t stream) {
  return (p.flags & kFlagZoh) ? launch_nsplit_z<S, K, true, WIN>(p, stream)
                              : launch_nsplit_z<S, K, false, WIN>(p, stream);
}

}  // namespace nsplit_detail
}  // namespace ssm
