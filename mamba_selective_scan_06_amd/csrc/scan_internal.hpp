// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// A validated problem: shapes, pointers and the chosen plan.
struct Problem {
  int64_t batch, seqlen, dim, dstate;
  int dtype;  // 0 = fp32, 1 = bf16
  int flags;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  const float* h0;
  float* hT;
  void* y;
  // time splitting (NSPLIT family only)
  int splits;        // number of segments (1 = none)
  int64_t seg_len;   // timesteps per segment (multiple of the tile length)
  float* ws_state;   // (B, splits, D, N) segment end states from a zero start
  float* ws_dsum;    // (B, splits, D) sum of softplus(delta) over each segment
  bool windowed;     // a row of x or B spans 2 GiB or more: move the descriptors along it
  // (B, ceil(L / T) - 1, 4, D, ceil(N / 4)): the state after every T-th token
  // (T = ckpt_tokens(N)) for the backward, or nullptr
  float* checkpoints = nullptr;
};

constexpr int kFlagGenericA = 1;
constexpr int kFlagZoh = 2;
constexpr int kFlagCarryScan = 4;  // time split: compose segment summaries with the wave-level scan launch

// Tile length (timesteps) of the NSPLIT family; segment lengths are multiples of it.
constexpr int kNsplitTile = 16;
// Tokens past the current position (the end of a row, or the start of a
// descriptor window) that the NSPLIT kernels' prefetching loads can reach.
constexpr int64_t kNsplitReach = 320;
// Tiles per loop turn of the NSPLIT kernels; a segment runs whole turns and
// at most one half turn, so its padded length is a multiple of half a turn.
constexpr int kNsplitTurn = 8;

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
hipError_t launch_nsplit(const Problem& p, hipStream_t stream);
// Time split: turn the segment summaries in p.ws_state into the state
// entering each segment (wave-level associative scan; carry_scan.hip).
hipError_t launch_carry_scan(const Problem& p, hipStream_t stream);

// Size of the device array behind ssm_scan_fwd_noalloc (segment summaries of
// a time-split forward), and its address on the current device (looked up
// once per device).
constexpr int64_t kNoallocScratchBytes = int64_t{8} << 20;
hipError_t noalloc_scratch(void** out);
hipError_t launch_lane(const Problem& p, hipStream_t stream);
hipError_t launch_decode(const Problem& p, hipStream_t stream);
hipError_t launch_state_copy(const Problem& p, hipStream_t stream);  // seqlen == 0: hT <- h0 or 0

// ---- backward -----------------------------------------------------------------------
// Largest state size of the backward kernels.
constexpr int kBwdMaxState = 64;

// Lane layout of the backward kernels: G = ceil(N / K) adjacent lanes share a
// channel and each owns K consecutive states (K = 4 for N <= 4, else 8).
constexpr int bwd_lane_states(int64_t dstate) { return dstate <= 4 ? 4 : 8; }
constexpr int bwd_lanes_per_channel(int64_t dstate) {
  return dstate <= 8 ? 1 : (dstate <= 16 ? 2 : (dstate <= 32 ? 4 : 8));
}
// Tokens per checkpoint chunk: the chunk's recomputed states live in
// registers, (T + 1) * K of them per lane.
constexpr int bwd_chunk_len(int64_t dstate) { return bwd_lane_states(dstate) == 4 ? 16 : 8; }
// Spacing of the checkpoints a forward writes for the backward: its chunk.
constexpr int ckpt_tokens(int64_t dstate) { return bwd_chunk_len(dstate); }
// States per quarter of a checkpoint entry, laid out (4, D, M): state n of
// channel d at [n / M][d][n % M].
constexpr int ckpt_quarter(int64_t dstate) { return static_cast<int>((dstate + 3) / 4); }

struct BwdProblem {
  int64_t batch, seqlen, dim, dstate;
  int dtype;        // 0 = fp32, 1 = bf16
  int flags;        // ssm_flags (kFlagGenericA)
  int splits;       // time segments, >= 1
  int64_t seg_len;  // tokens per segment, a multiple of the chunk length
  int64_t nck;      // checkpoint chunks per sequence, ceil(L / chunk)
  int64_t nblk;     // waves per (batch row, segment): ceil(D / 64) * G, one partial dB / dC row each
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  const float* h0;
  const void* dy;
  const float* dhT;
  void* dx;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dD;
  void* dz;
  float* ddelta_bias;
  float* dh0;
  // workspace regions (fp32)
  float* ck;     // (B, nck, D, N) state entering each chunk, from a zero state at its segment start
  float* ckds;   // (B, nck, D) sum of softplus(delta) from the segment start to the chunk start
  float* segh;   // (B, S, D, N) segment end state from zero -> true state entering the segment
  float* segc;   // (B, S, D, N) adjoint at segment start from zero -> true adjoint leaving the segment end
  float* segds;  // (B, S, D) sum of softplus(delta) over each segment
  float* pA;     // (B, S, D, N) partial dA
  float* pD;     // (B, S, D) partial dD
  float* pbias;  // (B, S, D) partial d delta_bias
  float* pB;     // (B, L, nblk, N) partial dB, one row per wave (64 / G channels)
  float* pC;     // (B, L, nblk, N) partial dC
  // The forward's checkpoints ((B, nck - 1, 4, D, ceil(N / 4)), true states
  // after every chunk but the last), or nullptr.  With them the local pass skips the
  // forward recurrence, the combine its forward half, and ck, ckds and segh
  // are not used.
  const float* ck_in = nullptr;
};

hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream);

namespace bwd {
// Pieces of the backward launch sequence that live in different units.
hipError_t launch_combine(const BwdProblem& p, hipStream_t stream);
hipError_t launch_reduce_d(const BwdProblem& p, hipStream_t stream);
template <typename S>
hipError_t launch_typed(const BwdProblem& p, hipStream_t stream);  // S = float or uint16_t (bf16 bits)
extern template hipError_t launch_typed<float>(const BwdProblem& p, hipStream_t stream);
extern template hipError_t launch_typed<uint16_t>(const BwdProblem& p, hipStream_t stream);
}  // namespace bwd
// Outputs of a problem with no token (L == 0) or no chain (B == 0 or D == 0).
hipError_t launch_bwd_empty(const BwdProblem& p, hipStream_t stream);

// ---- conv1d + SiLU prologue ----------------------------------------------------------
struct ConvProblem {
  int64_t batch, seqlen, dim;
  int width;  // 1..4
  int dtype;  // 0 = fp32, 1 = bf16
  const void* x;
  const float* weight;
  const float* bias;
  const void* state;
  void* u;
  void* state_out;
};

hipError_t launch_conv(const ConvProblem& p, hipStream_t stream);

// ---- Mamba-2 state-space dual layer ---------------------------------------------------
// One kernel serves two recurrences over a P x N matrix state per (b, h):
//   mode 0 (SSD):  a_t = softplus(dt + dt_bias[h]) A[h],  i_t = softplus(dt + dt_bias[h]),  + D[h] x
//   mode 1 (gated linear attention): a_t = log_f[b,t,h] (0 if null), i_t = in_gate[b,t,h] (1 if null)
//   mode 2: mode 1 with the feature map elu(v) + 1 applied to B (keys) and C (queries)
// S_t = exp(a_t) S_{t-1} + i_t x_t B_t^T,  y_t = S_t C_t.
struct SsdProblem {
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate;
  int mode = 0;
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* dt_bias;
  const float* log_f = nullptr;
  const float* in_gate = nullptr;
  const float* h0;
  float* hT;
  void* y;
  // time segments: splits > 1 runs a state-only pass over the first splits - 1
  // segments of seg_chunks 64-token chunks, cut into sub-segments of
  // sub_chunks (a divisor of seg_chunks), into ws_state (B, R, H, P, N) and
  // ws_la (B, R, H) with R = (splits - 1) seg_chunks / sub_chunks, then the
  // full pass
  int splits = 1;
  int64_t seg_chunks = 0;
  int64_t sub_chunks = 0;
  float* ws_state = nullptr;
  float* ws_la = nullptr;
};

hipError_t launch_ssd(const SsdProblem& p, hipStream_t stream);
// phi(u) = elu(u) + 1 of n bf16 keys and n bf16 queries (n a multiple of 8,
// all four buffers 16-byte aligned), rounded to bf16 as the SSD kernel's own
// feature map rounds them.
hipError_t launch_gla_feature_map(const void* k, const void* q, void* pk, void* pq, int64_t n, hipStream_t stream);

}  // namespace ssm
