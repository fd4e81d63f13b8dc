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
};

constexpr int kFlagGenericA = 1;

// Tile length (timesteps) of the NSPLIT family; segment lengths are multiples of it.
constexpr int kNsplitTile = 16;

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
hipError_t launch_nsplit(const Problem& p, hipStream_t stream);
hipError_t launch_lane(const Problem& p, hipStream_t stream);
hipError_t launch_decode(const Problem& p, hipStream_t stream);
hipError_t launch_state_copy(const Problem& p, hipStream_t stream);  // seqlen == 0: hT <- h0 or 0

}  // namespace ssm
