// Device helpers shared by the scan kernels (gfx950, wave64).
//
// Element access for the two storage types, and the per-token scalar maths of
// the selective SSM in fp32: the softplus of the step size (selection, page
// youngju.dev "Mamba 논문 리뷰" section 3.1) and the SiLU of the output gate
// (section 3.4).  Transcendentals use the hardware v_exp_f32 / v_log_f32 /
// v_rcp_f32 directly; the one place where that alone would lose accuracy
// (log of 1 + w for small w) carries an explicit correction term.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- storage <-> fp32 --------------------------------------------------------
// bf16 is kept as its raw 16-bit pattern; widening to fp32 is an exact shift.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// Narrowing rounds to nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) {
  __hip_bfloat16 b = __float2bfloat16(v);
  *p = __bfloat16_as_ushort(b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^{-|v|}).
// log1p(w), w in (0, 1], is evaluated as ln(p) + (w - (p - 1)) with p = fl(1 + w):
// the second term is the exact rounding error of 1 + w (Sterbenz), so the
// result keeps its relative accuracy when w is tiny (v << 0), where a plain
// log(1 + w) would lose all of it.  Dividing that term by p is skipped; the
// neglected part is below 2^-24 * w.
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = fast_exp2(-fabsf(v) * kLog2e);
  const float p = 1.0f + w;
  const float corr = w - (p - 1.0f);
  return fmaxf(v, 0.0f) + __builtin_fmaf(fast_log2(p), kLn2, corr);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}); z -> -inf gives -0, not NaN.
__device__ __forceinline__ float silu_f32(float z) {
  return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// Wave index inside the workgroup as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace ssm
