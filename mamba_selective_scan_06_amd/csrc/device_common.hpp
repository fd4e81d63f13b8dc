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

// Zero-order-hold input coefficient of one state (page youngju.dev section
// 2.2: Bbar = (delta A)^-1 (exp(delta A) - I) delta B; for a diagonal A the
// factor multiplying B_n x is (exp(delta A_n) - 1) / A_n, with limit delta at
// A_n = 0).  `a` is exp(delta A_n) as computed for the decay.  Near a = 1 the
// difference a - 1 loses relative accuracy, so for |z| < 1/32, z = delta A_n,
// the factor is the series delta (1 + z/2 + z^2/6 + z^3/24) (truncation below
// 1e-8 relative); above it a - 1 is accurate to ~2e-6.  A_n = 0 always takes
// the series (inv_An is then unused).
//
// The choice is one v_cmp + v_cndmask written together, after both sides are
// computed: left to itself the compiler turns it into a branch per element.
__device__ __forceinline__ float select_small_z(float z, float if_small, float otherwise) {
  float r;
  asm("v_cmp_gt_f32_e64 vcc, %4, |%1|\n\tv_cndmask_b32_e32 %0, %3, %2, vcc"
      : "=v"(r)
      : "v"(z), "v"(if_small), "v"(otherwise), "s"(0.03125f)
      : "vcc");
  return r;
}

__device__ __forceinline__ float zoh_coef(float dt, float An, float inv_An, float a) {
  const float z = dt * An;
  const float series =
      dt * __builtin_fmaf(z, __builtin_fmaf(z, __builtin_fmaf(z, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
  return select_small_z(z, series, (a - 1.0f) * inv_An);
}

// expm1(z) for z <= 0, with `a` = exp(z): the same series / difference split.
__device__ __forceinline__ float expm1_neg(float z, float a) {
  const float series = z * __builtin_fmaf(z, __builtin_fmaf(z, __builtin_fmaf(z, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
  return select_small_z(z, series, a - 1.0f);
}

// Wave index inside the workgroup as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace ssm
