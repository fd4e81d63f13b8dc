// Two waves on one SIMD (gfx950), each running its own stream: does one wave's
// stream slow the other's?  Waves 0-3 of a 512-thread workgroup (one per SIMD)
// run 32k FMAs on 8 accumulators (plain, or with a DPP row-broadcast source);
// waves 4-7 (the other wave of each SIMD) idle, run plain FMAs, or run
// v_exp_f32.  Prints "<case> 1 <cycles of wave 0 per FMA instruction>" (the
// wave's own s_memtime clock, so the other waves' longer streams do not count).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); exit(3);} } while (0)
constexpr int ITER = 4096;
#define CLOB "v40", "v44", "v48", "v52", "v56", "v60", "v64", "v68", "v33", "v34"
#define INIT "v_mov_b32 v40, 1.0\n v_mov_b32 v44, 1.0\n v_mov_b32 v48, 1.0\n v_mov_b32 v52, 1.0\n v_mov_b32 v56, 1.0\n v_mov_b32 v60, 1.0\n v_mov_b32 v64, 1.0\n v_mov_b32 v68, 1.0\n v_mov_b32 v33, 1.0\n v_mov_b32 v34, 0\n"
#define F8 "v_fmac_f32_e32 v40, v33, v34\n v_fmac_f32_e32 v44, v33, v34\n v_fmac_f32_e32 v48, v33, v34\n v_fmac_f32_e32 v52, v33, v34\n v_fmac_f32_e32 v56, v33, v34\n v_fmac_f32_e32 v60, v33, v34\n v_fmac_f32_e32 v64, v33, v34\n v_fmac_f32_e32 v68, v33, v34\n"
#define E8 "v_exp_f32 v40, v33\n v_exp_f32 v44, v33\n v_exp_f32 v48, v33\n v_exp_f32 v52, v33\n v_exp_f32 v56, v33\n v_exp_f32 v60, v33\n v_exp_f32 v64, v33\n v_exp_f32 v68, v33\n"
#define DP " row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
#define D8 "v_fmac_f32_dpp v40, v33, v34" DP " v_fmac_f32_dpp v44, v33, v34" DP " v_fmac_f32_dpp v48, v33, v34" DP " v_fmac_f32_dpp v52, v33, v34" DP " v_fmac_f32_dpp v56, v33, v34" DP " v_fmac_f32_dpp v60, v33, v34" DP " v_fmac_f32_dpp v64, v33, v34" DP " v_fmac_f32_dpp v68, v33, v34" DP
// MODE 0: waves 0-3 FMA, waves 4-7 idle.  1: waves 4-7 exp.  2: waves 4-7 FMA.
// 3: waves 0-3 DPP-FMA, 4-7 idle.  4: waves 0-3 DPP-FMA, 4-7 plain FMA.  5: waves 0-3 DPP-FMA, 4-7 exp.
template <int MODE>
__global__ void probe(int* out, int* t) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  asm volatile(INIT ::: CLOB);
  long long t0 = clock64();
  if (w < 4) {
    for (int it = 0; it < ITER; ++it) {
      if constexpr (MODE < 3) asm volatile(F8 F8 F8 F8 ::: CLOB);
      else asm volatile(D8 D8 D8 D8 ::: CLOB);
    }
  } else if (MODE == 1 || MODE == 5) {
    for (int it = 0; it < ITER; ++it) asm volatile(E8 E8 ::: CLOB);
  } else if (MODE == 2 || MODE == 4) {
    for (int it = 0; it < ITER; ++it) asm volatile(F8 F8 F8 F8 ::: CLOB);
  }
  long long t1 = clock64();
  if (threadIdx.x == 0 && blockIdx.x == 0) t[0] = (int)(t1 - t0);
  if (threadIdx.x == 100000) out[0] = 1;
}
template <int MODE>
void run(const char* name) {
  int *out, *t; CK(hipMalloc(&out, 4)); CK(hipMalloc(&t, 4));
  hipLaunchKernelGGL(probe<MODE>, dim3(256), dim3(512), 0, 0, out, t);
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(probe<MODE>, dim3(256), dim3(512), 0, 0, out, t);
  CK(hipEventRecord(e1)); CK(hipDeviceSynchronize());
  float ms; CK(hipEventElapsedTime(&ms, e0, e1));
  int tc; CK(hipMemcpy(&tc, t, 4, hipMemcpyDeviceToHost));
  (void)ms;
  printf("%s 1 %.3f\n", name, tc / (32.0 * ITER));
  fflush(stdout); CK(hipFree(out)); CK(hipFree(t));
}
int main() {
  run<0>("fma_alone");
  run<1>("fma_with_exp");
  run<2>("fma_with_fma");
  run<3>("dppfma_alone");
  run<4>("dppfma_with_fma");
  run<5>("dppfma_with_exp");
  return 0;
}
