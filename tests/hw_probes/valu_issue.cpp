// Issue cost of wave64 VALU instructions on one SIMD (gfx950), by operand
// kind and number of waves per SIMD.  Every kernel runs ITER iterations of 32
// instructions: independent ones on 8 accumulators (registers fixed in asm so
// the VGPR banks, index mod 4, are known), or one dependent chain and the time per instruction per SIMD
// is the launch time over (instructions x waves per SIMD).  Prints one line
// per case: "<case> <waves per SIMD> <ns per instruction per SIMD>".
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      exit(3);                                                                   \
    }                                                                            \
  } while (0)

constexpr int ITER = 4096;
#define CLOB "v40", "v44", "v48", "v52", "v56", "v60", "v64", "v68", "v32", "v33", "v34", "v35", "v36", "s20"
#define INIT                                                                                                  \
  "v_mov_b32 v40, 1.0\n v_mov_b32 v44, 1.0\n v_mov_b32 v48, 1.0\n v_mov_b32 v52, 1.0\n v_mov_b32 v56, 1.0\n" \
  " v_mov_b32 v60, 1.0\n v_mov_b32 v64, 1.0\n v_mov_b32 v68, 1.0\n v_mov_b32 v32, 1.0\n v_mov_b32 v33, 1.0\n" \
  " v_mov_b32 v34, 0\n v_mov_b32 v35, 1.0\n v_mov_b32 v36, 1.0\n s_mov_b32 s20, 1.0\n"
// 8 instructions on the accumulators v40..v68 (all bank 0)
#define B8(OP, A, B, SUF)                                                                              \
  OP " v40, " A ", " B SUF "\n" OP " v44, " A ", " B SUF "\n" OP " v48, " A ", " B SUF "\n" OP " v52, " A \
     ", " B SUF "\n" OP " v56, " A ", " B SUF "\n" OP " v60, " A ", " B SUF "\n" OP " v64, " A ", " B SUF  \
     "\n" OP " v68, " A ", " B SUF "\n"
#define X4(x) x x x x
#define DPP " row_newbcast:3 row_mask:0xf bank_mask:0xf"

template <int KIND>
__global__ void probe(int* out) {
  asm volatile(INIT ::: CLOB);
  for (int it = 0; it < ITER; ++it) {
    // fused multiply-add v += a * b, sources in banks 1 and 2 (accumulator bank 0)
    if constexpr (KIND == 0) asm volatile(X4(B8("v_fmac_f32_e32", "v33", "v34", "")) ::: CLOB);
    // the same with both sources' banks equal to the accumulator's (bank 0)
    if constexpr (KIND == 1) asm volatile(X4(B8("v_fmac_f32_e32", "v36", "v32", "")) ::: CLOB);
    // a scalar (SGPR) first source
    if constexpr (KIND == 2) asm volatile(X4(B8("v_fmac_f32_e32", "s20", "v34", "")) ::: CLOB);
    // a DPP row broadcast on the first source (the source is never rewritten)
    if constexpr (KIND == 3) asm volatile(X4(B8("v_fmac_f32_dpp", "v33", "v34", DPP)) ::: CLOB);
    // a two-source multiply
    if constexpr (KIND == 4) asm volatile(X4(B8("v_mul_f32_e32", "v33", "v35", "")) ::: CLOB);
    // one dependent chain: all 32 FMAs accumulate into v40, so each waits for
    // the one before (what a lone wave pays for back-to-back dependences)
    if constexpr (KIND == 6)
      asm volatile(X4(X4("v_fmac_f32_e32 v40, v33, v34\n v_fmac_f32_e32 v40, v33, v34\n")) ::: CLOB);
    // the same chain with a DPP row-broadcast first source
    if constexpr (KIND == 7)
      asm volatile(X4(X4("v_fmac_f32_dpp v40, v33, v34" DPP "\n v_fmac_f32_dpp v40, v33, v34" DPP "\n")) ::: CLOB);
    // a transcendental (2^x), one source
    if constexpr (KIND == 5)
      asm volatile(X4("v_exp_f32 v40, v33\n v_exp_f32 v44, v33\n v_exp_f32 v48, v33\n v_exp_f32 v52, v33\n"
                      " v_exp_f32 v56, v33\n v_exp_f32 v60, v33\n v_exp_f32 v64, v33\n v_exp_f32 v68, v33\n") ::: CLOB);
  }
  if (threadIdx.x == 100000) out[0] = 1;  // never true: keeps the kernel's argument
}

template <int KIND>
void run(const char* name, int wps) {
  int* out;
  CK(hipMalloc(&out, 4));
  const int threads = 256 * wps;  // 4 SIMDs x wps waves, one workgroup per compute unit
  hipLaunchKernelGGL(probe<KIND>, dim3(256), dim3(threads), 0, 0, out);
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(probe<KIND>, dim3(256), dim3(threads), 0, 0, out);
  CK(hipEventRecord(e1));
  CK(hipDeviceSynchronize());
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  printf("%s %d %.4f\n", name, wps, ms * 1e6 / (32.0 * ITER * wps));
  fflush(stdout);
  CK(hipFree(out));
}

int main() {
  for (int w : {1, 2, 4}) {
    run<0>("fma", w);
    run<1>("fma_bank_conflict", w);
    run<2>("fma_sgpr", w);
    run<3>("fma_dpp", w);
    run<4>("mul", w);
    run<5>("exp", w);
    run<6>("fma_chain", w);
    run<7>("fma_dpp_chain", w);
  }
  return 0;
}
