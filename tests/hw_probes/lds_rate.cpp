// LDS throughput of one compute unit (gfx950) by access width: each wave
// reads or writes its own 4 KiB slice with lane-linear addresses (every
// 16-lane group touches 256 contiguous bytes), ITER times over 4 KiB.
// Prints "<case> <waves per CU> <bytes per ns per CU>".
#include <hip/hip_runtime.h>

#include <stdint.h>
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

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
constexpr int ITER = 2048;
constexpr int SLICE = 4096;  // bytes per wave

// KIND: 0 read b32, 1 read b64, 2 read b128, 3 write b32, 4 write b128
template <int KIND>
__global__ void probe(uint32_t* out, int salt) {
  __shared__ __align__(16) uint32_t lds[16 * SLICE / 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 16 * SLICE / 4; i += blockDim.x) lds[i] = i ^ salt;
  __syncthreads();
  const int base = (w % 16) * SLICE / 4;  // in words
  const u4 v4 = {static_cast<uint32_t>(lane), static_cast<uint32_t>(w), static_cast<uint32_t>(salt), 7u};
  for (int it = 0; it < ITER; ++it) {
    if constexpr (KIND <= 2) {
      u4 r[16];
      constexpr int n = KIND == 0 ? 16 : (KIND == 1 ? 8 : 4);  // accesses covering the 4 KiB slice
#pragma unroll
      for (int k = 0; k < n; ++k) {
        if constexpr (KIND == 0) r[k].x = lds[base + k * 64 + lane];
        if constexpr (KIND == 1) r[k].xy = *reinterpret_cast<u2*>(&lds[base + k * 128 + lane * 2]);
        if constexpr (KIND == 2) r[k] = *reinterpret_cast<u4*>(&lds[base + k * 256 + lane * 4]);
      }
#pragma unroll
      for (int k = 0; k < n; ++k) asm volatile("" ::"v"(r[k]));
    } else {
      constexpr int n = KIND == 3 ? 16 : 4;
#pragma unroll
      for (int k = 0; k < n; ++k) {
        if constexpr (KIND == 3) lds[base + k * 64 + lane] = v4.x + k + it;
        if constexpr (KIND == 4) {
          const u4 t = {v4.x + k + it, v4.y, v4.z, v4.w};
          *reinterpret_cast<u4*>(&lds[base + k * 256 + lane * 4]) = t;
        }
      }
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();
  if (lds[lane] == 0x12345678u) out[blockIdx.x * blockDim.x + threadIdx.x] = 1;
}

template <int KIND>
void run(const char* name, int waves) {
  uint32_t* out;
  CK(hipMalloc(&out, 256 * waves * 64 * 4));
  hipLaunchKernelGGL(probe<KIND>, dim3(256), dim3(64 * waves), 0, 0, out, 3);
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(probe<KIND>, dim3(256), dim3(64 * waves), 0, 0, out, 3);
  CK(hipEventRecord(e1));
  CK(hipDeviceSynchronize());
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const double bytes = static_cast<double>(ITER) * SLICE * waves;  // per compute unit
  printf("%s %d %.1f\n", name, waves, bytes / (ms * 1e6));
  fflush(stdout);
  CK(hipFree(out));
}

int main() {
  for (int w : {8, 16}) {
    run<0>("read_2x_b32", w);  // compiled as ds_read2st64_b32
    run<1>("read_2x_b64", w);  // ds_read2st64_b64
    run<2>("read_b128", w);
    run<3>("write_2x_b32", w);  // ds_write2st64_b32
    run<4>("write_b128", w);
  }
  return 0;
}
