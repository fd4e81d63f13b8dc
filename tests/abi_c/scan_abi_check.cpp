// A caller of libssm_scan.so through its C ABI alone: plain HIP device memory,
// no Python and no torch.  It loads one problem's inputs from raw files in a
// directory (written by the test from the shared seeded generator), runs
// ssm_scan_fwd on a stream of its own, and writes y and hT back for the test to
// compare with the oracle.  It also checks the error path (a NULL argument)
// and the ABI version.
//
//   scan_abi_check DIR B L D N DTYPE
//     DIR/{x,delta,B,C,z}.bin  (B,L,D) / (B,L,N) in DTYPE (0 = fp32, 1 = bf16 bits)
//     DIR/{A,D,bias,h0}.bin    fp32; D, z, bias, h0 may be absent (NULL)
//     writes DIR/y.bin (DTYPE) and DIR/hT.bin (fp32)
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "ssm_scan.h"

#define CHECK_HIP(e)                                                        \
  do {                                                                      \
    hipError_t r_ = (e);                                                    \
    if (r_ != hipSuccess) {                                                 \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(r_), __LINE__); \
      std::exit(2);                                                         \
    }                                                                       \
  } while (0)

static std::vector<char> read_file(const std::string& path, size_t expect, bool optional) {
  std::vector<char> buf;
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) {
    if (optional) return buf;
    std::fprintf(stderr, "missing %s\n", path.c_str());
    std::exit(3);
  }
  buf.resize(expect);
  const size_t got = std::fread(buf.data(), 1, expect, f);
  std::fclose(f);
  if (got != expect) {
    std::fprintf(stderr, "%s: %zu bytes, expected %zu\n", path.c_str(), got, expect);
    std::exit(3);
  }
  return buf;
}

// Device copy of a file's bytes, or NULL when the file is absent and optional.
static void* to_device(const std::string& dir, const char* name, size_t bytes, bool optional) {
  std::vector<char> h = read_file(dir + "/" + name + ".bin", bytes, optional);
  if (h.empty()) return nullptr;
  void* d = nullptr;
  CHECK_HIP(hipMalloc(&d, bytes));
  CHECK_HIP(hipMemcpy(d, h.data(), bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: %s DIR B L D N DTYPE\n", argv[0]);
    return 1;
  }
  const std::string dir = argv[1];
  const int64_t B = std::atoll(argv[2]), L = std::atoll(argv[3]), D = std::atoll(argv[4]), N = std::atoll(argv[5]);
  const int dtype = std::atoi(argv[6]);
  const size_t es = dtype == SSM_DTYPE_F32 ? 4 : 2;
  if (ssm_scan_abi_version() != SSM_SCAN_ABI_VERSION) {
    std::fprintf(stderr, "ABI version mismatch\n");
    return 4;
  }

  ssm_scan_args a = {};
  a.batch = B, a.seqlen = L, a.dim = D, a.dstate = N;
  a.dtype = dtype;
  // error path first: no x
  const int rc_null = ssm_scan_fwd(&a, nullptr);
  if (rc_null != SSM_ERR_NULL) {
    std::fprintf(stderr, "expected SSM_ERR_NULL for a missing x, got %d (%s)\n", rc_null, ssm_scan_strerror(rc_null));
    return 5;
  }

  const size_t bld = static_cast<size_t>(B * L * D), bln = static_cast<size_t>(B * L * N);
  const size_t bdn = static_cast<size_t>(B * D * N);
  a.x = to_device(dir, "x", bld * es, false);
  a.delta = to_device(dir, "delta", bld * es, false);
  a.A = static_cast<const float*>(to_device(dir, "A", static_cast<size_t>(D * N) * 4, false));
  a.B = to_device(dir, "B", bln * es, false);
  a.C = to_device(dir, "C", bln * es, false);
  a.D = static_cast<const float*>(to_device(dir, "D", static_cast<size_t>(D) * 4, true));
  a.z = to_device(dir, "z", bld * es, true);
  a.delta_bias = static_cast<const float*>(to_device(dir, "bias", static_cast<size_t>(D) * 4, true));
  a.h0 = static_cast<const float*>(to_device(dir, "h0", bdn * 4, true));
  void *y = nullptr, *hT = nullptr;
  CHECK_HIP(hipMalloc(&y, bld * es));
  CHECK_HIP(hipMalloc(&hT, bdn * 4));
  a.y = y;
  a.hT = static_cast<float*>(hT);

  // time splitting needs a caller-provided workspace when the plan asks for one
  const int64_t ws = ssm_scan_workspace_bytes(&a);
  if (ws < 0) {
    std::fprintf(stderr, "workspace query: %s\n", ssm_scan_strerror(static_cast<int>(ws)));
    return 6;
  }
  void* wsp = nullptr;
  if (ws > 0) CHECK_HIP(hipMalloc(&wsp, static_cast<size_t>(ws)));
  a.workspace = wsp;
  a.workspace_bytes = ws;
  const int64_t plan = ssm_scan_plan(&a);

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  const int rc = ssm_scan_fwd(&a, stream);
  if (rc != SSM_OK) {
    std::fprintf(stderr, "ssm_scan_fwd: %s\n", ssm_scan_strerror(rc));
    return 7;
  }
  CHECK_HIP(hipStreamSynchronize(stream));

  std::vector<char> hy(bld * es), hh(bdn * 4);
  CHECK_HIP(hipMemcpy(hy.data(), y, hy.size(), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hh.data(), hT, hh.size(), hipMemcpyDeviceToHost));
  FILE* f = std::fopen((dir + "/y.bin").c_str(), "wb");
  std::fwrite(hy.data(), 1, hy.size(), f);
  std::fclose(f);
  f = std::fopen((dir + "/hT.bin").c_str(), "wb");
  std::fwrite(hh.data(), 1, hh.size(), f);
  std::fclose(f);
  std::printf("ok plan=%lld workspace=%lld\n", static_cast<long long>(plan), static_cast<long long>(ws));

  CHECK_HIP(hipStreamDestroy(stream));
  const void* bufs[] = {a.x, a.delta, a.A, a.B, a.C, a.D, a.z, a.delta_bias, a.h0, y, hT, wsp};
  for (const void* p : bufs)
    if (p) CHECK_HIP(hipFree(const_cast<void*>(p)));
  return 0;
}
