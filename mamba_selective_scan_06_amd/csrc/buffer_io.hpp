// Raw buffer access for the NSPLIT kernels (gfx950).
//
// A buffer descriptor covers part of one batch row of a tensor (under 2 GiB);
// the whole byte offset goes in the VGPR operand, which is the part the
// hardware range check covers on this GPU family.  Loads past the end return 0
// and stores past the end are dropped, which lets the kernels prefetch past the
// end of a sequence and run padded tiles without bounds branches.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace ssm {

// Word 3 of a raw buffer descriptor on the gfx9 family: 32-bit data format.
constexpr int kRawBufferFlags = 0x00020000;

// Largest byte count a descriptor here covers, and an offset that fails the
// range check of every such descriptor.
constexpr int64_t kMaxRecords = 0x7FFFFFFF;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
// A base offset past every window: adding any in-window offset (below 2^31)
// neither wraps nor comes back into range.
constexpr uint32_t kPastWindow = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRawBufferFlags);
}

// Cache-policy operand of the buffer intrinsics that sets the non-temporal
// bit (`nt`) on gfx950: the token tensors these helpers move (x, delta, z in,
// y out) are touched once, so they stream past the caches (1% faster on the
// forward scan).
constexpr int kStreamPolicy = 2;

// One element's raw bits (bf16 zero-extended, or fp32) at byte offset `off`.
template <typename S>
__device__ __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(S) == 4)
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kStreamPolicy);
  else
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, kStreamPolicy);
}

template <typename S>
__device__ __forceinline__ float bits_to_f32(uint32_t v) {
  if constexpr (sizeof(S) == 4) return __uint_as_float(v);
  else return __uint_as_float(v << 16);
}

// Store one fp32 value as S (bf16: round to nearest even) at byte offset `off`.
template <typename S>
__device__ __forceinline__ void store_val(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  if constexpr (sizeof(S) == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, kStreamPolicy);
  } else {
    __hip_bfloat16 hb = __float2bfloat16(v);
    __builtin_amdgcn_raw_buffer_store_b16(__bfloat16_as_ushort(hb), r, static_cast<int>(off), 0, kStreamPolicy);
  }
}

}  // namespace ssm
