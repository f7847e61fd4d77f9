// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kMaxExperts = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 <-> fp32.  A bf16 value is the high half of the fp32 with the same
// value, so widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t pair) {
  return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t pair) {
  return __uint_as_float(pair & 0xffff0000u);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two values in one v_cvt_pk_bf16_f32 (the same rounding as one at a time).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Unpack 8 bf16 (one 16-byte vector) to fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Prefix count of set bits in `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  const uint64_t below = (lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()));
  return __popcll(mask & below);
}

// Buffer descriptor of a byte range: loads at offsets past `bytes` return
// zero and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes,
                                           0x00020000);
}

// Offset used for chunks that lie outside the data: at or beyond every
// descriptor's byte count, so such loads return zero.
constexpr uint32_t kOutOfRange = 0xfffffff0u;

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

}  // namespace moe
