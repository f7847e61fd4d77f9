// Weighted combine of the expert outputs for the DiT-MoE layer.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters": eq. MoE(x) sums
// the selected experts' outputs weighted by the gate, and every token also
// receives the outputs of the n_s shared experts (shared expert routing),
// with weight 1.
//
// One thread owns 8 consecutive features of one token: it reads the token's
// slot rows and weights, gathers 8 features of each selected expert output
// (16 or 32 bytes), accumulates w * y in fp32 in slot order, adds the shared
// output and rounds once.  No atomics: the result is the same on every run.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t row, int D,
                                      int c, float* f) {
  if constexpr (BF16) {
    const uint4 v = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(base) + row * D)[c];
    unpack8(v, f);
  } else {
    const float4* p = reinterpret_cast<const float4*>(
        static_cast<const float*>(base) + row * D) + 2 * c;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t row, int D, int c,
                                       const float* f) {
  if constexpr (BF16) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + row * D)[c] = v;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + row * D) +
                2 * c;
    p[0] = make_float4(f[0], f[1], f[2], f[3]);
    p[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

constexpr int kSlotGroup = 4;

template <bool YB, bool SB, bool OB>
__global__ __launch_bounds__(256) void combine_kernel(
    const void* __restrict__ y_rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ w, int64_t N, int D, int Kmax,
    const void* __restrict__ y_shared, void* __restrict__ y) {
  // N * D / 8 < 2^31 is checked on the host: 32-bit index arithmetic.
  const uint32_t nch = static_cast<uint32_t>(D / 8);
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= static_cast<uint32_t>(N) * nch) return;
  const uint32_t tq = i / nch;
  const int64_t t = tq;
  const int c = static_cast<int>(i - tq * nch);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  // Slots go in groups of kSlotGroup: the group's slot rows, weights and
  // expert-output rows are all loaded before the first multiply-add, so the
  // row loads do not wait on one another; the sum stays in slot order.
  for (int k0 = 0; k0 < Kmax; k0 += kSlotGroup) {
    int32_t r[kSlotGroup];
    float wk[kSlotGroup];
#pragma unroll
    for (int q = 0; q < kSlotGroup; ++q) {
      r[q] = -1;
      wk[q] = 0.0f;
      if (k0 + q < Kmax) {
        r[q] = slot_row[t * Kmax + k0 + q];
        wk[q] = w[t * Kmax + k0 + q];
      }
    }
    float v[kSlotGroup][8];
#pragma unroll
    for (int q = 0; q < kSlotGroup; ++q)
      if (r[q] >= 0) load8<YB>(y_rows, r[q], D, c, v[q]);
#pragma unroll
    for (int q = 0; q < kSlotGroup; ++q)
      if (r[q] >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(wk[q], v[q][j], acc[j]);
      }
  }
  if (y_shared != nullptr) {
    float v[8];
    load8<SB>(y_shared, t, D, c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += v[j];
  }
  store8<OB>(y, t, D, c, acc);
}

template <bool YB, bool SB>
hipError_t launch_c2(const void* y_rows, const int32_t* slot_row,
                     const float* w, int64_t N, int D, int Kmax,
                     const void* y_shared, void* y, bool out_bf16,
                     hipStream_t stream) {
  const int64_t total = N * (D / 8);
  const dim3 grid(static_cast<unsigned>(ceil_div(total, 256)));
  if (out_bf16)
    hipLaunchKernelGGL((combine_kernel<YB, SB, true>), grid, dim3(256), 0,
                       stream, y_rows, slot_row, w, N, D, Kmax, y_shared, y);
  else
    hipLaunchKernelGGL((combine_kernel<YB, SB, false>), grid, dim3(256), 0,
                       stream, y_rows, slot_row, w, N, D, Kmax, y_shared, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y_rows, bool y_bf16,
                          const int32_t* slot_row, const float* w, int64_t N,
                          int D, int Kmax, const void* y_shared, bool sh_bf16,
                          void* y, bool out_bf16, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (y_bf16) {
    if (sh_bf16)
      return launch_c2<true, true>(y_rows, slot_row, w, N, D, Kmax, y_shared,
                                   y, out_bf16, stream);
    return launch_c2<true, false>(y_rows, slot_row, w, N, D, Kmax, y_shared, y,
                                  out_bf16, stream);
  }
  if (sh_bf16)
    return launch_c2<false, true>(y_rows, slot_row, w, N, D, Kmax, y_shared, y,
                                  out_bf16, stream);
  return launch_c2<false, false>(y_rows, slot_row, w, N, D, Kmax, y_shared, y,
                                 out_bf16, stream);
}

}  // namespace moe
