// Expert-level balance statistic of the DiT-MoE layer.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE-DiT, eq.
// L_balance:  L = alpha * sum_i (n/(K T) sum_t I(t,i)) * (1/T sum_t P(t,i)),
// with T the patch-sequence length, I(t,i) the selection indicator and
// P(t,i) the token's probability of expert i.
//
//  * balance_seq_kernel: workgroup b owns image b.  Thread (r, e) of an
//    R x E grid (R = 1024 / E) sums tokens t = r, r+R, ... of expert e in
//    order; the R partial sums of each expert are then added by a
//    fixed-order tree in LDS.  Counts are exact integers.  Same inputs, same
//    bits.
//  * balance_loss_kernel: one workgroup turns counts and prob_sums into the
//    loss, summing in a fixed order (per image, then over images).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBalThreads = 256;
constexpr int kSeqThreads = 1024;

__global__ __launch_bounds__(kSeqThreads) void balance_seq_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx, int T,
    int E, int Kmax, int32_t* __restrict__ counts, float* __restrict__ psum) {
  __shared__ float sp[kSeqThreads];
  __shared__ int32_t sc[kSeqThreads];
  const int R = kSeqThreads / E;
  const int r = threadIdx.x / E;
  const int e = threadIdx.x - r * E;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * T;
  float p = 0.0f;
  int32_t c = 0;
  if (r < R) {
    // tokens r, r + R, ...; unrolled so that several loads are in flight
    int t = r;
    for (; t + 3 * R < T; t += 4 * R) {
      float q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = probs[(t0 + t + u * R) * E + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p += q[u];
        const int64_t tt = t0 + t + u * R;
        for (int k = 0; k < Kmax; ++k) c += (idx[tt * Kmax + k] == e) ? 1 : 0;
      }
    }
    for (; t < T; t += R) {
      const int64_t tt = t0 + t;
      p += probs[tt * E + e];
      for (int k = 0; k < Kmax; ++k) c += (idx[tt * Kmax + k] == e) ? 1 : 0;
    }
  }
  sp[threadIdx.x] = p;
  sc[threadIdx.x] = c;
  __syncthreads();
  // fixed-order tree over the R rows of each expert
  for (int h = 1; h < R; h *= 2) {
    if (r < R && (r % (2 * h)) == 0 && r + h < R) {
      sp[threadIdx.x] += sp[threadIdx.x + h * E];
      sc[threadIdx.x] += sc[threadIdx.x + h * E];
    }
    __syncthreads();
  }
  if (threadIdx.x < E) {
    psum[static_cast<int64_t>(blockIdx.x) * E + threadIdx.x] = sp[threadIdx.x];
    counts[static_cast<int64_t>(blockIdx.x) * E + threadIdx.x] = sc[threadIdx.x];
  }
}

__global__ __launch_bounds__(kBalThreads) void balance_loss_kernel(
    const int32_t* __restrict__ counts, const float* __restrict__ psum, int B,
    int T, int E, int K, float alpha, int global, float* __restrict__ loss) {
  __shared__ float part[kBalThreads];
  const int tid = threadIdx.x;
  if (!global) {
    // L_b = alpha * sum_i (E/(K T)) c[b][i] * (S[b][i] / T); loss = mean_b.
    const float f = static_cast<float>(E) / (static_cast<float>(K) * T);
    float acc = 0.0f;
    for (int b = tid; b < B; b += kBalThreads) {
      float lb = 0.0f;
      for (int i = 0; i < E; ++i) {
        const int64_t o = static_cast<int64_t>(b) * E + i;
        lb += (f * static_cast<float>(counts[o])) * (psum[o] / T);
      }
      acc += alpha * lb;
    }
    part[tid] = acc;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int j = 0; j < kBalThreads; ++j) s += part[j];
      loss[0] = (B > 0) ? s / static_cast<float>(B) : 0.0f;
    }
  } else {
    // One pool of B*T tokens.
    const float Tg = static_cast<float>(B) * T;
    const float f = static_cast<float>(E) / (static_cast<float>(K) * Tg);
    float term = 0.0f;
    if (tid < E) {
      int64_t c = 0;
      float s = 0.0f;
      for (int b = 0; b < B; ++b) {
        c += counts[static_cast<int64_t>(b) * E + tid];
        s += psum[static_cast<int64_t>(b) * E + tid];
      }
      term = (f * static_cast<float>(c)) * (s / Tg);
    }
    part[tid] = term;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int j = 0; j < E; ++j) s += part[j];
      loss[0] = alpha * s;
    }
  }
}

}  // namespace

hipError_t launch_balance(const float* probs, const int32_t* idx, int B, int T,
                          int E, int Kmax, int K, float alpha, bool global,
                          int32_t* counts, float* psum, float* loss,
                          hipStream_t stream) {
  if (B > 0) {
    hipLaunchKernelGGL(balance_seq_kernel, dim3(B), dim3(kSeqThreads), 0,
                       stream, probs, idx, T, E, Kmax, counts, psum);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(balance_loss_kernel, dim3(1), dim3(kBalThreads), 0, stream,
                     counts, psum, B, T, E, K, alpha, global ? 1 : 0, loss);
  return hipGetLastError();
}

}  // namespace moe
