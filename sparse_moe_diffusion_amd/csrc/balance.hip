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
//  * balance_partials_kernel: when the gate kernel has already reduced each
//    16-token group (partials [N/16][E]), one workgroup adds each image's
//    T/16 partials in group order and then computes the loss as above.
//  * route_finish_kernel (the fused routing call): the same in workgroup 0,
//    and in workgroup 1 the permutation's expert scan over the gate's
//    per-16-token selection counts.
#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace moe {

namespace {

constexpr int kBalThreads = 256;
constexpr int kSeqThreads = 1024;

__global__ __launch_bounds__(kSeqThreads) void balance_seq_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx, int T,
    int E, int Kmax, int32_t* __restrict__ counts, float* __restrict__ psum) {
  __shared__ float sp[kSeqThreads];
  __shared__ int32_t sc[kSeqThreads];
  // Each chunk of kSeqThreads tokens: every thread first turns one token's
  // Kmax slots into a bit mask of its experts, so the (r, e) threads read
  // a mask per token instead of Kmax slots.
  __shared__ uint64_t tmask[kSeqThreads];
  const int R = kSeqThreads / E;
  const int r = threadIdx.x / E;
  const int e = threadIdx.x - r * E;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * T;
  float p = 0.0f;
  int32_t c = 0;
  // Token t of the image is summed by thread (t % R, e), in ascending t:
  // chunks of R * (kSeqThreads / R) tokens keep that order.
  const int chunk = R * (kSeqThreads / R);
  for (int c0 = 0; c0 < T; c0 += chunk) {
    {
      // the token's slots 8 at a time, all 8 loads in flight (slots past
      // Kmax and tokens past T re-read a valid slot and are not counted)
      const int t = c0 + static_cast<int>(threadIdx.x);
      const bool in = threadIdx.x < chunk && t < T;
      const int32_t* s = idx + (t0 + (t < T ? t : T - 1)) * Kmax;
      uint64_t m = 0;
      for (int k0 = 0; k0 < Kmax; k0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s[k0 + u < Kmax ? k0 + u : Kmax - 1];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k0 + u < Kmax && v[u] >= 0 && v[u] < 64) m |= 1ull << v[u];
      }
      tmask[threadIdx.x] = in ? m : 0ull;
    }
    __syncthreads();
    if (r < R) {
      const int c1 = min(T, c0 + chunk);
      // tokens c0 + r, c0 + r + R, ...; eight loads in flight, added in
      // token order
      int t = c0 + r;
      for (; t + 7 * R < c1; t += 8 * R) {
        float q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = probs[(t0 + t + u * R) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          p += q[u];
          c += static_cast<int32_t>((tmask[t + u * R - c0] >> e) & 1ull);
        }
      }
      for (; t < c1; t += R) {
        p += probs[(t0 + t) * E + e];
        c += static_cast<int32_t>((tmask[t - c0] >> e) & 1ull);
      }
    }
    __syncthreads();
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

// part[0] = sum of part[0 .. kBalThreads), by a fixed pairwise tree (the
// same association every call).  Every thread calls it; tid >= kBalThreads
// only passes the barriers.
__device__ __forceinline__ void tree_sum(float* part, int tid) {
  for (int h = kBalThreads / 2; h > 0; h /= 2) {
    if (tid < h) part[tid] += part[tid + h];
    __syncthreads();
  }
}

// The loss from counts and prob_sums.  Every thread of the workgroup calls
// it (it holds barriers); threads kBalThreads and up only pass them.
__device__ void balance_loss_body(const int32_t* __restrict__ counts,
                                  const float* __restrict__ psum, int B, int T,
                                  int E, int K, float alpha, int global,
                                  float* __restrict__ loss) {
  __shared__ float part[kBalThreads];
  const int tid = threadIdx.x < kBalThreads ? threadIdx.x : kBalThreads;
  if (B == 0) {   // no tokens: no load (uniform, so no thread skips a barrier)
    if (tid == 0) loss[0] = 0.0f;
    return;
  }
  if (!global) {
    // L_b = alpha * sum_i (E/(K T)) c[b][i] * (S[b][i] / T); loss = mean_b.
    const float f = static_cast<float>(E) / (static_cast<float>(K) * T);
    float acc = 0.0f;
    for (int b = tid; tid < kBalThreads && b < B; b += kBalThreads) {
      float lb = 0.0f;
      for (int i = 0; i < E; ++i) {
        const int64_t o = static_cast<int64_t>(b) * E + i;
        lb += (f * static_cast<float>(counts[o])) * (psum[o] / T);
      }
      acc += alpha * lb;
    }
    if (tid < kBalThreads) part[tid] = acc;
    __syncthreads();
    tree_sum(part, tid);
    if (tid == 0) loss[0] = part[0] / static_cast<float>(B);
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
    if (tid < kBalThreads) part[tid] = term;
    __syncthreads();
    tree_sum(part, tid);
    if (tid == 0) loss[0] = alpha * part[0];
  }
}

__global__ __launch_bounds__(kBalThreads) void balance_loss_kernel(
    const int32_t* __restrict__ counts, const float* __restrict__ psum, int B,
    int T, int E, int K, float alpha, int global, float* __restrict__ loss) {
  balance_loss_body(counts, psum, B, T, E, K, alpha, global, loss);
}

// Partials of 16-token groups -> counts and prob_sums per image, then the
// loss.  With B*E outputs of T/16 groups each, R = 1024 / (B*E) threads
// (a power of two, at most 16) share an output: thread j of output (b, e)
// adds groups j, j + R, ... of image b in order, all its loads issued
// before the first addition (up to kPartBatch per round), and the R sums
// are then added in j order.  Partial rows are E apart, so the threads of
// one j read neighbouring words.  The results also stay in LDS (up to
// kPartLds outputs), where the loss reads them.  Fixed association
// throughout: same bits every call.
constexpr int kPartBatch = 16;
constexpr int kPartLds = 2048;

__device__ inline void balance_from_partials(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c,
    int B, int T, int E, int K, float alpha, int global,
    int32_t* __restrict__ counts, float* __restrict__ psum,
    float* __restrict__ loss) {
  __shared__ float sp[kSeqThreads];
  __shared__ int32_t sc[kSeqThreads];
  __shared__ float lps[kPartLds];
  __shared__ int32_t lcn[kPartLds];
  const int G = T / 16;
  const int64_t outs = static_cast<int64_t>(B) * E;
  int R = 1;
  while (R < 16 && outs * (2 * R) <= kSeqThreads) R *= 2;
  for (int64_t o0 = 0; o0 < outs; o0 += kSeqThreads / R) {
    const int64_t o = o0 + threadIdx.x / R;
    const int j = threadIdx.x % R;
    float s = 0.0f;
    int32_t c = 0;
    if (o < outs) {
      const int64_t b = o / E;
      const int64_t base = b * G * E + (o - b * E);
      for (int g0 = j; g0 < G; g0 += kPartBatch * R) {
        float q[kPartBatch];
        int32_t n[kPartBatch];
#pragma unroll
        for (int u = 0; u < kPartBatch; ++u) {
          const int g = g0 + u * R;
          q[u] = g < G ? part_p[base + static_cast<int64_t>(g) * E] : 0.0f;
          n[u] = g < G ? part_c[base + static_cast<int64_t>(g) * E] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPartBatch; ++u) {
          if (g0 + u * R < G) {
            s += q[u];
            c += n[u];
          }
        }
      }
    }
    sp[threadIdx.x] = s;
    sc[threadIdx.x] = c;
    __syncthreads();
    if (j == 0 && o < outs) {
      for (int i = 1; i < R; ++i) {
        s += sp[threadIdx.x + i];
        c += sc[threadIdx.x + i];
      }
      psum[o] = s;
      counts[o] = c;
      if (o < kPartLds) {
        lps[o] = s;
        lcn[o] = c;
      }
    }
    __syncthreads();
  }
  // The loss from the LDS copies when they hold every output; otherwise it
  // reads what this workgroup just wrote to global memory (a workgroup
  // barrier orders those writes before the reads; the loop ended on one).
  if (outs <= kPartLds)
    balance_loss_body(lcn, lps, B, T, E, K, alpha, global, loss);
  else
    balance_loss_body(counts, psum, B, T, E, K, alpha, global, loss);
}

__global__ __launch_bounds__(kSeqThreads) void balance_partials_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c,
    int B, int T, int E, int K, float alpha, int global,
    int32_t* __restrict__ counts, float* __restrict__ psum,
    float* __restrict__ loss) {
  balance_from_partials(part_p, part_c, B, T, E, K, alpha, global, counts,
                        psum, loss);
}

// The fused routing call's second launch, two workgroups side by side.
// Workgroup 0 finishes the balance statistic from the gate's partials, as
// balance_partials_kernel does.  Workgroup 1 is the permutation's expert
// scan, fed with the gate's per-16-token selection counts (part_c), 16 of
// them per 256-token block: the block counts the permute's count kernel
// would form, so that kernel is not needed.
__global__ __launch_bounds__(kSeqThreads) void route_finish_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c,
    int B, int T, int E, int K, float alpha, int global,
    int32_t* __restrict__ counts, float* __restrict__ psum,
    float* __restrict__ loss, int32_t* __restrict__ expert_counts,
    int64_t* __restrict__ expert_offsets, int64_t* __restrict__ block_base) {
  static_assert(kSeqThreads == kScanThreads && kPermTokens % 16 == 0,
                "one workgroup size; whole 16-token groups per block");
  if (blockIdx.x == 0) {
    balance_from_partials(part_p, part_c, B, T, E, K, alpha, global, counts,
                          psum, loss);
  } else {
    const int64_t N = static_cast<int64_t>(B) * T;
    const int nblocks = static_cast<int>(ceil_div(N, kPermTokens));
    expert_scan<kPermTokens / 16>(part_c, nblocks, N / 16, E, expert_counts,
                expert_offsets, block_base);
  }
}

}  // namespace

size_t balance_partials_bytes(int64_t N, int E) {
  const size_t words = static_cast<size_t>((N + 15) / 16) * E;
  const size_t half = (words * 4 + 255) / 256 * 256;
  return 2 * half;
}

hipError_t launch_route_finish(const void* partials, int B, int T, int E,
                               int K, float alpha, bool global, int32_t* counts,
                               float* psum, float* loss, int32_t* expert_counts,
                               int64_t* expert_offsets, int64_t* block_base,
                               hipStream_t stream) {
  const int64_t N = static_cast<int64_t>(B) * T;
  const float* part_p = static_cast<const float*>(partials);
  const int32_t* part_c = reinterpret_cast<const int32_t*>(
      static_cast<const char*>(partials) + balance_partials_bytes(N, E) / 2);
  hipLaunchKernelGGL(route_finish_kernel, dim3(2), dim3(kSeqThreads), 0, stream,
                     part_p, part_c, B, T, E, K, alpha, global ? 1 : 0, counts,
                     psum, loss, expert_counts, expert_offsets, block_base);
  return hipGetLastError();
}

hipError_t launch_balance_from_partials(const void* partials, int B, int T,
                                        int E, int K, float alpha, bool global,
                                        int32_t* counts, float* psum,
                                        float* loss, hipStream_t stream) {
  const int64_t N = static_cast<int64_t>(B) * T;
  const float* part_p = static_cast<const float*>(partials);
  const int32_t* part_c = reinterpret_cast<const int32_t*>(
      static_cast<const char*>(partials) + balance_partials_bytes(N, E) / 2);
  hipLaunchKernelGGL(balance_partials_kernel, dim3(1), dim3(kSeqThreads), 0,
                     stream, part_p, part_c, B, T, E, K, alpha, global ? 1 : 0,
                     counts, psum, loss);
  return hipGetLastError();
}

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
