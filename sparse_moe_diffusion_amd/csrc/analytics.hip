// Routing analytics: expert-selection counts by patch position and by a
// per-image tag.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", Expert
// Specialization Analysis: the frequency with which each expert is selected,
// seen by spatial position, by image class and by denoising time step
// (heatmaps of figures 5-7); "DiT-MoE" project hub page, section 4 (analysis
// tools).  The counts of one batch are added into caller-owned totals, so a
// sweep over many batches (classes, sampling steps) accumulates on the
// device.
//
// Kernel layout (gfx950): a workgroup owns 64 positions x 8 images.  Each
// thread takes one position of several images and adds every valid slot
// into two LDS histograms (by position, by image of the block) with LDS
// atomics; the block's non-zero counts then go to the totals with 64-bit
// global integer atomics.  Integer addition is exact in any order, so the
// result does not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kHistPos = 64;       // positions per workgroup (one per lane)
constexpr int kHistImgs = 8;       // images per workgroup
constexpr int kHistThreads = 256;

__global__ __launch_bounds__(kHistThreads) void routing_hist_kernel(
    const int32_t* __restrict__ idx, int B, int T, int E, int Kmax,
    const int32_t* __restrict__ tags, int n_tags,
    unsigned long long* __restrict__ pos_counts,
    unsigned long long* __restrict__ tag_counts) {
  __shared__ uint32_t hp[kHistPos][kMaxExperts];
  __shared__ uint32_t ht[kHistImgs][kMaxExperts];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * kHistPos;
  const int b0 = blockIdx.y * kHistImgs;
  for (int i = tid; i < kHistPos * kMaxExperts; i += kHistThreads)
    (&hp[0][0])[i] = 0;
  for (int i = tid; i < kHistImgs * kMaxExperts; i += kHistThreads)
    (&ht[0][0])[i] = 0;
  __syncthreads();

  const int pl = tid % kHistPos;
  const int p = p0 + pl;
  for (int bl = tid / kHistPos; bl < kHistImgs; bl += kHistThreads / kHistPos) {
    const int b = b0 + bl;
    if (p < T && b < B) {
      const int32_t* row = idx + (static_cast<int64_t>(b) * T + p) * Kmax;
      for (int k = 0; k < Kmax; ++k) {
        const int e = row[k];
        if (e >= 0 && e < E) {
          atomicAdd(&hp[pl][e], 1u);
          atomicAdd(&ht[bl][e], 1u);
        }
      }
    }
  }
  __syncthreads();

  for (int i = tid; i < kHistPos * E; i += kHistThreads) {
    const int l = i / E, e = i - l * E;
    const uint32_t c = hp[l][e];
    if (p0 + l < T && c != 0)
      atomicAdd(&pos_counts[static_cast<int64_t>(p0 + l) * E + e],
                static_cast<unsigned long long>(c));
  }
  if (tags == nullptr) return;
  for (int i = tid; i < kHistImgs * E; i += kHistThreads) {
    const int l = i / E, e = i - l * E;
    const int b = b0 + l;
    if (b >= B) continue;
    const int g = tags[b];
    const uint32_t c = ht[l][e];
    if (g >= 0 && g < n_tags && c != 0)
      atomicAdd(&tag_counts[static_cast<int64_t>(g) * E + e],
                static_cast<unsigned long long>(c));
  }
}

}  // namespace

hipError_t launch_routing_hist(const int32_t* idx, int B, int T, int E,
                               int Kmax, const int32_t* tags, int n_tags,
                               int64_t* pos_counts, int64_t* tag_counts,
                               hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kHistPos)),
                  static_cast<unsigned>(ceil_div(B, kHistImgs)));
  hipLaunchKernelGGL(routing_hist_kernel, grid, dim3(kHistThreads), 0, stream,
                     idx, B, T, E, Kmax, tags, n_tags,
                     reinterpret_cast<unsigned long long*>(pos_counts),
                     reinterpret_cast<unsigned long long*>(tag_counts));
  return hipGetLastError();
}

}  // namespace moe
