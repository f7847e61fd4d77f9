// Token permutation by expert for the DiT-MoE layer.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE recap: with
// a sparse router only the selected experts are evaluated.  The selected
// (token, slot) pairs are grouped by expert so that each expert's MLP runs
// as one dense row block.  Rows of expert e are its selections in ascending
// (token, slot) order.
//
// Three launches, no host synchronisation:
//  1. permute_count_kernel: workgroup b covers 256 consecutive tokens (one
//     per thread); each token's experts form a bit mask, and one wave ballot
//     per expert counts the wave's selections.  Writes block_counts[b][e].
//  2. permute_scan_kernel: one 1024-thread workgroup scans the block counts
//     (chunks of blocks x experts, then a scan over chunks and experts):
//     expert counts, exclusive offsets and block bases.
//  3. permute_scatter_kernel: repeats the ballots (one per expert), so a
//     selection's row is block base + earlier waves' count + set lanes below
//     it; writes row_token, the block's slot_row (coalesced, from LDS), then
//     copies each token row once from HBM to its K destination rows with
//     16-byte lanes (row copy skipped when x_perm is null).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPermTokens = 256;
constexpr int kPermWaves = kPermTokens / kWave;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ uint64_t token_mask(const int32_t* __restrict__ idx,
                                               int64_t t, int Kmax, int E) {
  uint64_t m = 0;
  for (int k = 0; k < Kmax; ++k) {
    const int e = idx[t * Kmax + k];
    if (e >= 0 && e < E) m |= 1ull << e;
  }
  return m;
}

__global__ __launch_bounds__(kPermTokens) void permute_count_kernel(
    const int32_t* __restrict__ idx, int64_t N, int E, int Kmax,
    int32_t* __restrict__ block_counts) {
  __shared__ int32_t wc[kPermWaves][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermTokens + threadIdx.x;
  const uint64_t m = (t < N) ? token_mask(idx, t, Kmax, E) : 0ull;
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot((m >> e) & 1ull);
    if (lane == 0) wc[wave][e] = __popcll(b);
  }
  __syncthreads();
  if (threadIdx.x < E) {
    int32_t c = 0;
    for (int w = 0; w < kPermWaves; ++w) c += wc[w][threadIdx.x];
    block_counts[static_cast<int64_t>(blockIdx.x) * E + threadIdx.x] = c;
  }
}

// Thread (c, e) of a C x E grid (C = 1024 / E chunks of consecutive count
// blocks) sums its chunk's counts of expert e; a scan over the chunks in
// LDS gives each chunk its base within the expert, a scan over the experts
// gives the expert offsets, and each thread then writes the block bases of
// its chunk in block order.
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    const int32_t* __restrict__ block_counts, int nblocks, int E,
    int32_t* __restrict__ counts, int64_t* __restrict__ offsets,
    int64_t* __restrict__ block_base) {
  __shared__ int64_t part[kScanThreads];
  __shared__ int64_t tot[kMaxExperts];
  const int C = kScanThreads / E;
  const int tid = threadIdx.x;
  const int c = tid / E;
  const int e = tid - c * E;
  const bool active = c < C;
  const int b0 = static_cast<int>(static_cast<int64_t>(c) * nblocks / C);
  const int b1 = static_cast<int>(static_cast<int64_t>(c + 1) * nblocks / C);
  int64_t sum = 0;
  if (active)
    for (int b = b0; b < b1; ++b)
      sum += block_counts[static_cast<int64_t>(b) * E + e];
  part[tid] = sum;
  __syncthreads();
  // inclusive scan over chunks, per expert (Hillis-Steele)
  for (int off = 1; off < C; off *= 2) {
    int64_t v = part[tid];
    if (active && c >= off) v += part[tid - off * E];
    __syncthreads();
    part[tid] = v;
    __syncthreads();
  }
  if (active && c == C - 1) tot[e] = part[tid];
  __syncthreads();
  if (!active) return;
  int64_t base = 0;
  for (int j = 0; j < e; ++j) base += tot[j];
  if (c == 0) {
    counts[e] = static_cast<int32_t>(tot[e]);
    offsets[e] = base;
    if (e == E - 1) offsets[E] = base + tot[e];
  }
  int64_t run = base + (c > 0 ? part[tid - E] : 0);
  for (int b = b0; b < b1; ++b) {
    block_base[static_cast<int64_t>(b) * E + e] = run;
    run += block_counts[static_cast<int64_t>(b) * E + e];
  }
}

template <int VEC_BYTES>
__global__ __launch_bounds__(kPermTokens) void permute_scatter_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ idx, int64_t N,
    int row_bytes, int E, int Kmax, int64_t A,
    const int64_t* __restrict__ block_base, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token, void* __restrict__ x_perm) {
  extern __shared__ int32_t s_rows[];  // [kPermTokens][Kmax]
  __shared__ int32_t wc[kPermWaves][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPermTokens;
  const int64_t t = t0 + threadIdx.x;
  const bool valid = t < N;
  const uint64_t m = valid ? token_mask(idx, t, Kmax, E) : 0ull;
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot((m >> e) & 1ull);
    if (lane == 0) wc[wave][e] = __popcll(b);
  }
  __syncthreads();
  const int64_t* base = block_base + static_cast<int64_t>(blockIdx.x) * E;
  // The token's slots, then one ballot per expert (taken by the whole
  // wave): a lane holding expert ee finds its rank and writes it into the
  // slot that names ee.  Slots naming no valid expert keep -1.
  int32_t* const my = s_rows + threadIdx.x * Kmax;
  for (int k = 0; k < Kmax; ++k) {
    const int v = valid ? idx[t * Kmax + k] : -1;
    my[k] = (v >= 0 && v < E) ? v : -1;   // contents outside [0, E): empty
  }
  for (int ee = 0; ee < E; ++ee) {
    const bool has = (m >> ee) & 1ull;
    const uint64_t b = __ballot(has);
    if (has) {
      int64_t r = base[ee] + lanes_below(b);
      for (int w = 0; w < wave; ++w) r += wc[w][ee];
      const int32_t row = (r < A) ? static_cast<int32_t>(r) : -1;
      for (int k = 0; k < Kmax; ++k)
        if (my[k] == ee) my[k] = -2 - row;   // marked: no longer an expert
      if (row >= 0) row_token[row] = static_cast<int32_t>(t);
    }
  }
  // Marked slots hold -2 - row; the rest (empty or invalid) become -1.
  for (int k = 0; k < Kmax; ++k) my[k] = my[k] <= -2 ? -2 - my[k] : -1;
  __syncthreads();
  // slot_row of the block's tokens, coalesced.
  const int ntok = static_cast<int>(min<int64_t>(kPermTokens, N - t0));
  for (int i = threadIdx.x; i < ntok * Kmax; i += kPermTokens)
    slot_row[t0 * Kmax + i] = s_rows[i];
  if (x_perm == nullptr) return;

  // Row copy: each wave takes tokens wave, wave+4, ...; lanes cover the row
  // in VEC_BYTES pieces.
  typedef uint4 vec_t;
  static_assert(VEC_BYTES == 16, "16-byte lanes");
  const int nvec = row_bytes / VEC_BYTES;
  const char* xb = static_cast<const char*>(x);
  char* pb = static_cast<char*>(x_perm);
  for (int tl = wave; tl < ntok; tl += kPermWaves) {
    const vec_t* src = reinterpret_cast<const vec_t*>(xb + (t0 + tl) * row_bytes);
    for (int c = lane; c < nvec; c += kWave) {
      const vec_t v = src[c];
      for (int k = 0; k < Kmax; ++k) {
        const int32_t r = s_rows[tl * Kmax + k];
        if (r >= 0)
          reinterpret_cast<vec_t*>(pb + static_cast<int64_t>(r) * row_bytes)[c] = v;
      }
    }
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t N, int E) {
  const int64_t nb = ceil_div(N, kPermTokens);
  // block_counts (int32) + block_base (int64), each [nb][E], 256-B aligned
  const size_t a = ((nb * E * sizeof(int32_t)) + 255) / 256 * 256;
  return a + nb * E * sizeof(int64_t) + 256;
}

hipError_t launch_permute(const void* x, bool bf16, const int32_t* idx,
                          int64_t N, int D, int E, int Kmax, int64_t A,
                          int32_t* counts, int64_t* offsets, int32_t* row_token,
                          int32_t* slot_row, void* x_perm, void* workspace,
                          hipStream_t stream) {
  const int64_t nb = ceil_div(N, kPermTokens);
  int32_t* block_counts = static_cast<int32_t*>(workspace);
  const size_t a = ((nb * E * sizeof(int32_t)) + 255) / 256 * 256;
  int64_t* block_base =
      reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + a);
  if (nb > 0) {
    hipLaunchKernelGGL(permute_count_kernel, dim3(static_cast<unsigned>(nb)),
                       dim3(kPermTokens), 0, stream, idx, N, E, Kmax,
                       block_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                     block_counts, static_cast<int>(nb), E, counts, offsets,
                     block_base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nb == 0) return err;
  const int row_bytes = D * (bf16 ? 2 : 4);
  const size_t shmem = static_cast<size_t>(kPermTokens) * Kmax * sizeof(int32_t);
  if (shmem > 32768) {
    err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&permute_scatter_kernel<16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_scatter_kernel<16>, dim3(static_cast<unsigned>(nb)),
                     dim3(kPermTokens), shmem, stream, x, idx, N, row_bytes, E,
                     Kmax, A, block_base, slot_row, row_token, x_perm);
  return hipGetLastError();
}

}  // namespace moe
