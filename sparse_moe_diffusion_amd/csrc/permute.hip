// Token permutation by expert for the DiT-MoE layer.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE recap: with
// a sparse router only the selected experts are evaluated.  The selected
// (token, slot) pairs are grouped by expert so that each expert's MLP runs
// as one dense row block.  Rows of expert e are its selections in ascending
// (token, slot) order.
//
// Three launches (a fourth with x_perm), no host synchronisation:
//  1. permute_count_kernel: workgroup b covers 256 consecutive tokens (one
//     per thread); the block's slots are read into LDS together, each
//     token's experts form a bit mask, and one wave ballot per expert counts
//     the wave's selections.  Writes block_counts[b][e].
//  2. permute_scan_kernel: one 1024-thread workgroup scans the block counts
//     (chunks of blocks x experts, then a scan over chunks and experts):
//     expert counts, exclusive offsets and block bases.
//  3. permute_scatter_kernel: repeats the slot read and the ballots (one per
//     expert, kept in LDS), so each slot's row is block base (read once into
//     LDS) + earlier waves' count + set lanes below it in its expert's
//     ballot; writes row_token and the block's slot_row (coalesced, from
//     LDS).
//  4. permute_copy_kernel (only with x_perm): one thread per 16-byte chunk
//     of every token row reads the chunk once and writes it to the token's
//     selected rows; consecutive threads cover consecutive chunks, so both
//     the reads and the writes are row-contiguous, and the grid is large
//     enough to keep every CU streaming.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace moe {

namespace {

constexpr int kPermWaves = kPermTokens / kWave;

// The block's slots, idx[t0 .. t0 + ntok) (ntok Kmax values, contiguous),
// into s_rows: consecutive threads read consecutive values, 8 loads in
// flight per thread (past the end they re-read the last value and are not
// stored, so no branch separates the loads).  Then each thread's own Kmax
// slots are sanitised in place (outside [0, E), or a token past N: -1) and
// their experts returned as a bit mask.  Called by every thread of the
// block; ends with the slots in place for this thread only.
constexpr int kSlotLoads = 8;
__device__ __forceinline__ uint64_t block_slots(const int32_t* __restrict__ idx,
                                                int64_t t0, int ntok, int Kmax,
                                                int E, int32_t* s_rows) {
  const int n = ntok * Kmax;
  const int32_t* const src = idx + t0 * Kmax;
  for (int i0 = 0; i0 < n; i0 += kPermTokens * kSlotLoads) {
    int32_t v[kSlotLoads];
#pragma unroll
    for (int u = 0; u < kSlotLoads; ++u) {
      const int i = i0 + u * kPermTokens + static_cast<int>(threadIdx.x);
      v[u] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kSlotLoads; ++u) {
      const int i = i0 + u * kPermTokens + static_cast<int>(threadIdx.x);
      if (i < n) s_rows[i] = v[u];
    }
  }
  __syncthreads();
  int32_t* const my = s_rows + threadIdx.x * Kmax;
  const bool valid = static_cast<int>(threadIdx.x) < ntok;
  uint64_t m = 0;
  for (int k = 0; k < Kmax; ++k) {
    const int e = valid ? my[k] : -1;
    const bool ok = e >= 0 && e < E;   // contents outside [0, E): empty
    my[k] = ok ? e : -1;
    if (ok) m |= 1ull << e;
  }
  return m;
}

__global__ __launch_bounds__(kPermTokens) void permute_count_kernel(
    const int32_t* __restrict__ idx, int64_t N, int E, int Kmax,
    int32_t* __restrict__ block_counts) {
  extern __shared__ int32_t s_rows[];  // [kPermTokens][Kmax]
  __shared__ int32_t wc[kPermWaves][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPermTokens;
  const int ntok = static_cast<int>(min<int64_t>(kPermTokens, N - t0));
  const uint64_t m = block_slots(idx, t0, ntok, Kmax, E, s_rows);
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

// One workgroup: expert counts, offsets and block bases from the block
// counts (see expert_scan).
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    const int32_t* __restrict__ block_counts, int nblocks, int E,
    int32_t* __restrict__ counts, int64_t* __restrict__ offsets,
    int64_t* __restrict__ block_base) {
  expert_scan<1>(block_counts, nblocks, nblocks, E, counts, offsets, block_base);
}

__global__ __launch_bounds__(kPermTokens) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t N, int E, int Kmax, int64_t A,
    const int64_t* __restrict__ block_base, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token) {
  extern __shared__ int32_t s_rows[];  // [kPermTokens][Kmax]
  __shared__ int32_t wc[kPermWaves][kMaxExperts];
  __shared__ uint64_t wb[kPermWaves][kMaxExperts];
  __shared__ int64_t sbase[kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPermTokens;
  const int64_t t = t0 + threadIdx.x;
  const int ntok = static_cast<int>(min<int64_t>(kPermTokens, N - t0));
  // the block's first row of each expert, read once (the expert loop below
  // would otherwise wait on one global load per expert)
  if (static_cast<int>(threadIdx.x) < E)
    sbase[threadIdx.x] = block_base[static_cast<int64_t>(blockIdx.x) * E + threadIdx.x];
  // the token's slots, sanitised, in s_rows (see block_slots; its barrier
  // also orders sbase)
  const uint64_t m = block_slots(idx, t0, ntok, Kmax, E, s_rows);
  // One ballot per expert (taken by the whole wave), kept with its count.
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot((m >> e) & 1ull);
    if (lane == 0) {
      wc[wave][e] = __popcll(b);
      wb[wave][e] = b;
    }
  }
  __syncthreads();
  // Each slot naming expert e takes row block base + earlier waves' count +
  // set lanes below it in the wave's ballot of e (a token naming e twice
  // gets the same row in both slots).  Slots naming no valid expert, and
  // rows past A, keep -1.
  int32_t* const my = s_rows + threadIdx.x * Kmax;
  for (int k = 0; k < Kmax; ++k) {
    const int e = my[k];
    if (e < 0) continue;
    int64_t r = sbase[e] + lanes_below(wb[wave][e]);
    for (int w = 0; w < wave; ++w) r += wc[w][e];
    const int32_t row = (r < A) ? static_cast<int32_t>(r) : -1;
    my[k] = row;
    if (row >= 0) row_token[row] = static_cast<int32_t>(t);
  }
  __syncthreads();
  // slot_row of the block's tokens, coalesced.
  for (int i = threadIdx.x; i < ntok * Kmax; i += kPermTokens)
    slot_row[t0 * Kmax + i] = s_rows[i];
}

// x_perm[slot_row[t][k]] = x[t] for every slot k >= 0 of token t, 16 bytes
// per thread: thread i copies chunk i % nvec of token i / nvec.  The token's
// slot rows are read once per thread (the same few words for the nvec
// threads of a token, served by the caches).
__global__ __launch_bounds__(256) void permute_copy_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ slot_row,
    int64_t N, int nvec, int Kmax, uint4* __restrict__ x_perm) {
  const int64_t n = N * nvec;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / nvec;
    const int c = static_cast<int>(i - t * nvec);
    const uint4 v = x[i];
    for (int k = 0; k < Kmax; ++k) {
      const int32_t r = slot_row[t * Kmax + k];
      if (r >= 0) x_perm[static_cast<int64_t>(r) * nvec + c] = v;
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

// ------------------------------------------------ allocation-free variant --
// moe_permute_noalloc keeps the block counts and block bases in this array
// instead of a caller's workspace.  Each device holds its own copy for the
// life of the process.  On the host the array's name only stands in for the
// device copies and is never passed to a kernel: permute_scratch() returns
// the current device's address, looked up once per device.
constexpr size_t kPermScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kPermScratchBytes];

size_t permute_scratch_bytes() { return kPermScratchBytes; }

hipError_t permute_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

namespace {

// Dynamic LDS of the count and scatter kernels: the block's slots.  Past
// 32 KB (Kmax > 32) the kernel must opt in.
size_t slots_lds(int Kmax) {
  return static_cast<size_t>(kPermTokens) * Kmax * sizeof(int32_t);
}

hipError_t opt_in_lds(const void* kernel, size_t shmem) {
  if (shmem <= 32768) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(shmem));
}

}  // namespace

hipError_t launch_permute_scatter(const int32_t* idx, int64_t N, int E,
                                  int Kmax, int64_t A, const int64_t* block_base,
                                  int32_t* slot_row, int32_t* row_token,
                                  hipStream_t stream) {
  const int64_t nb = ceil_div(N, kPermTokens);
  if (nb == 0) return hipSuccess;
  const size_t shmem = slots_lds(Kmax);
  const hipError_t err = opt_in_lds(
      reinterpret_cast<const void*>(&permute_scatter_kernel), shmem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(static_cast<unsigned>(nb)),
                     dim3(kPermTokens), shmem, stream, idx, N, E, Kmax, A,
                     block_base, slot_row, row_token);
  return hipGetLastError();
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
    const size_t shmem = slots_lds(Kmax);
    hipError_t err = opt_in_lds(
        reinterpret_cast<const void*>(&permute_count_kernel), shmem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_count_kernel, dim3(static_cast<unsigned>(nb)),
                       dim3(kPermTokens), shmem, stream, idx, N, E, Kmax,
                       block_counts);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                     block_counts, static_cast<int>(nb), E, counts, offsets,
                     block_base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_permute_scatter(idx, N, E, Kmax, A, block_base, slot_row,
                               row_token, stream);
  if (err != hipSuccess || nb == 0 || x_perm == nullptr) return err;
  // D is a multiple of 8, so a row is a whole number of 16-byte chunks.
  const int nvec = D * (bf16 ? 2 : 4) / 16;
  const int64_t chunks = N * nvec;
  const unsigned grid =
      static_cast<unsigned>(std::min<int64_t>(ceil_div(chunks, 256), 16384));
  hipLaunchKernelGGL(permute_copy_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint4*>(x), slot_row, N, nvec, Kmax,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
