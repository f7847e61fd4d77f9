// The permutation's expert scan, shared by the permute's own scan kernel and
// the fused routing call's finish kernel.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE recap: only
// the selected experts are evaluated, so the selected (token, slot) pairs are
// grouped by expert, each expert's rows in ascending token order.  From the
// selection counts of every token block this computes each expert's count and
// row offset and, for every block, the first row of each expert's selections
// in it; the scatter then ranks the selections inside the block.
#pragma once

#include "common.hpp"

namespace moe {

// Tokens per permutation block (one thread per token in the count and
// scatter kernels) and the scan's threads.
constexpr int kPermTokens = 256;
constexpr int kScanThreads = 1024;

// Selections of expert e in token block b.  The counts come as GPB
// consecutive groups per block, ngroups in all (GPB = 1: one count per
// block).  Integer sums: the grouping does not change the result.  The GPB
// loads are independent, so they are in flight together (the counts were
// just written by another kernel, so each load may go past the L2).
template <int GPB>
__device__ __forceinline__ int64_t block_count(const int32_t* __restrict__ cnt,
                                               int64_t b, int e, int E,
                                               int64_t ngroups) {
  // groups past the end re-read the last one (no branch around the loads)
  // and count zero; a block holds at most 256 x 64 selections, so the sum
  // fits int32
  int32_t v[GPB];
#pragma unroll
  for (int u = 0; u < GPB; ++u) {
    const int64_t g = b * GPB + u;
    v[u] = cnt[(g < ngroups ? g : ngroups - 1) * E + e];
  }
  int32_t s = 0;
#pragma unroll
  for (int u = 0; u < GPB; ++u)
    if (b * GPB + u < ngroups) s += v[u];
  return s;
}

// Called by all kScanThreads threads of one workgroup, with GPB count
// groups per block.  Thread (c, e) of a C x E grid (C = kScanThreads / E
// chunks of consecutive blocks) sums its chunk's counts of expert e; a scan
// over the chunks in LDS gives each chunk its base within the expert, a scan
// over the experts gives the expert offsets, and each thread then writes the
// block bases of its chunk in block order:
//   counts[e] (int32), offsets[e] (exclusive, offsets[E] = total),
//   block_base[b][e] = offsets[e] + selections of e in blocks before b.
template <int GPB>
__device__ inline void expert_scan(const int32_t* __restrict__ cnt,
                                   int nblocks, int64_t ngroups,
                                   int E, int32_t* __restrict__ counts,
                                   int64_t* __restrict__ offsets,
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
    for (int b = b0; b < b1; ++b) sum += block_count<GPB>(cnt, b, e, E, ngroups);
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
    run += block_count<GPB>(cnt, b, e, E, ngroups);
  }
}

}  // namespace moe
