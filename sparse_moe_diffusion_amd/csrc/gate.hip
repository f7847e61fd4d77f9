// Gate scores, softmax and expert selection for the DiT-MoE layer.
//
// "DiT-MoE" project hub page, section 1 (MoE gate routing): a [E][D] gate
// weight scores every token against the routed experts, a softmax turns the
// scores into probabilities and the top-k experts are kept.  "Expert Race"
// (abstract): tokens and experts compete in one pool for the top
// candidates.
//
// Kernel layout (gfx950):
//  * gate_kernel: one workgroup = 64 tokens (one per lane) x 4 waves; wave w
//    accumulates the fp32 logits of its 64 tokens over the w-th quarter of
//    the features.  Gate weights are wave-uniform and arrive through scalar
//    loads; each lane streams its own token row with 16-byte loads.  The
//    four partial sums meet in LDS in a fixed order, then wave 0 runs the
//    softmax and the top-K selection in registers (ties: lower index).
//  * race_select_kernel: one 1024-thread workgroup finds the exact K*N-th
//    largest probability key by an MSB-first radix select (4 passes of 8
//    bits, per-wave LDS histograms) and the flat index of the last kept
//    entry among keys equal to it.
//  * race_emit_kernel: one thread per token writes its kept experts in
//    ascending order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kGateTokens = 64;
constexpr int kGateWaves = 4;

template <bool BF16>
__device__ __forceinline__ void load_x8(const void* x, int64_t row, int D,
                                        int chunk, float* f) {
  if constexpr (BF16) {
    const uint4 v =
        reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) +
                                       row * D)[chunk];
    unpack8(v, f);
  } else {
    const float4* p = reinterpret_cast<const float4*>(
        static_cast<const float*>(x) + row * D) + 2 * chunk;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// Selection key of a probability: NaN ranks below every number.
__device__ __forceinline__ float sel_key(float p) { return p == p ? p : -1.0f; }

template <int EP, bool BF16>
__global__ __launch_bounds__(kGateTokens * kGateWaves) void gate_kernel(
    const void* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ bias, int64_t N, int D, int E, int K, int topk,
    float* __restrict__ probs, int32_t* __restrict__ idx,
    float* __restrict__ wout) {
  __shared__ float part[kGateWaves][EP][kGateTokens];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kGateTokens + lane;
  const bool valid = t < N;
  const int nchunk = D / 8;
  const int c0 = wave * nchunk / kGateWaves;
  const int c1 = (wave + 1) * nchunk / kGateWaves;

  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0f;

  if (valid) {
#pragma unroll 2
    for (int c = c0; c < c1; ++c) {
      float xf[8];
      load_x8<BF16>(x, t, D, c, xf);
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        if (e < E) {
          const float* w = wg + static_cast<int64_t>(e) * D + 8 * c;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[e] = fmaf(xf[j], w[j], acc[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) part[wave][e][lane] = acc[e];
  __syncthreads();
  if (wave != 0 || !valid) return;

  float p[EP];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    if (e < E) {
      float l = part[0][e][lane] + part[1][e][lane];
      l += part[2][e][lane];
      l += part[3][e][lane];
      if (bias != nullptr) l += bias[e];
      p[e] = l;
      m = fmaxf(m, l);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    if (e < E) {
      p[e] = expf(p[e] - m);
      s += p[e];
    }
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    if (e < E) {
      p[e] = p[e] / s;
      probs[t * E + e] = p[e];
    }
  }
  if (!topk) return;

  uint64_t taken = 0;
  for (int k = 0; k < K; ++k) {
    int best = -1;
    float bkey = 0.0f, bp = 0.0f;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      if (e < E && !((taken >> e) & 1ull)) {
        const float key = sel_key(p[e]);
        if (best < 0 || key > bkey) {
          best = e;
          bkey = key;
          bp = p[e];
        }
      }
    }
    taken |= 1ull << best;
    idx[t * K + k] = best;
    wout[t * K + k] = bp;
  }
}

// ---------------------------------------------------------- Expert Race --

constexpr int kRaceThreads = 1024;
constexpr int kRaceWaves = kRaceThreads / kWave;

// Order-preserving key of a probability: the fp32 bit pattern of a
// non-negative float orders like its value.  NaN and negatives map to 0.
__device__ __forceinline__ uint32_t race_key(float p) {
  return (p > 0.0f) ? __float_as_uint(p) : 0u;
}

// out[0] = threshold key tau, out[1] = flat index of the last kept entry
// whose key equals tau.  Entries with key > tau, or key == tau and flat
// index <= out[1], are kept: exactly A of them.
__global__ __launch_bounds__(kRaceThreads) void race_select_kernel(
    const float* __restrict__ probs, int64_t total, int64_t A,
    uint32_t* __restrict__ out) {
  __shared__ uint32_t hist[kRaceWaves][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t s_prefix, s_mask, s_need;
  __shared__ uint32_t wcnt[kRaceWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (tid == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_need = static_cast<uint32_t>(A);
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kRaceWaves * 256; i += kRaceThreads)
      (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int64_t i = tid; i < total; i += kRaceThreads) {
      const uint32_t k = race_key(probs[i]);
      if ((k & mask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
      for (int w = 0; w < kRaceWaves; ++w) c += hist[w][tid];
      tot[tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t need = s_need, above = 0;
      int digit = 0;
      for (int d = 255; d >= 0; --d) {
        if (above + tot[d] >= need) {
          digit = d;
          break;
        }
        above += tot[d];
      }
      s_need = need - above;
      s_prefix = prefix | (static_cast<uint32_t>(digit) << shift);
      s_mask = mask | (255u << shift);
    }
    __syncthreads();
  }
  // The s_need-th (1-based) entry equal to tau in flat order is the last
  // one kept.  Walk the keys in tiles of 1024 flat entries.
  const uint32_t tau = s_prefix;
  const uint32_t need = s_need;
  uint32_t running = 0;
  for (int64_t base = 0; base < total; base += kRaceThreads) {
    const int64_t i = base + tid;
    const bool eq = (i < total) && race_key(probs[i]) == tau;
    const uint64_t bal = __ballot(eq);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    uint32_t before = 0, tile = 0;
    for (int w = 0; w < kRaceWaves; ++w) {
      if (w < wave) before += wcnt[w];
      tile += wcnt[w];
    }
    if (running + tile >= need) {
      const uint32_t rank = running + before + lanes_below(bal);
      if (eq && rank + 1 == need) {
        out[0] = tau;
        out[1] = static_cast<uint32_t>(i);
      }
      return;
    }
    running += tile;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void race_emit_kernel(
    const float* __restrict__ probs, int64_t N, int E,
    const uint32_t* __restrict__ sel, int32_t* __restrict__ idx,
    float* __restrict__ w) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const uint32_t tau = sel[0];
  const int64_t cut = sel[1];
  int n = 0;
  for (int e = 0; e < E; ++e) {
    const float p = probs[t * E + e];
    const uint32_t k = race_key(p);
    const int64_t flat = t * E + e;
    if (k > tau || (k == tau && flat <= cut)) {
      idx[t * E + n] = e;
      w[t * E + n] = p;
      ++n;
    }
  }
  for (; n < E; ++n) {
    idx[t * E + n] = -1;
    w[t * E + n] = 0.0f;
  }
}

template <int EP>
hipError_t launch_gate_ep(const void* x, bool bf16, const float* wg,
                          const float* bias, int64_t N, int D, int E, int K,
                          bool topk, float* probs, int32_t* idx, float* w,
                          hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kGateTokens)));
  const dim3 block(kGateTokens * kGateWaves);
  if (bf16)
    hipLaunchKernelGGL((gate_kernel<EP, true>), grid, block, 0, stream, x, wg,
                       bias, N, D, E, K, topk ? 1 : 0, probs, idx, w);
  else
    hipLaunchKernelGGL((gate_kernel<EP, false>), grid, block, 0, stream, x,
                       wg, bias, N, D, E, K, topk ? 1 : 0, probs, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const float* w_gate,
                       const float* bias, int64_t N, int D, int E, int K,
                       bool topk, float* probs, int32_t* idx, float* w,
                       hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (E <= 8)
    return launch_gate_ep<8>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                             idx, w, stream);
  if (E <= 16)
    return launch_gate_ep<16>(x, x_bf16, w_gate, bias, N, D, E, K, topk,
                              probs, idx, w, stream);
  if (E <= 32)
    return launch_gate_ep<32>(x, x_bf16, w_gate, bias, N, D, E, K, topk,
                              probs, idx, w, stream);
  return launch_gate_ep<64>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                            idx, w, stream);
}

size_t race_workspace_bytes() { return 256; }

hipError_t launch_race(const float* probs, int64_t N, int E, int K,
                       int32_t* idx, float* w, void* workspace,
                       hipStream_t stream) {
  if (N == 0) return hipSuccess;
  uint32_t* sel = static_cast<uint32_t*>(workspace);
  hipLaunchKernelGGL(race_select_kernel, dim3(1), dim3(kRaceThreads), 0,
                     stream, probs, N * E, static_cast<int64_t>(K) * N, sel);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(race_emit_kernel,
                     dim3(static_cast<unsigned>(ceil_div(N, 256))), dim3(256),
                     0, stream, probs, N, E, sel, idx, w);
  return hipGetLastError();
}

}  // namespace moe
