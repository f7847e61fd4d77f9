// Gate scores, softmax and expert selection for the DiT-MoE layer.
//
// "DiT-MoE" project hub page, section 1 (MoE gate routing): a [E][D] gate
// weight scores every token against the routed experts, a softmax turns the
// scores into probabilities and the top-k experts are kept.  "Expert Race"
// (abstract): tokens and experts compete in one pool for the top
// candidates.
//
// Kernel layout (gfx950):
//  * gate_mfma_kernel (bf16 tokens): logits on the matrix cores from an
//    exact three-way bf16 split of the fp32 gate weights, partial sums
//    added in fp64; see the kernel.  gate_f32_kernel (fp32 tokens): the same
//    logits from VALU fp64 FMAs.  Both leave 64 tokens' logits in LDS after
//    a fixed-order sum over 4 waves, and wave 0 runs the fp32 softmax and the
//    top-K selection in registers, one token per lane (ties: lower index).
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
constexpr int kGateChunk = 5;   // 32-wide k slices loaded ahead per wave
constexpr int kGateGroups = 4;  // 16-token groups per workgroup (MFMA path)

// Selection key of a probability: NaN ranks below every number.
__device__ __forceinline__ float sel_key(float p) { return p == p ? p : -1.0f; }

// Softmax over the E logits of one token (one lane) and, for top-K routing,
// the K experts first in (probability descending, index ascending) order.
template <int EP>
__device__ __forceinline__ void softmax_topk(float (&p)[EP], int64_t t, int E,
                                             int K, bool topk,
                                             float* __restrict__ probs,
                                             int32_t* __restrict__ idx,
                                             float* __restrict__ wout) {
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (e < E) m = fmaxf(m, p[e]);
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

// fp32 tokens: VALU dot products with fp64 accumulation.  One workgroup =
// 64 tokens (one per lane) x 4 waves; wave w covers the w-th quarter of the
// features, with the gate weights as wave-uniform scalar loads.
template <int EP>
__global__ __launch_bounds__(kGateTokens * kGateWaves) void gate_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ bias, int64_t N, int D, int E, int K, int topk,
    float* __restrict__ probs, int32_t* __restrict__ idx,
    float* __restrict__ wout) {
  __shared__ double red[kGateTokens][EP];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kGateTokens + lane;
  const bool valid = t < N;
  const int c0 = wave * D / kGateWaves, c1 = (wave + 1) * D / kGateWaves;
  double acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0;
  if (valid) {
    for (int c = c0; c < c1; ++c) {
      const double xv = x[t * D + c];
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E) acc[e] = fma(xv, static_cast<double>(wg[e * D + c]), acc[e]);
    }
  }
  // fixed-order cross-wave sum
  for (int w = 0; w < kGateWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int e = 0; e < EP; ++e)
        red[lane][e] = (w == 0) ? acc[e] : red[lane][e] + acc[e];
    }
    __syncthreads();
  }
  if (wave != 0 || !valid) return;
  float p[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (e < E)
      p[e] = static_cast<float>(red[lane][e] + (bias ? bias[e] : 0.0));
  softmax_topk<EP>(p, t, E, K, topk != 0, probs, idx, wout);
}

// bf16 tokens on the matrix cores.  The fp32 gate weight is split exactly
// into three bf16 parts, w = hi + mid + lo (each remainder of a
// round-to-nearest-even has at most 16, then 8, significant bits), so
// x * w = x*hi + x*mid + x*lo with every product exact in fp32.  One
// v_mfma_f32_16x16x32_bf16 per part sums a 32-wide k slice for 16 experts x
// 16 tokens; the fp32 slice sums are added in fp64, and the logit is
// rounded once to fp32.
//
// Workgroup: 16 GG tokens (GG groups of 16) x 4 waves; wave w covers the
// w-th quarter of the 32-wide k slices for all of them.  MFMA operands come
// straight from memory: lane l loads 8 consecutive features (16 bytes) of
// token (l % 16) and the matching 8 gate weights of expert (l % 16); lane
// l's results are token (l % 16), experts 4 (l / 16) + 0..3.
template <int EB, int GG>
__global__ __launch_bounds__(64 * kGateWaves) void gate_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ bias, int64_t N, int D, int E, int K, int topk,
    float* __restrict__ probs, int32_t* __restrict__ idx,
    float* __restrict__ wout) {
  constexpr int EP = 16 * EB;
  constexpr int TPB = 16 * GG;   // tokens per workgroup
  __shared__ double red[TPB][EP];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TPB;
  const int nsteps = (D + 31) / 32;
  const int s0 = wave * nsteps / kGateWaves;
  const int s1 = (wave + 1) * nsteps / kGateWaves;

  bool tok_ok[GG];
  const uint16_t* xrow[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) {
    const int64_t t = t0 + g * 16 + col;
    tok_ok[g] = t < N;
    xrow[g] = x + (tok_ok[g] ? t : 0) * D;
  }
  bool e_ok[EB];
  const float* wrow[EB];
#pragma unroll
  for (int b = 0; b < EB; ++b) {
    const int e = b * 16 + col;
    e_ok[b] = e < E;
    wrow[b] = wg + static_cast<int64_t>(e_ok[b] ? e : 0) * D;
  }

  double acc[GG][EB][4];
#pragma unroll
  for (int g = 0; g < GG; ++g)
#pragma unroll
    for (int b = 0; b < EB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[g][b][i] = 0.0;

  // Slices go in chunks of kGateChunk: the chunk's token and weight loads
  // are all issued before its first MFMA, so several slices of x are in
  // flight per wave (a dependent load per slice leaves HBM idle).
  for (int st0 = s0; st0 < s1; st0 += kGateChunk) {
    uint4 xv[kGateChunk][GG];
    float4 wv[kGateChunk][EB][2];
#pragma unroll
    for (int c = 0; c < kGateChunk; ++c) {
      const int k0 = (st0 + c) * 32 + kq * 8;
      const bool k_ok = st0 + c < s1 && k0 < D;
#pragma unroll
      for (int g = 0; g < GG; ++g) {
        xv[c][g] = make_uint4(0, 0, 0, 0);
        if (tok_ok[g] && k_ok) xv[c][g] = *reinterpret_cast<const uint4*>(xrow[g] + k0);
      }
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        wv[c][b][0] = make_float4(0, 0, 0, 0);
        wv[c][b][1] = wv[c][b][0];
        if (e_ok[b] && k_ok) {
          wv[c][b][0] = *reinterpret_cast<const float4*>(wrow[b] + k0);
          wv[c][b][1] = *reinterpret_cast<const float4*>(wrow[b] + k0 + 4);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kGateChunk; ++c) {
      if (st0 + c >= s1) break;
      bf16x8 whi[EB], wmid[EB], wlo[EB];
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        const float4 wa = wv[c][b][0], wb = wv[c][b][1];
        const float w8[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a0 = w8[2 * j], a1 = w8[2 * j + 1];
          h[j] = pack_bf16x2(a0, a1);
          const float r0 = a0 - bf16_lo(h[j]), r1 = a1 - bf16_hi(h[j]);
          m[j] = pack_bf16x2(r0, r1);
          const float q0 = r0 - bf16_lo(m[j]), q1 = r1 - bf16_hi(m[j]);
          l[j] = pack_bf16x2(q0, q1);
        }
        whi[b] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
        wmid[b] = __builtin_bit_cast(bf16x8, make_uint4(m[0], m[1], m[2], m[3]));
        wlo[b] = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
      }
#pragma unroll
      for (int g = 0; g < GG; ++g) {
        const bf16x8 xb = __builtin_bit_cast(bf16x8, xv[c][g]);
#pragma unroll
        for (int b = 0; b < EB; ++b) {
          f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[b], xb, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wmid[b], xb, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[b], xb, a, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[g][b][i] += static_cast<double>(a[i]);
        }
      }
    }
  }
  // fixed-order cross-wave sum into red[token][expert]
  for (int w = 0; w < kGateWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int g = 0; g < GG; ++g)
#pragma unroll
        for (int b = 0; b < EB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            double& r = red[g * 16 + col][b * 16 + kq * 4 + i];
            r = (w == 0) ? acc[g][b][i] : r + acc[g][b][i];
          }
    }
    __syncthreads();
  }
  const int64_t t = t0 + lane;
  if (wave != 0 || lane >= TPB || t >= N) return;
  float p[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (e < E)
      p[e] = static_cast<float>(red[lane][e] + (bias ? bias[e] : 0.0));
  softmax_topk<EP>(p, t, E, K, topk != 0, probs, idx, wout);
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

template <int EB>
hipError_t launch_gate_eb(const void* x, bool bf16, const float* wg,
                          const float* bias, int64_t N, int D, int E, int K,
                          bool topk, float* probs, int32_t* idx, float* w,
                          hipStream_t stream) {
  const dim3 block(64 * kGateWaves);
  if (bf16)
    hipLaunchKernelGGL((gate_mfma_kernel<EB, kGateGroups>),
                       dim3(static_cast<unsigned>(ceil_div(N, 16 * kGateGroups))),
                       block, 0, stream, static_cast<const uint16_t*>(x), wg,
                       bias, N, D, E, K, topk ? 1 : 0, probs, idx, w);
  else
    hipLaunchKernelGGL((gate_f32_kernel<16 * EB>),
                       dim3(static_cast<unsigned>(ceil_div(N, kGateTokens))),
                       block, 0, stream, static_cast<const float*>(x), wg, bias,
                       N, D, E, K, topk ? 1 : 0, probs, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const float* w_gate,
                       const float* bias, int64_t N, int D, int E, int K,
                       bool topk, float* probs, int32_t* idx, float* w,
                       hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (E <= 16)
    return launch_gate_eb<1>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                             idx, w, stream);
  if (E <= 32)
    return launch_gate_eb<2>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                             idx, w, stream);
  return launch_gate_eb<4>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
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
