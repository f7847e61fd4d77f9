// Gate scores, softmax and expert selection for the DiT-MoE layer.
//
// "DiT-MoE" project hub page, section 1 (MoE gate routing): a [E][D] gate
// weight scores every token against the routed experts, a softmax turns the
// scores into probabilities and the top-k experts are kept.  "Expert Race"
// (abstract): tokens and experts compete in one pool for the top
// candidates.
//
// Kernel layout (gfx950):
//  * gate_stream_kernel (bf16 tokens, E <= 16, the layer's gate): each wave
//    streams its own 16 tokens' features through a ring of register loads
//    and multiplies them on the matrix cores against an exact three-way
//    bf16 split of the fp32 gate weights held in LDS (slice sums in fp64);
//    softmax, top-K and, for top-K routing, the balance statistic's
//    per-16-token partial sums follow in registers.  See the kernel.
//  * gate_mfma_kernel (bf16 tokens, E > 16): logits on the matrix cores from an
//    exact three-way bf16 split of the fp32 gate weights, partial sums
//    added in fp64; see the kernel.  gate_f32_kernel (fp32 tokens): the same
//    logits from VALU fp64 FMAs.  Both leave 64 tokens' logits in LDS after
//    a fixed-order sum over 4 waves, and wave 0 runs the fp32 softmax and the
//    top-K selection in registers, one token per lane (ties: lower index).
//  * race_hist_kernel / race_digit_kernel / race_cut_kernel: the exact
//    K*N-th largest probability key by an MSB-first radix select (4 passes
//    of 8 bits; each pass a histogram over 256 workgroups and a one-
//    workgroup digit choice), then the flat index of the last kept entry
//    among keys equal to it.
//  * race_emit_kernel: one thread per token finds its kept experts in
//    ascending order, staged in LDS and written out by the block with
//    consecutive threads on consecutive slots.
#include <atomic>

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
// p is left holding the probabilities; the result has bit e set when expert
// e was selected (0 without top-K routing).
template <int EP>
__device__ __forceinline__ uint64_t softmax_topk(float (&p)[EP], int64_t t, int E,
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
  if (!topk) return 0;
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
  return taken;
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

// bf16 tokens, E <= 16, streaming form of the same arithmetic: three MFMAs
// per 32-wide slice on the exact split of the gate weight, slice sums added
// in fp64 in slice order, one rounding to fp32.
//
// A workgroup of W waves (8, 4 or 2: enough workgroups to occupy every CU)
// owns 16 W tokens; each wave streams the features of its own 16 tokens
// with kRing 32-wide slices in flight (a ring of register loads refilled as
// each slice is consumed), so HBM sees a steady stream, and keeps its
// tokens' logits in registers: no cross-wave sum.  Lane l's logits are
// token (l % 16), experts 4 (l / 16) + 0..3.
//
// The split weights live in LDS, P slices at a time (a phase; P is all the
// slices when they fit, else a multiple of kRing): chunk
// ((part * P + s) * 4 + kq) * EC + e holds the 8 bf16 of part `part` (hi,
// mid, lo) of expert e for features 32 s + 8 kq .. + 7 of the phase, so the
// lanes of a wave read one slice's operand as consecutive 16-byte chunks.
// The first phase's fp32 weights are loaded before the token ring (loads
// return in order, so they are not queued behind it) and split while the
// ring's slices are in flight; a later phase is split when every wave has
// finished the previous one, the ring still loading tokens.
//
// The softmax and the selection run on all 64 lanes: the four lanes of a
// token combine their maxima, sums and candidates with cross-lane swaps
// (the same bits on all four).  With bal_p != nullptr (top-K routing,
// 16-token groups that never straddle two images) each wave also writes
// the balance statistic's partial sums of its 16 tokens, added as a
// pairwise tree over the tokens: bal_p[g][e] (probabilities) and
// bal_c[g][e] (selections), for group g = first token / 16.
constexpr int kStreamWaves = 8;            // most waves per workgroup
constexpr int kRing = 12;                  // slices in flight per wave
constexpr int kStreamLdsMax = 144 * 1024;  // split weights, bytes
constexpr int kSplitBatch = 6;             // weight chunks loaded per thread at once

// Slices per phase of the split weights: all of them if they fit the LDS
// budget, else the largest multiple of kRing that does.
__host__ __device__ constexpr int stream_phase_slices(int D, int EC) {
  const int nsteps = (D + 31) / 32;
  const int fit = kStreamLdsMax / (3 * 4 * EC * 16);
  return nsteps <= fit ? nsteps : fit / kRing * kRing;
}

__host__ __device__ constexpr size_t stream_lds_bytes(int D, int EC) {
  return static_cast<size_t>(3) * stream_phase_slices(D, EC) * 4 * EC * 16;
}

template <int EC>
__global__ __launch_bounds__(64 * kStreamWaves) void gate_stream_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ bias, int64_t N, int D, int E, int K, int topk,
    float* __restrict__ probs, int32_t* __restrict__ idx,
    float* __restrict__ wout, float* __restrict__ bal_p,
    int32_t* __restrict__ bal_c, int P) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ u32x4 wsplit[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int waves = static_cast<int>(blockDim.x) / kWave;
  const int nthreads = static_cast<int>(blockDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int nsteps = (D + 31) / 32;
  const int stride = P * 4 * EC;        // chunks per part
  const int nchunks = EC * P * 4;       // weight chunks of one phase

  // This wave's 16 token rows; rows past N read zero.
  const int64_t t0 =
      static_cast<int64_t>(blockIdx.x) * (16 * waves) + 16 * wave;
  const int64_t left = N - t0;
  const int nrows = left <= 0 ? 0 : (left >= 16 ? 16 : static_cast<int>(left));
  const uint32_t row_bytes = static_cast<uint32_t>(D) * 2u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(
      x + (nrows > 0 ? t0 : int64_t(0)) * D,
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(nrows) * row_bytes));
  const uint32_t off0 = static_cast<uint32_t>(col) * row_bytes + kq * 16u;
  // Byte offset of this lane's 8 features of slice s (zero past D).
  auto xoff = [&](int s) -> uint32_t {
    return (s * 32 + kq * 8 < D) ? off0 + static_cast<uint32_t>(s) * 64u
                                 : kOutOfRange;
  };

  // One batch of the split: thread i takes chunks C0 + nthreads b of phase
  // PH (chunk c: expert c % EC, phase features 8 (c / EC) ..).  Macros over
  // the kernel's own registers (a helper taking these arrays by reference
  // would put them in scratch memory).
  float4 wa4[kSplitBatch], wb4[kSplitBatch];
#define MOE_SPLIT_LOAD(PH, C0)                                               \
  do {                                                                       \
    _Pragma("unroll") for (int b_ = 0; b_ < kSplitBatch; ++b_) {             \
      const int c_ = (C0) + nthreads * b_;                                   \
      const int e_ = c_ % EC;                                                \
      const int k_ = (PH) * P * 32 + 8 * (c_ / EC);                          \
      wa4[b_] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);                         \
      wb4[b_] = wa4[b_];                                                     \
      if (c_ < nchunks && e_ < E && k_ < D) {                                \
        const float* src_ = wg + static_cast<int64_t>(e_) * D + k_;          \
        wa4[b_] = *reinterpret_cast<const float4*>(src_);                    \
        wb4[b_] = *reinterpret_cast<const float4*>(src_ + 4);                \
      }                                                                      \
    }                                                                        \
  } while (0)
#define MOE_SPLIT_STORE(C0)                                                  \
  do {                                                                       \
    _Pragma("unroll") for (int b_ = 0; b_ < kSplitBatch; ++b_) {             \
      const int c_ = (C0) + nthreads * b_;                                   \
      if (c_ < nchunks) {                                                    \
        const int e_ = c_ % EC;                                              \
        const int k_ = 8 * (c_ / EC);                                        \
        const float w8_[8] = {wa4[b_].x, wa4[b_].y, wa4[b_].z, wa4[b_].w,    \
                              wb4[b_].x, wb4[b_].y, wb4[b_].z, wb4[b_].w};   \
        u32x4 h_, m_, l_;                                                    \
        _Pragma("unroll") for (int q_ = 0; q_ < 4; ++q_) {                   \
          const float a0_ = w8_[2 * q_], a1_ = w8_[2 * q_ + 1];              \
          h_[q_] = pack_bf16x2(a0_, a1_);                                    \
          const float r0_ = a0_ - bf16_lo(h_[q_]);                           \
          const float r1_ = a1_ - bf16_hi(h_[q_]);                           \
          m_[q_] = pack_bf16x2(r0_, r1_);                                    \
          l_[q_] = pack_bf16x2(r0_ - bf16_lo(m_[q_]), r1_ - bf16_hi(m_[q_])); \
        }                                                                    \
        const int chunk_ = ((k_ >> 5) * 4 + ((k_ >> 3) & 3)) * EC + e_;      \
        wsplit[chunk_] = h_;                                                 \
        wsplit[stride + chunk_] = m_;                                        \
        wsplit[2 * stride + chunk_] = l_;                                    \
      }                                                                      \
    }                                                                        \
  } while (0)
#define MOE_SPLIT_REST(PH, FIRST)                                            \
  for (int c0_ = (FIRST); c0_ < nchunks; c0_ += nthreads * kSplitBatch) {    \
    MOE_SPLIT_LOAD(PH, c0_);                                                 \
    MOE_SPLIT_STORE(c0_);                                                    \
  }

  // Phase 0: the weights' first batch, then the token ring, then the split.
  MOE_SPLIT_LOAD(0, tid);
  u32x4 xr[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j)
    xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, xoff(j), 0, 0);
  MOE_SPLIT_STORE(tid);
  MOE_SPLIT_REST(0, tid + nthreads * kSplitBatch)
  __syncthreads();

  // Straight-line ring over each phase's slices: slices past nsteps load
  // zero features and read the (finite) weights of the last slice, so they
  // add exactly zero.  Lanes past the stored expert columns (E <= 8) read
  // expert 0's chunk: their output rows are experts >= E, never used.  The
  // three weight parts of slice s + 1 are read from LDS while slice s is
  // multiplied (kRing is even, so the two register sets alternate in a
  // fixed pattern); the first slice of a phase is read after its split.
  static_assert(kRing % 2 == 0, "even ring");
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const u32x4* const wl = wsplit + kq * EC + (col < EC ? col : 0);
  u32x4 wa[3], wb[3];
  for (int s_begin = 0; s_begin < nsteps; s_begin += P) {
    const int ph = s_begin / P;
    const int s_last = (s_begin + P < nsteps ? s_begin + P : nsteps) - 1;
    if (ph > 0) {
      __syncthreads();   // every wave is done with the previous phase
      MOE_SPLIT_REST(ph, tid)
      __syncthreads();
    }
    auto wslice = [&](int s, u32x4 (&w)[3]) {
      const int sw = ((s < s_last ? s : s_last) - s_begin) * 4 * EC;
      w[0] = wl[sw];
      w[1] = wl[stride + sw];
      w[2] = wl[2 * stride + sw];
    };
    wslice(s_begin, wa);
    // P is a multiple of kRing unless this is the only phase, so the ring
    // position of slice s_begin is 0.
    for (int s0 = s_begin; s0 <= s_last; s0 += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int s = s0 + j;
        u32x4 (&cur)[3] = (j % 2 == 0) ? wa : wb;
        u32x4 (&nxt)[3] = (j % 2 == 0) ? wb : wa;
        wslice(s + 1, nxt);
        const bf16x8 xb = __builtin_bit_cast(bf16x8, xr[j]);
        xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, xoff(s + kRing), 0, 0);
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int part = 0; part < 3; ++part)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, cur[part]), xb, a, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += static_cast<double>(a[i]);
      }
    }
  }

#undef MOE_SPLIT_LOAD
#undef MOE_SPLIT_STORE
#undef MOE_SPLIT_REST

  // Softmax of token col over the four lanes col + 16 q.
  const int64_t t = t0 + col;
  const bool tok = t < N;
  float p[4];
  bool ok[4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * kq + i;
    ok[i] = e < E;
    const double b = (bias != nullptr && ok[i]) ? static_cast<double>(bias[e]) : 0.0;
    p[i] = static_cast<float>(acc[i] + b);
    if (ok[i]) m = fmaxf(m, p[i]);
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = ok[i] ? expf(p[i] - m) : 0.0f;
    sum += p[i];
  }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = ok[i] ? p[i] / sum : 0.0f;
    if (tok && ok[i]) probs[t * E + 4 * kq + i] = p[i];
  }

  // Top-K: K rounds of the largest remaining (key, expert) pair, ties to
  // the lower expert; each lane offers its best, the four lanes agree.
  uint32_t sel = 0;   // experts selected by token col (bit e)
  if (topk) {
    for (int k = 0; k < K; ++k) {
      float bk = -INFINITY, bp = 0.0f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * kq + i;
        if (ok[i] && !((sel >> e) & 1u)) {
          const float key = sel_key(p[i]);
          if (be == 0x7fffffff || key > bk) {
            bk = key;
            be = e;
            bp = p[i];
          }
        }
      }
#pragma unroll
      for (int off = 16; off <= 32; off *= 2) {
        const float ok2 = __shfl_xor(bk, off);
        const int oe = __shfl_xor(be, off);
        const float op = __shfl_xor(bp, off);
        if (ok2 > bk || (ok2 == bk && oe < be)) {
          bk = ok2;
          be = oe;
          bp = op;
        }
      }
      sel |= 1u << be;
      if (kq == 0 && tok) {
        idx[t * K + k] = be;
        wout[t * K + k] = bp;
      }
    }
  }
  if (bal_p == nullptr) return;
  // Whole groups only: the host takes this path when N is a multiple of 16.
  const uint64_t row = 0xffffull << (16 * kq);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = tok ? p[i] : 0.0f;
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    const int e = 4 * kq + i;
    const uint64_t hit = __ballot(tok && ((sel >> e) & 1u));
    if (col == 0 && ok[i] && t0 < N) {
      const int64_t o = (t0 / 16) * E + e;
      bal_p[o] = v;
      bal_c[o] = __popcll(hit & row);
    }
  }
}

// Split weights of E experts: the streaming kernel takes E <= 16 (bf16
// tokens, any D).
bool gate_stream_fits(int D, int E) {
  (void)D;
  return E <= 16;
}

// Waves per workgroup of the streaming gate: 8, or fewer when that leaves
// CUs without a workgroup (short inputs).
int gate_stream_waves(int64_t N) {
  const int cus = cu_count();
  int w = kStreamWaves;
  while (w > 2 && ceil_div(N, 16 * w) < cus) w /= 2;
  return w;
}

template <int EC>
hipError_t launch_gate_stream(const void* x, const float* wg, const float* bias,
                              int64_t N, int D, int E, int K, bool topk,
                              float* probs, int32_t* idx, float* w,
                              float* bal_p, int32_t* bal_c,
                              hipStream_t stream) {
  // the LDS opt-in is a property of the kernel on each device: set once per
  // device
  static std::atomic<bool> lds_opt_in[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!lds_opt_in[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gate_stream_kernel<EC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kStreamLdsMax);
    if (e != hipSuccess) return e;
    lds_opt_in[dev].store(true, std::memory_order_release);
  }
  const int waves = gate_stream_waves(N);
  hipLaunchKernelGGL((gate_stream_kernel<EC>),
                     dim3(static_cast<unsigned>(ceil_div(N, 16 * waves))),
                     dim3(64 * waves),
                     static_cast<unsigned>(stream_lds_bytes(D, EC)), stream,
                     static_cast<const uint16_t*>(x), wg, bias, N, D, E, K,
                     topk ? 1 : 0, probs, idx, w, bal_p, bal_c,
                     stream_phase_slices(D, EC));
  return hipGetLastError();
}

// ---------------------------------------------------------- Expert Race --

constexpr int kRaceThreads = 1024;
constexpr int kRaceWaves = kRaceThreads / kWave;

// Order-preserving key of a probability: the fp32 bit pattern of a
// non-negative float orders like its value.  NaN and negatives map to 0.
__device__ __forceinline__ uint32_t race_key(float p) {
  return (p > 0.0f) ? __float_as_uint(p) : 0u;
}

// The global top-A of the N*E probabilities as a threshold: tau (a key)
// and the flat index `cut` of the last kept entry equal to tau.  Entries
// with key > tau, or key == tau and flat index <= cut, are kept: exactly A.
//
// Four 8-bit radix passes, most significant digit first.  Each pass is two
// launches: race_hist_kernel, where kRaceBlocks workgroups each count the
// digits of their slice of the keys that still match the prefix in an LDS
// histogram and write it out, and race_digit_kernel, where one workgroup
// adds the kRaceBlocks histograms bin by bin in workgroup order (integer
// counts: exact in any order) and narrows the prefix.  The state after pass
// p (prefix, mask, how many of the matching entries are still needed) is
// RaceState p + 1 in the workspace; the state before pass 0 (no prefix,
// A needed) is implicit.  Probabilities share their sign and high
// exponent bits, so in the first pass most keys of a wave fall in a few
// bins: the wave counts each distinct digit with one ballot and one LDS
// atomic instead of 64 colliding atomics.
constexpr int kRaceBlocks = 256;
constexpr int kRaceHistThreads = 256;
constexpr int kRaceHistLoads = 4;
static_assert(kRaceBlocks % 64 == 0, "whole batches of 16 per quarter");

struct RaceState {
  uint32_t prefix, mask, need, all;
};

size_t race_hist_offset() { return 256; }   // RaceState[5] first

__global__ __launch_bounds__(kRaceHistThreads) void race_hist_kernel(
    const float* __restrict__ probs, int64_t total, int pass,
    const RaceState* __restrict__ st, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  h[tid] = 0;
  __syncthreads();
  // pass 0 matches every key (st[0] is never written)
  const uint32_t prefix = pass == 0 ? 0u : st[pass].prefix;
  const uint32_t mask = pass == 0 ? 0u : st[pass].mask;
  const int shift = 24 - 8 * pass;
  const int64_t per = (total + kRaceBlocks - 1) / kRaceBlocks;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = min(total, b0 + per);
  // kRaceHistLoads keys per thread in flight (past the slice they re-read
  // its last key and are not counted)
  for (int64_t i0 = b0; i0 < b1; i0 += kRaceHistThreads * kRaceHistLoads) {
    float pv[kRaceHistLoads];
#pragma unroll
    for (int u = 0; u < kRaceHistLoads; ++u) {
      const int64_t i = i0 + u * kRaceHistThreads + tid;
      pv[u] = probs[i < b1 ? i : b1 - 1];
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
#pragma unroll
    for (int u = 0; u < kRaceHistLoads; ++u) {
      const int64_t i = i0 + u * kRaceHistThreads + tid;
      const uint32_t k = race_key(pv[u]);
      bool live = i < b1 && (k & mask) == prefix;
      const uint32_t d = (k >> shift) & 255u;
      if (pass == 0) {
        // one round per distinct digit among the wave's live lanes
        uint64_t left = __ballot(live);
        while (left != 0) {
          const int leader = __builtin_ctzll(left);
          const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
          const uint64_t same = __ballot(live && d == dl);
          if (lane == leader) atomicAdd(&h[dl], static_cast<uint32_t>(__popcll(same)));
          if (d == dl) live = false;
          left = __ballot(live);
        }
      } else if (live) {
        atomicAdd(&h[d], 1u);
      }
    }
  }
  __syncthreads();
  hist[static_cast<int64_t>(blockIdx.x) * 256 + tid] = h[tid];
}

// One workgroup: the pass's digit.  Thread (q, d) adds bin d over the
// q-th quarter of the histogram workgroups (16 loads in flight), the four
// quarter sums are added in order, and thread 0 walks the digits from the
// top.
__global__ __launch_bounds__(1024) void race_digit_kernel(
    const uint32_t* __restrict__ hist, int pass, uint32_t a_first,
    RaceState* __restrict__ st) {
  __shared__ uint32_t part[4][256];
  __shared__ uint32_t tot[256];
  const int tid = threadIdx.x;
  const int d = tid & 255, q = tid >> 8;
  constexpr int kQuarter = kRaceBlocks / 4;
  uint32_t c = 0;
  for (int b0 = q * kQuarter; b0 < (q + 1) * kQuarter; b0 += 16) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = hist[static_cast<int64_t>(b0 + u) * 256 + d];
#pragma unroll
    for (int u = 0; u < 16; ++u) c += v[u];
  }
  part[q][d] = c;
  __syncthreads();
  // above[d] = entries in bins above d (a suffix sum: 8 doubling steps)
  __shared__ uint32_t above[2][256];
  if (tid < 256) {
    tot[tid] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    above[0][tid] = tot[tid];
  }
  __syncthreads();
  int cur = 0;
  for (int h = 1; h < 256; h *= 2) {
    if (tid < 256)
      above[cur ^ 1][tid] = above[cur][tid] + (tid + h < 256 ? above[cur][tid + h] : 0u);
    __syncthreads();
    cur ^= 1;
  }
  if (tid < 256) {
    // inclusive suffix sum -> exclusive
    const uint32_t ab = above[cur][tid] - tot[tid];
    const RaceState in = pass == 0 ? RaceState{0u, 0u, a_first, 0u} : st[pass];
    // The bins' ranges [ab, ab + tot) partition the matching entries from
    // the top: exactly one digit holds the need-th (bin 0 takes the
    // remainder if the counts fall short, as the serial walk would).
    const bool hit = ab < in.need && (ab + tot[tid] >= in.need || tid == 0);
    if (hit) {
      const int shift = 24 - 8 * pass;
      RaceState out;
      out.prefix = in.prefix | (static_cast<uint32_t>(tid) << shift);
      out.mask = in.mask | (255u << shift);
      out.need = in.need - ab;
      // after the last pass tot[digit] counts the entries equal to tau
      out.all = (pass == 3 && out.need == tot[tid]) ? 1u : 0u;
      st[pass + 1] = out;
    }
  }
}

// sel[0] = tau, sel[1] = cut.  When every entry equal to tau is kept (no
// tie straddles the cut: the usual case) cut is the last flat index;
// otherwise one workgroup finds the need-th entry equal to tau in flat
// order, in tiles of 1024 entries.
__global__ __launch_bounds__(kRaceThreads) void race_cut_kernel(
    const float* __restrict__ probs, int64_t total,
    const RaceState* __restrict__ st4, uint32_t* __restrict__ sel) {
  __shared__ uint32_t wcnt[kRaceWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint32_t tau = st4->prefix;
  const uint32_t need = st4->need;
  if (st4->all != 0) {
    if (tid == 0) {
      sel[0] = tau;
      sel[1] = static_cast<uint32_t>(total - 1);
    }
    return;
  }
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
        sel[0] = tau;
        sel[1] = static_cast<uint32_t>(i);
      }
      return;
    }
    running += tile;
    __syncthreads();
  }
}

// A block of tokens (256 when E <= 16, else 64: at most 4096 slots) finds
// each token's kept experts from its probabilities (loaded 16 at a time, all
// in flight) into LDS rows padded to E + 1 entries (no bank conflicts
// between consecutive tokens), then copies the block's [tokens][E] slots
// out with consecutive threads on consecutive slots.
constexpr int kEmitSlots = 4096;
__host__ __device__ constexpr int emit_tokens(int E) { return E <= 16 ? 256 : 64; }

__global__ __launch_bounds__(256) void race_emit_kernel(
    const float* __restrict__ probs, int64_t N, int E,
    const uint32_t* __restrict__ sel, int32_t* __restrict__ idx,
    float* __restrict__ w) {
  __shared__ int32_t s_i[kEmitSlots + 256];
  __shared__ float s_w[kEmitSlots + 256];
  const int tid = threadIdx.x, TB = blockDim.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int ntok = static_cast<int>(min<int64_t>(TB, N - t0));
  const int pitch = E + 1;
  if (tid < ntok) {
    const int64_t t = t0 + tid;
    const uint32_t tau = sel[0];
    const int64_t cut = sel[1];
    int32_t* const ri = s_i + tid * pitch;
    float* const rw = s_w + tid * pitch;
    int n = 0;
    // past E the loads re-read the last probability and are not used
    for (int e0 = 0; e0 < E; e0 += 16) {
      float pv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) pv[u] = probs[t * E + (e0 + u < E ? e0 + u : E - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + u;
        if (e >= E) break;
        const uint32_t k = race_key(pv[u]);
        const int64_t flat = t * E + e;
        if (k > tau || (k == tau && flat <= cut)) {
          ri[n] = e;
          rw[n] = pv[u];
          ++n;
        }
      }
    }
    for (; n < E; ++n) {
      ri[n] = -1;
      rw[n] = 0.0f;
    }
  }
  __syncthreads();
  const int nslots = ntok * E;
  for (int i = tid; i < nslots; i += TB) {
    const int tk = i / E;
    const int j = tk * pitch + (i - tk * E);
    idx[t0 * E + i] = s_i[j];
    w[t0 * E + i] = s_w[j];
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
  if (x_bf16 && gate_stream_fits(D, E))
    return E <= 8 ? launch_gate_stream<8>(x, w_gate, bias, N, D, E, K, topk,
                                          probs, idx, w, nullptr, nullptr,
                                          stream)
                  : launch_gate_stream<16>(x, w_gate, bias, N, D, E, K, topk,
                                           probs, idx, w, nullptr, nullptr,
                                           stream);
  if (E <= 16)
    return launch_gate_eb<1>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                             idx, w, stream);
  if (E <= 32)
    return launch_gate_eb<2>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                             idx, w, stream);
  return launch_gate_eb<4>(x, x_bf16, w_gate, bias, N, D, E, K, topk, probs,
                           idx, w, stream);
}

bool gate_balance_fuses(bool x_bf16, int64_t N, int T, int D, int E) {
  return x_bf16 && N > 0 && T % 16 == 0 && gate_stream_fits(D, E);
}

hipError_t launch_gate_balance_partials(const void* x, const float* w_gate,
                                        const float* bias, int64_t N, int D,
                                        int E, int K, float* probs,
                                        int32_t* idx, float* w, float* bal_p,
                                        int32_t* bal_c, hipStream_t stream) {
  return E <= 8 ? launch_gate_stream<8>(x, w_gate, bias, N, D, E, K, true,
                                        probs, idx, w, bal_p, bal_c, stream)
                : launch_gate_stream<16>(x, w_gate, bias, N, D, E, K, true,
                                         probs, idx, w, bal_p, bal_c, stream);
}

// [0, 80): RaceState[5]; [96, 104): sel; [256, ...): 4 passes of
// kRaceBlocks x 256 histogram words.
size_t race_workspace_bytes() {
  return race_hist_offset() + static_cast<size_t>(4) * kRaceBlocks * 256 * 4;
}

hipError_t launch_race(const float* probs, int64_t N, int E, int K,
                       int32_t* idx, float* w, void* workspace,
                       hipStream_t stream) {
  if (N == 0) return hipSuccess;
  char* ws = static_cast<char*>(workspace);
  RaceState* st = reinterpret_cast<RaceState*>(ws);
  uint32_t* sel = reinterpret_cast<uint32_t*>(ws + 96);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + race_hist_offset());
  const int64_t total = N * E;
  hipError_t err;
  for (int pass = 0; pass < 4; ++pass) {
    uint32_t* hp = hist + static_cast<size_t>(pass) * kRaceBlocks * 256;
    hipLaunchKernelGGL(race_hist_kernel, dim3(kRaceBlocks),
                       dim3(kRaceHistThreads), 0, stream, probs, total, pass,
                       st, hp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(race_digit_kernel, dim3(1), dim3(1024), 0, stream, hp,
                       pass, static_cast<uint32_t>(K * N), st);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(race_cut_kernel, dim3(1), dim3(kRaceThreads), 0, stream,
                     probs, total, st + 4, sel);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int tb = emit_tokens(E);
  static_assert(emit_tokens(16) * 17 <= kEmitSlots + 256 &&
                    emit_tokens(kMaxExperts) * (kMaxExperts + 1) <= kEmitSlots + 256,
                "a block's padded slot rows fit the LDS rows");
  hipLaunchKernelGGL(race_emit_kernel,
                     dim3(static_cast<unsigned>(ceil_div(N, tb))), dim3(tb),
                     0, stream, probs, N, E, sel, idx, w);
  return hipGetLastError();
}

}  // namespace moe
