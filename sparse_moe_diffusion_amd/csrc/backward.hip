// Backward of the DiT-MoE layer: everything except the expert GEMMs.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE-DiT: the
// layer is trained with the expert-level balance loss added to the
// denoising loss.  The gradients are those of the forward definitions (eq. MoE(x),
// eq. MLP, eq. L_balance, the gate softmax of the "DiT-MoE" project hub
// page, section 1) with the routing held fixed: the selection itself has no
// gradient, the slot weights (gate probabilities) do.
//
// Kernels (gfx950):
//  * transpose_kernel: [G][R][C] -> [G][C][R] bf16 through 64x64 LDS tiles
//    (W1's transposed copy for the dx GEMM; W2 is read as stored).
//  * rows_kernel: a row copy, optionally gathered through a row index and
//    optionally through GELU (the row-major operands of the K-grouped
//    weight-gradient GEMM when they are not already in HBM).
//  * combine_bwd_kernel: one wave per token; the routed rows' output
//    gradients w * dy and the slot-weight gradients <dy, y_row>.
//  * gate_bwd_token_kernel, gate_bwd_wgrad_kernel, gate_bwd_reduce_kernel,
//    gate_bwd_dx_tok_kernel (E <= 8) / gate_bwd_dx_kernel: dP -> dlogits
//    per token; dW_g and dbias partials per token chunk and their
//    fixed-order sum; dx assembled per token.
#include <algorithm>

#include "common.hpp"
#include "gather.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float gelu_fwd(float u) {
  constexpr float kC1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
  constexpr float kC2 = kC1 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(u * fmaf(kC2, u * u, kC1));
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------------ transposes --

constexpr int kTile = 64;

// 64 x 64 tile: 16-byte loads along the source rows, scattered 2-byte LDS
// writes into the transposed tile, 16-byte LDS reads and 16-byte stores
// along the destination rows (R and C are multiples of 8).
constexpr int kTp = kTile + 8;   // LDS row pitch (elements), keeps 16 B rows

__device__ __forceinline__ void tile_store_t(uint16_t (*t)[kTp], int j, int c8,
                                             uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[c8 + 2 * i][j] = static_cast<uint16_t>(w[i] & 0xffffu);
    t[c8 + 2 * i + 1][j] = static_cast<uint16_t>(w[i] >> 16);
  }
}

__global__ __launch_bounds__(256) void transpose_kernel(
    const uint16_t* __restrict__ src, int R, int C,
    uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kTile][kTp];
  const int c0 = blockIdx.x * kTile, r0 = blockIdx.y * kTile;
  const int64_t g = blockIdx.z;
  const uint16_t* s = src + g * R * C;
  uint16_t* d = dst + g * R * C;
  const int ch = threadIdx.x & 7, jr = threadIdx.x >> 3;   // 8 chunks x 32 rows
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = jr + 32 * h;
    const int rr = r0 + j, cc = c0 + 8 * ch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < R && cc < C)
      v = *reinterpret_cast<const uint4*>(s + static_cast<int64_t>(rr) * C + cc);
    tile_store_t(t, j, 8 * ch, v);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = jr + 32 * h;
    const int cc = c0 + c, rr = r0 + 8 * ch;
    if (cc < C && rr < R)
      *reinterpret_cast<uint4*>(d + static_cast<int64_t>(cc) * R + rr) =
          *reinterpret_cast<const uint4*>(&t[c][8 * ch]);
  }
}

// dst [total][C] = f(src rows): row r is source row row_index[r] (or r),
// with GELU applied when asked.  One 16-byte chunk per thread (C a multiple
// of 8); consecutive threads along a row.
template <bool GELU>
__global__ __launch_bounds__(256) void rows_kernel(
    const uint16_t* __restrict__ src, const int32_t* __restrict__ row_index,
    int64_t src_rows, int64_t total, int C, uint16_t* __restrict__ dst) {
  const int cpr = C / 8;
  const int64_t n = total * cpr;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
       i < n; i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / cpr;
    const int c = static_cast<int>(i - r * cpr) * 8;
    const int64_t sr = row_index ? row_index[r] : r;
    // an index entry outside [0, src_rows) gives a zero row
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row_index == nullptr || gather_row_valid(sr, src_rows))
      v = *reinterpret_cast<const uint4*>(src + sr * C + c);
    if constexpr (GELU) {
      float f[8];
      unpack8(v, f);
      v.x = pack_bf16x2(gelu_fwd(f[0]), gelu_fwd(f[1]));
      v.y = pack_bf16x2(gelu_fwd(f[2]), gelu_fwd(f[3]));
      v.z = pack_bf16x2(gelu_fwd(f[4]), gelu_fwd(f[5]));
      v.w = pack_bf16x2(gelu_fwd(f[6]), gelu_fwd(f[7]));
    }
    *reinterpret_cast<uint4*>(dst + r * C + c) = v;
  }
}

template <bool BF16>
__device__ __forceinline__ void ld8(const void* base, int64_t row, int D, int c,
                                    float* f) {
  if constexpr (BF16) {
    unpack8(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) +
                                           row * D)[c], f);
  } else {
    const float4* p =
        reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * D) + 2 * c;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void st8(void* base, int64_t row, int D, int c,
                                    const float* f) {
  if constexpr (BF16) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + row * D)[c] = v;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + row * D) + 2 * c;
    p[0] = make_float4(f[0], f[1], f[2], f[3]);
    p[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

// Wave sum in a fixed order (xor butterfly): the same bits on every run.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

constexpr int kCbWaves = 4;

// Token t: for each slot k with row r = slot_row[t][k] >= 0,
//   dy_rows[r] = topk_w[t][k] * dy[t]   and   dw[t][k] = <dy[t], y_rows[r]>;
// empty slots get dw = 0.
template <bool DB, bool YB>
__global__ __launch_bounds__(64 * kCbWaves) void combine_bwd_kernel(
    const void* __restrict__ dy, const void* __restrict__ y_rows,
    const int32_t* __restrict__ slot_row, const float* __restrict__ w,
    int64_t N, int D, int Kmax, void* __restrict__ dy_rows,
    float* __restrict__ dw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCbWaves + (threadIdx.x >> 6);
  if (t >= N) return;
  const int nch = D / 8;
  for (int k = 0; k < Kmax; ++k) {
    const int32_t r = slot_row[t * Kmax + k];
    if (r < 0) {
      if (lane == 0) dw[t * Kmax + k] = 0.0f;
      continue;
    }
    const float wk = w[t * Kmax + k];
    float part = 0.0f;
    for (int c = lane; c < nch; c += 64) {
      float g[8], y[8], o[8];
      ld8<DB>(dy, t, D, c, g);
      ld8<YB>(y_rows, r, D, c, y);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        part = fmaf(g[j], y[j], part);
        o[j] = wk * g[j];
      }
      st8<YB>(dy_rows, r, D, c, o);
    }
    const float s = wave_sum(part);
    if (lane == 0) dw[t * Kmax + k] = s;
  }
}

// ------------------------------------------------------------------ gate --

// Per token: dP[i] = sum_k [idx[t][k] == i] dw[t][k] + dloss * dL/dP[t][i],
// dlogits = P (dP - sum_j P_j dP_j), written to dl [N][E].  EP >= E bounds
// the experts, so dP stays in registers (a slot adds to the expert it names
// through unrolled compares, in slot order).  In global mode the balance
// term is the same for every token: each workgroup forms it once, from the
// counts summed over the images.
template <int EP>
__global__ __launch_bounds__(256) void gate_bwd_token_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, const int32_t* __restrict__ counts, int B,
    int T, int E, int Kmax, int K, float alpha, float dloss, int global,
    float* __restrict__ dl) {
  __shared__ float gcoef[EP];
  const int64_t N = static_cast<int64_t>(B) * T;
  if (global && dloss != 0.0f) {   // uniform: every thread reaches the barrier
    if (static_cast<int>(threadIdx.x) < E) {
      const int i = threadIdx.x;
      int64_t c = 0;
      for (int bb = 0; bb < B; ++bb) c += counts[static_cast<int64_t>(bb) * E + i];
      const float Tg = static_cast<float>(N);
      float g = alpha * (static_cast<float>(E) / (static_cast<float>(K) * Tg)) *
                static_cast<float>(c) / Tg;
      gcoef[i] = g * dloss;
    }
    __syncthreads();
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const int b = static_cast<int>(t / T);
  float dP[EP];
#pragma unroll
  for (int i = 0; i < EP; ++i) {
    float g = 0.0f;
    if (i < E && dloss != 0.0f) {
      if (global) {
        g = gcoef[i];
      } else {
        g = alpha / static_cast<float>(B) *
            (static_cast<float>(E) / (static_cast<float>(K) * T)) *
            static_cast<float>(counts[static_cast<int64_t>(b) * E + i]) /
            static_cast<float>(T);
        g *= dloss;
      }
    }
    dP[i] = g;
  }
  for (int k = 0; k < Kmax; ++k) {
    const int e = idx[t * Kmax + k];
    const float d = dw[t * Kmax + k];
#pragma unroll
    for (int i = 0; i < EP; ++i)
      if (i == e && i < E) dP[i] += d;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < EP; ++i)
    if (i < E) s = fmaf(probs[t * E + i], dP[i], s);
#pragma unroll
  for (int i = 0; i < EP; ++i) {
    if (i < E) {
      const float p = probs[t * E + i];
      dl[t * E + i] = p * (dP[i] - s);
    }
  }
}

constexpr int kGbTokens = 64;    // tokens per workgroup of the dW_g pass
constexpr int kGbBatch = 8;      // x rows loaded ahead in that pass

// dx[t] = sum_k dx_rows[slot_row[t][k]] + dx_shared[t] + sum_i dl[t][i] W_g[i]
// in fp32, rounded once, added in that order.  One thread per 8 features of
// a token.  No load sits behind a branch, so they go out together: the
// shared row and the first 8 experts' dl and W_g before the slot rows, the
// slot rows in groups of 4 (an empty slot, or a missing operand, reads the
// token's own dx chunk, a valid address, and is not added).
template <bool OB>
__global__ __launch_bounds__(256) void gate_bwd_dx_kernel(
    const float* __restrict__ wg, const float* __restrict__ dl, int64_t N,
    int D, int E, int Kmax, const void* __restrict__ dx_rows,
    const int32_t* __restrict__ slot_row, const void* __restrict__ dx_shared,
    void* __restrict__ dx) {
  const uint32_t nch = static_cast<uint32_t>(D / 8);
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= static_cast<uint32_t>(N) * nch) return;
  const uint32_t tq = i / nch;
  const int64_t t = tq;
  const int c = static_cast<int>(i - tq * nch);
  // the shared experts' row and the first 8 experts, loaded first
  float sh[8];
  ld8<OB>(dx_shared != nullptr ? dx_shared : dx, t, D, c, sh);
  float d[8];
  float4 wa[8], wb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = u < E ? u : E - 1;
    d[u] = dl[t * E + e];
    const float4* wp =
        reinterpret_cast<const float4*>(wg + static_cast<int64_t>(e) * D) + 2 * c;
    wa[u] = wp[0];
    wb[u] = wp[1];
  }
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.0f;
  if (slot_row != nullptr) {
    for (int k0 = 0; k0 < Kmax; k0 += 4) {
      int32_t r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        r[q] = slot_row[t * Kmax + (k0 + q < Kmax ? k0 + q : Kmax - 1)];
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = k0 + q < Kmax && r[q] >= 0;
        ld8<OB>(ok ? dx_rows : static_cast<const void*>(dx), ok ? r[q] : t, D, c,
                v[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (k0 + q < Kmax && r[q] >= 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] += v[q][j];
        }
    }
  }
  if (dx_shared != nullptr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] += sh[j];
  }
  for (int e0 = 0; e0 < E; e0 += 8) {
    if (e0 > 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u < E ? e0 + u : E - 1;
        d[u] = dl[t * E + e];
        const float4* wp =
            reinterpret_cast<const float4*>(wg + static_cast<int64_t>(e) * D) + 2 * c;
        wa[u] = wp[0];
        wb[u] = wp[1];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (e0 + u >= E) break;
      const float4 a = wa[u], b = wb[u];
      o[0] = fmaf(d[u], a.x, o[0]); o[1] = fmaf(d[u], a.y, o[1]);
      o[2] = fmaf(d[u], a.z, o[2]); o[3] = fmaf(d[u], a.w, o[3]);
      o[4] = fmaf(d[u], b.x, o[4]); o[5] = fmaf(d[u], b.y, o[5]);
      o[6] = fmaf(d[u], b.z, o[6]); o[7] = fmaf(d[u], b.w, o[7]);
    }
  }
  st8<OB>(dx, t, D, c, o);
}

// The same for E <= EB (8): a thread owns one 8-feature chunk of kDxTokens
// consecutive tokens and keeps that chunk of W_g (EB x 8 floats) in
// registers, so W_g is read once per kDxTokens tokens instead of once per
// token (at D = 1152, E = 8 that is 37 KB per token).  Same order of
// additions, same bits.
constexpr int kDxTokens = 8;
template <bool OB, int EB>
__global__ __launch_bounds__(256) void gate_bwd_dx_tok_kernel(
    const float* __restrict__ wg, const float* __restrict__ dl, int64_t N,
    int D, int E, int Kmax, const void* __restrict__ dx_rows,
    const int32_t* __restrict__ slot_row, const void* __restrict__ dx_shared,
    void* __restrict__ dx) {
  const uint32_t nch = static_cast<uint32_t>(D / 8);
  const uint32_t ng = static_cast<uint32_t>((N + kDxTokens - 1) / kDxTokens);
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ng * nch) return;
  const uint32_t tg = i / nch;
  const int c = static_cast<int>(i - tg * nch);
  float4 wa[EB], wb[EB];
#pragma unroll
  for (int u = 0; u < EB; ++u) {
    const float4* wp = reinterpret_cast<const float4*>(
                           wg + static_cast<int64_t>(u < E ? u : E - 1) * D) + 2 * c;
    wa[u] = wp[0];
    wb[u] = wp[1];
  }
  const int64_t tb = static_cast<int64_t>(tg) * kDxTokens;
  const int64_t t1 = min<int64_t>(N, tb + kDxTokens);
  // The first four slot rows of the next token are read while this token's
  // rows are in flight, so a token costs one round trip to memory, not two
  // (an index, then the rows it names).
  int32_t rn[4];
  if (slot_row != nullptr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) rn[q] = slot_row[tb * Kmax + (q < Kmax ? q : Kmax - 1)];
  }
  for (int64_t t = tb; t < t1; ++t) {
    float sh[8];
    ld8<OB>(dx_shared != nullptr ? dx_shared : dx, t, D, c, sh);
    float d[EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) d[u] = dl[t * E + (u < E ? u : E - 1)];
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.0f;
    if (slot_row != nullptr) {
      {
        int32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = rn[q];
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = q < Kmax && r[q] >= 0;
          ld8<OB>(ok ? dx_rows : static_cast<const void*>(dx), ok ? r[q] : t, D, c,
                  v[q]);
        }
        const int64_t tn = t + 1 < t1 ? t + 1 : t;
#pragma unroll
        for (int q = 0; q < 4; ++q) rn[q] = slot_row[tn * Kmax + (q < Kmax ? q : Kmax - 1)];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < Kmax && r[q] >= 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] += v[q][j];
          }
      }
      for (int k0 = 4; k0 < Kmax; k0 += 4) {
        int32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          r[q] = slot_row[t * Kmax + (k0 + q < Kmax ? k0 + q : Kmax - 1)];
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = k0 + q < Kmax && r[q] >= 0;
          ld8<OB>(ok ? dx_rows : static_cast<const void*>(dx), ok ? r[q] : t, D,
                  c, v[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (k0 + q < Kmax && r[q] >= 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] += v[q][j];
          }
      }
    }
    if (dx_shared != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] += sh[j];
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      if (u >= E) break;
      const float4 a = wa[u], b = wb[u];
      o[0] = fmaf(d[u], a.x, o[0]); o[1] = fmaf(d[u], a.y, o[1]);
      o[2] = fmaf(d[u], a.z, o[2]); o[3] = fmaf(d[u], a.w, o[3]);
      o[4] = fmaf(d[u], b.x, o[4]); o[5] = fmaf(d[u], b.y, o[5]);
      o[6] = fmaf(d[u], b.z, o[6]); o[7] = fmaf(d[u], b.w, o[7]);
    }
    st8<OB>(dx, t, D, c, o);
  }
}

// Workgroup = kGbTokens tokens; their dl rows are staged in LDS.  Thread =
// one (8 consecutive features c, block of 8 experts) pair: it sums, over
// the chunk's tokens, dl[t][i] x[t][c..c+8], loading kGbBatch x rows ahead,
// and writes its part of the chunk's partial [E][D].  Threads i < E also sum
// dl over the chunk (the dbias partial).
template <bool XB>
__global__ __launch_bounds__(256) void gate_bwd_wgrad_kernel(
    const void* __restrict__ x, const float* __restrict__ dl, int64_t N, int D,
    int E, float* __restrict__ part_w, float* __restrict__ part_b) {
  __shared__ float sdl[kGbTokens][kMaxExperts];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kGbTokens;
  const int nt = static_cast<int>(min<int64_t>(kGbTokens, N - t0));
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x)
    sdl[i / E][i % E] = dl[t0 * E + i];
  __syncthreads();
  const int nch = D / 8;
  const int neb = (E + 7) / 8;
  float* pw = part_w + static_cast<int64_t>(blockIdx.x) * E * D;
  for (int pr = threadIdx.x; pr < nch * neb; pr += blockDim.x) {
    const int c = pr % nch;
    {
      const int e0 = 8 * (pr / nch);
      float acc[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
      for (int tb = 0; tb < nt; tb += kGbBatch) {
        // every row of the batch in flight (past the chunk: its last token's
        // row again, not used)
        float xv[kGbBatch][8];
#pragma unroll
        for (int b = 0; b < kGbBatch; ++b)
          ld8<XB>(x, t0 + (tb + b < nt ? tb + b : nt - 1), D, c, xv[b]);
#pragma unroll
        for (int b = 0; b < kGbBatch; ++b) {
          if (tb + b >= nt) break;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (e0 + i < E) {
              const float d = sdl[tb + b][e0 + i];
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(d, xv[b][j], acc[i][j]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (e0 + i >= E) break;
        float4* q = reinterpret_cast<float4*>(pw + static_cast<int64_t>(e0 + i) * D) + 2 * c;
        q[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        q[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
      }
    }
  }
  for (int i = threadIdx.x; i < E; i += blockDim.x) {
    float s = 0.0f;
    for (int t = 0; t < nt; ++t) s += sdl[t][i];
    part_b[static_cast<int64_t>(blockIdx.x) * E + i] = s;
  }
}

// Fixed-order sum of the chunk partials into dW_g [E][D] (entries
// i < E*D) and dbias [E] (entries E*D + e).  A workgroup takes 32 entries;
// its 8 groups of 32 threads each sum one eighth of the chunks in chunk
// order (loads in batches of 8), and the 8 sums are added in group order:
// a fixed association, the same bits on every run.
__global__ __launch_bounds__(256) void gate_bwd_reduce_kernel(
    const float* __restrict__ part_w, const float* __restrict__ part_b,
    int nchunks, int E, int D, float* __restrict__ dw_gate,
    float* __restrict__ dbias) {
  __shared__ float ps[8][32];
  const int64_t ED = static_cast<int64_t>(E) * D;
  const int64_t nout = ED + (dbias != nullptr ? E : 0);
  const int io = threadIdx.x & 31, seg = threadIdx.x >> 5;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 32 + io;
  const int per = (nchunks + 7) / 8;
  const int c_begin = seg * per, c_end = min(nchunks, c_begin + per);
  float sum = 0.0f;
  if (i < nout) {
    for (int c0 = c_begin; c0 < c_end; c0 += 8) {
      float v[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = c0 + b;
        v[b] = 0.0f;
        if (c < c_end)
          v[b] = i < ED ? part_w[static_cast<int64_t>(c) * ED + i]
                        : part_b[static_cast<int64_t>(c) * E + (i - ED)];
      }
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (c0 + b < c_end) sum += v[b];
    }
  }
  ps[seg][io] = sum;
  __syncthreads();
  if (seg == 0 && i < nout) {
    float t = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) t += ps[g][io];
    if (i < ED)
      dw_gate[i] = t;
    else
      dbias[i - ED] = t;
  }
}

}  // namespace

hipError_t launch_transpose(const void* src, int G, int R, int C, void* dst,
                            hipStream_t stream) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(C, kTile)),
                  static_cast<unsigned>(ceil_div(R, kTile)),
                  static_cast<unsigned>(G));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), R, C,
                     static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_rows(const void* src, const int32_t* row_index,
                       int64_t src_rows, int64_t total, int C, bool gelu,
                       void* dst, hipStream_t stream) {
  if (total == 0 || C == 0) return hipSuccess;
  const int64_t n = total * (C / 8);
  const unsigned grid =
      static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192));
  if (gelu)
    hipLaunchKernelGGL(rows_kernel<true>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), row_index, src_rows,
                       total, C, static_cast<uint16_t*>(dst));
  else
    hipLaunchKernelGGL(rows_kernel<false>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), row_index, src_rows,
                       total, C, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_combine_backward(const void* dy, bool dy_bf16,
                                   const void* y_rows, bool y_bf16,
                                   const int32_t* slot_row, const float* w,
                                   int64_t N, int D, int Kmax, void* dy_rows,
                                   float* dw, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kCbWaves)));
  const dim3 block(64 * kCbWaves);
  if (dy_bf16 && y_bf16)
    hipLaunchKernelGGL((combine_bwd_kernel<true, true>), grid, block, 0, stream,
                       dy, y_rows, slot_row, w, N, D, Kmax, dy_rows, dw);
  else if (dy_bf16)
    hipLaunchKernelGGL((combine_bwd_kernel<true, false>), grid, block, 0, stream,
                       dy, y_rows, slot_row, w, N, D, Kmax, dy_rows, dw);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_bwd_kernel<false, true>), grid, block, 0, stream,
                       dy, y_rows, slot_row, w, N, D, Kmax, dy_rows, dw);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<false, false>), grid, block, 0, stream,
                       dy, y_rows, slot_row, w, N, D, Kmax, dy_rows, dw);
  return hipGetLastError();
}

// Workspace: dl [N][E], padded to 64 floats so that the 16-byte stores of
// the partials stay aligned, then part_w [chunks][E][D], part_b [chunks][E].
size_t gate_backward_workspace_bytes(int64_t N, int E, int D) {
  const int64_t chunks = ceil_div(N, kGbTokens);
  const int64_t dl = (N * E + 63) / 64 * 64;
  return static_cast<size_t>(dl + chunks * E * D + chunks * E) * 4;
}

hipError_t launch_gate_backward(const void* x, bool x_bf16, const float* wg,
                                const float* probs, const int32_t* idx,
                                const float* dw, const int32_t* counts, int B,
                                int T, int D, int E, int Kmax, int K, float alpha,
                                float dloss, bool global, const void* dx_rows,
                                const int32_t* slot_row, const void* dx_shared,
                                bool dx_bf16, void* dx, float* dw_gate,
                                float* dbias, void* workspace,
                                hipStream_t stream) {
  const int64_t N = static_cast<int64_t>(B) * T;
  const int64_t chunks = ceil_div(N, kGbTokens);
  float* dl = static_cast<float*>(workspace);
  float* part_w = dl + (N * E + 63) / 64 * 64;
  float* part_b = part_w + chunks * E * D;
  if (N > 0) {
    const dim3 tgrid(static_cast<unsigned>(ceil_div(N, 256)));
#define MOE_TOKEN_BWD(EP_)                                                   \
    hipLaunchKernelGGL(gate_bwd_token_kernel<EP_>, tgrid, dim3(256), 0, stream, \
                       probs, idx, dw, counts, B, T, E, Kmax, K, alpha, dloss, \
                       global ? 1 : 0, dl)
    if (E <= 8)
      MOE_TOKEN_BWD(8);
    else if (E <= 16)
      MOE_TOKEN_BWD(16);
    else if (E <= 32)
      MOE_TOKEN_BWD(32);
    else
      MOE_TOKEN_BWD(64);
#undef MOE_TOKEN_BWD
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // dW_g / dbias partials: threads = the feature chunks rounded up to
    // whole waves, at most 256
    const int nch = D / 8;
    const int wthreads = min(256, (nch * ((E + 7) / 8) + 63) / 64 * 64);
    if (x_bf16)
      hipLaunchKernelGGL(gate_bwd_wgrad_kernel<true>,
                         dim3(static_cast<unsigned>(chunks)), dim3(wthreads), 0,
                         stream, x, dl, N, D, E, part_w, part_b);
    else
      hipLaunchKernelGGL(gate_bwd_wgrad_kernel<false>,
                         dim3(static_cast<unsigned>(chunks)), dim3(wthreads), 0,
                         stream, x, dl, N, D, E, part_w, part_b);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (dx != nullptr) {
      // E <= 8: W_g's chunk in registers over kDxTokens tokens per thread
      // (16 experts' chunks would be kept in scratch memory)
      const dim3 gt(static_cast<unsigned>(ceil_div(ceil_div(N, kDxTokens) * nch, 256)));
      const dim3 g2(static_cast<unsigned>(ceil_div(N * nch, 256)));
#define MOE_DX(KERNEL, GRID)                                                 \
      hipLaunchKernelGGL(KERNEL, GRID, dim3(256), 0, stream, wg, dl, N, D, E, \
                         Kmax, dx_rows, slot_row, dx_shared, dx)
      if (E <= 8 && dx_bf16)
        MOE_DX((gate_bwd_dx_tok_kernel<true, 8>), gt);
      else if (E <= 8)
        MOE_DX((gate_bwd_dx_tok_kernel<false, 8>), gt);
      else if (dx_bf16)
        MOE_DX(gate_bwd_dx_kernel<true>, g2);
      else
        MOE_DX(gate_bwd_dx_kernel<false>, g2);
#undef MOE_DX
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  const int64_t nout = static_cast<int64_t>(E) * D + (dbias != nullptr ? E : 0);
  hipLaunchKernelGGL(gate_bwd_reduce_kernel,
                     dim3(static_cast<unsigned>(ceil_div(nout, 32))), dim3(256),
                     0, stream, part_w, part_b, static_cast<int>(chunks), E, D,
                     dw_gate, dbias);
  return hipGetLastError();
}

}  // namespace moe
