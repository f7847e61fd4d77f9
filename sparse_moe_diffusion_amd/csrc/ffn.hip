// Grouped expert MLPs of the DiT-MoE layer on gfx950.
//
// "Scaling Diffusion Transformers to 16 Billion Parameters", MoE-DiT eq. MLP:
// each expert is W2 gelu(W1 x); "Scalable Diffusion Models with Transformers
// (DiT)", model architecture: the GELU is the tanh approximation.
//
// moe_grouped_ffn runs two grouped GEMMs over G row groups whose bounds
// live in device memory (no host synchronisation):
//   stage 1:  h = gelu_tanh(A W1[g]^T + b1[g])   A rows gathered by index
//   stage 2:  y = h W2[g]^T + b2[g]
//
// bf16 path (the hot path): one workgroup of 8 waves (two per SIMD) owns a
// 256-token x 256-feature (up-projection) or 256 x 192 (down-projection)
// output tile; each wave accumulates its 128 x 64 or 64 x 96 slice with
// v_mfma_f32_32x32x16_bf16 in fp32.  Operands move from HBM straight into
// LDS with buffer_load ... lds transfers (no staging registers), in 64-wide
// k stages: the next stage is in flight while the current one feeds the
// matrix cores, and its transfers are spread between the MFMAs.  The
// down-projection's large tiles keep a third stage of token rows, so each of
// those transfers has two stages of MFMAs to arrive in.
// Both operands are k-contiguous rows; LDS rows are 128 bytes and the
// 16-byte chunk c of row r sits at slot c ^ swz(r), which keeps the MFMA
// fragment reads free of bank conflicts (measured: zero).  Fragments are
// read one k step ahead of the MFMAs that use them.  Buffer descriptors
// make out-of-range rows and k chunks load as zero, so ragged tiles need no
// branches.  With bf16 output the finished tile goes through LDS and leaves
// in row-contiguous 16-byte stores.
//
// The weight gradients of the backward run the same kernel in a K-grouped
// form: the reduction runs down the token rows of row-major operands, which
// land in LDS as [64 tokens][256 features] stage tiles and reach the matrix
// cores through LDS transpose reads (ds_read_b64_tr_b16).  The backward's
// du GEMM reads W2 as stored (k-major) the same way, on the weight tile only.
//
// The MFMA computes out^T: weight rows are the 32-row "A" operand and token
// rows the "B" operand, so each lane ends up holding 4 consecutive output
// features of one token and stores 8 (bf16) or 16 (fp32) bytes at a time.
//
// Tile order: the bf16 kernels are persistent, about one workgroup per CU;
// workgroups are dealt round-robin to the 8 XCDs, and the workgroups of an
// XCD walk chunks of consecutive tiles; within a group, tiles go in bands of
// about GM row-tiles, feature-tile major, so tiles running at once share both
// their token rows and their weight rows in the XCD's L2.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "gather.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// kEpiCombine: the stage-2 store of the shared experts fused with the
// weighted combine of the routed outputs (one group holding every token).
// kEpiGeluGrad: the product (rounded to bf16 in the staged tile) times
// GELU'(u) at the same position, u read from GemmParams::aux, rounded again
// (backward of the first expert matrix).
enum Epi { kEpiGelu = 0, kEpiStore = 1, kEpiCombine = 2, kEpiGeluGrad = 3 };

// Most slots per token the fused combine takes: top-K routing (K <= 4) uses
// the kernel form with 4 slot columns, Expert Race (Kmax = E <= 16) the one
// with 16 (a larger slot table in LDS).
constexpr int kCombineMaxSlots = 16;

struct GemmParams {
  const void* a;           // activation rows [*][Kd]
  const int32_t* a_index;  // source row of each output row, or null
  const void* w;           // [G][Nd][Kd]
  const float* bias;       // [G][Nd] or null
  void* c;                 // [total][Nd]
  const int64_t* offsets;  // [G+1], device; null: one group of all rows
  int64_t total;
  int G, Nd, Kd;
  // kEpiCombine only: c[t] = this GEMM's (bf16) output for token t plus, in
  // slot order, cmb_w[t][k] * cmb_rows[cmb_slot[t][k]] for the slots >= 0.
  const void* cmb_rows;      // [*][Nd] bf16 routed expert outputs
  const int32_t* cmb_slot;   // [total][cmb_kmax]
  const float* cmb_w;        // [total][cmb_kmax]
  int cmb_kmax;              // 1..kCombineMaxSlots (at most the kernel's CMAX)
  // kEpiGeluGrad only: the pre-activations u [total][Nd] bf16.
  const void* aux;
  // K-grouped form (weight gradients): C[g] [mrows][Nd] fp32 = A[rows g]^T
  // B[rows g], A [total][mrows] and B (in w) [total][Nd] bf16 row-major,
  // rows g = group g's token rows.
  int mrows;
  // K-grouped form split over the reduction: each group's rows are cut
  // into ksplit pieces (multiples of 64 rows but the last) whose products
  // go to separate fp32 partials, C [ksplit][G][mrows][Nd] (0 or 1: no
  // split).
  int ksplit;
  // kEpiGelu with bf16 output: if set, also the pre-activations u = A W^T
  // + bias, [total][Nd] bf16 (kept by a training forward for the backward).
  void* u_out;
  // With a_index: the rows of a.  Index entries outside [0, a_rows) read
  // zero rows (the gathered rows' descriptor spans exactly a_rows rows).
  int64_t a_rows;
  // Large store-form tiles (three token-row stages, plain operands): if
  // set, the last, partial round of tiles is split along k over the
  // workgroups that would otherwise idle, each piece's fp32 partial sums
  // going to this workspace (layout: kSplitHdrBytes of header, then one
  // BM x BN fp32 slot per workgroup), and splitk_tail_kernel finishes
  // those tiles.
  float* sk_ws = nullptr;
};

// The split workspace's header: int64 [0] pieces per tile S (0: no split),
// [1] split tiles R, then per split tile r: [2 + 3 r] first row, [3 + 3 r]
// row end, [4 + 3 r] group << 32 | first feature.  At most 1023 split tiles.
constexpr size_t kSplitHdrBytes = 3 * 8 * 1024;

struct TileLoc {
  int g;
  int64_t row0, row_end;
  int n0;
  int kofs, klen;   // K-grouped form: the split's first token row and row count
};

// tanh-GELU via 0.5 (1 + tanh z) = 1 / (1 + exp(-2z)),
// z = sqrt(2/pi) (u + 0.044715 u^3).  The exponent -2 z log2(e) is formed as
// u (c1 + c2 u^2) with the constants folded, then the hardware exp2.
__device__ __forceinline__ float gelu_tanh(float u) {
  constexpr float kC1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
  constexpr float kC2 = kC1 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(u * fmaf(kC2, u * u, kC1));
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int q = n / 8, r = n % 8;
  const int xcd = pid % 8, j = pid / 8;
  return xcd * q + min(xcd, r) + j;
}

// Tile Lg of a group of mt row-tiles and ntn feature tiles: its row tile m
// and feature tile n.  The row tiles form nb = max(1, round(mt / GM)) bands
// of near-equal size (the first mt % nb bands one row tile larger), each
// walked feature-tile major.  Balanced bands keep a group's last band from
// holding one or two row tiles: such a band's tiles running at once would
// share their token rows but each read weight rows of its own.
template <int GM>
__device__ __forceinline__ void band_tile(int Lg, int mt, int ntn, int& m,
                                          int& n) {
  const int nb = max(1, (mt + GM / 2) / GM);
  const int q = mt / nb, r = mt - q * nb;
  const int big = r * (q + 1) * ntn;   // tiles of the larger bands
  int m_first, gm, rem;
  if (Lg < big) {
    const int band = Lg / ((q + 1) * ntn);
    m_first = band * (q + 1);
    gm = q + 1;
    rem = Lg - band * (q + 1) * ntn;
  } else {
    const int band = (Lg - big) / (q * ntn);
    m_first = r * (q + 1) + band * q;
    gm = q;
    rem = Lg - big - band * q * ntn;
  }
  m = m_first + rem % gm;
  n = rem / gm;
}

template <int BM, int BN, int GM>
__device__ __forceinline__ bool locate_tile(const GemmParams& p, int L,
                                            TileLoc& loc) {
  const int ntn = (p.Nd + BN - 1) / BN;
  for (int g = 0; g < p.G; ++g) {
    int64_t r0 = p.offsets[g], r1 = p.offsets[g + 1];
    r0 = min(max(r0, int64_t(0)), p.total);
    r1 = min(max(r1, r0), p.total);
    const int mt = static_cast<int>((r1 - r0 + BM - 1) / BM);
    const int tiles = mt * ntn;
    if (L < tiles) {
      int m, n;
      band_tile<GM>(L, mt, ntn, m, n);
      // All wave-uniform: keep them in scalar registers.
      loc.g = __builtin_amdgcn_readfirstlane(g);
      loc.row0 = uniform64(r0 + static_cast<int64_t>(m) * BM);
      loc.row_end = uniform64(r1);
      loc.n0 = __builtin_amdgcn_readfirstlane(n * BN);
      return true;
    }
    L -= tiles;
  }
  return false;
}

// Group table of the persistent kernels, in LDS: for every group g its
// clamped row range [row0, row_end) and the index of its first tile; entry G
// of the first-tile column holds the total tile count.  Built once per
// workgroup, so that finding a tile reads no global memory: a global load at
// a tile boundary would wait on the previous tile's output stores (the
// vector-memory counter retires in order).
constexpr int kTabCol = kMaxFfnGroups + 1;
constexpr int kTabInts = 3 * kTabCol;

template <int BM, int BN>
__device__ void build_group_table(const GemmParams& p, int32_t* tab, int wave,
                                  int lane) {
  if (wave == 0) {
    const int ntn = (p.Nd + BN - 1) / BN;
    int base = 0;
    for (int c = 0; c < p.G; c += 64) {
      const int g = c + lane;
      int64_t r0 = 0, r1 = 0;
      int tiles = 0;
      if (g < p.G) {
        r0 = p.offsets ? min(max(p.offsets[g], int64_t(0)), p.total) : 0;
        r1 = p.offsets ? min(max(p.offsets[g + 1], r0), p.total) : p.total;
        tiles = static_cast<int>((r1 - r0 + BM - 1) / BM) * ntn;
      }
      int inc = tiles;   // inclusive scan of tile counts over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d);
        if (lane >= d) inc += v;
      }
      if (g < p.G) {
        tab[g] = static_cast<int32_t>(r0);
        tab[kTabCol + g] = static_cast<int32_t>(r1);
        tab[2 * kTabCol + g] = base + inc - tiles;
      }
      base += __shfl(inc, 63);
    }
    if (lane == 0) tab[2 * kTabCol + p.G] = base;
  }
  __syncthreads();
}

// Tile L of the launch from the group table (same order as locate_tile).
// Every lane of the wave must take part.  Table entries are read at
// wave-uniform addresses and declared uniform, so that the branches and the
// descriptors built from them stay scalar.
template <int BM, int BN, int GM>
__device__ __forceinline__ bool locate_tile_tab(const GemmParams& p,
                                                const int32_t* tab, int lane,
                                                int L, TileLoc& loc) {
  const int32_t* const first = tab + 2 * kTabCol;
  if (L >= __builtin_amdgcn_readfirstlane(first[p.G])) return false;
  // The one group whose tile range holds L (empty groups have none).
  int g = 0;
  for (int c = 0; c < p.G; c += 64) {
    const int gg = c + lane;
    const bool in = gg < p.G && first[gg] <= L && L < first[gg + 1];
    const uint64_t m = __ballot(in);
    if (m != 0) {
      g = c + __builtin_ctzll(m);
      break;
    }
  }
  g = __builtin_amdgcn_readfirstlane(g);
  const int r0 = __builtin_amdgcn_readfirstlane(tab[g]);
  const int r1 = __builtin_amdgcn_readfirstlane(tab[kTabCol + g]);
  const int ntn = (p.Nd + BN - 1) / BN;
  const int mt = (r1 - r0 + BM - 1) / BM;
  const int Lg = L - __builtin_amdgcn_readfirstlane(first[g]);
  int m, n;
  band_tile<GM>(Lg, mt, ntn, m, n);
  loc.g = g;
  loc.row0 = uniform64(static_cast<int64_t>(r0) + static_cast<int64_t>(m) * BM);
  loc.row_end = uniform64(r1);
  loc.n0 = __builtin_amdgcn_readfirstlane(n * BN);
  return true;
}

// d/du of gelu_tanh: with s = 0.5 (1 + tanh z) = 1 / (1 + exp(-2z)),
// gelu'(u) = s + 2 sqrt(2/pi) u s (1 - s) (1 + 3 0.044715 u^2).
__device__ __forceinline__ float gelu_tanh_grad(float u) {
  constexpr float kC1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
  constexpr float kC2 = kC1 * 0.044715f;
  const float s = __builtin_amdgcn_rcpf(
      1.0f + __builtin_amdgcn_exp2f(u * fmaf(kC2, u * u, kC1)));
  return fmaf(2.0f * 0.7978845608028654f * u * s * (1.0f - s),
              fmaf(3.0f * 0.044715f, u * u, 1.0f), s);
}

// K-grouped form: the group table holds each group's token rows of the
// row-major operands, [kofs, kofs + klen) (offsets clamped to [0, total]).
__device__ __forceinline__ void build_kseg_table(const GemmParams& p,
                                                 int32_t* tab, int wave,
                                                 int lane) {
  if (wave == 0) {
    for (int c = 0; c < p.G; c += 64) {
      const int g = c + lane;
      if (g < p.G) {
        const int64_t r0 = p.offsets ? min(max(p.offsets[g], int64_t(0)), p.total) : 0;
        const int64_t r1 = p.offsets ? min(max(p.offsets[g + 1], r0), p.total) : p.total;
        tab[g] = static_cast<int>(r0);
        tab[kTabCol + g] = static_cast<int>(r1 - r0);
      }
    }
  }
  __syncthreads();
}

// Tile L of a K-grouped launch: virtual group v = L / (row tiles x feature
// tiles) is split v / G of group g = v % G, bands of about GM row tiles
// within it.  Output rows are v * mrows + row (the split's partial).
template <int BM, int BN, int GM>
__device__ __forceinline__ bool locate_tile_kg(const GemmParams& p,
                                               const int32_t* tab, int L,
                                               TileLoc& loc) {
  const int mt = (p.mrows + BM - 1) / BM;
  const int ntn = (p.Nd + BN - 1) / BN;
  const int per = mt * ntn;
  const int S = p.ksplit > 1 ? p.ksplit : 1;
  if (L >= S * p.G * per) return false;
  const int v = L / per;
  const int g = v % p.G, sp = v / p.G;
  const int Lg = L - v * per;
  int m, n;
  band_tile<GM>(Lg, mt, ntn, m, n);
  const int64_t base = static_cast<int64_t>(v) * p.mrows;
  loc.g = __builtin_amdgcn_readfirstlane(v);
  loc.row0 = uniform64(base + static_cast<int64_t>(m) * BM);
  loc.row_end = uniform64(base + p.mrows);
  loc.n0 = __builtin_amdgcn_readfirstlane(n * BN);
  // the split's piece of the group's rows (a multiple of 64 rows except
  // the last piece, possibly empty: the partial is then zero)
  const int kofs = __builtin_amdgcn_readfirstlane(tab[g]);
  const int klen = __builtin_amdgcn_readfirstlane(tab[kTabCol + g]);
  const int cs = ((klen + 63) / 64 + S - 1) / S * 64;
  loc.kofs = kofs + sp * cs;
  loc.klen = max(0, min(cs, klen - sp * cs));
  return true;
}

template <bool KG, int BM, int BN, int GM>
__device__ __forceinline__ bool locate_any(const GemmParams& p,
                                           const int32_t* tab, int lane, int L,
                                           TileLoc& loc) {
  if constexpr (KG) {
    return locate_tile_kg<BM, BN, GM>(p, tab, L, loc);
  } else {
    loc.kofs = 0;
    loc.klen = 0;
    return locate_tile_tab<BM, BN, GM>(p, tab, lane, L, loc);
  }
}

// Bias and activation of 4 consecutive output features f..f+3 of group g,
// output row `row`.  BIAS: whether to add p.bias here; the staged bf16
// epilogue adds it to the accumulators beforehand and passes false, so that
// its loops over a tile's outputs hold no branch (the activations of
// consecutive groups of 4 can then be interleaved).
template <int EPI, bool BIAS>
__device__ __forceinline__ f32x4 finish4(const GemmParams& p, int g,
                                         int64_t row, int f, f32x4 v) {
  if constexpr (BIAS) {
    const float* b = p.bias + static_cast<int64_t>(g) * p.Nd + f;
    v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
  }
  if constexpr (EPI == kEpiGelu) {
    v[0] = gelu_tanh(v[0]); v[1] = gelu_tanh(v[1]);
    v[2] = gelu_tanh(v[2]); v[3] = gelu_tanh(v[3]);
  }
  if constexpr (EPI == kEpiGeluGrad) {
    // bf16 output only: the factor gelu'(u) is applied in the copy-out
    // loop, where u is read row-contiguous.
    (void)row;
  }
  return v;
}

template <int EPI, bool OUT_BF16>
__device__ __forceinline__ void store4(const GemmParams& p, int g, int64_t row,
                                       int f, f32x4 v) {
  v = p.bias != nullptr ? finish4<EPI, true>(p, g, row, f, v)
                        : finish4<EPI, false>(p, g, row, f, v);
  if constexpr (OUT_BF16) {
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.c) + row * p.Nd + f) = o;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.c) + row * p.Nd + f) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ------------------------------------------------------- bf16 / MFMA ----

constexpr int kBK = 64, kGM = 8;   // kGM: band of the fp32 path

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }


typedef __attribute__((address_space(3))) void lds_void;

// Wait until this wave's global->LDS transfers have landed (vmcnt = 0) and
// its LDS reads have returned (lgkmcnt = 0), then the workgroup barrier:
// afterwards every wave may read the new stage and refill the old one.
__device__ __forceinline__ void stage_barrier() {
  // s_waitcnt fields on gfx9: vmcnt [3:0] and [15:14], expcnt [6:4],
  // lgkmcnt [11:8]; expcnt all-ones leaves it unconstrained.
  __builtin_amdgcn_s_waitcnt(0x7 << 4);
  __builtin_amdgcn_s_barrier();
}

// The same with the wave's newest KEEP transfers still allowed in flight
// (the next-but-one stage of a three-stage ring): vmcnt(KEEP).
template <int KEEP>
__device__ __forceinline__ void stage_barrier_keep() {
  static_assert(KEEP >= 0 && KEEP < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((KEEP & 0xf) | ((KEEP >> 4) << 14) | (0x7 << 4));
  __builtin_amdgcn_s_barrier();
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((lds_void*)(const_cast<void*>(p))));
}

// MFMA fragment of a [k][rows] LDS tile (rows contiguous within each k row,
// row pitch PITCH bytes): 8 consecutive k values of one row, from two
// transpose reads of 4 k rows each.  In every 16-lane group the transpose
// read hands lane j element y of the 8-byte piece addressed by lane
// 4y + j/4, position j % 4; the caller's per-lane address makes that piece
// (k row 4y.., rows 4(j/4)..) so lane j ends up with row j's k values.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int PITCH>
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint16_t* base, int off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  char* b = const_cast<char*>(reinterpret_cast<const char*>(base)) + off;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + 4 * PITCH));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3,
                                                            4, 5, 6, 7));
}

// SZ bytes per lane (16 or 4) from global memory straight into LDS: lane l
// of the wave writes bytes [SZ l, SZ l + SZ) of the block at LDS byte
// address `dst`.  The destination reaches the instruction as a plain
// wave-uniform 32-bit address, so the compiler cannot attribute the
// transfer to a particular LDS region and adds no waits of its own before
// LDS reads (its alias tracking would otherwise wait for transfers into
// other stages); the kernel orders every transfer against its readers
// explicitly (vmcnt wait, then workgroup barrier).
template <int SZ>
__device__ __forceinline__ void dma_untracked(__amdgpu_buffer_rsrc_t r,
                                              uint32_t dst, uint32_t off) {
  static_assert(SZ == 16 || SZ == 4, "16- or 4-byte transfers");
  lds_void* const a = (lds_void*)(
      static_cast<uintptr_t>(__builtin_amdgcn_readfirstlane(dst)));
  if constexpr (SZ == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, a, 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, a, 4, off, 0, 0, 0);
}

// The same 16-byte transfer, written out (for the K-grouped form): the
// compiler waits for every outstanding transfer before each LDS transpose
// read that follows a transfer it can see, which would stall the pipeline
// at every k step.  The descriptor is rebuilt from a uniform base and byte
// count (stride 0, the flags make_rsrc uses); offsets at or past the count
// read zero.  The transfer writes no register, and the kernel orders it
// against its readers itself (vmcnt wait, then workgroup barrier).  The
// compiler's hazard checks do not see into the block, so it carries its own
// wait states: the descriptor's SGPRs may come straight from
// v_readfirstlane, and a VMEM instruction needs 5 wait states after a VALU
// write of an SGPR it reads (the M0 write needs 1).  The M0 write and
// s_nop 4 give 6.
// M0 is a reserved register: the compiler neither saves it around the block
// nor learns that the block changed it (hipcc warns of the clobber).  That is
// safe only because the two forms that use this transfer (K-grouped, and
// k-major weights) contain no compiler-built LDS transfer, the only M0
// reader in these kernels: their gathered-row fetch is compiled out, and
// they take no prefetch and no combine table (static checks in the
// kernel), so no value of the compiler's own is live in M0 across the
// block.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16_raw(const char* base, uint32_t bytes,
                                          uint32_t dst, uint32_t off) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(b));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(off), "s"(r)
      : "memory", "m0");
}

// Tile of BM token rows x BN output features; waves form a WT x WF grid, each
// owning (BM/WT) tokens x (BN/WF) features as (BN/WF/32) x (BM/WT/32)
// v_mfma_f32_32x32x16_bf16 tiles.  LDS holds two k-stages of both operands
// (rows of 64 k = 128 bytes, 16-byte chunks swizzled by swz(row)).  Each
// k-stage is loaded by (BM+BN)/8 wave-wide 1 KB DMA transfers; lane l of a
// transfer covering rows r0..r0+7 fetches chunk (l % 8) ^ swz(r0 + l / 8) of
// row r0 + l / 8, which is exactly the swizzled LDS slot it lands in.  One
// workgroup per CU.
//
// BT: the weight operand is stored k-major, [G][Kd][Nd] (a forward weight
// read as its own transpose), and is brought to LDS and read as the
// K-grouped form reads its operands ([64][BN] stage tiles, transpose reads);
// the token operand stays row-major and is read in place (no gather).
//
// NST: token-row k stages held in LDS (the weight rows always have two).
// With 2, stage k + 1 of both operands streams in while stage k is
// multiplied.  With 3, stage k + 2 of the token rows streams in (with stage
// k + 1 of the weight rows, issued first), so each token-row transfer has
// two stages of MFMAs to arrive in: the wait at a stage's end leaves the
// wave's newest QA transfers (the token rows of stage k + 2) in flight.
template <int EPI, bool OUT_BF16, int BM, int BN, int WT, int WF, int GM,
          bool PF, bool KG = false, int CMAX = 4, bool BT = false, int NST = 2>
__global__ __launch_bounds__(64 * WT * WF, 1) void gemm_bf16_kernel(GemmParams p) {
  static_assert(EPI != kEpiGeluGrad || OUT_BF16, "gelu'(u) is applied on bf16 output");
  static_assert(NST == 2 || (NST == 3 && !PF && !KG && !BT),
                "three token-row stages: plain operands, no prefetch transfers "
                "in the wait count");
  static_assert(!BT || (!KG && !PF && EPI != kEpiCombine && (BN == 128 || BN == 256)),
                "k-major weights: whole 256- or 512-byte k rows, no prefetch, "
                "no combine");
  static_assert(!KG || (!OUT_BF16 && !PF && EPI == kEpiStore),
                "the K-grouped form writes fp32 without prefetch");
  static_assert(!KG || (BM == 256 && BN == 256),
                "the K-grouped stage tiles are two 512-byte k rows per transfer");
  constexpr int kWaves = WT * WF;
  constexpr int TB = BM / WT / 32;   // token blocks per wave
  constexpr int FB = BN / WF / 32;   // feature blocks per wave
  constexpr int NQ = (BM + BN) / 8 / kWaves;  // DMA transfers per wave per stage
  constexpr int QA = BM / 8 / kWaves;         // ... of which token rows
  static_assert((BM + BN) % (8 * kWaves) == 0 && BM % (8 * kWaves) == 0,
                "whole transfers");
  // LDS: the two k stages during the main loop; afterwards (bf16 output)
  // the finished tile, row-major with a 16-byte pad per row, so that it
  // leaves in whole-row 16-byte-per-lane stores.
  constexpr int kStageBytes = (NST * BM + 2 * BN) * kBK * 2;
  constexpr int kOutPitch = BN + 8;   // staged row pitch, elements
  constexpr int kOutBytes = OUT_BF16 ? BM * kOutPitch * 2 : 0;
  constexpr int kMainElems = (kStageBytes > kOutBytes ? kStageBytes : kOutBytes) / 2;
  constexpr int kPfElems = PF ? 256 : 0;
  // slot rows and weights, [BM][CMAX] each, and (CMAX > 4) each row's
  // count of non-empty slots.  With three token-row stages and CMAX > 4
  // they do not fit beside the stages: they are loaded after the main loop
  // into the idle stage area, past the staged output tile (kLateCmb).
  constexpr bool kLateCmb = EPI == kEpiCombine && NST == 3 && CMAX > 4;
  constexpr int kCmbInts =
      EPI == kEpiCombine ? 2 * BM * CMAX + (CMAX > 4 ? BM : 0) : 0;
  static_assert(!kLateCmb || kOutBytes + kCmbInts * 4 <= kMainElems * 2,
                "the late slot table fits in the stage area");
  static_assert(EPI != kEpiCombine || OUT_BF16, "the combine writes bf16");
  __shared__ __attribute__((aligned(1024)))
  uint16_t lds[kMainElems + kPfElems + 2 * (kTabInts + 2 * BM + (kLateCmb ? 0 : kCmbInts))];
  int32_t* const tab = reinterpret_cast<int32_t*>(lds + kMainElems + kPfElems);
  int32_t* const sidx = tab + kTabInts;   // 2 x BM gathered source rows
  // kEpiCombine: the tile's slot rows and weights, [BM][cmb_kmax] each
  // (cmb_kmax <= CMAX).
  int32_t* const cslot =
      kLateCmb ? reinterpret_cast<int32_t*>(lds + kOutBytes / 2) : sidx + 2 * BM;
  float* const cwt = reinterpret_cast<float*>(cslot + BM * CMAX);
  int32_t* const ccnt = cslot + 2 * BM * CMAX;
  // Token-row stage s at lds + s BM kBK, then the two weight-row stages.
  uint16_t* const sA0 = lds;
  uint16_t* const sA1 = sA0 + BM * kBK;
  uint16_t* const sA2 = sA1 + BM * kBK;   // NST == 3 only
  uint16_t* const sB0 = lds + NST * BM * kBK;
  uint16_t* const sB1 = sB0 + BN * kBK;

  // The same as LDS byte addresses, for the transfers.
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t bA0 = lds0, bA1 = bA0 + BM * kBK * 2, bA2 = bA1 + BM * kBK * 2;
  const uint32_t bB0 = lds0 + NST * BM * kBK * 2, bB1 = bB0 + BN * kBK * 2;
  const uint32_t bPf = lds0 + kMainElems * 2;
  const uint32_t bIdx = bPf + kPfElems * 2 + kTabInts * 4;
  const uint32_t bCmb = kLateCmb ? lds0 + kOutBytes : bIdx + 2 * BM * 4;

  // Persistent: the grid is a multiple of 8 workgroups, about one per CU,
  // dealt round-robin to the 8 XCDs.  The pw workgroups of one XCD take
  // chunks of pw consecutive tiles (chunks dealt round-robin to the XCDs), so
  // the tiles running at once on an XCD are neighbours in tile order.  The
  // loop ends when the tile index passes the last tile of the last group.
  const int tid0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int wt = wave % WT;   // token slice of the tile
  const int wf = wave / WT;   // feature slice of the tile
  const int Kd0 = p.Kd;
  const uint32_t row_bytes0 = static_cast<uint32_t>(Kd0) * 2u;
  if constexpr (KG)
    build_kseg_table(p, tab, wave, tid0 & 63);
  else
    build_group_table<BM, BN>(p, tab, wave, tid0 & 63);

  // Split of the last round (see GemmParams::sk_ws): T tiles on Gw
  // workgroups are F whole rounds and R more tiles.  With S = min(Gw / R,
  // k stages) >= 2 and R within the header (at most 1023 tiles), workgroup
  // w < R S takes, after its F tiles, piece w % S of the k stages of tile
  // F Gw + w / S.
  constexpr bool kCanSplit = EPI == kEpiStore && NST == 3 && !KG && !BT && !PF;
  int skS = 0, skF = 0, skR = 0, piece_s = -1;
  const int nkt = (Kd0 + kBK - 1) / kBK;
  if constexpr (kCanSplit) {
    if (p.sk_ws != nullptr && p.a_index == nullptr) {
      const int T = __builtin_amdgcn_readfirstlane(tab[2 * kTabCol + p.G]);
      const int Gw = gridDim.x;
      const int F = T / Gw, R = T - F * Gw;
      const int S = R > 0 ? min(Gw / R, nkt) : 0;
      if (S >= 2 && R <= 1023) {
        skS = S;
        skF = F;
        skR = R;
      }
      if (blockIdx.x == 0 && tid0 == 0) {
        int64_t* const h = reinterpret_cast<int64_t*>(p.sk_ws);
        h[0] = skS;
        h[1] = skR;
      }
    }
  }

  // Token rows: gathered through a_index from the whole activation matrix,
  // or read in place from the tile's first row.  Rows past the group end
  // re-read row 0 (gather) or the tile's first row; their results are never
  // stored.  In gather mode the tile's source rows sit in LDS buffer
  // (tile count & 1) of sidx: the next tile's are transferred there before
  // this tile's first k stage, so a tile starts without waiting on global
  // memory.
  // (never in the K-grouped and k-major forms: their transfers write M0
  // themselves, see dma16_raw)
  const bool gather = !KG && !BT && p.a_index != nullptr;
#define MOE_FETCH_ROWS(L, B, LANE)                                           \
  do {                                                                       \
    if (wave < BM / 64) {                                                    \
      const uint32_t n_ =                                                    \
          static_cast<uint32_t>(min(static_cast<int>((L).row_end - (L).row0), BM)); \
      const __amdgpu_buffer_rsrc_t rs_ = make_rsrc(                          \
          reinterpret_cast<const void*>(uniform64(                           \
              reinterpret_cast<int64_t>(p.a_index + (L).row0))),             \
          __builtin_amdgcn_readfirstlane(n_ * 4u));                          \
      dma_untracked<4>(rs_, bIdx + ((B) * BM + wave * 64) * 4,               \
                       static_cast<uint32_t>(wave * 64 + (LANE)) * 4u);      \
    }                                                                        \
  } while (0)
  const int pj = blockIdx.x >> 3, pxcd = blockIdx.x & 7, pw = gridDim.x >> 3;
  int pc = pxcd, it = 0;
  TileLoc loc;
  // The next tile of this workgroup: its share of the whole rounds, then
  // (split) its piece of a tile of the last round.
#define MOE_NEXT_TILE(LANE)                                                  \
  do {                                                                       \
    const int l_ = pc * pw + pj;                                             \
    have = (skS == 0 || l_ < skF * static_cast<int>(gridDim.x)) &&           \
           locate_any<KG, BM, BN, GM>(p, tab, (LANE), l_, loc);              \
    if constexpr (kCanSplit) {                                               \
      if (piece_s >= 0) {                                                    \
        have = false;                                                        \
      } else if (!have && skS > 0 &&                                         \
                 static_cast<int>(blockIdx.x) < skR * skS) {                 \
        piece_s = static_cast<int>(blockIdx.x) % skS;                        \
        have = locate_any<KG, BM, BN, GM>(                                   \
            p, tab, (LANE),                                                  \
            skF * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x) / skS, \
            loc);                                                            \
      }                                                                      \
    }                                                                        \
  } while (0)
  bool have = false;
  MOE_NEXT_TILE(tid0 & 63);
  if (gather && have) MOE_FETCH_ROWS(loc, 0, tid0 & 63);
  stage_barrier();
  while (have) {
  // A fresh, opaque copy of the thread index per tile: no lane-dependent
  // value is hoisted out of the tile loop (it would stay live through the
  // main loop and spill).
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  // The previous tile's readers of the LDS are done.
  __builtin_amdgcn_s_barrier();

  // Reduction length of this tile: the feature width, or in the K-grouped
  // form this split's piece of the group's token rows.  The K-grouped
  // operands are row-major [rows][C] (C = mrows for A, Nd for W): a k stage
  // is 64 token rows, kept in LDS as [64][BM] and [64][BN] tiles.
  const int Kd = KG ? loc.klen : Kd0;
  const uint32_t row_bytes = row_bytes0;
  // A piece of a split tile: k stages [pk0, pk1) of it.  Its operand
  // descriptors start pk0 stages into every row, and its reduction length Kl
  // ends at the piece (or at Kd), so the k-tail checks below zero-fill
  // whatever lies past it.  Otherwise Kl = Kd.
  const bool piece = kCanSplit && piece_s >= 0;
  const int pk0 = piece ? piece_s * nkt / skS : 0;
  const int pk1 = piece ? (piece_s + 1) * nkt / skS : nkt;
  const int Kl = piece ? min(Kd - pk0 * kBK, (pk1 - pk0) * kBK) : Kd;
  const int64_t kshift = piece ? static_cast<int64_t>(pk0) * kBK : 0;
  const uint32_t kstep_a = static_cast<uint32_t>(p.mrows) * 128u;   // KG only
  const uint32_t kstep_b = static_cast<uint32_t>(p.Nd) * 128u;
  const int64_t kg_m = KG ? loc.row0 - static_cast<int64_t>(loc.g) * p.mrows : 0;
  const uint16_t* a_base =
      static_cast<const uint16_t*>(p.a) +
      (gather ? int64_t(0)
              : KG ? static_cast<int64_t>(loc.kofs) * p.mrows + kg_m
                   : loc.row0 * Kd + kshift);
  // KG: from the tile's first feature of the piece's first row to the end
  // of its last row.  Rows past the piece read zero; tile features past the
  // operand's C read the next row's (finite) values, which only reach
  // output rows and features that are not stored.
  const int64_t kg_a =
      KG ? (static_cast<int64_t>(loc.klen) * p.mrows - kg_m) * 2 : 0;
  const uint32_t a_bytes =
      gather ? static_cast<uint32_t>(p.a_rows) * row_bytes
      : KG   ? static_cast<uint32_t>(kg_a > 0 ? kg_a : 0)
             : static_cast<uint32_t>(min(static_cast<int>(loc.row_end - loc.row0), BM)) *
                       row_bytes -
                   static_cast<uint32_t>(kshift * 2);
  const __amdgpu_buffer_rsrc_t rsA =
      make_rsrc(reinterpret_cast<const void*>(
                    uniform64(reinterpret_cast<int64_t>(a_base))),
                __builtin_amdgcn_readfirstlane(a_bytes));
  // Weight rows of group g: features past Nd fall outside the descriptor.
  // BT: group g's [Kd][Nd] block from the tile's first feature of k row 0
  // to its end; a stage's 64 k rows lie at a byte offset of 128 Nd per
  // stage from there, so k rows past Kd fall outside the range and read
  // zero (features past Nd read the next row's values, which only reach
  // features that are not stored).
  const uint16_t* w_base =
      static_cast<const uint16_t*>(p.w) +
      (KG   ? static_cast<int64_t>(loc.kofs) * p.Nd + loc.n0
       : BT ? static_cast<int64_t>(loc.g) * Kd * p.Nd + loc.n0
            : (static_cast<int64_t>(loc.g) * p.Nd + loc.n0) * Kd + kshift);
  const int64_t kg_w =
      KG   ? (static_cast<int64_t>(loc.klen) * p.Nd - loc.n0) * 2
      : BT ? (static_cast<int64_t>(Kd) * p.Nd - loc.n0) * 2
           : 0;
  const uint32_t w_bytes =
      (KG || BT) ? static_cast<uint32_t>(kg_w > 0 ? kg_w : 0)
                 : static_cast<uint32_t>(min(p.Nd - loc.n0, BN)) * row_bytes -
                       static_cast<uint32_t>(kshift * 2);
  const __amdgpu_buffer_rsrc_t rsB =
      make_rsrc(reinterpret_cast<const void*>(
                    uniform64(reinterpret_cast<int64_t>(w_base))),
                __builtin_amdgcn_readfirstlane(w_bytes));
  const char* const kg_abase =
      reinterpret_cast<const char*>(uniform64(reinterpret_cast<int64_t>(a_base)));
  const char* const kg_wbase =
      reinterpret_cast<const char*>(uniform64(reinterpret_cast<int64_t>(w_base)));

  // Per DMA transfer q of this wave: byte offset of this lane's chunk at
  // k = 0, the chunk's k index, and the LDS destination (elements).
  uint32_t goff[NQ];
  uint32_t ldst[NQ];   // LDS byte offset of the transfer in its stage
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = wave + kWaves * q;          // transfer index in the stage
    const bool isA = q < QA;                  // uniform across the wave
    if (KG || (BT && !isA)) {
      // 1 KB of the operand's [64][R] stage tile per transfer: lane l lands
      // at byte 16 l of it, i.e. k row kr, 16-byte slot pc, which holds
      // chunk pc ^ 4 (kr % 4) of that token row (so the transpose reads of
      // four consecutive k rows hit four different bank quarters).
      const int ta = isA ? t : t - BM / 8;
      const int rb = (isA ? BM : BN) * 2;
      const int byte = ta * 1024 + lane * 16;
      const int kr = byte / rb;
      const int pc = (byte - kr * rb) / 16;
      const int lc = pc ^ (4 * (kr & 3));
      ldst[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ta * 1024));
      goff[q] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(isA ? p.mrows : p.Nd) * 2u +
                static_cast<uint32_t>(lc) * 16u;
      continue;
    }
    const int r0 = (isA ? t : t - BM / 8) * 8;
    const int r = r0 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    ldst[q] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(r0 * kBK * 2));
    if (isA) {
      const bool valid = loc.row0 + r < loc.row_end;
      goff[q] = gather ? gather_row_offset(sidx[(it & 1) * BM + r],
                                           static_cast<uint32_t>(p.a_rows),
                                           row_bytes, c * 16u)
                       : static_cast<uint32_t>(valid ? r : 0) * row_bytes +
                             c * 16u;
    } else {
      goff[q] = static_cast<uint32_t>(r) * row_bytes + c * 16u;
    }
  }

  const int nk = (Kl + kBK - 1) / kBK;

  // L2 prefetch (PF, in-place token rows only): the tiles an XCD runs at once
  // read the same row chunks at about the same time, so without it they all
  // wait on the same misses.  Each tile touches one dword of its share of the
  // rows two stages ahead: token rows split by feature tile (all feature
  // tiles of a row-tile run together), weight rows split by row-tile index
  // mod 4.  Wave 0 touches token rows, wave 1 weight rows; the landing area
  // in LDS is never read.
  uint32_t pf_off = kOutOfRange;
  __amdgpu_buffer_rsrc_t pf_rs = rsB;
  if constexpr (PF) {
    const int ntn = (p.Nd + BN - 1) / BN;
    if (wave == 0) {
      const int r = (loc.n0 / BN) + ntn * lane;
      pf_rs = rsA;
      if (!gather && r < BM) pf_off = static_cast<uint32_t>(r) * row_bytes;
    } else if (wave == 1) {
      const int r = static_cast<int>((loc.row0 / BM) & 3) + 4 * lane;
      if (r < BN) pf_off = static_cast<uint32_t>(r) * row_bytes;
    }
  }
  const uint32_t pf_lds = bPf + (wave & 1) * 256;
#define MOE_PREFETCH(KT)                                                     \
  do {                                                                       \
    if constexpr (PF) {                                                      \
      if (wave < 2) {                                                        \
        const int pkt_ = (KT);                                               \
        const uint32_t o_ = (pf_off == kOutOfRange || pkt_ * kBK >= Kl)      \
                                ? kOutOfRange                                \
                                : pf_off + static_cast<uint32_t>(pkt_) * (kBK * 2); \
        dma_untracked<4>(pf_rs, pf_lds, o_);                                 \
      }                                                                      \
    }                                                                        \
  } while (0)

// DMA transfers Q0 <= q < Q1 of k-stage KT into the LDS buffers at byte
// addresses DA / DB.
// K-grouped form: the descriptors' base moves to the stage's first token
// row and their range shrinks with it, so rows past the piece read zero and
// the per-lane offsets stay fixed (held in registers for the whole tile).
#define MOE_ISSUE(KT, DA, DB, Q0, Q1)                                        \
  do {                                                                       \
    const int ikt_ = (KT);                                                   \
    if constexpr (KG) {                                                      \
      const uint32_t sa_ = static_cast<uint32_t>(ikt_) * kstep_a;            \
      const uint32_t sb_ = static_cast<uint32_t>(ikt_) * kstep_b;            \
      _Pragma("unroll") for (int q = (Q0); q < (Q1); ++q) {                  \
        if (q < QA)                                                          \
          dma16_raw(kg_abase + sa_, a_bytes > sa_ ? a_bytes - sa_ : 0u,      \
                    (DA) + ldst[q], goff[q]);                                \
        else                                                                 \
          dma16_raw(kg_wbase + sb_, w_bytes > sb_ ? w_bytes - sb_ : 0u,      \
                    (DB) + ldst[q], goff[q]);                                \
      }                                                                      \
    } else if constexpr (BT) {                                               \
      /* every transfer written out (the compiler would otherwise wait for */ \
      /* builtin transfers before the weight's transpose reads); the      */ \
      /* weight's k stage is a byte offset from k row 0, so k rows past   */ \
      /* Kd fall outside the descriptor and read zero                     */ \
      const bool full_ = (ikt_ + 1) * kBK <= Kl;                             \
      const uint32_t sb_ = static_cast<uint32_t>(ikt_) * kstep_b;            \
      _Pragma("unroll") for (int q = (Q0); q < (Q1); ++q) {                  \
        if (q < QA) {                                                        \
          uint32_t off_ = goff[q] + static_cast<uint32_t>(ikt_) * (kBK * 2); \
          if (!full_) {                                                      \
            const int r_ = (wave + kWaves * q) * 8 + (lane >> 3);            \
            const int c_ = (lane & 7) ^ swz(r_);                             \
            if (ikt_ * kBK + c_ * 8 >= Kl) off_ = kOutOfRange;               \
          }                                                                  \
          dma16_raw(kg_abase, a_bytes, (DA) + ldst[q], off_);                \
        } else {                                                             \
          dma16_raw(kg_wbase, w_bytes, (DB) + ldst[q], goff[q] + sb_);       \
        }                                                                    \
      }                                                                      \
    } else {                                                                 \
      const bool full_ = (ikt_ + 1) * kBK <= Kl;                             \
      _Pragma("unroll") for (int q = (Q0); q < (Q1); ++q) {                  \
        const bool isA_ = q < QA;                                            \
        uint32_t off_ = goff[q] + static_cast<uint32_t>(ikt_) * (kBK * 2);   \
        if (!full_) {                                                        \
          /* this lane's chunk of the transfer: row r, k index 8 c */        \
          const int t_ = wave + kWaves * q;                                  \
          const int r_ = (isA_ ? t_ : t_ - BM / 8) * 8 + (lane >> 3);        \
          const int c_ = (lane & 7) ^ swz(r_);                               \
          if (ikt_ * kBK + c_ * 8 >= Kl) off_ = kOutOfRange;                 \
        }                                                                    \
        dma_untracked<16>(isA_ ? rsA : rsB, (isA_ ? (DA) : (DB)) + ldst[q], off_); \
      }                                                                      \
    }                                                                        \
  } while (0)

  // NST == 3: transfers in issue order i (weight rows first): i < QB are
  // weight-row transfers QA + i of stage KTB into DB, the rest token-row
  // transfers i - QB of stage KTA into DA.
#define MOE_ISSUE3(KTA, KTB, DA, DB, I0, I1)                                 \
  do {                                                                       \
    _Pragma("unroll") for (int i_ = (I0); i_ < (I1); ++i_) {                 \
      constexpr int QB_ = NQ - QA;                                           \
      const int q = i_ < QB_ ? QA + i_ : i_ - QB_;                           \
      const bool isA_ = q < QA;                                              \
      const int ikt_ = isA_ ? (KTA) : (KTB);                                 \
      uint32_t off_ = goff[q] + static_cast<uint32_t>(ikt_) * (kBK * 2);     \
      if ((ikt_ + 1) * kBK > Kl) {                                           \
        const int t_ = wave + kWaves * q;                                    \
        const int r_ = (isA_ ? t_ : t_ - BM / 8) * 8 + (lane >> 3);          \
        const int c_ = (lane & 7) ^ swz(r_);                                 \
        if (ikt_ * kBK + c_ * 8 >= Kl) off_ = kOutOfRange;                   \
      }                                                                      \
      dma_untracked<16>(isA_ ? rsA : rsB, (isA_ ? (DA) : (DB)) + ldst[q], off_); \
    }                                                                        \
  } while (0)

  // Fragment rows: (lane & 31) within each 32-row block; at k step ks of a
  // stage the lane reads chunk kc = 2 ks + (lane >> 5), stored at slot
  // kc ^ swz(row).  Element offsets for all four k steps are precomputed.
  const int khalf = lane >> 5;
  // Non-K-grouped form: oa[i][0] / ob[j][0] hold row * 64 + 8 (khalf ^
  // swz(row)), the chunk of k step 0; step ks reads chunk (2 ks + khalf) ^
  // swz(row), i.e. that offset XOR 16 ks (the row part has its low 6 bits
  // clear), so one register per fragment serves all four steps.
  int oa[FB][1], ob[TB][1];
  if constexpr (KG || BT) {
    // Transposed fragments (byte offsets at k step 0): lane l addresses k
    // row 8 (l / 32) + (l / 4) % 4 and the 8-byte piece of features
    // 16 ((l / 16) % 2) + 4 (l % 4) .. + 3 of its 32-row block, in the
    // swizzled slot of that k row (see the transfers).
    const int kr = 8 * khalf + ((lane >> 2) & 3);
    const int sw = 4 * ((lane >> 2) & 3);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int hb = (lane & 1) * 8;
#pragma unroll
    for (int i = 0; i < FB; ++i) {
      const int c0 = (wf * (BN / WF) + i * 32) / 8;
      oa[i][0] = kr * BN * 2 + ((c0 + cl) ^ sw) * 16 + hb;
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if constexpr (KG) {
        const int c0 = (wt * (BM / WT) + j * 32) / 8;
        ob[j][0] = kr * BM * 2 + ((c0 + cl) ^ sw) * 16 + hb;
      } else {
        const int row = wt * (BM / WT) + j * 32 + (lane & 31);
        ob[j][0] = row * kBK + ((khalf ^ swz(row)) * 8);
      }
    }
  } else {
#pragma unroll
  for (int i = 0; i < FB; ++i) {
    const int row = wf * (BN / WF) + i * 32 + (lane & 31);
    oa[i][0] = row * kBK + ((khalf ^ swz(row)) * 8);
  }
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int row = wt * (BM / WT) + j * 32 + (lane & 31);
    ob[j][0] = row * kBK + ((khalf ^ swz(row)) * 8);
  }
  }

  f32x16 acc[FB][TB];
#pragma unroll
  for (int i = 0; i < FB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Two fragment register sets: while the MFMAs of k step ks run on one,
  // the LDS reads of step ks + 1 fill the other.
  bf16x8 fa0[FB], fb0[TB], fa1[FB], fb1[TB];

#define MOE_FRAGS(FA, FB_, SA, SB, KS)                                       \
  do {                                                                       \
    if constexpr (KG) {                                                      \
      _Pragma("unroll") for (int i = 0; i < FB; ++i) FA[i] =                 \
          lds_frag_tr<BN * 2>((SB), oa[i][0] + (KS) * 16 * BN * 2);          \
      _Pragma("unroll") for (int j = 0; j < TB; ++j) FB_[j] =                \
          lds_frag_tr<BM * 2>((SA), ob[j][0] + (KS) * 16 * BM * 2);          \
    } else if constexpr (BT) {                                               \
      _Pragma("unroll") for (int i = 0; i < FB; ++i) FA[i] =                 \
          lds_frag_tr<BN * 2>((SB), oa[i][0] + (KS) * 16 * BN * 2);          \
      _Pragma("unroll") for (int j = 0; j < TB; ++j) FB_[j] =                \
          *reinterpret_cast<const bf16x8*>(&(SA)[ob[j][0] ^ (16 * (KS))]);   \
    } else {                                                                 \
      _Pragma("unroll") for (int i = 0; i < FB; ++i) FA[i] =                 \
          *reinterpret_cast<const bf16x8*>(&(SB)[oa[i][0] ^ (16 * (KS))]);   \
      _Pragma("unroll") for (int j = 0; j < TB; ++j) FB_[j] =                \
          *reinterpret_cast<const bf16x8*>(&(SA)[ob[j][0] ^ (16 * (KS))]);   \
    }                                                                        \
  } while (0)

#define MOE_MFMAS(FA, FB_, I0, I1)                                           \
  do {                                                                       \
    _Pragma("unroll") for (int i = (I0); i < (I1); ++i)                      \
      _Pragma("unroll") for (int j = 0; j < TB; ++j) acc[i][j] =             \
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB_[j], acc[i][j],  \
                                                  0, 0, 0);                  \
  } while (0)

  // One 64-wide k stage read from CA / CB while stage KT + 1 streams into
  // NA / NB.  The order of the groups is pinned with scheduling barriers.
  // The next stage's transfers are spread over the MFMAs of the first two
  // k steps (one transfer per MFMA_PER_DMA MFMAs): issued in one burst they
  // fill the address unit's queue and stall every wave at issue, leaving
  // the matrix cores idle.  The last k step's MFMAs straddle the stage
  // barrier so that the matrix cores stay busy while the next stage's first
  // fragments are read.
  constexpr int kQH = (NQ + 1) / 2;                 // transfers in k step 0
  constexpr int kMfmaPerDma = (FB * TB) / kQH > 0 ? (FB * TB) / kQH : 1;
#define MOE_INTERLEAVE(NDMA)                                                 \
  do {                                                                       \
    _Pragma("unroll") for (int d_ = 0; d_ < (NDMA); ++d_) {                  \
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerDma, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                     \
    }                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x008, FB * TB, 0);                 \
  } while (0)

#define MOE_STAGE(KT, CA, CB, NA, NB, DNA, DNB)                              \
  do {                                                                       \
    const int skt_ = (KT);                                                   \
    const bool more_ = skt_ + 1 < nk;                                        \
    MOE_PREFETCH(skt_ + 2);                                                  \
    MOE_FRAGS(fa1, fb1, CA, CB, 1);                                          \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_MFMAS(fa0, fb0, 0, FB);                                              \
    if constexpr (NST == 3)                                                  \
      MOE_ISSUE3(skt_ + 2, skt_ + 1, DNA, DNB, 0, kQH);                      \
    else                                                                     \
      MOE_ISSUE(skt_ + 1, DNA, DNB, 0, kQH);                                 \
    MOE_INTERLEAVE(kQH);                                                     \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_FRAGS(fa0, fb0, CA, CB, 2);                                          \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_MFMAS(fa1, fb1, 0, FB);                                              \
    if constexpr (NST == 3)                                                  \
      MOE_ISSUE3(skt_ + 2, skt_ + 1, DNA, DNB, kQH, NQ);                     \
    else                                                                     \
      MOE_ISSUE(skt_ + 1, DNA, DNB, kQH, NQ);                                \
    MOE_INTERLEAVE(NQ - kQH);                                                \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_FRAGS(fa1, fb1, CA, CB, 3);                                          \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_MFMAS(fa0, fb0, 0, FB);                                              \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_MFMAS(fa1, fb1, 0, FB - FB / 2);                                     \
    __builtin_amdgcn_sched_barrier(0);                                       \
    if (more_) {                                                             \
      stage_barrier_keep<NST == 3 ? QA : 0>();                               \
      __builtin_amdgcn_sched_barrier(0);                                     \
      MOE_FRAGS(fa0, fb0, NA, NB, 0);                                        \
    }                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                       \
    MOE_MFMAS(fa1, fb1, FB - FB / 2, FB);                                    \
    __builtin_amdgcn_sched_barrier(0);                                       \
  } while (0)

  // In gather mode, the source rows of this workgroup's next tile.
  if (gather) {
    TileLoc nloc;
    if (locate_any<KG, BM, BN, GM>(p, tab, lane, (pc + 8) * pw + pj, nloc))
      MOE_FETCH_ROWS(nloc, (it + 1) & 1, lane);
  }

  // kEpiCombine: the slot rows and weights of this tile's tokens, for the
  // epilogue (rows past the end read zero and are never stored); in the
  // late form, issued at the start of the epilogue instead.
#define MOE_CMB_DMA()                                                        \
  do {                                                                       \
    const int km_ = p.cmb_kmax;                                              \
    const uint32_t nb_ = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>( \
        min(static_cast<int>(loc.row_end - loc.row0), BM) * km_ * 4));       \
    const __amdgpu_buffer_rsrc_t rsS_ = make_rsrc(                           \
        reinterpret_cast<const void*>(                                       \
            uniform64(reinterpret_cast<int64_t>(p.cmb_slot + loc.row0 * km_))), \
        nb_);                                                                \
    const __amdgpu_buffer_rsrc_t rsW_ = make_rsrc(                           \
        reinterpret_cast<const void*>(                                       \
            uniform64(reinterpret_cast<int64_t>(p.cmb_w + loc.row0 * km_))),  \
        nb_);                                                                \
    for (int q = wave; q < BM * km_ / 64; q += kWaves) {                     \
      const uint32_t o_ = static_cast<uint32_t>(q * 64 + lane) * 4u;         \
      dma_untracked<4>(rsS_, bCmb + q * 256, o_);                            \
      dma_untracked<4>(rsW_, bCmb + BM * CMAX * 4 + q * 256, o_);            \
    }                                                                        \
  } while (0)
  if constexpr (EPI == kEpiCombine && !kLateCmb) {
    MOE_CMB_DMA();
  }

  MOE_ISSUE(0, bA0, bB0, 0, NQ);
  if constexpr (NST == 3) MOE_ISSUE(1, bA1, bB1, 0, QA);   // token rows only
  stage_barrier_keep<NST == 3 ? QA : 0>();
  MOE_FRAGS(fa0, fb0, sA0, sB0, 0);
  // Stages rotate through the buffers.  The last stages' transfers address
  // k-stages from nk on, which lie wholly past Kd: they load zeros into
  // idle buffers (no branch around them, so they interleave with the MFMAs)
  // and are drained before the epilogue.
  if constexpr (NST == 2) {
    for (int kt = 0; kt < nk; kt += 2) {
      MOE_STAGE(kt, sA0, sB0, sA1, sB1, bA1, bB1);
      if (kt + 1 < nk) MOE_STAGE(kt + 1, sA1, sB1, sA0, sB0, bA0, bB0);
    }
  } else {
    // token rows in three buffers, weight rows in two: the pair of buffers
    // of stage kt is (kt % 3, kt % 2), six stages per turn
    for (int kt = 0; kt < nk; kt += 6) {
      MOE_STAGE(kt, sA0, sB0, sA1, sB1, bA2, bB1);
      if (kt + 1 < nk) MOE_STAGE(kt + 1, sA1, sB1, sA2, sB0, bA0, bB0);
      if (kt + 2 < nk) MOE_STAGE(kt + 2, sA2, sB0, sA0, sB1, bA1, bB1);
      if (kt + 3 < nk) MOE_STAGE(kt + 3, sA0, sB1, sA1, sB0, bA2, bB0);
      if (kt + 4 < nk) MOE_STAGE(kt + 4, sA1, sB0, sA2, sB1, bA0, bB1);
      if (kt + 5 < nk) MOE_STAGE(kt + 5, sA2, sB1, sA0, sB0, bA1, bB0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x7 << 4);
#undef MOE_STAGE
#undef MOE_ISSUE3
#undef MOE_PREFETCH
#undef MOE_INTERLEAVE
#undef MOE_MFMAS
#undef MOE_FRAGS
#undef MOE_ISSUE

  // acc[i][j] register r: feature 8 (r / 4) + 4 (lane >> 5) + r % 4 of
  // feature block i, token (lane & 31) of token block j.
  if (piece) {
    // A piece of a split tile: its fp32 partial sums, [BM][BN] row-major in
    // this workgroup's slot (every row and feature, as they are; the
    // finishing kernel adds the bias and skips what is not stored), and,
    // from the tile's first piece, where the tile lies.
    float* const part = p.sk_ws + kSplitHdrBytes / 4 +
                        static_cast<int64_t>(blockIdx.x) * (BM * BN);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int t = wt * (BM / WT) + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < FB; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int fl = wf * (BN / WF) + i * 32 + 8 * q + 4 * khalf;
          f32x4 v;
          v[0] = acc[i][j][4 * q + 0];
          v[1] = acc[i][j][4 * q + 1];
          v[2] = acc[i][j][4 * q + 2];
          v[3] = acc[i][j][4 * q + 3];
          *reinterpret_cast<f32x4*>(part + t * BN + fl) = v;
        }
      }
    }
    if (piece_s == 0 && tid == 0) {
      int64_t* const h = reinterpret_cast<int64_t*>(p.sk_ws) +
                         2 + 3 * (static_cast<int>(blockIdx.x) / skS);
      h[0] = loc.row0;
      h[1] = loc.row_end;
      h[2] = (static_cast<int64_t>(loc.g) << 32) | loc.n0;
    }
  } else if constexpr (OUT_BF16) {
    // The bias, if any, joins the accumulators first, in one loop behind a
    // uniform branch (u = A W^T + b, as the staging below would form it), so
    // that the staging loops carry no bias code: two forms of them in one
    // kernel raised the register count past 256 and spilled.
    if (p.bias != nullptr) {
      const float* const bg =
          p.bias + static_cast<int64_t>(loc.g) * p.Nd + loc.n0;
#pragma unroll
      for (int i = 0; i < FB; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int fl = wf * (BN / WF) + i * 32 + 8 * q + 4 * khalf;
          if (loc.n0 + fl >= p.Nd) continue;
          const float b0 = bg[fl], b1 = bg[fl + 1], b2 = bg[fl + 2],
                      b3 = bg[fl + 3];
#pragma unroll
          for (int j = 0; j < TB; ++j) {
            acc[i][j][4 * q + 0] += b0;
            acc[i][j][4 * q + 1] += b1;
            acc[i][j][4 * q + 2] += b2;
            acc[i][j][4 * q + 3] += b3;
          }
        }
      }
    }
    // Every wave is done with the stages: stage the tile in LDS.  Rows past
    // the group end are staged too (finite values from the zero or re-read
    // operand rows; the copy-out skips them).  Features past Nd are skipped;
    // a tile that holds none takes the branch-free form.
    stage_barrier();
    // the late slot table lands past the staged tile (waited for by the
    // barrier after the staging)
    if constexpr (kLateCmb) MOE_CMB_DMA();
#define MOE_STAGE_OUT(CHECK, E_)                                             \
    _Pragma("unroll") for (int j = 0; j < TB; ++j) {                         \
      const int t = wt * (BM / WT) + j * 32 + (lane & 31);                   \
      _Pragma("unroll") for (int i = 0; i < FB; ++i) {                       \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                      \
          const int fl = wf * (BN / WF) + i * 32 + 8 * q + 4 * khalf;        \
          if ((CHECK) && loc.n0 + fl >= p.Nd) continue;                      \
          f32x4 v;                                                           \
          v[0] = acc[i][j][4 * q + 0];                                       \
          v[1] = acc[i][j][4 * q + 1];                                       \
          v[2] = acc[i][j][4 * q + 2];                                       \
          v[3] = acc[i][j][4 * q + 3];                                       \
          v = finish4<E_, false>(p, loc.g, loc.row0 + t, loc.n0 + fl, v);    \
          uint2 o;                                                           \
          o.x = pack_bf16x2(v[0], v[1]);                                     \
          o.y = pack_bf16x2(v[2], v[3]);                                     \
          *reinterpret_cast<uint2*>(&lds[t * kOutPitch + fl]) = o;           \
        }                                                                    \
      }                                                                      \
    }
    constexpr int kChunks = BN / 8;
    uint16_t* const c = static_cast<uint16_t*>(p.c);
    const bool full_n = loc.n0 + BN <= p.Nd;
    // Copy out the staged tile to `dst`: 16 bytes per lane, consecutive
    // lanes along a row, as non-temporal stores (the tile is not read again
    // by this kernel; without the hint the write burst at the end of every
    // tile allocates L2 lines).
#define MOE_COPY_OUT(DST)                                                    \
    for (int idx = tid; idx < BM * kChunks; idx += 64 * kWaves) {            \
      const int r = idx / kChunks;                                           \
      const int f = loc.n0 + (idx - r * kChunks) * 8;                        \
      const int64_t row = loc.row0 + r;                                      \
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));        \
      if (row < loc.row_end && f < p.Nd)                                     \
        __builtin_nontemporal_store(                                         \
            *reinterpret_cast<const u32x4*>(&lds[r * kOutPitch + (f - loc.n0)]), \
            reinterpret_cast<u32x4*>((DST) + row * p.Nd + f));               \
    }
    if constexpr (EPI == kEpiGelu) {
      // Training forward: the pre-activations first, through the same
      // staging area, then the activations below.
      if (p.u_out != nullptr) {
        if (full_n) {
          MOE_STAGE_OUT(false, kEpiStore)
        } else {
          MOE_STAGE_OUT(true, kEpiStore)
        }
        stage_barrier();
        MOE_COPY_OUT(static_cast<uint16_t*>(p.u_out))
        stage_barrier();
      }
    }
    if (full_n) {
      MOE_STAGE_OUT(false, EPI)
    } else {
      MOE_STAGE_OUT(true, EPI)
    }
#undef MOE_STAGE_OUT
#undef MOE_CMB_DMA
    stage_barrier();
    if constexpr (EPI == kEpiCombine) {
      // y[t] = sum over the slots >= 0, in slot order, of w * routed row,
      // then plus the staged (bf16) shared output, in fp32, rounded once:
      // the arithmetic of the separate combine kernel.  Chunks go in
      // batches of kB, slots in groups of kG: a group's routed-row loads
      // for the whole batch are all issued before its first multiply-add.
      constexpr int kIters = (BM * kChunks + 64 * kWaves - 1) / (64 * kWaves);
      constexpr int kB = CMAX > 4 ? 4 : 6;
      constexpr int kG = 4;
      const uint16_t* const yr = static_cast<const uint16_t*>(p.cmb_rows);
      int km = p.cmb_kmax;
      if constexpr (CMAX > 4) {
        // Many slots, few of them used (Expert Race): move each row's
        // non-empty slots to its front, in slot order, and count them, so
        // that a chunk visits only the groups holding its row's slots (the
        // sum keeps its slot order).  The table is [BM][km] from here on.
        for (int r = tid; r < BM; r += 64 * kWaves) {
          int n = 0;
          for (int k = 0; k < km; ++k) {
            const int32_t sv = cslot[r * km + k];
            const float wv = cwt[r * km + k];
            if (sv >= 0) {
              cslot[r * km + n] = sv;
              cwt[r * km + n] = wv;
              ++n;
            }
          }
          for (int k = n; k < km; ++k) cslot[r * km + k] = -1;
          ccnt[r] = n;
        }
        stage_barrier();
      }
      for (int i0 = 0; i0 < kIters; i0 += kB) {
        float a8[kB][8];
#pragma unroll
        for (int b = 0; b < kB; ++b)
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[b][j] = 0.0f;
        // slot groups this lane's chunks need
        int kend = km;
        if constexpr (CMAX > 4) {
          kend = 0;
#pragma unroll
          for (int b = 0; b < kB; ++b) {
            const int idx = tid + (i0 + b) * 64 * kWaves;
            if (idx < BM * kChunks) kend = max(kend, ccnt[idx / kChunks]);
          }
        }
        for (int k0 = 0; k0 < kend; k0 += kG) {
          uint4 v[kB][kG];
          int32_t sl[kB][kG];
          float wk[kB][kG];
#pragma unroll
          for (int b = 0; b < kB; ++b) {
            const int idx = tid + (i0 + b) * 64 * kWaves;
            const int r = idx / kChunks;
            const int f = loc.n0 + (idx - r * kChunks) * 8;
            const bool ok = idx < BM * kChunks && loc.row0 + r < loc.row_end &&
                            f < p.Nd;
#pragma unroll
            for (int k = 0; k < kG; ++k) {
              sl[b][k] = -1;
              wk[b][k] = 0.0f;
              v[b][k] = make_uint4(0, 0, 0, 0);
              if (ok && k0 + k < km) {
                sl[b][k] = cslot[r * km + k0 + k];
                wk[b][k] = cwt[r * km + k0 + k];
              }
              if (sl[b][k] >= 0)
                v[b][k] = *reinterpret_cast<const uint4*>(
                    yr + static_cast<int64_t>(sl[b][k]) * p.Nd + f);
            }
          }
#pragma unroll
          for (int b = 0; b < kB; ++b) {
#pragma unroll
            for (int k = 0; k < kG; ++k) {
              if (sl[b][k] < 0) continue;
              float yv[8];
              unpack8(v[b][k], yv);
#pragma unroll
              for (int j = 0; j < 8; ++j) a8[b][j] = fmaf(wk[b][k], yv[j], a8[b][j]);
            }
          }
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int idx = tid + (i0 + b) * 64 * kWaves;
          const int r = idx / kChunks;
          const int f = loc.n0 + (idx - r * kChunks) * 8;
          const int64_t row = loc.row0 + r;
          if (idx >= BM * kChunks || row >= loc.row_end || f >= p.Nd) continue;
          float sh[8];
          unpack8(*reinterpret_cast<const uint4*>(
                      &lds[r * kOutPitch + (f - loc.n0)]), sh);
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[b][j] += sh[j];
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          u32x4 o;
          o[0] = pack_bf16x2(a8[b][0], a8[b][1]);
          o[1] = pack_bf16x2(a8[b][2], a8[b][3]);
          o[2] = pack_bf16x2(a8[b][4], a8[b][5]);
          o[3] = pack_bf16x2(a8[b][6], a8[b][7]);
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(c + row * p.Nd + f));
        }
      }
    } else if constexpr (EPI == kEpiGeluGrad) {
      // du = staged product * gelu'(u): u in batches of kB row-contiguous
      // 16-byte chunks, all loaded before the first multiply.
      constexpr int kIters = (BM * kChunks + 64 * kWaves - 1) / (64 * kWaves);
      constexpr int kB = 8;
      const uint16_t* const ua = static_cast<const uint16_t*>(p.aux);
      for (int i0 = 0; i0 < kIters; i0 += kB) {
        uint4 uv[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int idx = tid + (i0 + b) * 64 * kWaves;
          const int r = idx / kChunks;
          const int f = loc.n0 + (idx - r * kChunks) * 8;
          uv[b] = make_uint4(0, 0, 0, 0);
          if (i0 + b < kIters && idx < BM * kChunks &&
              loc.row0 + r < loc.row_end && f < p.Nd)
            uv[b] = *reinterpret_cast<const uint4*>(ua + (loc.row0 + r) * p.Nd + f);
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int idx = tid + (i0 + b) * 64 * kWaves;
          const int r = idx / kChunks;
          const int f = loc.n0 + (idx - r * kChunks) * 8;
          const int64_t row = loc.row0 + r;
          if (i0 + b >= kIters || idx >= BM * kChunks || row >= loc.row_end ||
              f >= p.Nd)
            continue;
          float a8[8], u8[8];
          unpack8(*reinterpret_cast<const uint4*>(
                      &lds[r * kOutPitch + (f - loc.n0)]), a8);
          unpack8(uv[b], u8);
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[j] *= gelu_tanh_grad(u8[j]);
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          u32x4 o;
          o[0] = pack_bf16x2(a8[0], a8[1]);
          o[1] = pack_bf16x2(a8[2], a8[3]);
          o[2] = pack_bf16x2(a8[4], a8[5]);
          o[3] = pack_bf16x2(a8[6], a8[7]);
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(c + row * p.Nd + f));
        }
      }
    } else {
      MOE_COPY_OUT(c)
    }
#undef MOE_COPY_OUT
  } else {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int64_t row = loc.row0 + wt * (BM / WT) + j * 32 + (lane & 31);
      if (row >= loc.row_end) continue;
#pragma unroll
      for (int i = 0; i < FB; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = loc.n0 + wf * (BN / WF) + i * 32 + 8 * q + 4 * khalf;
          if (f >= p.Nd) continue;
          f32x4 v;
          v[0] = acc[i][j][4 * q + 0];
          v[1] = acc[i][j][4 * q + 1];
          v[2] = acc[i][j][4 * q + 2];
          v[3] = acc[i][j][4 * q + 3];
          store4<EPI, OUT_BF16>(p, loc.g, row, f, v);
        }
      }
    }
  }
  pc += 8;
  ++it;
  MOE_NEXT_TILE(lane);
  }  // tile loop
#undef MOE_NEXT_TILE
}

// Finishes the tiles of a split last round (GemmParams::sk_ws): the S
// partials of each split tile added in piece order, then the bias, stored
// as the store epilogue does (rounded once).  A tile's BM x BN outputs are
// cut into split_finish_wgs() chunks of 1024 (4 consecutive features per
// thread); the workgroups (four per CU, so about one chunk each) walk the R
// tiles' chunks, and the loads of a batch of up to 16 pieces are issued
// before their additions: a chunk costs the header read and one round trip
// per batch.  Rows past the group end and features past Nd are skipped.
// With no split every workgroup returns after reading the header.
constexpr int kSplitFinishBatch = 16;
constexpr int kSplitFinishPerCu = 4;
template <int BM, int BN>
constexpr int split_finish_wgs() { return BM * BN / (256 * 4); }

template <bool OUT_BF16, int BM, int BN>
__global__ __launch_bounds__(256) void splitk_tail_kernel(GemmParams p) {
  static_assert(BM * BN % (256 * 4) == 0, "whole workgroups per tile");
  constexpr int kW = split_finish_wgs<BM, BN>();
  const int64_t* const h = reinterpret_cast<const int64_t*>(p.sk_ws);
  const int S = static_cast<int>(h[0]), R = static_cast<int>(h[1]);
  if (S < 2) return;
  for (int item = blockIdx.x; item < R * kW; item += gridDim.x) {
    const int r = item / kW;
    const int idx = (item - r * kW) * 1024 + threadIdx.x * 4;
    const int64_t row0 = h[2 + 3 * r], row_end = h[3 + 3 * r];
    const int g = static_cast<int>(h[4 + 3 * r] >> 32);
    const int n0 = static_cast<int>(h[4 + 3 * r] & 0xffffffff);
    const int t = idx / BN, f = idx - t * BN;
    const int64_t row = row0 + t;
    if (row >= row_end || n0 + f >= p.Nd) continue;
    const float* const part = p.sk_ws + kSplitHdrBytes / 4 +
                              static_cast<int64_t>(r) * S * (BM * BN) + idx;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += kSplitFinishBatch) {
      f32x4 w[kSplitFinishBatch];
#pragma unroll
      for (int b = 0; b < kSplitFinishBatch; ++b)
        if (s0 + b < S)
          w[b] = *reinterpret_cast<const f32x4*>(
              part + static_cast<int64_t>(s0 + b) * (BM * BN));
#pragma unroll
      for (int b = 0; b < kSplitFinishBatch; ++b) {
        if (s0 + b < S) {
          if (s0 + b == 0) {
            v = w[b];
          } else {
            v[0] += w[b][0]; v[1] += w[b][1]; v[2] += w[b][2]; v[3] += w[b][3];
          }
        }
      }
    }
    store4<kEpiStore, OUT_BF16>(p, g, row, n0 + f, v);
  }
}

// ------------------------------------------- single-kernel expert MLP ----
// Both matrices of an expert MLP in one kernel, for narrow layers (D = 128,
// 256 or 384): the hidden activation never leaves the CU.  A workgroup of
// 8 waves owns 128 token rows of one group and walks the hidden width in
// chunks of 64:
//   phase A:  hc = gelu(W1[chunk] x^T + b1[chunk])   -> LDS (bf16, 128 x 64)
//   phase B:  y^T += W2[:, chunk] hc^T               -> registers (fp32)
// Wave w owns tokens 32 (w % 4) .. +32; in phase A hidden rows 32 (w / 4)
// .. +32 of the chunk, in phase B output features (w / 4) D/2 .. +D/2.  Its
// token rows stay in registers as MFMA operands for the whole tile.  The
// weights of the chunk reach LDS by buffer_load ... lds: W2's while phase A
// runs, the next chunk's W1 while phase B runs.  LDS rows are 64 k (128
// bytes) with the 16-byte chunks swizzled as in the GEMMs.  Rounding and
// summation order are those of the two-stage path (h rounded to bf16 once,
// y summed over the hidden width in the same order), so both give the same
// bits.
constexpr int kMlpBM = 128, kMlpHC = 64, kMlpWaves = 8;

template <int DT>   // D = 128 DT
__global__ __launch_bounds__(64 * kMlpWaves, 1) void mlp_fused_kernel(
    GemmParams p, const void* __restrict__ w2, const float* __restrict__ b2,
    int H, int y_f32) {
  constexpr int D = 128 * DT;
  constexpr int KS = D / 16;          // phase-A k steps (16 wide)
  constexpr int FBY = D / 64;         // phase-B output blocks of 32 per wave
  constexpr int NT = D / 8;           // 1 KB transfers per weight chunk
  constexpr int NTW = NT / kMlpWaves; // ... per wave
  static_assert(NT % kMlpWaves == 0, "whole transfers per wave");
  constexpr int kW1Bytes = kMlpHC * D * 2;   // [D/64 slices][64 rows][128 B]
  constexpr int kW2Bytes = D * 128;          // [D rows][128 B]
  constexpr int kHBytes = kMlpBM * 128;      // [128 tokens][128 B]
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[kW1Bytes + kW2Bytes + kHBytes + kTabInts * 4];
  int32_t* const tab = reinterpret_cast<int32_t*>(lds + kW1Bytes + kW2Bytes + kHBytes);
  const uint16_t* const sW1 = reinterpret_cast<const uint16_t*>(lds);
  const uint16_t* const sW2 = reinterpret_cast<const uint16_t*>(lds + kW1Bytes);
  uint8_t* const sH = lds + kW1Bytes + kW2Bytes;
  const uint32_t bW1 = lds_addr(lds), bW2 = bW1 + kW1Bytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = wave & 3, fh = wave >> 2;
  const int khalf = lane >> 5;
  build_group_table<kMlpBM, D>(p, tab, wave, lane);
  TileLoc loc;
  if (!locate_tile_tab<kMlpBM, D, 1>(p, tab, lane,
                                     xcd_remap(blockIdx.x, gridDim.x), loc))
    return;
  const int g = loc.g;
  const uint16_t* const w1g =
      static_cast<const uint16_t*>(p.w) + static_cast<int64_t>(g) * H * D;
  const uint16_t* const w2g =
      static_cast<const uint16_t*>(w2) + static_cast<int64_t>(g) * D * H;

  // Transfer q of this wave for a weight chunk: rows r0 .. r0 + 7; lane l
  // fetches chunk (l % 8) ^ swz(row) of row r0 + l / 8 into slot l % 8.
  // W1 chunk (hidden rows hc0 .. hc0 + 63, all D k): transfer t covers
  // slice t / 8 (k 64 (t / 8) ..), rows 8 (t % 8) ..; W2 chunk (all D
  // output rows, hidden k hc0 .. hc0 + 63): transfer t covers rows 8 t ...
  // Lane-dependent offsets are recomputed from an opaque copy of the lane
  // index in every chunk (a few VALU operations), instead of being hoisted
  // into registers that would stay live through the MFMA loops next to the
  // token fragments and accumulators.
#define MOE_MLP_ISSUE_W1(HC0)                                                \
  do {                                                                       \
    const __amdgpu_buffer_rsrc_t rs_ = make_rsrc(                            \
        reinterpret_cast<const void*>(uniform64(reinterpret_cast<int64_t>(   \
            w1g + static_cast<int64_t>(HC0) * D))),                          \
        static_cast<uint32_t>(kW1Bytes));                                    \
    _Pragma("unroll") for (int q = 0; q < NTW; ++q) {                        \
      const int t_ = wave + kMlpWaves * q;                                   \
      const int r_ = (t_ % 8) * 8 + (ol >> 3);                               \
      const uint32_t o_ = static_cast<uint32_t>(r_) * (D * 2) +              \
                          (t_ / 8) * 128 + (((ol & 7) ^ swz(r_)) * 16);      \
      dma_untracked<16>(rs_, bW1 + (t_ / 8) * (kMlpHC * 128) + (t_ % 8) * 1024, o_); \
    }                                                                        \
  } while (0)
#define MOE_MLP_ISSUE_W2(HC0)                                                \
  do {                                                                       \
    const __amdgpu_buffer_rsrc_t rs_ = make_rsrc(                            \
        reinterpret_cast<const void*>(                                       \
            uniform64(reinterpret_cast<int64_t>(w2g + (HC0)))),              \
        static_cast<uint32_t>((D - 1) * H * 2 + kMlpHC * 2));                \
    _Pragma("unroll") for (int q = 0; q < NTW; ++q) {                        \
      const int t_ = wave + kMlpWaves * q;                                   \
      const int r_ = t_ * 8 + (ol >> 3);                                     \
      const uint32_t o_ = static_cast<uint32_t>(r_) * static_cast<uint32_t>(H * 2) + \
                          (((ol & 7) ^ swz(r_)) * 16);                       \
      dma_untracked<16>(rs_, bW2 + t_ * 1024, o_);                           \
    }                                                                        \
  } while (0)

  {
    const int ol = lane;
    MOE_MLP_ISSUE_W1(0);
  }
  // This lane's token row as phase A's B operand: k 16 s + 8 khalf .. + 8
  // of step s.  Rows past the group end re-read the tile's first row (never
  // stored).
  // An index entry outside [0, a_rows) gives a zero row.
  bf16x8 xf[KS];
  {
    const int64_t row = loc.row0 + tb * 32 + (lane & 31);
    const int64_t r = row < loc.row_end ? row : loc.row0;
    const int64_t src = p.a_index != nullptr ? p.a_index[r] : r;
    const bool ok = p.a_index == nullptr || gather_row_valid(src, p.a_rows);
    const uint16_t* const xr =
        static_cast<const uint16_t*>(p.a) + (ok ? src : 0) * D + 8 * khalf;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = ok ? *reinterpret_cast<const uint4*>(xr + 16 * s)
                         : make_uint4(0, 0, 0, 0);
      xf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 acc[FBY];
#pragma unroll
  for (int i = 0; i < FBY; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  stage_barrier();

  // LDS element offsets.  Phase A: W1 row 32 fh + (lane & 31) of the
  // chunk, k step s -> slice s / 4, chunk 2 (s % 4) + khalf.  Phase B: W2
  // row (output feature) fh D/2 + 32 i + (lane & 31); h row (token)
  // 32 tb + (lane & 31); k step s -> chunk 2 s + khalf.
  const int nc = H / kMlpHC;
  for (int c = 0; c < nc; ++c) {
    int ol = lane;
    asm volatile("" : "+v"(ol));
    const int kh = ol >> 5;
    const int ra = fh * 32 + (ol & 31);
    const int rt = tb * 32 + (ol & 31);
    const int hc0 = c * kMlpHC;
    MOE_MLP_ISSUE_W2(hc0);
    // phase A
    f32x16 ah;
#pragma unroll
    for (int r = 0; r < 16; ++r) ah[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ck = 2 * (s % 4) + kh;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          &sW1[(s / 4) * kMlpHC * 64 + ra * 64 + ((ck ^ swz(ra)) * 8)]);
      ah = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[s], ah, 0, 0, 0);
    }
    // bias, GELU, bf16 into hc: register 4 q + j holds hidden feature
    // 32 fh + 8 q + 4 khalf + j of token rt.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int hf = fh * 32 + 8 * q + 4 * kh;
      f32x4 v;
      v[0] = ah[4 * q + 0]; v[1] = ah[4 * q + 1];
      v[2] = ah[4 * q + 2]; v[3] = ah[4 * q + 3];
      if (p.bias != nullptr) {
        const float* b = p.bias + static_cast<int64_t>(g) * H + hc0 + hf;
        v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
      }
      uint2 o;
      o.x = pack_bf16x2(gelu_tanh(v[0]), gelu_tanh(v[1]));
      o.y = pack_bf16x2(gelu_tanh(v[2]), gelu_tanh(v[3]));
      const int ch = hf >> 3;
      *reinterpret_cast<uint2*>(sH + rt * 128 + ((ch ^ swz(rt)) * 16) + kh * 8) = o;
    }
    stage_barrier();   // hc written, W2 chunk landed, W1 chunk read by all
    if (c + 1 < nc) MOE_MLP_ISSUE_W1(hc0 + kMlpHC);
    // phase B, k step outermost: one h fragment live at a time.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 hb = *reinterpret_cast<const bf16x8*>(
          sH + rt * 128 + (((2 * s + kh) ^ swz(rt)) * 16));
#pragma unroll
      for (int i = 0; i < FBY; ++i) {
        const int ro = fh * (D / 2) + 32 * i + (ol & 31);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &sW2[ro * 64 + (((2 * s + kh) ^ swz(ro)) * 8)]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hb, acc[i], 0, 0, 0);
      }
    }
    stage_barrier();   // next W1 chunk landed; W2 chunk and hc read by all
  }

  // y row rt: register 4 q + j of block i is output feature
  // fh D/2 + 32 i + 8 q + 4 khalf + j.
  int el = lane;
  asm volatile("" : "+v"(el));
  const int rt = tb * 32 + (el & 31);
  const int64_t row = loc.row0 + rt;
  if (row >= loc.row_end) return;
#pragma unroll
  for (int i = 0; i < FBY; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = fh * (D / 2) + 32 * i + 8 * q + 4 * (el >> 5);
      f32x4 v;
      v[0] = acc[i][4 * q + 0]; v[1] = acc[i][4 * q + 1];
      v[2] = acc[i][4 * q + 2]; v[3] = acc[i][4 * q + 3];
      if (b2 != nullptr) {
        const float* b = b2 + static_cast<int64_t>(g) * D + f;
        v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
      }
      if (y_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.c) + row * D + f) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else {
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.c) + row * D + f) = o;
      }
    }
  }
#undef MOE_MLP_ISSUE_W1
#undef MOE_MLP_ISSUE_W2
}

// Tile shapes: the up-projection (N = H, a multiple of 256 in every DiT-MoE
// shape) uses 256 x 256 tiles, 2 x 4 waves of 128 tokens x 64 features; the
// down-projection (N = D, e.g. 1152 = 6 x 192) uses 256 x 192 tiles, 4 x 2
// waves of 64 tokens x 96 features.
constexpr int kUpBM = 256, kUpBN = 256, kUpWT = 2, kUpWF = 4;
constexpr int kDnBM = 256, kDnBN = 192, kDnWT = 4, kDnWF = 2;
// Tile order within a group (bands of about GM row-tiles, feature-tile
// major).
// Stage 2 has few feature tiles (1152 / 192 = 6) and a large token operand
// (h): with GM = 1 all feature tiles of a row-tile run at once, so each row
// of h leaves HBM once.  Stage 1 (18+ feature tiles) keeps bands of 8.
constexpr int kUpGM = 8, kDnGM = 1;
// Stage 2 streams a long token operand (K = H) whose rows mostly miss L2:
// its large tiles keep three token-row stages in LDS, so each transfer has
// two stages of MFMAs to land in (0.65 -> 0.56-0.59 ms per XL launch, where
// the two-stage form was bound by that latency: without its MFMAs it took
// 0.61 ms).  That form takes no L2 prefetch (measured to add nothing to it);
// the small-tile form keeps two stages and the prefetch.
constexpr int kDnNST = 3;
constexpr bool kDnPF = true;
// Small problems (short sequences, narrow layers): when the large tiles
// would occupy fewer than 3/4 of the CUs, most of the chip idles.  Those
// launches take 128 x 128 tiles (2 x 4 waves of 64 tokens x 32 features;
// about 94 VGPRs and 64 KB of stages), two workgroups per CU.  Small tiles
// run at about half the large tiles' rate per CU, so they only pay when
// they bring that many more CUs in.  Measured on the S-sized layer (8192
// tokens, D = 384): the shared experts' stage 2 with the combine (64 large
// tiles) 89 -> 53 us, routed stage 2 (158 large tiles) 49 -> 42 us; the
// 768-wide layer's shared stage 2 (256 large tiles, one full round) takes
// 159 us with large tiles and 380 us with small ones.
constexpr int kSmBM = 128, kSmBN = 128, kSmWT = 2, kSmWF = 4, kSmOcc = 2;

// ---------------------------------------------------------- fp32 path ----
// Plain fp32 FMA tiles (64 x 64 x 16, 4 x 4 outputs per thread) for fp32
// layers; same tile order and epilogue as the bf16 path.

constexpr int kFM = 64, kFN = 64, kFK = 16;
constexpr int kF32Threads = 256;

template <int EPI>
__global__ __launch_bounds__(kF32Threads) void gemm_f32_kernel(GemmParams p) {
  __shared__ float sA[kFK][kFM + 4];
  __shared__ float sB[kFK][kFN + 4];
  TileLoc loc;
  if (!locate_tile<kFM, kFN, kGM>(p, xcd_remap(blockIdx.x, gridDim.x), loc))
    return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int Kd = p.Kd;
  const float* A = static_cast<const float*>(p.a);
  const float* W = static_cast<const float*>(p.w) +
                   static_cast<int64_t>(loc.g) * p.Nd * Kd;
  // loads: row tid >> 2 (0..63), k quad (tid & 3) * 4
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int64_t grow = loc.row0 + lrow;
  bool a_ok = grow < loc.row_end;
  int64_t src = 0;
  if (a_ok) src = (p.a_index != nullptr) ? p.a_index[grow] : grow;
  // an index entry outside [0, a_rows) gives a zero row
  if (a_ok && p.a_index != nullptr && !gather_row_valid(src, p.a_rows)) {
    a_ok = false;
    src = 0;
  }
  const float* a_src = A + src * Kd + lk;
  const int f = loc.n0 + lrow;
  const bool b_ok = f < p.Nd;
  const float* b_src = W + static_cast<int64_t>(b_ok ? f : 0) * Kd + lk;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < Kd; k0 += kFK) {
    const bool kok = k0 + lk < Kd;
    const float4 av = (a_ok && kok) ? *reinterpret_cast<const float4*>(a_src + k0)
                                    : make_float4(0, 0, 0, 0);
    const float4 bv = (b_ok && kok) ? *reinterpret_cast<const float4*>(b_src + k0)
                                    : make_float4(0, 0, 0, 0);
    sA[lk + 0][lrow] = av.x; sA[lk + 1][lrow] = av.y;
    sA[lk + 2][lrow] = av.z; sA[lk + 3][lrow] = av.w;
    sB[lk + 0][lrow] = bv.x; sB[lk + 1][lrow] = bv.y;
    sB[lk + 2][lrow] = bv.z; sB[lk + 3][lrow] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = loc.row0 + ty * 4 + i;
    const int fo = loc.n0 + tx * 4;
    if (row < loc.row_end && fo < p.Nd) {
      f32x4 v;
      v[0] = acc[i][0]; v[1] = acc[i][1]; v[2] = acc[i][2]; v[3] = acc[i][3];
      store4<EPI, false>(p, loc.g, row, fo, v);
    }
  }
}

int tile_grid(const GemmParams& p, int BM, int BN) {
  const int64_t mt = (p.total + static_cast<int64_t>(p.G) * (BM - 1)) / BM;
  return static_cast<int>(mt * ((p.Nd + BN - 1) / BN));
}

}  // namespace

// The CU count of the current device, read once per device.
int cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n < 8)
      n = 8;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

// Workgroups of a persistent launch: the CU count of the current device,
// rounded down to a multiple of 8, and no more than the tile bound rounded
// up to a multiple of 8.
// occ workgroups per CU (the kernel's resources allow that many).
int persistent_grid(int tiles, int occ = 1) {
  const int cap = cu_count() / 8 * 8 * occ;
  const int want = (tiles + 7) / 8 * 8;
  return want < cap ? want : cap;
}

// Launch one forward GEMM stage: large tiles (BM x BN) or, for a problem
// with fewer large tiles than 3/4 of the CUs, the small-tile form.
template <int EPI, bool OUT_BF16, int BM, int BN, int WT, int WF, int GM, bool PF,
          int CMAX = 4, bool BT = false, int NST = 2>
void launch_stage(const GemmParams& p, hipStream_t stream) {
  const int big = tile_grid(p, BM, BN);
  if (static_cast<int64_t>(big) * 4 < static_cast<int64_t>(cu_count()) * 3) {
    hipLaunchKernelGGL(
        (gemm_bf16_kernel<EPI, OUT_BF16, kSmBM, kSmBN, kSmWT, kSmWF, GM, PF,
                          false, CMAX, BT, 2>),
        dim3(persistent_grid(tile_grid(p, kSmBM, kSmBN), kSmOcc)),
        dim3(64 * kSmWT * kSmWF), 0, stream, p);
    return;
  }
  const int grid = persistent_grid(big);
  hipLaunchKernelGGL(
      (gemm_bf16_kernel<EPI, OUT_BF16, BM, BN, WT, WF, GM, NST == 3 ? false : PF,
                        false, CMAX, BT, NST>),
      dim3(grid), dim3(64 * WT * WF), 0, stream, p);
  // the split last round's tiles (at most one per two workgroups)
  if constexpr (EPI == kEpiStore && NST == 3 && !BT) {
    if (p.sk_ws != nullptr && p.a_index == nullptr)
      hipLaunchKernelGGL((splitk_tail_kernel<OUT_BF16, BM, BN>),
                         dim3(grid * kSplitFinishPerCu), dim3(256), 0, stream, p);
  }
}

}  // namespace

namespace {

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Reduction splits of the K-grouped weight-gradient GEMMs ([G][M][N] out,
// 256 x 256 tiles, `total` token rows over G groups).  Splitting a group's
// token rows into S pieces makes S x more tiles, each 1/S as long, and adds
// the fp32 partials' traffic (S written, S read back by the reduction).  The
// estimate for S: ceil(S x tiles / CUs) rounds of tiles of ceil(rows / S)
// tokens at about 4 TFLOP/s per CU, plus 2 S G M N 4 bytes at about 5 TB/s.
// S runs up to 8, with pieces of at least 2048 tokens of an average group,
// and a split is taken only when its estimate is below 0.9 of the unsplit
// one (the estimate ignores the clock, which rises when fewer CUs are busy).
// The CU count is the current device's, as the persistent grids use; the
// workspace query and the launch take the same count, so the partials always
// fit.  Measured: the shared experts' weight gradients of the S layer (24
// tiles, 8192 tokens) take 0.28 instead of 0.46 ms per backward call with
// S = 4; those of the XL layer (180 tiles over 184 of 256 CUs, 32768
// tokens) split in 4 as well.
int choose_ksplit(int G, int M, int N, int64_t total) {
  const int64_t tiles = static_cast<int64_t>(G) * ((M + kUpBM - 1) / kUpBM) *
                        ((N + kUpBN - 1) / kUpBN);
  if (G <= 0 || tiles <= 0 || total <= 0) return 1;
  constexpr int64_t kMinTokens = 2048;
  constexpr double kCuFlops = 4.0e12, kHbmBytes = 5.0e12;
  const int64_t cus = cu_count();
  const int64_t per_group = total / G;
  const double tile_flops_per_token = 2.0 * kUpBM * kUpBN;
  const double out_bytes = 4.0 * G * static_cast<double>(M) * N;
  auto estimate = [&](int S) {
    const int64_t rounds = (S * tiles + cus - 1) / cus;
    const int64_t piece = (per_group + S - 1) / S;
    return static_cast<double>(rounds) * piece * tile_flops_per_token / kCuFlops +
           (S > 1 ? 2.0 * S * out_bytes / kHbmBytes : 0.0);
  };
  int best = 1;
  double best_t = estimate(1);
  const double unsplit = best_t;
  for (int S = 2; S <= 8 && per_group / S >= kMinTokens; ++S) {
    const double t = estimate(S);
    if (t < best_t) {
      best = S;
      best_t = t;
    }
  }
  return best_t < 0.9 * unsplit ? best : 1;
}

// out[i] = part[0][i] + part[1][i] + ... in split order (same bits every
// call), four floats per thread.
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(
    const float4* __restrict__ part, int S, int64_t n4, float4* __restrict__ out) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float4 a = part[i];
    for (int s = 1; s < S; ++s) {
      const float4 b = part[static_cast<int64_t>(s) * n4 + i];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    out[i] = a;
  }
}

struct BwdLayout {
  size_t u, h, du, w1t, xr, part, total;
};

BwdLayout bwd_layout(int64_t total, int G, int D, int H) {
  BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.u = take(static_cast<size_t>(total) * H * 2);
  L.h = take(static_cast<size_t>(total) * H * 2);
  L.du = take(static_cast<size_t>(total) * H * 2);
  L.w1t = take(static_cast<size_t>(G) * D * H * 2);
  L.xr = take(static_cast<size_t>(total) * D * 2);
  const int S = choose_ksplit(G, D, H, total);
  L.part = take(S > 1 ? static_cast<size_t>(S) * G * D * H * 4 : 0);
  L.total = o;
  return L;
}

}  // namespace

size_t ffn_backward_workspace_bytes(int64_t total, int G, int D, int H) {
  return bwd_layout(total, G, D, H).total;
}

// Backward of the grouped expert MLPs, given dy_rows = dLoss/d(expert output):
//   u       = x_rows W1^T (+ b1)                   (recomputed, bf16)
//   du      = (dy_rows W2) * gelu'(u)              (W2 read k-major as stored)
//   dx_rows = du W1                                (W1 transposed once)
//   dW2[g]  = dy_rows[g]^T gelu(u[g]),  dW1[g] = du[g]^T x_rows[g]
// the last two as K-grouped GEMMs that read the row-major operands and
// transpose them on the way from LDS.
hipError_t launch_ffn_backward(const FfnBwdArgs& a, hipStream_t stream) {
  const BwdLayout L = bwd_layout(a.total_rows, a.G, a.D, a.H);
  char* ws = static_cast<char*>(a.workspace);
  void* u = ws + L.u;
  void* du = ws + L.du;
  void* w1t = ws + L.w1t;
  // a = gelu(u) and the expert's input rows, row-major, for the weight
  // gradients: the forward's, or formed here.
  const void* hh = a.h_saved != nullptr ? a.h_saved : ws + L.h;
  const void* xr = a.row_index != nullptr ? ws + L.xr : a.x;
  const int G = a.G, D = a.D, H = a.H;
  hipError_t err;
#define MOE_TRY(call)                      \
  do {                                     \
    err = (call);                          \
    if (err != hipSuccess) return err;     \
  } while (0)

  // W1's transpose for dx (its 192-wide tiles take no k-major weights); W2
  // is read as stored, k-major, by the du GEMM
  MOE_TRY(launch_transpose(a.w1, G, H, D, w1t, stream));
  if (a.total_rows > 0) {
    // u: the forward's saved pre-activations, or recomputed (with
    // h = gelu(u) beside it when h was not kept either).
    const void* uu = a.u_saved;
    if (uu == nullptr) {
      GemmParams pu{a.x, a.row_index, a.w1, a.b1, u, a.offsets, a.total_rows,
                    G, H, D};
      pu.a_rows = a.src_rows;
      if (a.h_saved == nullptr) {
        pu.c = ws + L.h;
        pu.u_out = u;
        launch_stage<kEpiGelu, true, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false>(
            pu, stream);
      } else {
        launch_stage<kEpiStore, true, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false>(
            pu, stream);
      }
      MOE_TRY(hipGetLastError());
      uu = u;
    } else if (a.h_saved == nullptr) {
      MOE_TRY(launch_rows(uu, nullptr, 0, a.total_rows, H, true, ws + L.h,
                          stream));
    }
    GemmParams pd{a.dy_rows, nullptr, a.w2, nullptr, du, a.offsets,
                  a.total_rows, G, H, D};
    pd.aux = uu;
    launch_stage<kEpiGeluGrad, true, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false,
                 4, true>(pd, stream);
    MOE_TRY(hipGetLastError());
    GemmParams px{du, nullptr, w1t, nullptr, a.dx_rows, a.offsets,
                  a.total_rows, G, D, H};
    if (a.dx_f32)
      launch_stage<kEpiStore, false, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF,
                   4, false, kDnNST>(
          px, stream);
    else
      launch_stage<kEpiStore, true, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF,
                   4, false, kDnNST>(
          px, stream);
    MOE_TRY(hipGetLastError());
    if (a.row_index != nullptr)
      MOE_TRY(launch_rows(a.x, a.row_index, a.src_rows, a.total_rows, D, false,
                          ws + L.xr, stream));
  }
  // dW2[g] [D][H] = dy_rows[g]^T h[g];  dW1[g] [H][D] = du[g]^T x_rows[g].
  // With no rows every segment is empty and the products are zero.
  // When the tiles would not fill the chip, the reduction is split and the
  // partials are added in split order afterwards.
  const int S = choose_ksplit(G, D, H, a.total_rows);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const int64_t n4 = static_cast<int64_t>(G) * D * H / 4;
  const unsigned rgrid =
      static_cast<unsigned>(std::min<int64_t>((n4 + 255) / 256, 4096));
  GemmParams pw2{a.dy_rows, nullptr, hh, nullptr, S > 1 ? part : a.dw2,
                 a.offsets, a.total_rows, G, H, 0};
  pw2.mrows = D;
  pw2.ksplit = S;
  const int tiles2 =
      S * G * ((D + kUpBM - 1) / kUpBM) * ((H + kUpBN - 1) / kUpBN);
  hipLaunchKernelGGL(
      (gemm_bf16_kernel<kEpiStore, false, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false, true>),
      dim3(persistent_grid(tiles2)), dim3(64 * kUpWT * kUpWF), 0, stream, pw2);
  MOE_TRY(hipGetLastError());
  if (S > 1) {
    hipLaunchKernelGGL(ksplit_reduce_kernel, dim3(rgrid), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(part), S, n4,
                       reinterpret_cast<float4*>(a.dw2));
    MOE_TRY(hipGetLastError());
  }
  GemmParams pw1{du, nullptr, xr, nullptr, S > 1 ? part : a.dw1, a.offsets,
                 a.total_rows, G, D, 0};
  pw1.mrows = H;
  pw1.ksplit = S;
  const int tiles1 =
      S * G * ((H + kUpBM - 1) / kUpBM) * ((D + kUpBN - 1) / kUpBN);
  hipLaunchKernelGGL(
      (gemm_bf16_kernel<kEpiStore, false, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false, true>),
      dim3(persistent_grid(tiles1)), dim3(64 * kUpWT * kUpWF), 0, stream, pw1);
  MOE_TRY(hipGetLastError());
  if (S > 1) {
    hipLaunchKernelGGL(ksplit_reduce_kernel, dim3(rgrid), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(part), S, n4,
                       reinterpret_cast<float4*>(a.dw1));
    MOE_TRY(hipGetLastError());
  }
#undef MOE_TRY
  return hipSuccess;
}

hipError_t launch_ffn_down_combine(const void* h, int64_t N, int D, int H,
                                  const void* w2, const float* b2,
                                  const void* y_rows, const int32_t* slot_row,
                                  const float* topk_w, int Kmax, void* y,
                                  hipStream_t stream) {
  if (N == 0) return hipSuccess;
  GemmParams p{h,       nullptr, w2,       b2,     y, nullptr, N, 1, D, H,
               y_rows, slot_row, topk_w, Kmax};
  if (Kmax <= 4)
    launch_stage<kEpiCombine, true, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF, 4,
                 false, kDnNST>(
        p, stream);
  else
    launch_stage<kEpiCombine, true, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF,
                 kCombineMaxSlots, false, kDnNST>(p, stream);
  return hipGetLastError();
}

bool mlp_fused_supported(int D, int H) {
  return (D == 128 || D == 256 || D == 384) && H > 0 && H % kMlpHC == 0;
}

hipError_t launch_mlp_fused(const FfnArgs& a, hipStream_t stream) {
  if (a.total_rows == 0) return hipSuccess;
  GemmParams p{a.x, a.row_index, a.w1, a.b1, a.y, a.offsets, a.total_rows,
               a.G, a.D, a.D};
  p.a_rows = a.src_rows;
  const int tiles = tile_grid(p, kMlpBM, a.D);
  const dim3 grid(static_cast<unsigned>(tiles)), block(64 * kMlpWaves);
  const int yf = a.y_f32 ? 1 : 0;
  switch (a.D) {
    case 128:
      hipLaunchKernelGGL((mlp_fused_kernel<1>), grid, block, 0, stream, p,
                         a.w2, a.b2, a.H, yf);
      break;
    case 256:
      hipLaunchKernelGGL((mlp_fused_kernel<2>), grid, block, 0, stream, p,
                         a.w2, a.b2, a.H, yf);
      break;
    default:
      hipLaunchKernelGGL((mlp_fused_kernel<3>), grid, block, 0, stream, p,
                         a.w2, a.b2, a.H, yf);
  }
  return hipGetLastError();
}

size_t ffn_split_workspace_bytes() {
  // one slot per workgroup of the largest persistent grid
  return kSplitHdrBytes + static_cast<size_t>(cu_count() / 8 * 8) * kDnBM *
                              kDnBN * sizeof(float);
}

hipError_t launch_ffn(const FfnArgs& a, bool up, bool down,
                      hipStream_t stream) {
  if (a.total_rows == 0) return hipSuccess;
  GemmParams p1{a.x, a.row_index, a.w1, a.b1, a.h, a.offsets, a.total_rows,
                a.G, a.H, a.D};
  p1.u_out = a.u;
  p1.a_rows = a.src_rows;
  GemmParams p2{a.h, nullptr, a.w2, a.b2, a.y, a.offsets, a.total_rows,
                a.G, a.D, a.H};
  p2.sk_ws = a.split_ws;
  if (a.bf16) {
    if (up) {
      launch_stage<kEpiGelu, true, kUpBM, kUpBN, kUpWT, kUpWF, kUpGM, false>(
          p1, stream);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (down) {
      if (a.y_f32)
        launch_stage<kEpiStore, false, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF,
                     4, false, kDnNST>(
            p2, stream);
      else
        launch_stage<kEpiStore, true, kDnBM, kDnBN, kDnWT, kDnWF, kDnGM, kDnPF,
                     4, false, kDnNST>(
            p2, stream);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  if (up) {
    hipLaunchKernelGGL((gemm_f32_kernel<kEpiGelu>),
                       dim3(tile_grid(p1, kFM, kFN)), dim3(kF32Threads), 0,
                       stream, p1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (down) {
    hipLaunchKernelGGL((gemm_f32_kernel<kEpiStore>),
                       dim3(tile_grid(p2, kFM, kFN)), dim3(kF32Threads), 0,
                       stream, p2);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
