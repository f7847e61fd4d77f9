// Host-side launchers of the gfx950 kernels (internal to libmoe).
// Every launcher only enqueues work on `stream` and returns the launch
// status; argument validation lives in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ffn.hip: the CU count of the current device (read once per device).
int cu_count();

// gate.hip
hipError_t launch_gate(const void* x, bool x_bf16, const float* w_gate,
                       const float* bias, int64_t N, int D, int E, int K,
                       bool topk, float* probs, int32_t* idx, float* w,
                       hipStream_t stream);
// Top-K gate that also writes the balance statistic's per-16-token partial
// sums (bal_p [N/16][E] fp32, bal_c [N/16][E] int32); fuses when x is bf16,
// the streaming gate holds the weights and T is a multiple of 16.
bool gate_balance_fuses(bool x_bf16, int64_t N, int T, int D, int E);
hipError_t launch_gate_balance_partials(const void* x, const float* w_gate,
                                        const float* bias, int64_t N, int D,
                                        int E, int K, float* probs,
                                        int32_t* idx, float* w, float* bal_p,
                                        int32_t* bal_c, hipStream_t stream);
size_t race_workspace_bytes();
hipError_t launch_race(const float* probs, int64_t N, int E, int K,
                       int32_t* idx, float* w, void* workspace,
                       hipStream_t stream);

// permute.hip
size_t permute_workspace_bytes(int64_t N, int E);
// The allocation-free variant's static scratch: its size, and its address on
// the current device (looked up once per device).
size_t permute_scratch_bytes();
hipError_t permute_scratch(void** ptr);
hipError_t launch_permute(const void* x, bool bf16, const int32_t* idx,
                          int64_t N, int D, int E, int Kmax, int64_t A,
                          int32_t* counts, int64_t* offsets, int32_t* row_token,
                          int32_t* slot_row, void* x_perm, void* workspace,
                          hipStream_t stream);
// The permute's last step alone: ranks every selection inside its 256-token
// block from the block bases (block_base [ceil(N/256)][E] int64, as the
// scan writes them) and writes slot_row and row_token.
hipError_t launch_permute_scatter(const int32_t* idx, int64_t N, int E,
                                  int Kmax, int64_t A, const int64_t* block_base,
                                  int32_t* slot_row, int32_t* row_token,
                                  hipStream_t stream);

// ffn.hip
// Most groups (experts) one grouped-FFN launch takes.
constexpr int kMaxFfnGroups = 128;
struct FfnArgs {
  const void* x;            // [*][D]
  const int32_t* row_index; // [total] or null
  int64_t total_rows;
  const int64_t* offsets;   // [G+1] device
  int G, D, H;
  const void* w1;           // [G][H][D]
  const float* b1;          // [G][H] or null
  const void* w2;           // [G][D][H]
  const float* b2;          // [G][D] or null
  void* h;                  // [total][H]
  void* y;                  // [total][D]
  bool bf16;                // input / weight / h dtype
  bool y_f32;               // output dtype
  void* u = nullptr;        // [total][H] bf16 pre-activations out, or null
  int64_t src_rows = 0;     // rows of x when row_index is given
  // stage 2 (bf16 inputs): ffn_split_workspace_bytes() of device scratch
  // for splitting its last round of tiles along k, or null
  float* split_ws = nullptr;
};
size_t ffn_split_workspace_bytes();
hipError_t launch_ffn(const FfnArgs& a, bool up, bool down, hipStream_t stream);
// Both stages in one kernel (bf16, D in {128, 256, 384}, H % 64 == 0); h is
// not used.
bool mlp_fused_supported(int D, int H);
hipError_t launch_mlp_fused(const FfnArgs& a, hipStream_t stream);
// Stage 2 of the shared experts (one group of all N tokens, bf16) fused with
// the weighted combine of the routed outputs; Kmax <= 4.
hipError_t launch_ffn_down_combine(const void* h, int64_t N, int D, int H,
                                  const void* w2, const float* b2,
                                  const void* y_rows, const int32_t* slot_row,
                                  const float* topk_w, int Kmax, void* y,
                                  hipStream_t stream);

// combine.hip
hipError_t launch_combine(const void* y_rows, bool y_bf16,
                          const int32_t* slot_row, const float* w, int64_t N,
                          int D, int Kmax, const void* y_shared, bool sh_bf16,
                          void* y, bool out_bf16, hipStream_t stream);

// balance.hip
// Bytes of the partial-sum buffer for N tokens (fp32 half, then int32 half).
size_t balance_partials_bytes(int64_t N, int E);
hipError_t launch_balance_from_partials(const void* partials, int B, int T,
                                        int E, int K, float alpha, bool global,
                                        int32_t* counts, float* psum,
                                        float* loss, hipStream_t stream);
// Fused routing call, second launch: the balance finish from the gate's
// partials and the permutation's expert scan over its per-16-token
// selection counts (two workgroups of one launch).
hipError_t launch_route_finish(const void* partials, int B, int T, int E,
                               int K, float alpha, bool global, int32_t* counts,
                               float* psum, float* loss, int32_t* expert_counts,
                               int64_t* expert_offsets, int64_t* block_base,
                               hipStream_t stream);
hipError_t launch_balance(const float* probs, const int32_t* idx, int B, int T,
                          int E, int Kmax, int K, float alpha, bool global,
                          int32_t* counts, float* psum, float* loss,
                          hipStream_t stream);

// backward.hip
hipError_t launch_transpose(const void* src, int G, int R, int C, void* dst,
                            hipStream_t stream);
// dst[r] = src[row_index[r]] (or src[r]), optionally through GELU; index
// entries outside [0, src_rows) give zero rows.
hipError_t launch_rows(const void* src, const int32_t* row_index,
                       int64_t src_rows, int64_t total, int C, bool gelu,
                       void* dst, hipStream_t stream);
hipError_t launch_combine_backward(const void* dy, bool dy_bf16,
                                   const void* y_rows, bool y_bf16,
                                   const int32_t* slot_row, const float* w,
                                   int64_t N, int D, int Kmax, void* dy_rows,
                                   float* dw, hipStream_t stream);
size_t gate_backward_workspace_bytes(int64_t N, int E, int D);
hipError_t launch_gate_backward(const void* x, bool x_bf16, const float* wg,
                                const float* probs, const int32_t* idx,
                                const float* dw, const int32_t* counts, int B,
                                int T, int D, int E, int Kmax, int K, float alpha,
                                float dloss, bool global, const void* dx_rows,
                                const int32_t* slot_row, const void* dx_shared,
                                bool dx_bf16, void* dx, float* dw_gate,
                                float* dbias, void* workspace,
                                hipStream_t stream);

// ffn.hip, backward of the grouped expert MLPs (bf16)
struct FfnBwdArgs {
  const void* x;            // [*][D]
  const int32_t* row_index; // [total] or null
  int64_t total_rows;
  const int64_t* offsets;   // [G+1] device
  int G, D, H;
  const void* w1;           // [G][H][D]
  const float* b1;          // [G][H] or null
  const void* w2;           // [G][D][H]
  const void* dy_rows;      // [total][D] gradient of the expert outputs
  void* workspace;
  void* dx_rows;            // [total][D]
  bool dx_f32;
  float* dw1;               // [G][H][D]
  float* dw2;               // [G][D][H]
  const void* u_saved = nullptr;  // [total][H] forward pre-activations, or null
  const void* h_saved = nullptr;  // [total][H] forward activations, or null
  int64_t src_rows = 0;           // rows of x when row_index is given
};
size_t ffn_backward_workspace_bytes(int64_t total, int G, int D, int H);
hipError_t launch_ffn_backward(const FfnBwdArgs& a, hipStream_t stream);

// analytics.hip
hipError_t launch_routing_hist(const int32_t* idx, int B, int T, int E,
                               int Kmax, const int32_t* tags, int n_tags,
                               int64_t* pos_counts, int64_t* tag_counts,
                               hipStream_t stream);

}  // namespace moe
