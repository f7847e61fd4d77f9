/*
 * moe.h -- C ABI of the DiT-MoE sparse mixture-of-experts feed-forward layer
 * on one MI355X (gfx950).
 *
 * The layer, per image-patch token x (a row of D features):
 *   y = sum over the token's selected routed experts i of P(t,i) * e_i(x)
 *     + sum over the n_s shared experts s of e_s(x),
 *   e(x) = W2 gelu_tanh(W1 x),
 * with P the softmax of the gate scores over the E routed experts, plus the
 * expert-level balance statistic of the routing.
 *
 * Sources, by page title and section:
 *   "DiT-MoE" project hub page, section 1 (MoE gate routing): the gate weight
 *     is [n_routed_experts][gating_dim], softmax scoring, top-k selection and
 *     an auxiliary balance loss.
 *   "Scaling Diffusion Transformers to 16 Billion Parameters", Methods: eq.
 *     MoE(x) = sum_i g(x)_i e_i(x) (MoE recap); eq. MLP(x) = W2 gelu(W1 x),
 *     shared expert routing and the expert-level balance loss eq. L_balance
 *     (MoE-DiT).
 *   "Scalable Diffusion Models with Transformers (DiT)", model architecture:
 *     the GELU is the tanh approximation.
 *   "Expert Race: A Flexible Routing Strategy for Scaling Diffusion
 *     Transformer with Mixture of Experts", abstract: tokens and experts
 *     compete together for the top candidates.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     allocated and owned by the caller.  The library never allocates,
 *     frees or synchronises; every call only validates its arguments on the
 *     host and enqueues kernels on `stream` (asynchronous).
 *   - All layouts are row-major and dense.  Expert weights follow the
 *     y = x W^T convention: W1 is [G][H][D], W2 is [G][D][H].
 *   - A pointer to an empty tensor (a size of 0) may be NULL.
 *   - A call that fails validation returns a non-zero status and launches
 *     nothing; moe_last_error() then describes the failure (thread-local).
 *     MOE_ERR_HIP reports a launch error from the HIP runtime.  Device data
 *     are not validated: NaN/Inf inputs are outside the contract, and every
 *     kernel stays in bounds on any input values, except that the slot rows
 *     passed to moe_combine, moe_ffn_down_combine and moe_combine_backward
 *     must name rows of y_rows, or be -1.  Row indices of the expert MLPs
 *     (row_index) come with the row count of the matrix they index: an
 *     entry outside it reads a zero row.
 *   - The library keeps no state between calls and is thread-safe.
 *   - Supported ranges: 1 <= E <= 64, 1 <= K <= E, D and H multiples of 8,
 *     N * Kmax < 2^31, every row count < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* null pointer, negative size, K > E ...  */
  MOE_ERR_UNSUPPORTED = 2,         /* legal but outside the supported range   */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the queried size  */
  MOE_ERR_HIP = 4                  /* the HIP runtime reported an error       */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_ROUTE_TOPK = 0, MOE_ROUTE_EXPERT_RACE = 1 } moe_route;

typedef enum { MOE_BAL_PER_SEQUENCE = 0, MOE_BAL_GLOBAL = 1 } moe_balance_mode;

/* Which GEMM stages of moe_grouped_ffn to run (bit mask). */
typedef enum {
  MOE_FFN_UP = 1,    /* h = gelu_tanh(W1 a + b1)  */
  MOE_FFN_DOWN = 2,  /* y = W2 h + b2             */
  MOE_FFN_BOTH = 3
} moe_ffn_stages;

/* Text of a status code (static storage). */
const char* moe_status_string(moe_status status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of device workspace moe_gate_topk needs: 0 for top-K routing; for
 * Expert Race a fixed ~1 MiB (the radix passes' per-workgroup histograms
 * and the threshold), whatever N and E.  The contents need no
 * initialisation. */
size_t moe_gate_workspace_size(int64_t N, int32_t E, int32_t K, moe_route route);

/*
 * Gate, softmax and expert selection ("DiT-MoE" hub page, section 1;
 * "Expert Race" abstract for MOE_ROUTE_EXPERT_RACE).
 *
 *   logit[t][i] = sum_d x[t][d] * w_gate[i][d] + logit_bias[i]   (fp32)
 *   probs[t][i] = softmax over the E routed experts of logit[t][.]  (fp32)
 *
 * MOE_ROUTE_TOPK (Kmax = K): each token keeps the K experts first in the
 *   order (probability descending, expert index ascending); slot k of token
 *   t holds the k-th of them: topk_idx[t][k], topk_w[t][k] = probs[t][idx].
 * MOE_ROUTE_EXPERT_RACE (Kmax = E): of all N*E probabilities the K*N first
 *   in the order (probability descending, flat index t*E+i ascending) are
 *   kept; each token lists its kept experts in ascending index order in
 *   topk_idx[t][0..], with topk_w the probabilities, and pads the rest of
 *   its E slots with idx = -1, w = 0.  A token may keep 0..E experts.
 *
 *   x          [N][D], x_dtype (MOE_F32 or MOE_BF16)
 *   w_gate     [E][D] fp32;   logit_bias [E] fp32 or NULL (no bias)
 *   probs      [N][E] fp32 out
 *   topk_idx   [N][Kmax] int32 out;  topk_w [N][Kmax] fp32 out
 *   workspace  device scratch of at least moe_gate_workspace_size() bytes
 *              (may be NULL when that size is 0)
 * Errors: INVALID_ARGUMENT for null pointers, N < 0, D < 1, K outside
 *   [1, E]; UNSUPPORTED for E > 64, D % 8 != 0, N*Kmax >= 2^31 or an unknown
 *   dtype; WORKSPACE_TOO_SMALL.
 */
moe_status moe_gate_topk(const void* x, moe_dtype x_dtype,
                         const float* w_gate, const float* logit_bias,
                         int64_t N, int32_t D, int32_t E, int32_t K,
                         moe_route route, float* probs, int32_t* topk_idx,
                         float* topk_w, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of device workspace moe_permute needs. */
size_t moe_permute_workspace_size(int64_t N, int32_t E, int32_t Kmax);

/*
 * Group the selected (token, slot) pairs by expert, so that only the
 * selected experts are evaluated ("Scaling Diffusion Transformers to 16
 * Billion Parameters", MoE recap: a sparse g needs no unused expert).
 *
 * A = K*N routed rows.  Rows of expert e are its selections in ascending
 * (token, slot) order and occupy [expert_offsets[e], expert_offsets[e+1]).
 *
 *   topk_idx        [N][Kmax] int32 in: expert per slot, -1 = empty slot;
 *                   a token names an expert at most once and exactly A slots
 *                   in total are non-empty
 *   expert_counts   [E] int32 out
 *   expert_offsets  [E+1] int64 out (exclusive scan, offsets[E] = A)
 *   row_token       [A] int32 out: token of each routed row
 *   slot_row        [N][Kmax] int32 out: routed row of each slot, -1 if empty
 *   x_perm          [A][D] dtype out, or NULL: row r = x[row_token[r]]
 *                   (with NULL only the index tensors are written and the
 *                   expert FFN gathers rows through row_token instead)
 * Errors: as moe_gate_topk; Kmax must be K or E.  Slot contents outside
 *   [-1, E) are not an error: such slots are treated as empty.
 */
moe_status moe_permute(const void* x, moe_dtype dtype, const int32_t* topk_idx,
                       int64_t N, int32_t D, int32_t E, int32_t Kmax, int32_t K,
                       int32_t* expert_counts, int64_t* expert_offsets,
                       int32_t* row_token, int32_t* slot_row, void* x_perm,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of the static scratch moe_permute_noalloc works in. */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as moe_permute,
 * minus the workspace: its block counts and bases live in a static device
 * array of MOE_PERMUTE_NOALLOC_SCRATCH_BYTES bytes, one per device, held
 * until the process ends.  The call allocates nothing.
 *
 * Limit: moe_permute_workspace_size(N, E, Kmax) must not exceed the scratch
 *   (about N * E <= 22 million, e.g. N <= 2.7 million tokens at E = 8);
 *   larger inputs return MOE_ERR_UNSUPPORTED.
 * Concurrency: every call on a device shares that device's scratch.  Calls
 *   that may overlap on one device (different streams, or several host
 *   threads) race and give wrong results; order them, e.g. on one stream.
 *   Nothing in the scratch needs to start at zero.
 * The first call on a device looks up the scratch's address on that
 *   device (hipGetSymbolAddress); a failure there returns MOE_ERR_HIP.
 */
moe_status moe_permute_noalloc(const void* x, moe_dtype dtype,
                               const int32_t* topk_idx, int64_t N, int32_t D,
                               int32_t E, int32_t Kmax, int32_t K,
                               int32_t* expert_counts, int64_t* expert_offsets,
                               int32_t* row_token, int32_t* slot_row,
                               void* x_perm, hipStream_t stream);

/*
 * The experts' MLPs over row groups ("Scaling Diffusion Transformers to 16
 * Billion Parameters", MoE-DiT eq. MLP; "Scalable Diffusion Models with
 * Transformers (DiT)": tanh GELU):
 *
 *   for each group g and each row r in [group_offsets[g], group_offsets[g+1]):
 *     h[r]      = gelu_tanh(W1[g] a_r + b1[g])         (h_ws, dtype)
 *     y_rows[r] = W2[g] h[r] + b2[g]                    (y_dtype)
 *   with a_r = x_rows[row_index[r]] if row_index != NULL, else x_rows[r];
 *   gelu_tanh(u) = 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).
 *
 * Routed experts: G = E, group_offsets = expert_offsets from moe_permute and
 * either x_perm or (x, row_token).  Shared experts: G = 1, offsets {0, N},
 * x itself, and the n_s shared experts stacked into one MLP of hidden width
 * n_s*H (W1 rows concatenated, W2 columns concatenated) -- their outputs
 * sum with weight 1, which is exactly that wider MLP.
 *
 *   x_rows         [src_rows][D] dtype with row_index, else [total_rows][D]
 *   row_index      [total_rows] int32 or NULL; an entry outside
 *                  [0, src_rows) reads a zero row (never memory outside
 *                  x_rows)
 *   src_rows       rows of x_rows, read only with row_index (then >= 1 when
 *                  stage 1 runs on rows, and (src_rows + 1) * D * element
 *                  bytes + 256 <= 2^32)
 *   group_offsets  [G+1] int64 DEVICE array, non-decreasing, from 0 to
 *                  total_rows (total_rows is also passed by value)
 *   w1 [G][H][D], w2 [G][D][H] dtype;  b1 [G][H], b2 [G][D] fp32 or NULL
 *   h_ws           [total_rows][H] dtype scratch (caller-owned)
 *   u_ws           [total_rows][H] bf16 out, or NULL: with stage 1, the
 *                  pre-activations u[r] = W1[g] a_r + b1[g] rounded once to
 *                  bf16 (what the training backward needs; passing them to
 *                  moe_grouped_ffn_backward skips its recomputation).  bf16
 *                  inputs only.
 *   y_rows         [total_rows][D] y_dtype out (MOE_F32, or MOE_BF16 when
 *                  dtype is MOE_BF16)
 *   stages         MOE_FFN_BOTH, or one stage alone (MOE_FFN_UP writes h_ws;
 *                  MOE_FFN_DOWN reads it): the two stages are two kernels,
 *                  and running them as two calls gives identical results.
 *                  With MOE_FFN_DOWN alone x_rows, row_index and w1 are not
 *                  read; with MOE_FFN_UP alone w2 and y_rows are not.
 * Arithmetic: bf16 inputs use bf16 MFMA with fp32 accumulation; h and bf16
 *   outputs are rounded to nearest even.  fp32 inputs compute in fp32.
 * Errors: INVALID_ARGUMENT for null pointers, negative sizes, stages
 *   outside 1..3 or src_rows < 1 with row_index; UNSUPPORTED for G > 128,
 *   D or H not multiples of 8, an unsupported dtype pair, total_rows >=
 *   2^31 or a gathered x_rows past the 4 GiB range above.
 */
moe_status moe_grouped_ffn(const void* x_rows, const int32_t* row_index,
                           int64_t src_rows, moe_dtype dtype,
                           int64_t total_rows,
                           const int64_t* group_offsets, int32_t G, int32_t D,
                           int32_t H, const void* w1, const float* b1,
                           const void* w2, const float* b2, void* h_ws,
                           void* u_ws, void* y_rows, moe_dtype y_dtype,
                           moe_ffn_stages stages, hipStream_t stream);

/* Bytes of device workspace moe_grouped_ffn_split needs on the current
 * device (a small header and one 256 x 192 fp32 tile per compute unit). */
size_t moe_grouped_ffn_split_workspace_size(void);

/*
 * moe_grouped_ffn with a workspace that lets stage 2 (bf16 inputs, large
 * tiles) split its last round of tiles along k: the expert GEMM keeps one
 * workgroup per compute unit walking its tiles, and when the tile count is
 * not a multiple of the workgroups, the R tiles of the last, partial round
 * are cut into S = min(workgroups / R, k stages) >= 2 pieces each, which
 * the workgroups that would otherwise idle multiply; one small kernel then
 * adds each tile's pieces in piece order, adds b2 and rounds once.  Stage 1
 * and the other stage-2 forms run as in moe_grouped_ffn.  Same arguments
 * and checks as moe_grouped_ffn; y is computed as there (fp32 accumulation
 * of the same products), with the k sums of the split tiles associated
 * piece by piece: results agree to fp32 rounding, deterministically for a
 * given routing.
 *
 *   workspace  device scratch of at least
 *              moe_grouped_ffn_split_workspace_size() bytes, 16-byte
 *              aligned (contents need no initialisation; calls that share
 *              one workspace must not overlap)
 * Errors: as moe_grouped_ffn; WORKSPACE_TOO_SMALL; INVALID_ARGUMENT for a
 *   null or misaligned workspace.
 */
moe_status moe_grouped_ffn_split(const void* x_rows, const int32_t* row_index,
                                 int64_t src_rows, moe_dtype dtype,
                                 int64_t total_rows,
                                 const int64_t* group_offsets, int32_t G,
                                 int32_t D, int32_t H, const void* w1,
                                 const float* b1, const void* w2,
                                 const float* b2, void* h_ws, void* u_ws,
                                 void* y_rows, moe_dtype y_dtype,
                                 moe_ffn_stages stages, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * The experts' MLPs of moe_grouped_ffn in one kernel, for narrow layers
 * (same page and equations as moe_grouped_ffn): for each group g and row r,
 *   y_rows[r] = W2[g] gelu_tanh(W1[g] a_r + b1[g]) + b2[g]
 * with the hidden activation kept on chip (never written to memory).  The
 * hidden values are rounded to bf16 and the sums run in the same order as
 * in moe_grouped_ffn, so both calls give identical results.
 *
 *   arguments as moe_grouped_ffn, without h_ws and stages
 * Errors: INVALID_ARGUMENT for null pointers, negative sizes or src_rows
 *   < 1 with row_index; UNSUPPORTED unless dtype is MOE_BF16 (y_dtype
 *   MOE_BF16 or MOE_F32), D is 128, 256 or 384 and H is a multiple of 64,
 *   G <= 128, total_rows < 2^31 and a gathered x_rows fits the 4 GiB range
 *   of moe_grouped_ffn.
 */
moe_status moe_grouped_mlp_fused(const void* x_rows, const int32_t* row_index,
                                 int64_t src_rows, moe_dtype dtype,
                                 int64_t total_rows,
                                 const int64_t* group_offsets, int32_t G,
                                 int32_t D, int32_t H, const void* w1,
                                 const float* b1, const void* w2,
                                 const float* b2, void* y_rows,
                                 moe_dtype y_dtype, hipStream_t stream);

/*
 * Weighted combine ("Scaling Diffusion Transformers to 16 Billion
 * Parameters": eq. MoE(x) with g(x)_i the gate probability; shared experts
 * added with weight 1):
 *
 *   y[t] = sum over k < Kmax with slot_row[t][k] >= 0 of
 *            topk_w[t][k] * y_rows[slot_row[t][k]]     (in slot order)
 *        + y_shared[t]                                 (if not NULL)
 * accumulated in fp32 and rounded once to out_dtype.
 *
 *   y_rows [A][D] y_dtype;  slot_row, topk_w [N][Kmax] (slot_row entries
 *   are rows of y_rows or -1);
 *   y_shared [N][D] sh_dtype or NULL;  y [N][D] out_dtype out
 * Errors: INVALID_ARGUMENT for null pointers, N < 0 or Kmax < 1;
 *   UNSUPPORTED for D % 8 != 0, Kmax > 64, N*D/8 >= 2^31 or unknown dtypes.
 */
moe_status moe_combine(const void* y_rows, moe_dtype y_dtype,
                       const int32_t* slot_row, const float* topk_w, int64_t N,
                       int32_t D, int32_t Kmax, const void* y_shared,
                       moe_dtype sh_dtype, void* y, moe_dtype out_dtype,
                       hipStream_t stream);

/*
 * Expert-level balance statistic ("Scaling Diffusion Transformers to 16
 * Billion Parameters", MoE-DiT, eq. L_balance):
 *
 *   L = alpha * sum_i (n/(K T) sum_t I(t,i)) * (1/T sum_t P(t,i))
 *
 * n = E routed experts, T = tokens per image, I(t,i) = 1 when token t
 * selected expert i, P = probs.  Per image b (tokens [bT, (b+1)T)):
 *   counts[b][i]    = sum_t I(t,i)          (int32 out, [B][E])
 *   prob_sums[b][i] = sum_t P(t,i)          (fp32 out, [B][E])
 * MOE_BAL_PER_SEQUENCE: loss = mean over b of L_b.
 * MOE_BAL_GLOBAL: loss = L over one pool of B*T tokens.
 * B = 0 (no tokens): loss = 0 in both modes.
 * Sums use a fixed reduction order: repeated calls give identical bits.
 *
 *   probs [B*T][E] fp32;  topk_idx [B*T][Kmax] int32 (-1 = empty);
 *   loss [1] fp32 device out
 * Errors: INVALID_ARGUMENT for null pointers, B < 0, T < 1, K outside
 *   [1, E]; UNSUPPORTED for E > 64.
 */
moe_status moe_balance_stats(const float* probs, const int32_t* topk_idx,
                             int32_t B, int32_t T, int32_t E, int32_t Kmax,
                             int32_t K, float alpha, moe_balance_mode mode,
                             int32_t* counts, float* prob_sums, float* loss,
                             hipStream_t stream);

/* Bytes of device workspace moe_gate_topk_balance needs. */
size_t moe_gate_balance_workspace_size(int32_t B, int32_t T, int32_t E);

/*
 * Top-K gate and the balance statistic in one call ("DiT-MoE" hub page,
 * section 1: the gate returns the selected experts, their weights and the
 * auxiliary loss; "Scaling Diffusion Transformers to 16 Billion
 * Parameters", MoE-DiT, eq. L_balance).  Computes exactly what
 * moe_gate_topk (MOE_ROUTE_TOPK) followed by moe_balance_stats (Kmax = K)
 * compute, for N = B*T tokens, image b owning tokens [bT, (b+1)T).
 *
 * When x is bf16, T is a multiple of 16 and E <= 16 (the streaming gate
 * kernel), the gate kernel also reduces each 16-token group to partial
 * sums in the workspace and one small kernel finishes counts, prob_sums and
 * the loss; probs, topk_idx, topk_w and counts are then bit for bit those of
 * the separate calls, and prob_sums and loss differ from them only by the
 * order of the fp32 additions (pairwise over each 16-token group, then the
 * groups in order).  Otherwise the separate kernels run.  Either way the
 * result is deterministic.
 *
 *   arguments as moe_gate_topk and moe_balance_stats;
 *   workspace  device scratch of at least moe_gate_balance_workspace_size()
 *              bytes (contents need no initialisation)
 * Errors: as moe_gate_topk and moe_balance_stats; WORKSPACE_TOO_SMALL.
 */
moe_status moe_gate_topk_balance(const void* x, moe_dtype x_dtype,
                                 const float* w_gate, const float* logit_bias,
                                 int32_t B, int32_t T, int32_t D, int32_t E,
                                 int32_t K, float alpha, moe_balance_mode mode,
                                 float* probs, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, float* prob_sums, float* loss,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Bytes of device workspace moe_gate_route needs. */
size_t moe_gate_route_workspace_size(int32_t B, int32_t T, int32_t E);

/*
 * Top-K gate, balance statistic and expert permutation in one call
 * ("DiT-MoE" hub page, section 1: the gate returns the selected experts,
 * their weights and the auxiliary loss; "Scaling Diffusion Transformers to
 * 16 Billion Parameters", MoE-DiT eq. L_balance, and MoE recap: only the
 * selected experts are evaluated, so their rows are grouped by expert).
 * Computes exactly what moe_gate_topk_balance followed by moe_permute
 * (Kmax = K, x_perm = NULL) compute, bit for bit, for N = B*T tokens.
 *
 * When moe_gate_topk_balance takes its fused form (bf16 x, T a multiple of
 * 16, E <= 16) this runs three kernels: the gate, which also writes the
 * balance statistic's per-16-token partial sums and selection counts; one
 * launch of two workgroups, the balance finish beside the permutation's
 * expert scan over those selection counts (they replace the permutation's
 * count pass); and the permutation's scatter.  Otherwise it runs the two
 * calls' kernels in turn.
 *
 *   arguments as moe_gate_topk_balance, then as moe_permute's outputs
 *   (expert_counts [E], expert_offsets [E+1], row_token [K*N],
 *   slot_row [N][K]);
 *   workspace  device scratch of at least moe_gate_route_workspace_size()
 *              bytes, 256-byte aligned (contents need no initialisation)
 * Errors: as moe_gate_topk_balance and moe_permute (K*N below 2^31);
 *   WORKSPACE_TOO_SMALL.
 */
moe_status moe_gate_route(const void* x, moe_dtype x_dtype,
                          const float* w_gate, const float* logit_bias,
                          int32_t B, int32_t T, int32_t D, int32_t E, int32_t K,
                          float alpha, moe_balance_mode mode, float* probs,
                          int32_t* topk_idx, float* topk_w, int32_t* counts,
                          float* prob_sums, float* loss, int32_t* expert_counts,
                          int64_t* expert_offsets, int32_t* row_token,
                          int32_t* slot_row, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Stage 2 of the shared experts fused with the weighted combine ("Scaling
 * Diffusion Transformers to 16 Billion Parameters": eq. MLP for the shared
 * experts, eq. MoE(x) for the routed ones, shared experts added with
 * weight 1).  For every token t < N:
 *
 *   s[t] = bf16( h[t] . w2^T (+ b2) )                  (fp32 accumulation)
 *   y[t] = sum over k < Kmax with slot_row[t][k] >= 0, in slot order, of
 *            topk_w[t][k] * y_rows[slot_row[t][k]]  +  s[t]
 * in fp32, rounded once to bf16: bit for bit what moe_grouped_ffn (stage 2
 * of the shared experts, one group of all N tokens) followed by moe_combine
 * produce, without writing or reading the shared output.
 *
 *   h [N][H] bf16 (stage-1 output of the shared experts, H = n_s * hidden);
 *   w2 [D][H] bf16 (the shared experts' W2 side by side); b2 [D] fp32 or
 *   NULL;  y_rows [*][D] bf16 routed outputs;  slot_row, topk_w [N][Kmax];
 *   y [N][D] bf16 out
 * Errors: INVALID_ARGUMENT for null pointers (N > 0), N < 0, D, H or
 *   Kmax < 1; UNSUPPORTED for a dtype other than bf16, Kmax > 16 (top-K
 *   routing with K <= 16, or Expert Race with E <= 16), D or H not
 *   multiples of 8, N*Kmax >= 2^31.
 */
moe_status moe_ffn_down_combine(const void* h, moe_dtype dtype, int64_t N,
                                int32_t D, int32_t H, const void* w2,
                                const float* b2, const void* y_rows,
                                const int32_t* slot_row, const float* topk_w,
                                int32_t Kmax, void* y, hipStream_t stream);

/* ----------------------------------------------------------- backward ----
 *
 * Training ("Scaling Diffusion Transformers to 16 Billion Parameters",
 * MoE-DiT: the layer is trained with the expert-level balance loss added to
 * the denoising loss).  The three calls below give the gradients of
 *
 *   Loss = <dy, y> + dloss * L_balance
 *
 * for the routing the forward pass chose, held fixed: the selection has no
 * gradient, the slot weights (gate probabilities) do, the balance counts do
 * not.  Order: moe_combine_backward, moe_grouped_ffn_backward (routed
 * experts, then shared experts with dy as their output gradient),
 * moe_gate_backward.  Expert biases get no gradient here (the layer's
 * experts have none).
 */

/*
 * Backward of the weighted combine (eq. MoE(x)).  For every token t and
 * slot k with r = slot_row[t][k] >= 0:
 *   dy_rows[r]      = topk_w[t][k] * dy[t]           (y_dtype)
 *   slot_grad[t][k] = <dy[t], y_rows[r]>             (fp32, fixed order)
 * and slot_grad = 0 for empty slots.
 *   dy [N][D] dy_dtype;  y_rows [*][D] y_dtype (the forward's expert rows);
 *   dy_rows [*][D] y_dtype out;  slot_grad [N][Kmax] fp32 out
 * Errors: INVALID_ARGUMENT for null pointers (N > 0), N < 0, D or
 *   Kmax < 1; UNSUPPORTED for D % 8 != 0, Kmax > 64, unknown dtypes.
 */
moe_status moe_combine_backward(const void* dy, moe_dtype dy_dtype,
                                const void* y_rows, moe_dtype y_dtype,
                                const int32_t* slot_row, const float* topk_w,
                                int64_t N, int32_t D, int32_t Kmax,
                                void* dy_rows, float* slot_grad,
                                hipStream_t stream);

/* Bytes of workspace moe_grouped_ffn_backward needs (0 for bad sizes).  The
 * size depends on the shape and on the compute-unit count of the current
 * device (it holds the partials of a split reduction sized to fill that
 * device): query it with the device current that the call will run on. */
size_t moe_ffn_backward_workspace_size(int64_t total_rows, int32_t G,
                                       int32_t D, int32_t H);

/*
 * Backward of the grouped expert MLPs (eq. MLP, tanh GELU), bf16.  With
 * u = x_rows W1_g^T (+ b1_g) (bf16), h = gelu(u) (bf16) and dy_rows the
 * gradient of the expert outputs:
 *   du      = (dy_rows W2_g) * gelu'(u)
 *   dx_rows = du W1_g                                  (dx_dtype out)
 *   dW1[g]  = sum over the group's rows of du^T x_rows  (fp32 out)
 *   dW2[g]  = sum over the group's rows of dy_rows^T h  (fp32 out)
 * Rows, groups, row_index and src_rows (gather) and weights are those of
 * the forward moe_grouped_ffn call (an index entry outside [0, src_rows)
 * reads a zero row).  dW1 / dW2 are written whole (zero for empty
 * groups).
 *   u_rows  [total_rows][H] bf16: the forward's u_ws, or NULL to recompute
 *           u here (the same bits);
 *   h_rows  [total_rows][H] bf16: the forward's h_ws, or NULL: recomputed
 *           with u (the same bits) when u_rows is NULL too, else gelu of
 *           the bf16 u (it can differ from the forward's h by one bf16
 *           rounding);
 *   dy_rows [total_rows][D] bf16;  dx_rows [total_rows][D];
 *   dw1 [G][H][D], dw2 [G][D][H] fp32 out;  workspace of at least
 *   moe_ffn_backward_workspace_size bytes (recomputed activations,
 *   W1's transpose, the gathered input rows and, when few
 *   weight-gradient tiles meet long token segments, the fp32 partials of a
 *   split reduction, added in a fixed order); contents need no
 *   initialisation
 * Errors: INVALID_ARGUMENT for null pointers, bad sizes or src_rows < 1
 *   with row_index; UNSUPPORTED for non-bf16 inputs, G > 128, D or H not
 *   multiples of 8, (total_rows + 64) * max(D, H) * 2 >= 2^32,
 *   D * H * 2 >= 2^32, a gathered
 *   x_rows past the 4 GiB range of moe_grouped_ffn; WORKSPACE_TOO_SMALL.
 */
moe_status moe_grouped_ffn_backward(
    const void* x_rows, const int32_t* row_index, int64_t src_rows,
    moe_dtype dtype, int64_t total_rows, const int64_t* group_offsets, int32_t G, int32_t D,
    int32_t H, const void* w1, const float* b1, const void* w2,
    const void* dy_rows, const void* u_rows, const void* h_rows,
    void* workspace, size_t workspace_bytes, void* dx_rows, moe_dtype dx_dtype,
    float* dw1, float* dw2, hipStream_t stream);

/* Bytes of workspace moe_gate_backward needs (0 for bad sizes). */
size_t moe_gate_backward_workspace_size(int64_t N, int32_t E, int32_t D);

/*
 * Backward of the gate and assembly of dx.  With P = probs, N = B*T:
 *   dP[t][i]  = sum_k [topk_idx[t][k] == i] slot_grad[t][k]
 *               + dloss * dL_balance/dP[t][i]   (counts from
 *                 moe_balance_stats; sequence or global as in the forward)
 *   dl[t]     = P[t] * (dP[t] - sum_j P[t][j] dP[t][j])     (softmax)
 *   dw_gate   = sum_t dl[t]^T x[t]       [E][D] fp32 (fixed-order sums)
 *   dbias     = sum_t dl[t]              [E] fp32 (may be NULL)
 *   dx[t]     = sum_k dx_rows[slot_row[t][k]] + dx_shared[t] + dl[t] W_g
 * in fp32, rounded once to dx_dtype; dx_rows / dx_shared may be NULL.
 *   x [N][D] x_dtype;  w_gate [E][D] fp32;  topk_idx, slot_grad,
 *   slot_row [N][Kmax];  counts [B][E] int32 (needed when dloss != 0);
 *   dx_rows [*][D], dx_shared [N][D], dx [N][D] dx_dtype
 * Errors: INVALID_ARGUMENT for null pointers or bad sizes, K outside
 *   [1, E]; UNSUPPORTED for E or Kmax > 64, D % 8 != 0;
 *   WORKSPACE_TOO_SMALL.
 */
moe_status moe_gate_backward(
    const void* x, moe_dtype x_dtype, const float* w_gate, const float* probs,
    const int32_t* topk_idx, const float* slot_grad, const int32_t* counts,
    int32_t B, int32_t T, int32_t D, int32_t E, int32_t Kmax, int32_t K,
    float alpha, float dloss, moe_balance_mode mode, const void* dx_rows,
    const int32_t* slot_row, const void* dx_shared, moe_dtype dx_dtype,
    void* dx, float* dw_gate, float* dbias, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Routing analytics ("Scaling Diffusion Transformers to 16 Billion
 * Parameters", Expert Specialization Analysis: the frequency of expert
 * selection by spatial position, by image class and by denoising time step;
 * "DiT-MoE" project hub page, section 4, analysis tools).  Adds the counts
 * of one batch of B images x T tokens to caller-owned totals:
 *
 *   pos_counts[p][i] += number of (image b, slot k) with
 *                       topk_idx[b*T + p][k] == i
 *   tag_counts[g][i] += number of (token t, slot k) of the images b with
 *                       image_tag[b] == g and topk_idx[t][k] == i
 *
 * Entries of topk_idx outside [0, E) (the -1 of an empty slot) count
 * nowhere; an image whose tag lies outside [0, n_tags) counts only by
 * position.  Counts are exact integers, independent of scheduling.  The
 * caller zero-fills the totals before the first batch; the frequencies of
 * the analysis are the totals divided by their sums.
 *
 *   topk_idx [B*T][Kmax] int32 device;  image_tag [B] int32 device or NULL
 *   (then tag_counts is ignored);  pos_counts [T][E], tag_counts
 *   [n_tags][E] int64 device, read and written
 * Errors: INVALID_ARGUMENT for B < 0, T < 1, E < 1, Kmax < 1, a null
 *   topk_idx (B > 0) or pos_counts, or image_tag given without n_tags >= 1
 *   and tag_counts; UNSUPPORTED for E or Kmax > 64 or B*T*Kmax >= 2^31.
 */
moe_status moe_routing_histogram(const int32_t* topk_idx, int32_t B,
                                 int32_t T, int32_t E, int32_t Kmax,
                                 const int32_t* image_tag, int32_t n_tags,
                                 int64_t* pos_counts, int64_t* tag_counts,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
