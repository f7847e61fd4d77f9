// C ABI of the DiT-MoE layer library: argument validation and launch.
// The contract of every entry point is documented in include/moe.h.
#include "moe.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cstring>

#include <string>

#include "gather.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// The integer a caller passed for a C enum parameter.  Any int can arrive
// through the C ABI, and in C++ an enum object holding a value outside the
// range of its enumerators must not be read as that type (the bits are
// copied out instead); every check below works on the int.
template <class Enum>
int enum_value(const Enum& e) {
  static_assert(sizeof(Enum) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof(v));
  return v;
}

bool valid_dtype(int d) { return d == MOE_F32 || d == MOE_BF16; }

constexpr int64_t kI32Limit = int64_t(1) << 31;
constexpr int kMaxE = 64;
constexpr int kMaxGroups = moe::kMaxFfnGroups;

#define CHECK_PTR(p)                                                       \
  do {                                                                     \
    if ((p) == nullptr)                                                    \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is null", fn, #p);     \
  } while (0)

// A pointer to an empty tensor may be null.
#define CHECK_PTR_IF(cond, p)                                              \
  do {                                                                     \
    if ((cond) && (p) == nullptr)                                          \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is null", fn, #p);     \
  } while (0)

// Rows gathered through a row index: the source matrix needs at least one
// row, and its bytes must stay addressable by the kernels' 32-bit buffer
// offsets (index entries outside [0, src_rows) then read zero rows).
#define CHECK_GATHER(rows, row_index, src_rows, row_bytes)                 \
  do {                                                                     \
    if ((rows) && (row_index) != nullptr) {                                \
      if ((src_rows) < 1)                                                  \
        return fail(MOE_ERR_INVALID_ARGUMENT,                              \
                    "%s: src_rows=%lld, need >= 1 with row_index", fn,     \
                    (long long)(src_rows));                                \
      if (!moe::gather_fits((src_rows), (row_bytes)))                      \
        return fail(MOE_ERR_UNSUPPORTED,                                   \
                    "%s: src_rows=%lld rows of %lld bytes exceed the "     \
                    "4 GiB gather range",                                  \
                    fn, (long long)(src_rows), (long long)(row_bytes));    \
    }                                                                      \
  } while (0)

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status_arg) {
  const int status = enum_value(status_arg);
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_gate_workspace_size(int64_t N, int32_t E, int32_t K,
                               moe_route route_arg) {
  const int route = enum_value(route_arg);
  (void)N; (void)E; (void)K;
  return route == MOE_ROUTE_EXPERT_RACE ? moe::race_workspace_bytes() : 0;
}

moe_status moe_gate_topk(const void* x, moe_dtype x_dtype_arg,
                         const float* w_gate, const float* logit_bias,
                         int64_t N, int32_t D, int32_t E, int32_t K,
                         moe_route route_arg, float* probs, int32_t* topk_idx,
                         float* topk_w, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const int x_dtype = enum_value(x_dtype_arg);
  const int route = enum_value(route_arg);
  const char* fn = "moe_gate_topk";
  if (N < 0 || D < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need N >= 0, D >= 1, E >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (route != MOE_ROUTE_TOPK && route != MOE_ROUTE_EXPERT_RACE)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: unknown route %d", fn, (int)route);
  CHECK_PTR(w_gate);
  CHECK_PTR_IF(N > 0, x); CHECK_PTR_IF(N > 0, probs);
  CHECK_PTR_IF(N > 0, topk_idx); CHECK_PTR_IF(N > 0, topk_w);
  if (!valid_dtype(x_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)x_dtype);
  if (E > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d above %d", fn, E, kMaxE);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  const int64_t Kmax = route == MOE_ROUTE_TOPK ? K : E;
  if (N * Kmax >= kI32Limit || N * E >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*Kmax must stay below 2^31", fn);
  const size_t need =
      moe_gate_workspace_size(N, E, K, static_cast<moe_route>(route));
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, need);
  CHECK_PTR_IF(need > 0, workspace);
  hipError_t err = moe::launch_gate(x, x_dtype == MOE_BF16, w_gate, logit_bias,
                                    N, D, E, K, route == MOE_ROUTE_TOPK, probs,
                                    topk_idx, topk_w, stream);
  if (err != hipSuccess) return from_hip(err, fn);
  if (route == MOE_ROUTE_EXPERT_RACE)
    err = moe::launch_race(probs, N, E, K, topk_idx, topk_w, workspace, stream);
  return from_hip(err, fn);
}

size_t moe_permute_workspace_size(int64_t N, int32_t E, int32_t Kmax) {
  (void)Kmax;
  if (N < 0 || E < 1) return 0;
  return moe::permute_workspace_bytes(N, E);
}

}  // extern "C"

namespace {

// Argument checks shared by moe_permute and moe_permute_noalloc.
moe_status check_permute(const char* fn, const void* x, int dtype,
                         const int32_t* topk_idx, int64_t N, int32_t D,
                         int32_t E, int32_t Kmax, int32_t K,
                         const int32_t* expert_counts,
                         const int64_t* expert_offsets,
                         const int32_t* row_token, const int32_t* slot_row,
                         const void* x_perm) {
  if (N < 0 || D < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need N >= 0, D >= 1, E >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (Kmax != K && Kmax != E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: Kmax=%d must be K or E", fn, Kmax);
  CHECK_PTR(expert_counts); CHECK_PTR(expert_offsets);
  CHECK_PTR_IF(N > 0, topk_idx); CHECK_PTR_IF(N > 0, slot_row);
  CHECK_PTR_IF(N > 0, row_token);
  CHECK_PTR_IF(N > 0 && x_perm != nullptr, x);
  if (!valid_dtype(dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (E > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d above %d", fn, E, kMaxE);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  if (N * Kmax >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*Kmax must stay below 2^31", fn);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_permute(const void* x, moe_dtype dtype_arg, const int32_t* topk_idx,
                       int64_t N, int32_t D, int32_t E, int32_t Kmax, int32_t K,
                       int32_t* expert_counts, int64_t* expert_offsets,
                       int32_t* row_token, int32_t* slot_row, void* x_perm,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const int dtype = enum_value(dtype_arg);
  const char* fn = "moe_permute";
  const moe_status st =
      check_permute(fn, x, dtype, topk_idx, N, D, E, Kmax, K, expert_counts,
                    expert_offsets, row_token, slot_row, x_perm);
  if (st != MOE_OK) return st;
  const size_t need = moe_permute_workspace_size(N, E, Kmax);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, need);
  CHECK_PTR(workspace);
  const int64_t A = static_cast<int64_t>(K) * N;
  return from_hip(moe::launch_permute(x, dtype == MOE_BF16, topk_idx, N, D, E,
                                      Kmax, A, expert_counts, expert_offsets,
                                      row_token, slot_row, x_perm, workspace,
                                      stream),
                  fn);
}

moe_status moe_permute_noalloc(const void* x, moe_dtype dtype_arg,
                               const int32_t* topk_idx, int64_t N, int32_t D,
                               int32_t E, int32_t Kmax, int32_t K,
                               int32_t* expert_counts, int64_t* expert_offsets,
                               int32_t* row_token, int32_t* slot_row,
                               void* x_perm, hipStream_t stream) {
  const int dtype = enum_value(dtype_arg);
  const char* fn = "moe_permute_noalloc";
  const moe_status st =
      check_permute(fn, x, dtype, topk_idx, N, D, E, Kmax, K, expert_counts,
                    expert_offsets, row_token, slot_row, x_perm);
  if (st != MOE_OK) return st;
  const size_t need = moe_permute_workspace_size(N, E, Kmax);
  if (need > moe::permute_scratch_bytes())
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: N=%lld, E=%d need %zu bytes of scratch, above the %zu "
                "bytes of the static scratch (use moe_permute with a "
                "workspace)",
                fn, (long long)N, E, need, moe::permute_scratch_bytes());
  void* scratch = nullptr;
  const hipError_t err = moe::permute_scratch(&scratch);
  if (err != hipSuccess) return from_hip(err, fn);
  const int64_t A = static_cast<int64_t>(K) * N;
  return from_hip(moe::launch_permute(x, dtype == MOE_BF16, topk_idx, N, D, E,
                                      Kmax, A, expert_counts, expert_offsets,
                                      row_token, slot_row, x_perm, scratch,
                                      stream),
                  fn);
}

}  // extern "C"

namespace {

// moe_grouped_ffn and moe_grouped_ffn_split: the same checks and launches;
// split_ws (checked by the caller) is the latter's workspace or null.  The
// enum arguments arrive as the callers read them (enum_value).
moe_status grouped_ffn(const char* fn, const void* x_rows,
                       const int32_t* row_index, int64_t src_rows, int dtype,
                       int64_t total_rows, const int64_t* group_offsets,
                       int32_t G, int32_t D, int32_t H, const void* w1,
                       const float* b1, const void* w2, const float* b2,
                       void* h_ws, void* u_ws, void* y_rows, int y_dtype,
                       int stages, void* split_ws, hipStream_t stream) {
  if (total_rows < 0 || G < 1 || D < 1 || H < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need total_rows >= 0, G >= 1, D >= 1, H >= 1", fn);
  if (stages < MOE_FFN_UP || stages > MOE_FFN_BOTH)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: stages=%d outside 1..3", fn,
                (int)stages);
  const bool up = stages & MOE_FFN_UP, down = stages & MOE_FFN_DOWN;
  const bool rows = total_rows > 0;
  CHECK_PTR_IF(up, w1); CHECK_PTR_IF(down, w2);
  CHECK_PTR_IF(rows && up, x_rows); CHECK_PTR_IF(rows, group_offsets);
  CHECK_PTR_IF(rows, h_ws); CHECK_PTR_IF(rows && down, y_rows);
  if (!valid_dtype(dtype) || !valid_dtype(y_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (dtype == MOE_F32 && y_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "%s: fp32 inputs need fp32 outputs", fn);
  if (u_ws != nullptr && dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: u_ws needs bf16 inputs", fn);
  if (G > kMaxGroups)
    return fail(MOE_ERR_UNSUPPORTED, "%s: G=%d above %d", fn, G, kMaxGroups);
  if (D % 8 != 0 || H % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d and H=%d must be multiples of 8",
                fn, D, H);
  if (total_rows >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: total_rows must stay below 2^31", fn);
  CHECK_GATHER(rows && up, row_index, src_rows,
               static_cast<int64_t>(D) * (dtype == MOE_BF16 ? 2 : 4));
  moe::FfnArgs a{x_rows, row_index, total_rows, group_offsets, G, D, H,
                 w1,     b1,        w2,         b2,            h_ws, y_rows,
                 dtype == MOE_BF16,  y_dtype == MOE_F32};
  a.u = up ? u_ws : nullptr;
  a.src_rows = src_rows;
  a.split_ws = static_cast<float*>(split_ws);
  return from_hip(moe::launch_ffn(a, up, down, stream), fn);
}

}  // namespace

extern "C" {

moe_status moe_grouped_ffn(const void* x_rows, const int32_t* row_index,
                           int64_t src_rows, moe_dtype dtype_arg,
                           int64_t total_rows,
                           const int64_t* group_offsets, int32_t G, int32_t D,
                           int32_t H, const void* w1, const float* b1,
                           const void* w2, const float* b2, void* h_ws,
                           void* u_ws, void* y_rows, moe_dtype y_dtype_arg,
                           moe_ffn_stages stages_arg, hipStream_t stream) {
  return grouped_ffn("moe_grouped_ffn", x_rows, row_index, src_rows,
                     enum_value(dtype_arg), total_rows, group_offsets, G, D, H,
                     w1, b1, w2, b2, h_ws, u_ws, y_rows, enum_value(y_dtype_arg),
                     enum_value(stages_arg), nullptr, stream);
}

size_t moe_grouped_ffn_split_workspace_size(void) {
  return moe::ffn_split_workspace_bytes();
}

moe_status moe_grouped_ffn_split(const void* x_rows, const int32_t* row_index,
                                 int64_t src_rows, moe_dtype dtype_arg,
                                 int64_t total_rows,
                                 const int64_t* group_offsets, int32_t G,
                                 int32_t D, int32_t H, const void* w1,
                                 const float* b1, const void* w2,
                                 const float* b2, void* h_ws, void* u_ws,
                                 void* y_rows, moe_dtype y_dtype_arg,
                                 moe_ffn_stages stages_arg, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "moe_grouped_ffn_split";
  const size_t need = moe_grouped_ffn_split_workspace_size();
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, need);
  CHECK_PTR(workspace);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace not 16-byte aligned",
                fn);
  return grouped_ffn(fn, x_rows, row_index, src_rows, enum_value(dtype_arg),
                     total_rows, group_offsets, G, D, H, w1, b1, w2, b2, h_ws,
                     u_ws, y_rows, enum_value(y_dtype_arg),
                     enum_value(stages_arg), workspace, stream);
}

moe_status moe_grouped_mlp_fused(const void* x_rows, const int32_t* row_index,
                                 int64_t src_rows, moe_dtype dtype_arg,
                                 int64_t total_rows,
                                 const int64_t* group_offsets, int32_t G,
                                 int32_t D, int32_t H, const void* w1,
                                 const float* b1, const void* w2,
                                 const float* b2, void* y_rows,
                                 moe_dtype y_dtype_arg, hipStream_t stream) {
  const int dtype = enum_value(dtype_arg);
  const int y_dtype = enum_value(y_dtype_arg);
  const char* fn = "moe_grouped_mlp_fused";
  if (total_rows < 0 || G < 1 || D < 1 || H < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need total_rows >= 0, G >= 1, D >= 1, H >= 1", fn);
  const bool rows = total_rows > 0;
  CHECK_PTR(w1); CHECK_PTR(w2);
  CHECK_PTR_IF(rows, x_rows); CHECK_PTR_IF(rows, group_offsets);
  CHECK_PTR_IF(rows, y_rows);
  if (dtype != MOE_BF16 || (y_dtype != MOE_BF16 && y_dtype != MOE_F32))
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: needs bf16 inputs and a bf16 or fp32 output", fn);
  if (G > kMaxGroups)
    return fail(MOE_ERR_UNSUPPORTED, "%s: G=%d above %d", fn, G, kMaxGroups);
  if (!moe::mlp_fused_supported(D, H))
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: needs D in {128, 256, 384} and H a multiple of 64 "
                "(D=%d, H=%d)", fn, D, H);
  if (total_rows >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: total_rows must stay below 2^31", fn);
  CHECK_GATHER(rows, row_index, src_rows, static_cast<int64_t>(D) * 2);
  moe::FfnArgs a{x_rows, row_index, total_rows, group_offsets, G, D, H,
                 w1,     b1,        w2,         b2,            nullptr, y_rows,
                 true,   y_dtype == MOE_F32};
  a.src_rows = src_rows;
  return from_hip(moe::launch_mlp_fused(a, stream), fn);
}

moe_status moe_combine(const void* y_rows, moe_dtype y_dtype_arg,
                       const int32_t* slot_row, const float* topk_w, int64_t N,
                       int32_t D, int32_t Kmax, const void* y_shared,
                       moe_dtype sh_dtype_arg, void* y, moe_dtype out_dtype_arg,
                       hipStream_t stream) {
  const int y_dtype = enum_value(y_dtype_arg);
  const int sh_dtype = enum_value(sh_dtype_arg);
  const int out_dtype = enum_value(out_dtype_arg);
  const char* fn = "moe_combine";
  if (N < 0 || D < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need N >= 0, D >= 1, Kmax >= 1",
                fn);
  CHECK_PTR_IF(N > 0, y_rows); CHECK_PTR_IF(N > 0, slot_row);
  CHECK_PTR_IF(N > 0, topk_w); CHECK_PTR_IF(N > 0, y);
  if (!valid_dtype(y_dtype) || !valid_dtype(out_dtype) ||
      (y_shared != nullptr && !valid_dtype(sh_dtype)))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  if (Kmax > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: Kmax=%d above %d", fn, Kmax, kMaxE);
  if (N * (D / 8) >= kI32Limit || N * Kmax >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*D/8 must stay below 2^31", fn);
  return from_hip(moe::launch_combine(y_rows, y_dtype == MOE_BF16, slot_row,
                                      topk_w, N, D, Kmax, y_shared,
                                      sh_dtype == MOE_BF16, y,
                                      out_dtype == MOE_BF16, stream),
                  fn);
}

moe_status moe_balance_stats(const float* probs, const int32_t* topk_idx,
                             int32_t B, int32_t T, int32_t E, int32_t Kmax,
                             int32_t K, float alpha, moe_balance_mode mode_arg,
                             int32_t* counts, float* prob_sums, float* loss,
                             hipStream_t stream) {
  const int mode = enum_value(mode_arg);
  const char* fn = "moe_balance_stats";
  if (B < 0 || T < 1 || E < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need B >= 0, T >= 1, E >= 1, Kmax >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (mode != MOE_BAL_PER_SEQUENCE && mode != MOE_BAL_GLOBAL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, (int)mode);
  CHECK_PTR(loss);
  CHECK_PTR_IF(B > 0, probs); CHECK_PTR_IF(B > 0, topk_idx);
  CHECK_PTR_IF(B > 0, counts); CHECK_PTR_IF(B > 0, prob_sums);
  if (E > kMaxE || Kmax > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d / Kmax=%d above %d", fn, E, Kmax,
                kMaxE);
  const int64_t N = static_cast<int64_t>(B) * T;
  if (N * E >= kI32Limit || N * Kmax >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: B*T*E must stay below 2^31", fn);
  return from_hip(moe::launch_balance(probs, topk_idx, B, T, E, Kmax, K, alpha,
                                      mode == MOE_BAL_GLOBAL, counts, prob_sums,
                                      loss, stream),
                  fn);
}

size_t moe_gate_balance_workspace_size(int32_t B, int32_t T, int32_t E) {
  if (B < 0 || T < 1 || E < 1) return 0;
  return moe::balance_partials_bytes(static_cast<int64_t>(B) * T, E);
}

moe_status moe_gate_topk_balance(const void* x, moe_dtype x_dtype_arg,
                                 const float* w_gate, const float* logit_bias,
                                 int32_t B, int32_t T, int32_t D, int32_t E,
                                 int32_t K, float alpha, moe_balance_mode mode_arg,
                                 float* probs, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, float* prob_sums, float* loss,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  const int x_dtype = enum_value(x_dtype_arg);
  const int mode = enum_value(mode_arg);
  const char* fn = "moe_gate_topk_balance";
  if (B < 0 || T < 1 || D < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need B >= 0, T >= 1, D >= 1, E >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (mode != MOE_BAL_PER_SEQUENCE && mode != MOE_BAL_GLOBAL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, (int)mode);
  const int64_t N = static_cast<int64_t>(B) * T;
  CHECK_PTR(w_gate); CHECK_PTR(loss);
  CHECK_PTR_IF(N > 0, x); CHECK_PTR_IF(N > 0, probs);
  CHECK_PTR_IF(N > 0, topk_idx); CHECK_PTR_IF(N > 0, topk_w);
  CHECK_PTR_IF(N > 0, counts); CHECK_PTR_IF(N > 0, prob_sums);
  if (!valid_dtype(x_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)x_dtype);
  if (E > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d above %d", fn, E, kMaxE);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  if (N * E >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: B*T*E must stay below 2^31", fn);
  const size_t need = moe_gate_balance_workspace_size(B, T, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, need);
  CHECK_PTR_IF(need > 0, workspace);
  const bool bf16 = x_dtype == MOE_BF16;
  const bool global = mode == MOE_BAL_GLOBAL;
  hipError_t err;
  if (moe::gate_balance_fuses(bf16, N, T, D, E)) {
    float* part_p = static_cast<float*>(workspace);
    int32_t* part_c = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                 need / 2);
    err = moe::launch_gate_balance_partials(x, w_gate, logit_bias, N, D, E, K,
                                            probs, topk_idx, topk_w, part_p,
                                            part_c, stream);
    if (err != hipSuccess) return from_hip(err, fn);
    err = moe::launch_balance_from_partials(workspace, B, T, E, K, alpha, global,
                                            counts, prob_sums, loss, stream);
    return from_hip(err, fn);
  }
  err = moe::launch_gate(x, bf16, w_gate, logit_bias, N, D, E, K, true, probs,
                         topk_idx, topk_w, stream);
  if (err != hipSuccess) return from_hip(err, fn);
  return from_hip(moe::launch_balance(probs, topk_idx, B, T, E, K, K, alpha,
                                      global, counts, prob_sums, loss, stream),
                  fn);
}

size_t moe_gate_route_workspace_size(int32_t B, int32_t T, int32_t E) {
  if (B < 0 || T < 1 || E < 1) return 0;
  const int64_t N = static_cast<int64_t>(B) * T;
  return moe::balance_partials_bytes(N, E) + moe::permute_workspace_bytes(N, E);
}

moe_status moe_gate_route(const void* x, moe_dtype x_dtype_arg,
                          const float* w_gate, const float* logit_bias,
                          int32_t B, int32_t T, int32_t D, int32_t E, int32_t K,
                          float alpha, moe_balance_mode mode_arg, float* probs,
                          int32_t* topk_idx, float* topk_w, int32_t* counts,
                          float* prob_sums, float* loss, int32_t* expert_counts,
                          int64_t* expert_offsets, int32_t* row_token,
                          int32_t* slot_row, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  const int x_dtype = enum_value(x_dtype_arg);
  const int mode = enum_value(mode_arg);
  const char* fn = "moe_gate_route";
  if (B < 0 || T < 1 || D < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need B >= 0, T >= 1, D >= 1, E >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (mode != MOE_BAL_PER_SEQUENCE && mode != MOE_BAL_GLOBAL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, (int)mode);
  const int64_t N = static_cast<int64_t>(B) * T;
  CHECK_PTR(w_gate); CHECK_PTR(loss);
  CHECK_PTR_IF(N > 0, x); CHECK_PTR_IF(N > 0, probs);
  CHECK_PTR_IF(N > 0, topk_w); CHECK_PTR_IF(N > 0, counts);
  CHECK_PTR_IF(N > 0, prob_sums);
  // the permutation's own checks (the index form: no x_perm)
  const moe_status st =
      check_permute(fn, x, x_dtype, topk_idx, N, D, E, K, K, expert_counts,
                    expert_offsets, row_token, slot_row, nullptr);
  if (st != MOE_OK) return st;
  if (N * E >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: B*T*E must stay below 2^31", fn);
  const size_t need = moe_gate_route_workspace_size(B, T, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, need);
  CHECK_PTR(workspace);
  const bool bf16 = x_dtype == MOE_BF16;
  const bool global = mode == MOE_BAL_GLOBAL;
  const int64_t A = static_cast<int64_t>(K) * N;
  // the gate's partial sums (fp32 half, then the int32 selection counts),
  // then the permutation's workspace
  const size_t pbytes = moe::balance_partials_bytes(N, E);
  char* const pws = static_cast<char*>(workspace) + pbytes;
  hipError_t err;
  if (moe::gate_balance_fuses(bf16, N, T, D, E)) {
    float* part_p = static_cast<float*>(workspace);
    int32_t* part_c = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                 pbytes / 2);
    int64_t* block_base = reinterpret_cast<int64_t*>(pws);
    err = moe::launch_gate_balance_partials(x, w_gate, logit_bias, N, D, E, K,
                                            probs, topk_idx, topk_w, part_p,
                                            part_c, stream);
    if (err != hipSuccess) return from_hip(err, fn);
    err = moe::launch_route_finish(workspace, B, T, E, K, alpha, global, counts,
                                   prob_sums, loss, expert_counts,
                                   expert_offsets, block_base, stream);
    if (err != hipSuccess) return from_hip(err, fn);
    return from_hip(moe::launch_permute_scatter(topk_idx, N, E, K, A, block_base,
                                                slot_row, row_token, stream),
                    fn);
  }
  err = moe::launch_gate(x, bf16, w_gate, logit_bias, N, D, E, K, true, probs,
                         topk_idx, topk_w, stream);
  if (err != hipSuccess) return from_hip(err, fn);
  err = moe::launch_balance(probs, topk_idx, B, T, E, K, K, alpha, global,
                            counts, prob_sums, loss, stream);
  if (err != hipSuccess) return from_hip(err, fn);
  return from_hip(moe::launch_permute(x, bf16, topk_idx, N, D, E, K, A,
                                      expert_counts, expert_offsets, row_token,
                                      slot_row, nullptr, pws, stream),
                  fn);
}

moe_status moe_ffn_down_combine(const void* h, moe_dtype dtype_arg, int64_t N,
                                int32_t D, int32_t H, const void* w2,
                                const float* b2, const void* y_rows,
                                const int32_t* slot_row, const float* topk_w,
                                int32_t Kmax, void* y, hipStream_t stream) {
  const int dtype = enum_value(dtype_arg);
  const char* fn = "moe_ffn_down_combine";
  if (N < 0 || D < 1 || H < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need N >= 0, D >= 1, H >= 1, Kmax >= 1", fn);
  const bool rows = N > 0;
  CHECK_PTR_IF(rows, h); CHECK_PTR_IF(rows, w2); CHECK_PTR_IF(rows, y_rows);
  CHECK_PTR_IF(rows, slot_row); CHECK_PTR_IF(rows, topk_w); CHECK_PTR_IF(rows, y);
  if (dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (Kmax > 16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: Kmax=%d above 16", fn, Kmax);
  if (D % 8 != 0 || H % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d and H=%d must be multiples of 8",
                fn, D, H);
  if (N >= kI32Limit || N * Kmax >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*Kmax must stay below 2^31", fn);
  return from_hip(moe::launch_ffn_down_combine(h, N, D, H, w2, b2, y_rows,
                                               slot_row, topk_w, Kmax, y,
                                               stream),
                  fn);
}

moe_status moe_combine_backward(const void* dy, moe_dtype dy_dtype_arg,
                                const void* y_rows, moe_dtype y_dtype_arg,
                                const int32_t* slot_row, const float* topk_w,
                                int64_t N, int32_t D, int32_t Kmax,
                                void* dy_rows, float* slot_grad,
                                hipStream_t stream) {
  const int dy_dtype = enum_value(dy_dtype_arg);
  const int y_dtype = enum_value(y_dtype_arg);
  const char* fn = "moe_combine_backward";
  if (N < 0 || D < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need N >= 0, D >= 1, Kmax >= 1",
                fn);
  const bool rows = N > 0;
  CHECK_PTR_IF(rows, dy); CHECK_PTR_IF(rows, y_rows); CHECK_PTR_IF(rows, slot_row);
  CHECK_PTR_IF(rows, topk_w); CHECK_PTR_IF(rows, dy_rows);
  CHECK_PTR_IF(rows, slot_grad);
  if (!valid_dtype(dy_dtype) || !valid_dtype(y_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  if (Kmax > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: Kmax=%d above %d", fn, Kmax, kMaxE);
  if (N * Kmax >= kI32Limit || N * (D / 8) >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*Kmax must stay below 2^31", fn);
  return from_hip(moe::launch_combine_backward(dy, dy_dtype == MOE_BF16, y_rows,
                                               y_dtype == MOE_BF16, slot_row,
                                               topk_w, N, D, Kmax, dy_rows,
                                               slot_grad, stream),
                  fn);
}

size_t moe_ffn_backward_workspace_size(int64_t total_rows, int32_t G, int32_t D,
                                       int32_t H) {
  if (total_rows < 0 || G < 1 || D < 1 || H < 1) return 0;
  return moe::ffn_backward_workspace_bytes(total_rows, G, D, H);
}

moe_status moe_grouped_ffn_backward(
    const void* x_rows, const int32_t* row_index, int64_t src_rows,
    moe_dtype dtype_arg, int64_t total_rows, const int64_t* group_offsets, int32_t G, int32_t D,
    int32_t H, const void* w1, const float* b1, const void* w2,
    const void* dy_rows, const void* u_rows, const void* h_rows,
    void* workspace, size_t workspace_bytes, void* dx_rows, moe_dtype dx_dtype_arg,
    float* dw1, float* dw2, hipStream_t stream) {
  const int dtype = enum_value(dtype_arg);
  const int dx_dtype = enum_value(dx_dtype_arg);
  const char* fn = "moe_grouped_ffn_backward";
  if (total_rows < 0 || G < 1 || D < 1 || H < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need total_rows >= 0, G >= 1, D >= 1, H >= 1", fn);
  const bool rows = total_rows > 0;
  CHECK_PTR(w1); CHECK_PTR(w2); CHECK_PTR(dw1); CHECK_PTR(dw2);
  CHECK_PTR(workspace);
  CHECK_PTR_IF(rows, x_rows); CHECK_PTR_IF(rows, group_offsets);
  CHECK_PTR_IF(rows, dy_rows); CHECK_PTR_IF(rows, dx_rows);
  if (dtype != MOE_BF16 || !valid_dtype(dx_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 inputs only", fn);
  if (G > kMaxGroups)
    return fail(MOE_ERR_UNSUPPORTED, "%s: G=%d above %d", fn, G, kMaxGroups);
  if (D % 8 != 0 || H % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d and H=%d must be multiples of 8",
                fn, D, H);
  // the weight-gradient GEMMs address a group's rows of the row-major
  // operands (up to [total_rows + 64][max(D, H)] bf16) with 32-bit byte
  // offsets
  if (total_rows >= kI32Limit ||
      (total_rows + 64) * static_cast<int64_t>(D > H ? D : H) * 2 >=
          (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "%s: total_rows=%lld too large", fn,
                (long long)total_rows);
  // the du GEMM reads a group's W2 block [D][H] k-major with 32-bit byte
  // offsets
  if (static_cast<int64_t>(D) * H * 2 >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "%s: D*H=%lld too large", fn,
                (long long)D * H);
  CHECK_GATHER(rows, row_index, src_rows, static_cast<int64_t>(D) * 2);
  if (workspace_bytes < moe::ffn_backward_workspace_bytes(total_rows, G, D, H))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace below %zu bytes",
                fn, moe::ffn_backward_workspace_bytes(total_rows, G, D, H));
  moe::FfnBwdArgs a{x_rows, row_index, total_rows, group_offsets, G, D, H,
                    w1,     b1,        w2,         dy_rows,       workspace,
                    dx_rows, dx_dtype == MOE_F32, dw1, dw2};
  a.u_saved = u_rows;
  a.h_saved = h_rows;
  a.src_rows = src_rows;
  return from_hip(moe::launch_ffn_backward(a, stream), fn);
}

size_t moe_gate_backward_workspace_size(int64_t N, int32_t E, int32_t D) {
  if (N < 0 || E < 1 || D < 1) return 0;
  return moe::gate_backward_workspace_bytes(N, E, D);
}

moe_status moe_gate_backward(
    const void* x, moe_dtype x_dtype_arg, const float* w_gate, const float* probs,
    const int32_t* topk_idx, const float* slot_grad, const int32_t* counts,
    int32_t B, int32_t T, int32_t D, int32_t E, int32_t Kmax, int32_t K,
    float alpha, float dloss, moe_balance_mode mode_arg, const void* dx_rows,
    const int32_t* slot_row, const void* dx_shared, moe_dtype dx_dtype_arg,
    void* dx, float* dw_gate, float* dbias, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  const int x_dtype = enum_value(x_dtype_arg);
  const int mode = enum_value(mode_arg);
  const int dx_dtype = enum_value(dx_dtype_arg);
  const char* fn = "moe_gate_backward";
  if (B < 0 || T < 1 || D < 1 || E < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need B >= 0, T >= 1, D >= 1, E >= 1, Kmax >= 1", fn);
  if (K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: K=%d outside [1, E=%d]", fn, K, E);
  if (mode != MOE_BAL_PER_SEQUENCE && mode != MOE_BAL_GLOBAL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, (int)mode);
  if (dx_rows != nullptr && slot_row == nullptr)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: dx_rows needs slot_row", fn);
  const bool rows = B > 0;
  CHECK_PTR(w_gate); CHECK_PTR(dw_gate); CHECK_PTR(workspace);
  CHECK_PTR_IF(rows, x); CHECK_PTR_IF(rows, probs); CHECK_PTR_IF(rows, topk_idx);
  CHECK_PTR_IF(rows, slot_grad); CHECK_PTR_IF(rows, dx);
  CHECK_PTR_IF(rows && dloss != 0.0f, counts);
  if (!valid_dtype(x_dtype) || !valid_dtype(dx_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (E > kMaxE || Kmax > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d / Kmax=%d above %d", fn, E, Kmax,
                kMaxE);
  if (D % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 8", fn, D);
  const int64_t N = static_cast<int64_t>(B) * T;
  if (N * E >= kI32Limit || N * Kmax >= kI32Limit || N * (D / 8) >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: B*T*E must stay below 2^31", fn);
  if (workspace_bytes < moe::gate_backward_workspace_bytes(N, E, D))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace below %zu bytes",
                fn, moe::gate_backward_workspace_bytes(N, E, D));
  return from_hip(moe::launch_gate_backward(
                      x, x_dtype == MOE_BF16, w_gate, probs, topk_idx,
                      slot_grad, counts, B, T, D, E, Kmax, K, alpha, dloss,
                      mode == MOE_BAL_GLOBAL, dx_rows, slot_row, dx_shared,
                      dx_dtype == MOE_BF16, dx, dw_gate, dbias, workspace,
                      stream),
                  fn);
}

moe_status moe_routing_histogram(const int32_t* topk_idx, int32_t B,
                                 int32_t T, int32_t E, int32_t Kmax,
                                 const int32_t* image_tag, int32_t n_tags,
                                 int64_t* pos_counts, int64_t* tag_counts,
                                 hipStream_t stream) {
  const char* fn = "moe_routing_histogram";
  if (B < 0 || T < 1 || E < 1 || Kmax < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: need B >= 0, T >= 1, E >= 1, Kmax >= 1", fn);
  if (image_tag != nullptr && (n_tags < 1 || tag_counts == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "%s: image_tag needs n_tags >= 1 and tag_counts", fn);
  CHECK_PTR_IF(B > 0, topk_idx); CHECK_PTR(pos_counts);
  if (E > kMaxE || Kmax > kMaxE)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d / Kmax=%d above %d", fn, E, Kmax,
                kMaxE);
  if (static_cast<int64_t>(B) * T * Kmax >= kI32Limit ||
      static_cast<int64_t>(n_tags) * E >= kI32Limit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: B*T*Kmax must stay below 2^31", fn);
  return from_hip(moe::launch_routing_hist(topk_idx, B, T, E, Kmax, image_tag,
                                           image_tag ? n_tags : 0, pos_counts,
                                           image_tag ? tag_counts : nullptr,
                                           stream),
                  fn);
}

}  // extern "C"
