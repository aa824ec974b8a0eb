// Entry points of libaa.so: host-side argument checks, then the launches in
// aa_kernels.hip.  Every check happens before anything is enqueued, so a call
// that fails leaves the stream untouched.
#include <stdint.h>

#include <string>

#include "aa_internal.h"

using aa::fail;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

aa_status_t check_ptr(const void* p, const char* what, const char* fn) {
  if (!p) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": " + what + " is NULL");
  if (!aligned16(p)) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": " + what + " is not 16-byte aligned");
  return AA_OK;
}

size_t elem_size(aa_dtype_t t) { return t == AA_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks shared by the row-typed calls: M, the position offset and the type map.
aa_status_t check_rows(const aa_plan_s& plan, int64_t M, int64_t pos_offset, const int32_t* row_types,
                       const char* fn) {
  if (M < 0) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": M is negative");
  if (M >= (int64_t(1) << 31)) return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": M of 2^31 rows or more");
  if (pos_offset < 0) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": pos_offset is negative");
  if (plan.type_kind == AA_TYPES_EXPLICIT) {
    if (!row_types && M > 0) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": explicit type map needs row_types");
    if (row_types && (reinterpret_cast<uintptr_t>(row_types) & 3u))
      return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": row_types is not 4-byte aligned");
  } else if (row_types) {
    return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": row_types given for a plan without an explicit type map");
  }
  if (plan.type_kind == AA_TYPES_BLOCK_ROWS && M % plan.q)
    return fail(AA_ERR_SHAPE, std::string(fn) + ": block-row typing needs q to divide M");
  return AA_OK;
}

aa_status_t check_bwd(const aa_plan_s& plan, int64_t M, int64_t pos_offset, const int32_t* row_types,
                      const char* fn) {
  aa_status_t st;
  if ((st = check_rows(plan, M, pos_offset, row_types, fn)) != AA_OK) return st;
  if (plan.type_kind == AA_TYPES_EXPLICIT)
    return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": explicit type lists are not supported by the gradients");
  if (plan.in_dtype != AA_BF16) return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": gradients need bf16 operands");
  if (plan.law == AA_LAW_DIGRAPH)
    return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": digraph plans have no gradient kernels");
  if (plan.layout_version != 1)
    return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": blocks that are not multiples of 16 have no gradient kernels");
  return AA_OK;
}

// Checks shared by the two SwiGLU calls (everything but the hidden buffer).
aa_status_t check_swiglu(aa_plan_t up, aa_plan_t down, const void* X, const void* Wg_packed, const void* Wu_packed,
                         const void* Wd_packed, const void* Y, int64_t M, int64_t pos_offset,
                         const int32_t* row_types, const char* fn) {
  if (!up || !down) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  if (up->law != down->law || up->q != down->q)
    return fail(AA_ERR_SHAPE, std::string(fn) + ": up and down plans use different laws or q");
  if (up->type_kind != down->type_kind || up->period != down->period)
    return fail(AA_ERR_SHAPE, std::string(fn) + ": up and down plans use different type maps");
  if (up->d_out != down->d_in || up->d_in != down->d_out)
    return fail(AA_ERR_SHAPE, std::string(fn) + ": up must map D -> F and down F -> D");
  if (down->in_dtype != up->out_dtype)
    return fail(AA_ERR_SHAPE, std::string(fn) + ": down's input dtype must be up's output dtype (H)");
  aa_status_t st;
  if ((st = check_rows(*up, M, pos_offset, row_types, fn)) != AA_OK) return st;
  if (M == 0) return AA_OK;
  if ((st = check_ptr(X, "X", fn)) != AA_OK) return st;
  if ((st = check_ptr(Wg_packed, "Wg_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(Wu_packed, "Wu_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(Wd_packed, "Wd_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(Y, "Y", fn)) != AA_OK) return st;
  const size_t yb = size_t(M * down->d_out) * elem_size(down->out_dtype);
  const size_t xb = size_t(M * up->d_in) * elem_size(up->in_dtype);
  if (overlaps(Y, yb, X, xb)) return fail(AA_ERR_INVALID_ARG, std::string(fn) + ": X and Y must not overlap");
  return AA_OK;
}

// The two launches of a SwiGLU FFN, after the checks.
aa_status_t run_swiglu(const aa_plan_s& up, const aa_plan_s& down, const void* X, const void* Wg_packed,
                       const void* Wu_packed, const void* Wd_packed, void* H, void* Y, int64_t M,
                       int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  aa_status_t st;
  // A few tokens (at most one per row type on average: generation decodes one
  // new position per call) take the matrix-vector kernels, which read each
  // token's 2q - 1 blocks once; the leaf GEMMs would pad them to full tiles.
  // The down projection's decode falls back to the leaf kernels itself when
  // its blocks are too wide for the matrix-vector kernels.
  if (M <= up.q && up.type_kind != AA_TYPES_BLOCK_ROWS && aa::decode_swiglu_ok(up)) {
    if ((st = aa::launch_decode(up, X, Wg_packed, Wu_packed, H, M, pos_offset, row_types, stream)) != AA_OK)
      return st;
    return aa::launch_decode(down, H, Wd_packed, nullptr, Y, M, pos_offset, row_types, stream);
  }
  aa::LeafCall gate_up{X, Wg_packed, Wu_packed, H, M, pos_offset, row_types, true};
  if ((st = aa::launch_leaf_gemm(up, gate_up, stream)) != AA_OK) return st;
  aa::LeafCall proj_down{H, Wd_packed, nullptr, Y, M, pos_offset, row_types, false};
  return aa::launch_leaf_gemm(down, proj_down, stream);
}

}  // namespace

extern "C" {

aa_status_t aa_pack_weights(aa_plan_t plan, const void* W_rowmajor, void* W_packed, hipStream_t stream) {
  aa::clear_error();
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_pack_weights: plan is NULL");
  aa_status_t st;
  if ((st = check_ptr(W_rowmajor, "W_rowmajor", "aa_pack_weights")) != AA_OK) return st;
  if ((st = check_ptr(W_packed, "W_packed", "aa_pack_weights")) != AA_OK) return st;
  const size_t bytes = size_t(plan->d_in * plan->d_out) * elem_size(plan->in_dtype);
  if (overlaps(W_rowmajor, bytes, W_packed, bytes))
    return fail(AA_ERR_INVALID_ARG, "aa_pack_weights: source and destination overlap");
  return aa::launch_pack(*plan, W_rowmajor, W_packed, false, stream);
}

aa_status_t aa_unpack_weights(aa_plan_t plan, const void* W_packed, void* W_rowmajor, hipStream_t stream) {
  aa::clear_error();
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_unpack_weights: plan is NULL");
  aa_status_t st;
  if ((st = check_ptr(W_packed, "W_packed", "aa_unpack_weights")) != AA_OK) return st;
  if ((st = check_ptr(W_rowmajor, "W_rowmajor", "aa_unpack_weights")) != AA_OK) return st;
  const size_t bytes = size_t(plan->d_in * plan->d_out) * elem_size(plan->in_dtype);
  if (overlaps(W_rowmajor, bytes, W_packed, bytes))
    return fail(AA_ERR_INVALID_ARG, "aa_unpack_weights: source and destination overlap");
  return aa::launch_pack(*plan, W_packed, W_rowmajor, true, stream);
}

aa_status_t aa_project_fwd(aa_plan_t plan, const void* X, const void* W_packed, void* Y, int64_t M,
                           int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_project_fwd";
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_project_fwd: plan is NULL");
  aa_status_t st;
  if ((st = check_rows(*plan, M, pos_offset, row_types, fn)) != AA_OK) return st;
  if (M == 0) return AA_OK;
  if ((st = check_ptr(X, "X", fn)) != AA_OK) return st;
  if ((st = check_ptr(W_packed, "W_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(Y, "Y", fn)) != AA_OK) return st;
  const size_t xb = size_t(M * plan->d_in) * elem_size(plan->in_dtype);
  const size_t wb = size_t(plan->d_in * plan->d_out) * elem_size(plan->in_dtype);
  const size_t yb = size_t(M * plan->d_out) * elem_size(plan->out_dtype);
  if (overlaps(Y, yb, X, xb) || overlaps(Y, yb, W_packed, wb))
    return fail(AA_ERR_INVALID_ARG, "aa_project_fwd: Y overlaps X or W_packed");
  aa::LeafCall call{X, W_packed, nullptr, Y, M, pos_offset, row_types, false};
  return aa::launch_leaf_gemm(*plan, call, stream);
}

aa_status_t aa_swiglu_ffn_fwd(aa_plan_t up, aa_plan_t down, const void* X, const void* Wg_packed,
                              const void* Wu_packed, const void* Wd_packed, void* H, void* Y, int64_t M,
                              int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_swiglu_ffn_fwd";
  aa_status_t st;
  if ((st = check_swiglu(up, down, X, Wg_packed, Wu_packed, Wd_packed, Y, M, pos_offset, row_types, fn)) != AA_OK)
    return st;
  if (M == 0) return AA_OK;
  if ((st = check_ptr(H, "H", fn)) != AA_OK) return st;
  const size_t hb = size_t(M * up->d_out) * elem_size(up->out_dtype);
  const size_t yb = size_t(M * down->d_out) * elem_size(down->out_dtype);
  const size_t xb = size_t(M * up->d_in) * elem_size(up->in_dtype);
  if (overlaps(H, hb, Y, yb) || overlaps(H, hb, X, xb))
    return fail(AA_ERR_INVALID_ARG, "aa_swiglu_ffn_fwd: X, H and Y must not overlap");
  return run_swiglu(*up, *down, X, Wg_packed, Wu_packed, Wd_packed, H, Y, M, pos_offset, row_types, stream);
}

aa_status_t aa_swiglu_ffn_fwd_noalloc(aa_plan_t up, aa_plan_t down, const void* X, const void* Wg_packed,
                                      const void* Wu_packed, const void* Wd_packed, void* Y, int64_t M,
                                      int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_swiglu_ffn_fwd_noalloc";
  aa_status_t st;
  if ((st = check_swiglu(up, down, X, Wg_packed, Wu_packed, Wd_packed, Y, M, pos_offset, row_types, fn)) != AA_OK)
    return st;
  if (M == 0) return AA_OK;
  const size_t hb = size_t(M) * size_t(up->d_out) * elem_size(up->out_dtype);
  if (hb > aa::kNoAllocScratchBytes)
    return fail(AA_ERR_UNSUPPORTED, std::string(fn) + ": the hidden activation (" + std::to_string(hb) +
                                        " bytes) exceeds the library's static scratch (" +
                                        std::to_string(aa::kNoAllocScratchBytes) + " bytes)");
  void* H = nullptr;
  if ((st = aa::noalloc_scratch(&H)) != AA_OK) return st;
  return run_swiglu(*up, *down, X, Wg_packed, Wu_packed, Wd_packed, H, Y, M, pos_offset, row_types, stream);
}

aa_status_t aa_project_bwd_workspace(aa_plan_t plan, int64_t M, size_t* data_bytes, size_t* weight_bytes) {
  aa::clear_error();
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_workspace: plan is NULL");
  if (M < 0) return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_workspace: M is negative");
  const bool none = plan->law == AA_LAW_DIGRAPH || plan->layout_version != 1;   // no gradient kernels
  if (data_bytes) *data_bytes = none ? 0 : aa::bwd_data_workspace_bytes(*plan, M);
  if (weight_bytes) *weight_bytes = none ? 0 : aa::bwd_weight_workspace_bytes(*plan, M);
  return AA_OK;
}

aa_status_t aa_project_bwd_data(aa_plan_t plan, const void* dY, const void* W_packed, void* dX, int64_t M,
                                int64_t pos_offset, const int32_t* row_types, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_project_bwd_data";
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_data: plan is NULL");
  aa_status_t st;
  if ((st = check_bwd(*plan, M, pos_offset, row_types, fn)) != AA_OK) return st;
  if (plan->b_in > 512) return fail(AA_ERR_UNSUPPORTED, "aa_project_bwd_data: input blocks wider than 512 features");
  if (M == 0) return AA_OK;
  if ((st = check_ptr(dY, "dY", fn)) != AA_OK) return st;
  if ((st = check_ptr(W_packed, "W_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(dX, "dX", fn)) != AA_OK) return st;
  const size_t need = aa::bwd_data_workspace_bytes(*plan, M);
  if (workspace_bytes < need)
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_data: workspace smaller than aa_project_bwd_workspace reports");
  if (need > 0 && (st = check_ptr(workspace, "workspace", fn)) != AA_OK) return st;
  const size_t yb = size_t(M * plan->d_out) * elem_size(plan->in_dtype);
  const size_t wb = size_t(plan->d_in * plan->d_out) * elem_size(plan->in_dtype);
  const size_t xb = size_t(M * plan->d_in) * elem_size(plan->out_dtype);
  if (overlaps(dX, xb, dY, yb) || overlaps(dX, xb, W_packed, wb))
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_data: dX overlaps dY or W_packed");
  if (need > 0 && (overlaps(workspace, need, dX, xb) || overlaps(workspace, need, dY, yb) ||
                   overlaps(workspace, need, W_packed, wb)))
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_data: workspace overlaps an operand");
  return aa::launch_bwd_data(*plan, dY, W_packed, dX, M, pos_offset, need > 0 ? workspace : nullptr, stream);
}

aa_status_t aa_project_bwd_weight(aa_plan_t plan, const void* X, const void* dY, void* dW_packed, int64_t M,
                                  int64_t pos_offset, const int32_t* row_types, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_project_bwd_weight";
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_weight: plan is NULL");
  aa_status_t st;
  if ((st = check_bwd(*plan, M, pos_offset, row_types, fn)) != AA_OK) return st;
  if (plan->b_in > 384)
    return fail(AA_ERR_UNSUPPORTED, "aa_project_bwd_weight: input blocks wider than 384 features");
  if (M == 0) return AA_OK;
  if ((st = check_ptr(X, "X", fn)) != AA_OK) return st;
  if ((st = check_ptr(dY, "dY", fn)) != AA_OK) return st;
  if ((st = check_ptr(dW_packed, "dW_packed", fn)) != AA_OK) return st;
  const size_t xb = size_t(M * plan->d_in) * elem_size(plan->in_dtype);
  const size_t yb = size_t(M * plan->d_out) * elem_size(plan->in_dtype);
  const size_t wb = size_t(plan->d_in * plan->d_out) * elem_size(plan->out_dtype);
  if (overlaps(dW_packed, wb, X, xb) || overlaps(dW_packed, wb, dY, yb))
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_weight: dW_packed overlaps X or dY");
  const size_t need = aa::bwd_weight_workspace_bytes(*plan, M);
  if (workspace_bytes < need)
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_weight: workspace smaller than aa_project_bwd_workspace reports");
  if (need > 0 && (st = check_ptr(workspace, "workspace", fn)) != AA_OK) return st;
  if (need > 0 && (overlaps(workspace, need, dW_packed, wb) || overlaps(workspace, need, X, xb) ||
                   overlaps(workspace, need, dY, yb)))
    return fail(AA_ERR_INVALID_ARG, "aa_project_bwd_weight: workspace overlaps an operand");
  return aa::launch_bwd_weight(*plan, X, dY, dW_packed, M, pos_offset, need > 0 ? workspace : nullptr, stream);
}

aa_status_t aa_decode_gemv(aa_plan_t plan, const void* x, const void* W_packed, void* y, int64_t n,
                           int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  aa::clear_error();
  static const char* fn = "aa_decode_gemv";
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: plan is NULL");
  if (n < 0) return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: n is negative");
  if (n >= (int64_t(1) << 20) * 16) return fail(AA_ERR_UNSUPPORTED, "aa_decode_gemv: too many tokens");
  if (pos_offset < 0) return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: pos_offset is negative");
  if (!row_types && plan->type_kind != AA_TYPES_POS_MOD)
    return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: row_types is required unless the plan uses position typing");
  if (row_types && (reinterpret_cast<uintptr_t>(row_types) & 3u))
    return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: row_types is not 4-byte aligned");
  if (row_types && plan->layout_version != 1)
    return fail(AA_ERR_UNSUPPORTED, "aa_decode_gemv: per-token types with blocks that are not multiples of 16");
  if (n == 0) return AA_OK;
  aa_status_t st;
  if ((st = check_ptr(x, "x", fn)) != AA_OK) return st;
  if ((st = check_ptr(W_packed, "W_packed", fn)) != AA_OK) return st;
  if ((st = check_ptr(y, "y", fn)) != AA_OK) return st;
  const size_t xb = size_t(n * plan->d_in) * elem_size(plan->in_dtype);
  const size_t yb = size_t(n * plan->d_out) * elem_size(plan->out_dtype);
  if (overlaps(y, yb, x, xb)) return fail(AA_ERR_INVALID_ARG, "aa_decode_gemv: x and y overlap");
  return aa::launch_decode(*plan, x, W_packed, nullptr, y, n, pos_offset, row_types, stream);
}

}  // extern "C"
