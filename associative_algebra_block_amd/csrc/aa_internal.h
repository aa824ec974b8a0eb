// Internal declarations shared by the host plan code, the entry points and the
// kernel launchers of libaa.so.  Not installed; the public surface is aa.h.
#pragma once

#include <stdint.h>

#include <string>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "aa.h"

// Host-side plan: immutable after aa_plan_create.
struct aa_plan_s {
  aa_law_t law;
  int32_t q;
  int64_t d_in, d_out;
  int64_t b_in, b_out;
  aa_type_kind_t type_kind;
  int64_t period;
  aa_dtype_t in_dtype, out_dtype;
  int64_t n_block_products;  // one full product
  int64_t n_leaves;          // q * q
  int32_t layout_version;    // packed weight layout (aa_packed_layout_version)
  int32_t tile_override;     // -1: automatic; else a variant id (tuning only)
  int32_t wg_per_cu;         // persistent kernels: workgroups launched per CU (0: automatic)
  int32_t persist_pol;       // persistent kernels: cache policy bits (-1: automatic; tuning only)
  int32_t swiglu_persist;    // 1: SwiGLU gate/up of 128-wide input blocks on the persistent kernel (tuning only)
  uint64_t adj[64];          // AA_LAW_DIGRAPH: bit k of adj[i] = edge i -> k (else all zero)
  int32_t n_edges;
};

namespace aa {

// Thread-local error text.
void set_error(const std::string& msg);
void clear_error();
aa_status_t fail(aa_status_t st, const std::string& msg);

// Number of block products in the table row of type i that ends in output
// group k (1 for k == i under Q_q, 2 otherwise; 1, 2 or 4 under Q2 x Q2; for a
// digraph 1 for k == i, 2 for an edge i -> k, else 0).  adj_row: bit k set for
// the edges i -> k of a digraph.
int leaf_groups(aa_law_t law, int q, int i, int k, int* groups /* up to 4 */, uint64_t adj_row = 0);

// ---------------------------------------------------------------- launch ---

// What a leaf-GEMM launch needs besides the plan.
struct LeafCall {
  const void* X;    // M x ldx, in_dtype
  const void* W0;   // packed weight (projection, or SwiGLU gate)
  const void* W1;   // packed SwiGLU up weight, or nullptr
  void* Y;          // M x ldy, out_dtype
  int64_t M;
  int64_t pos_offset;
  const int32_t* row_types;  // device, EXPLICIT only
  bool swiglu;               // Y = silu(X*W0) * (X*W1)
};

aa_status_t launch_leaf_gemm(const aa_plan_s& plan, const LeafCall& call, hipStream_t stream);

aa_status_t launch_pack(const aa_plan_s& plan, const void* src, void* dst, bool unpack,
                        hipStream_t stream);

// Plans whose block sides are not both multiples of 16 use packed layout 2
// and the small-block kernel (aa_small.hip).  small_layout_ok is the shape
// rule plan creation applies to them: bf16 weights, Q_q or a digraph,
// position or block-row typing, b_in and b_out multiples of 4 and at most 128.
bool small_layout_ok(aa_law_t law, aa_type_kind_t kind, aa_dtype_t in_dtype, int64_t b_in, int64_t b_out);
aa_status_t launch_small_gemm(const aa_plan_s& plan, const LeafCall& call, hipStream_t stream);
aa_status_t launch_pack_v2(const aa_plan_s& plan, const void* src, void* dst, bool unpack, hipStream_t stream);

// SwiGLU gate/up of leaves with many rows per type (aa_tile32.hip): bf16
// input, Q_q or Q2 x Q2, position or block-row typing, b_in a multiple of 32.
// rows_max: the rows of the largest row type; taken from 257 rows per type.
bool tile32_ok(const aa_plan_s& plan, const LeafCall& call, int64_t rows_max);
aa_status_t launch_tile32(const aa_plan_s& plan, const LeafCall& call, int64_t rows_max, hipStream_t stream);

// W1 non-null: SwiGLU gate/up (W gate, W1 up, y = silu(x W) * (x W1)); bf16
// input and input blocks of at most 256 rows (decode_swiglu_ok).
aa_status_t launch_decode(const aa_plan_s& plan, const void* x, const void* W, const void* W1, void* y,
                          int64_t n, int64_t pos_offset, const int32_t* row_types, hipStream_t stream);
bool decode_swiglu_ok(const aa_plan_s& plan);

// Gradients (bf16 operands, position or block-row typing).  Each needs the
// device workspace its *_workspace_bytes reports (0: none).
size_t bwd_data_workspace_bytes(const aa_plan_s& plan, int64_t M);
size_t bwd_weight_workspace_bytes(const aa_plan_s& plan, int64_t M);
aa_status_t launch_bwd_data(const aa_plan_s& plan, const void* dY, const void* W, void* dX, int64_t M,
                            int64_t pos_offset, void* ws, hipStream_t stream);
aa_status_t launch_bwd_weight(const aa_plan_s& plan, const void* X, const void* dY, void* dW, int64_t M,
                              int64_t pos_offset, void* ws, hipStream_t stream);

// Allocation-free SwiGLU: the hidden activation goes to a static device
// array of this many bytes (one per GPU); noalloc_scratch returns its address
// on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(AA_NOALLOC_SCRATCH_BYTES);
aa_status_t noalloc_scratch(void** ptr);

// Dispatch events set by aa_set_kernel_events for the calling thread: the
// start event is handed out once (to the next launch), the stop event to every
// launch until the events are set again.
struct KernelEvents {
  hipEvent_t start, stop;
};
KernelEvents take_kernel_events();

// Every kernel of the library is launched through here, so that the timing
// events reach the dispatch itself (hipExtLaunchKernel records them from the
// kernel's own start and end).  Errors are picked up by after_launch.
template <typename... Args, typename F = void (*)(Args...)>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args... args) {
  const KernelEvents ev = take_kernel_events();
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev.start, ev.stop, 0u, args...);
}

// Compute units of the current device.
int device_cu_count();

// Synchronise and check when AA_DEBUG=1; map launch errors to AA_ERR_HIP.
aa_status_t after_launch(hipStream_t stream, const char* what);

}  // namespace aa
