/*
 * aa.h - C ABI of libaa.so, the MI355X (gfx950) library for the row-typed
 * associative-algebra projection Y = X * W.
 *
 * The operation (agihunt.info review of "Change the Product, Keep the
 * Parameters: Associative Algebra Layers for Transformers", paragraphs on the
 * graph multiplication table, on row typing and on the pilot law):
 *
 *   The d_in input features and d_out output features are each split into q
 *   contiguous groups of equal width, b_in = d_in / q and b_out = d_out / q,
 *   and W into q x q blocks W_jk of b_in x b_out.  Every token (row of X) has
 *   a row type i in [0, q) and computes only row i of the multiplication
 *   table:
 *
 *     law Q_q      y_k = x_i W_ik + x_k W_kk   (k != i),   y_i = x_i W_ii
 *                  which is 2q - 1 block products per token, 2q^2 - q for a
 *                  full product (q^3 for the ordinary one);
 *     law Q2 x Q2  (q = 4, group g = 2a + b) y_g'' = sum of x_g' W_g'g'' over
 *                  g' = (a', b') with a' in {a, a''} and b' in {b, b''}: 9 of
 *                  16 block products per token, 36 for a full product.
 *
 *   Every weight block is kept (the parameter count stays d_in * d_out); only
 *   which activation block meets which weight block changes.
 *
 * Conventions for every call below.
 *  - Tensors are dense, row-major, and live in device memory owned by the
 *    caller.  The library allocates nothing in a compute call; a plan holds
 *    only host memory.
 *  - Calls enqueue work on `stream` (NULL = the legacy default stream) and
 *    return without synchronising.
 *  - Arguments are checked on the host before anything is launched; on a
 *    failed check the call returns a status other than AA_OK, launches
 *    nothing and records a message for aa_last_error().  A failed launch
 *    returns AA_ERR_HIP.  With the environment variable AA_DEBUG=1 every call
 *    synchronises its stream after launching and reports asynchronous faults
 *    as AA_ERR_HIP.
 *  - Kernel selection is automatic.  For tuning experiments only, the
 *    environment variables AA_TILE (force one kernel variant), AA_WG_PER_CU
 *    (workgroups per compute unit of the persistent kernels) and
 *    AA_PERSIST_POL (their cache-policy bits) are read once, when a plan is
 *    created, and stay fixed for that plan; a forced variant that does not
 *    fit the plan falls back to the general kernel.  Results do not depend on
 *    them beyond fp32 summation order.
 *  - Device pointers must be 16-byte aligned.
 *  - A plan is immutable after creation and may be shared between threads
 *    and streams.  aa_plan_create and aa_plan_info make no HIP calls.
 *  - Shape limits of this implementation: q >= 1, q divides d_in and d_out,
 *    and either the block sides b_in and b_out are multiples of 16 (the MFMA
 *    fragment width; packed layout 1), or they are multiples of 4 of at most
 *    128 with bf16 weights, the Q_q or digraph law and position or block-row
 *    typing (packed layout 2, e.g. the Qwen3-32B widths 5120 -> 25600 at
 *    q = 256: 20 x 100 blocks).  Layout-2 plans have no gradient calls and no
 *    per-token types in aa_decode_gemv.  Other shapes return
 *    AA_ERR_UNSUPPORTED.
 */
#ifndef AA_H_
#define AA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct aa_plan_s* aa_plan_t;

/* The multiplication law.  AA_LAW_Q2XQ2 requires q == 4 (the tensor square of
 * the two-group law; agihunt.info review, pilot-law paragraph).
 * AA_LAW_DIGRAPH is the table of a directed graph on the q groups (same
 * review, multiplication-table paragraph: the vertices are the diagonal slots,
 * the edges the kept off-diagonal slots, and an edge times an edge is zero;
 * Q_q is the complete graph); such plans come from aa_plan_create_digraph. */
typedef enum { AA_LAW_QQ = 0, AA_LAW_Q2XQ2 = 1, AA_LAW_DIGRAPH = 2 } aa_law_t;

/* How a row's type is found (agihunt.info review, row-typing paragraph: by
 * the token's absolute position).
 *  AA_TYPES_POS_MOD    row t has position p = pos_offset + t; with period > 0
 *                      (a batch of sequences of that length laid end to end)
 *                      p is taken modulo period; the type is p mod q.  period
 *                      must be 0 or a multiple of q.
 *  AA_TYPES_BLOCK_ROWS row t of an M-row input has type t / (M / q): the
 *                      block-row typing of a full algebra product A * B.
 *                      M must be a multiple of q.  pos_offset is ignored.
 *  AA_TYPES_EXPLICIT   the caller passes one int32 type per row in device
 *                      memory.  Rows whose type is outside [0, q) are not
 *                      written.  Each workgroup scans the type array, so this
 *                      map is meant for small M (mixed-position batches). */
typedef enum { AA_TYPES_POS_MOD = 0, AA_TYPES_BLOCK_ROWS = 1, AA_TYPES_EXPLICIT = 2 } aa_type_kind_t;

/* Element types.  Accumulation is always float32. */
typedef enum { AA_BF16 = 0, AA_F32 = 1 } aa_dtype_t;

typedef enum {
  AA_OK = 0,
  AA_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad enum, negative size */
  AA_ERR_SHAPE = 2,        /* sizes that do not fit together */
  AA_ERR_UNSUPPORTED = 3,  /* a valid request this implementation does not handle */
  AA_ERR_HIP = 4           /* the HIP runtime reported an error */
} aa_status_t;

/* Create a plan for projections with the given law, group count and widths.
 * in_dtype is the type of X and W; out_dtype the type of Y.  Supported pairs:
 * (BF16, BF16), (BF16, F32), (F32, F32), (F32, BF16).  On success *out holds
 * a new plan owned by the caller (free it with aa_plan_destroy); on failure
 * *out is set to NULL. */
aa_status_t aa_plan_create(aa_plan_t* out, aa_law_t law, int32_t q, int64_t d_in, int64_t d_out,
                           aa_type_kind_t type_kind, int64_t period,
                           aa_dtype_t in_dtype, aa_dtype_t out_dtype);

/* Create a plan for the table of a directed graph on q groups.  adjacency is
 * a host array of q * q bytes read during the call (not kept):
 * adjacency[i * q + k] != 0 with i != k makes i -> k an edge; the diagonal is
 * ignored.  A row of type i then computes, for output group k,
 *     y_i = x_i W_ii,   y_k = x_i W_ik + x_k W_kk  if i -> k is an edge,
 *     y_k = 0           otherwise
 * (weight blocks W_ik of non-edges are read by no call).  Everything else is
 * as for aa_plan_create; aa_plan_create itself rejects AA_LAW_DIGRAPH.
 * Limits of this implementation: 1 <= q <= 64; the calls run the general
 * leaf-GEMM kernel; the gradient calls return AA_ERR_UNSUPPORTED. */
aa_status_t aa_plan_create_digraph(aa_plan_t* out, int32_t q, const uint8_t* adjacency, int64_t d_in,
                                   int64_t d_out, aa_type_kind_t type_kind, int64_t period,
                                   aa_dtype_t in_dtype, aa_dtype_t out_dtype);

/* Free a plan.  NULL is accepted and ignored. */
aa_status_t aa_plan_destroy(aa_plan_t plan);

/* Query a plan.  Any output pointer may be NULL.
 *  n_block_products  block products of one full product: 2q^2 - q for Q_q,
 *                    36 for Q2 x Q2 (agihunt.info review, rank paragraph),
 *                    q + 2 |E| for a digraph with edge set E;
 *  n_leaves          (row type, output group) pairs, q^2;
 *  packed_elems      elements of a packed weight, equal to d_in * d_out. */
aa_status_t aa_plan_info(aa_plan_t plan, int64_t* n_block_products, int64_t* n_leaves,
                         int64_t* packed_elems);

/* The version of the packed weight layout a plan's calls read and write (the
 * format a caller stores packed weights in; see aa_pack_weights): 1 when both
 * block sides are multiples of 16, else 2.  Packed weights written under one version
 * are only valid for plans that report the same version and the same law, q,
 * d_in, d_out and in_dtype. */
aa_status_t aa_packed_layout_version(aa_plan_t plan, int32_t* version);

/* Rearrange a row-major d_in x d_out weight into the block-packed layout the
 * compute calls read, and back.  The packed weight has exactly d_in * d_out
 * elements of the plan's in_dtype; the two calls are inverse permutations
 * (bit-exact).  Source and destination must not overlap.
 *
 * Packed layout (version 1): the q x q blocks W_jk in row-major block order
 * (block index j * q + k), each block b_in * b_out elements.  Inside a block,
 * 16-column strips follow each other; inside a strip, 32-row slabs follow
 * each other; a slab holds 64 runs of 8 elements, run r covering rows
 * 8 * (r / 16) .. + 7 of the slab in column r mod 16 of the strip.  When b_in
 * is an odd multiple of 16 the last slab of each strip has 16 rows and 32
 * runs.
 *
 * Packed layout (version 2, blocks whose sides are not both multiples of 16):
 * the blocks in the same order and size; inside a block, runs of 4 elements,
 * run (kq, n) covering rows 4 kq .. 4 kq + 3 of column n.  Columns are taken
 * 16 at a time; inside such a fragment the runs go kq-major, then n; the last
 * fragment holds the remaining b_out mod 16 columns in the same order. */
aa_status_t aa_pack_weights(aa_plan_t plan, const void* W_rowmajor, void* W_packed, hipStream_t stream);
aa_status_t aa_unpack_weights(aa_plan_t plan, const void* W_packed, void* W_rowmajor, hipStream_t stream);

/* Row-typed projection Y = X * W (agihunt.info review, row-typing paragraph:
 * every token computes only its own table row; all row types run in one
 * launch).  X is M x d_in (in_dtype), W_packed is the packed weight, Y is
 * M x d_out (out_dtype); Y must not overlap X or W.  row_types is required
 * for AA_TYPES_EXPLICIT plans and must be NULL otherwise.  M == 0 is a no-op. */
aa_status_t aa_project_fwd(aa_plan_t plan, const void* X, const void* W_packed, void* Y, int64_t M,
                           int64_t pos_offset, const int32_t* row_types, hipStream_t stream);

/* SwiGLU feed-forward with all three projections in the algebra (authors'
 * post, part three, and agihunt.info review, model paragraph: the FFN is
 * SwiGLU and only its projections change):
 *   H = silu(X * Wg) (elementwise) (X * Wu)     M x F, stored as up's out_dtype
 *   Y = H * Wd                                  M x D, stored as down's out_dtype
 * `up` is the plan of the D -> F projections (gate and up share it), `down`
 * the plan of F -> D.  Both plans must have the same law, q and type map, and
 * down's in_dtype must equal up's out_dtype.  H is caller-owned workspace
 * (M x F) that receives the hidden activation.  No biases. */
aa_status_t aa_swiglu_ffn_fwd(aa_plan_t up, aa_plan_t down, const void* X, const void* Wg_packed,
                              const void* Wu_packed, const void* Wd_packed, void* H, void* Y,
                              int64_t M, int64_t pos_offset, const int32_t* row_types,
                              hipStream_t stream);

/* The SwiGLU feed-forward of aa_swiglu_ffn_fwd without the caller's hidden
 * buffer, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The call itself allocates nothing: the hidden activation H (M x F of up's
 * out_dtype) goes to a static device array of AA_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends.
 * Arguments, checks, kernels and results are those of aa_swiglu_ffn_fwd with
 * H dropped; a call whose H would exceed the array returns
 * AA_ERR_UNSUPPORTED and launches nothing.  The first call on a device looks
 * the array's address up (a HIP call, made once per device; make one call
 * before capturing a graph).  All calls on one GPU share its array, which
 * keeps the last call's H: calls that overlap in time on one GPU (several
 * streams or threads) race and must be serialised by the caller. */
#define AA_NOALLOC_SCRATCH_BYTES (64u << 20)
aa_status_t aa_swiglu_ffn_fwd_noalloc(aa_plan_t up, aa_plan_t down, const void* X, const void* Wg_packed,
                                      const void* Wu_packed, const void* Wd_packed, void* Y, int64_t M,
                                      int64_t pos_offset, const int32_t* row_types, hipStream_t stream);

/* Decode: n new tokens, each computing only its own table row by a
 * matrix-vector kernel (agihunt.info review: decoding computes only the new
 * position's row, leaves the KV cache as it is, and is a separate
 * matrix-vector kernel).  x is n x d_in, y is n x d_out.  With row_types
 * NULL the plan must use AA_TYPES_POS_MOD and row r has position
 * pos_offset + r; otherwise row_types gives one int32 type per row (any plan;
 * rows with a type outside [0, q) are not written).  Under Q_q a token reads
 * 2q - 1 weight blocks: its own block-row and the other diagonal blocks. */
aa_status_t aa_decode_gemv(aa_plan_t plan, const void* x, const void* W_packed, void* y, int64_t n,
                           int64_t pos_offset, const int32_t* row_types, hipStream_t stream);

/* Gradients of the row-typed projection for an upstream gradient dY (the
 * pages report a backward pass of the projection beside the forward one:
 * agihunt.info review, paragraph on the kernel measurements; it is the exact
 * gradient of the bilinear map of aa_project_fwd).  With T the plan's table
 * and tau(t) the type of row t:
 *   dX[t, j] = sum over k with (tau(t), j, k) in T of dY[t, k] W_jk^T
 *   dW_jk    = sum over rows t with (tau(t), j, k) in T of X[t, j]^T dY[t, k]
 * dY is M x d_out and X M x d_in, both of the plan's in_dtype; W_packed is the
 * packed weight; dX (M x d_in) and dW_packed (packed layout, d_in * d_out
 * elements, the same order as W_packed) are written in the plan's out_dtype.
 * dW_packed is overwritten, not accumulated; every block is written (blocks
 * no row reaches are zero).  Outputs must not overlap inputs.  M, pos_offset
 * and the type map mean what they mean for aa_project_fwd; M == 0 is a no-op
 * (dW is then not written).
 * Limits of this implementation: in_dtype AA_BF16; AA_TYPES_POS_MOD or
 * AA_TYPES_BLOCK_ROWS (row_types must be NULL; explicit type lists return
 * AA_ERR_UNSUPPORTED); b_in <= 512 for dX and b_in <= 384 for dW.
 * Workspace: each call needs caller-owned device scratch of at least the size
 * aa_project_bwd_workspace reports for the same plan and M (data_bytes for
 * aa_project_bwd_data, weight_bytes for aa_project_bwd_weight; either may be
 * 0, and the workspace pointer may then be NULL).  Its contents are
 * overwritten; calls that share a workspace must not overlap in time.  Either
 * output pointer of aa_project_bwd_workspace may be NULL. */
aa_status_t aa_project_bwd_workspace(aa_plan_t plan, int64_t M, size_t* data_bytes, size_t* weight_bytes);
aa_status_t aa_project_bwd_data(aa_plan_t plan, const void* dY, const void* W_packed, void* dX, int64_t M,
                                int64_t pos_offset, const int32_t* row_types, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);
aa_status_t aa_project_bwd_weight(aa_plan_t plan, const void* X, const void* dY, void* dW_packed, int64_t M,
                                  int64_t pos_offset, const int32_t* row_types, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Kernel timing, for measurement only (no part of the method).  After
 * aa_set_kernel_events(start, stop) the next kernel that a call of this
 * library launches from the calling thread records `start` at the beginning
 * of its own dispatch, and every kernel launched from this thread after that
 * records `stop` at the end of its dispatch, until the next
 * aa_set_kernel_events call; (NULL, NULL) switches this off.  Once the stream
 * has passed the call, hipEventElapsedTime(start, stop) is the time from the
 * start of its first kernel to the end of its last one, without the queue
 * time before the first kernel.  The events must have been created with
 * timing enabled on the device that runs the kernels and stay owned by the
 * caller; either may be NULL.  The setting is per thread.  Leave it off (NULL,
 * NULL) for calls captured into a HIP graph.  Always returns AA_OK and makes
 * no HIP call. */
aa_status_t aa_set_kernel_events(hipEvent_t start, hipEvent_t stop);

/* A static English name of a status code. */
const char* aa_status_string(aa_status_t status);

/* Detail of the last failure in the calling thread ("" if none).  The
 * pointer stays valid until the next aa_* call in this thread. */
const char* aa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AA_H_ */
