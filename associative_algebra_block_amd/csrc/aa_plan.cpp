// Host-side plan construction and validation for libaa.so.  Nothing here
// calls the HIP runtime, so plans can be created and checked on a machine
// without a GPU.
//
// The interaction table (agihunt.info review of "Change the Product, Keep the
// Parameters", paragraph on the graph multiplication table, and the pilot-law
// paragraph) is kept in closed form: under Q_q output group k of a row of type
// i takes input groups {i, k}; under the tensor square of Q2 (q = 4, group
// g = 2a + b) it takes every (a', b') with a' in {a, a''} and b' in {b, b''}.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <string>
#include <type_traits>

#include "aa_internal.h"

namespace aa {

static thread_local std::string g_last_error;

static thread_local KernelEvents g_kernel_events = {nullptr, nullptr};

KernelEvents take_kernel_events() {
  const KernelEvents ev = g_kernel_events;
  g_kernel_events.start = nullptr;
  return ev;
}

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
aa_status_t fail(aa_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

int leaf_groups(aa_law_t law, int q, int i, int k, int* groups, uint64_t adj_row) {
  if (law == AA_LAW_DIGRAPH) {
    groups[0] = i;
    groups[1] = k;
    if (k == i) return 1;
    return (adj_row >> k) & 1 ? 2 : 0;
  }
  if (law == AA_LAW_QQ) {
    groups[0] = i;
    if (k == i) return 1;
    groups[1] = k;
    return 2;
  }
  // Q2 x Q2: factors (a, b) of the type and (a2, b2) of the output group.
  (void)q;
  const int a = i >> 1, b = i & 1, a2 = k >> 1, b2 = k & 1;
  int as[2], bs[2];
  int na = 0, nb = 0;
  as[na++] = a;
  if (a2 != a) as[na++] = a2;
  bs[nb++] = b;
  if (b2 != b) bs[nb++] = b2;
  int n = 0;
  for (int x = 0; x < na; ++x)
    for (int y = 0; y < nb; ++y) groups[n++] = 2 * as[x] + bs[y];
  return n;
}

bool small_layout_ok(aa_law_t law, aa_type_kind_t kind, aa_dtype_t in_dtype, int64_t b_in, int64_t b_out) {
  return in_dtype == AA_BF16 && law != AA_LAW_Q2XQ2 && kind != AA_TYPES_EXPLICIT && b_in % 4 == 0 &&
         b_out % 4 == 0 && b_in <= 128 && b_out <= 128;
}

}  // namespace aa

using aa::fail;

namespace {

// The integer a C caller passed for an enum argument.  A C caller may pass
// any int; reading a value outside the enumerators through the enum type is
// undefined in C++, so the checks look at its representation instead.
template <typename E>
int32_t raw(const E& e) {
  static_assert(std::is_enum<E>::value && sizeof(E) == sizeof(int32_t), "enum arguments are 32-bit");
  int32_t v;
  memcpy(&v, &e, sizeof v);
  return v;
}

}  // namespace

extern "C" {

const char* aa_status_string(aa_status_t s) {
  switch (raw(s)) {
    case AA_OK: return "AA_OK";
    case AA_ERR_INVALID_ARG: return "AA_ERR_INVALID_ARG";
    case AA_ERR_SHAPE: return "AA_ERR_SHAPE";
    case AA_ERR_UNSUPPORTED: return "AA_ERR_UNSUPPORTED";
    case AA_ERR_HIP: return "AA_ERR_HIP";
  }
  return "AA_ERR_UNKNOWN";
}

const char* aa_last_error(void) { return aa::g_last_error.c_str(); }

aa_status_t aa_set_kernel_events(hipEvent_t start, hipEvent_t stop) {
  aa::g_kernel_events.start = start;
  aa::g_kernel_events.stop = stop;
  return AA_OK;
}

}  // extern "C"

namespace {

// Validation and construction shared by both creation calls; adjacency is
// non-null exactly for AA_LAW_DIGRAPH.
aa_status_t create(aa_plan_t* out, aa_law_t law, int32_t q, const uint8_t* adjacency, int64_t d_in, int64_t d_out,
                   int32_t kind_raw, int64_t period, int32_t in_raw, int32_t out_raw) {
  if (kind_raw != AA_TYPES_POS_MOD && kind_raw != AA_TYPES_BLOCK_ROWS && kind_raw != AA_TYPES_EXPLICIT)
    return fail(AA_ERR_INVALID_ARG, "aa_plan_create: unknown type map");
  if ((in_raw != AA_BF16 && in_raw != AA_F32) || (out_raw != AA_BF16 && out_raw != AA_F32))
    return fail(AA_ERR_INVALID_ARG, "aa_plan_create: unknown dtype");
  // valid enumerators from here on
  const aa_type_kind_t type_kind = static_cast<aa_type_kind_t>(kind_raw);
  const aa_dtype_t in_dtype = static_cast<aa_dtype_t>(in_raw), out_dtype = static_cast<aa_dtype_t>(out_raw);
  if (q < 1) return fail(AA_ERR_INVALID_ARG, "aa_plan_create: q must be >= 1");
  if (q > 65536) return fail(AA_ERR_UNSUPPORTED, "aa_plan_create: q above 65536");
  if (law == AA_LAW_Q2XQ2 && q != 4)
    return fail(AA_ERR_INVALID_ARG, "aa_plan_create: the Q2xQ2 law has exactly q = 4 groups");
  if (d_in < 1 || d_out < 1) return fail(AA_ERR_INVALID_ARG, "aa_plan_create: widths must be positive");
  if (d_in % q || d_out % q)
    return fail(AA_ERR_SHAPE, "aa_plan_create: q must divide d_in and d_out");
  if (period < 0) return fail(AA_ERR_INVALID_ARG, "aa_plan_create: negative period");
  if (type_kind == AA_TYPES_POS_MOD && period % q)
    return fail(AA_ERR_UNSUPPORTED,
                "aa_plan_create: a period that q does not divide needs AA_TYPES_EXPLICIT");
  const int64_t b_in = d_in / q, b_out = d_out / q;
  // blocks whose sides are multiples of the 16-wide MFMA fragment use packed
  // layout 1; narrower ones layout 2 and the small-block kernel, in the
  // shapes that kernel takes
  const bool layout1 = b_in % 16 == 0 && b_out % 16 == 0;
  if (!layout1 && !aa::small_layout_ok(law, type_kind, in_dtype, b_in, b_out))
    return fail(AA_ERR_UNSUPPORTED,
                "aa_plan_create: block sides d_in/q and d_out/q must be multiples of 16, or multiples of 4 "
                "up to 128 with bf16 weights, position or block-row typing and the Q_q or digraph law");
  if (d_in > (int64_t(1) << 31) || d_out > (int64_t(1) << 31))
    return fail(AA_ERR_UNSUPPORTED, "aa_plan_create: widths above 2^31");

  aa_plan_s* p = new (std::nothrow) aa_plan_s;
  if (!p) return fail(AA_ERR_INVALID_ARG, "aa_plan_create: out of host memory");
  p->n_edges = 0;
  for (int i = 0; i < 64; ++i) p->adj[i] = 0;
  if (adjacency) {
    for (int i = 0; i < q; ++i)
      for (int k = 0; k < q; ++k)
        if (k != i && adjacency[int64_t(i) * q + k]) {
          p->adj[i] |= uint64_t(1) << k;
          ++p->n_edges;
        }
  }
  p->law = law;
  p->q = q;
  p->d_in = d_in;
  p->d_out = d_out;
  p->b_in = b_in;
  p->b_out = b_out;
  p->type_kind = type_kind;
  p->period = period;
  p->in_dtype = in_dtype;
  p->out_dtype = out_dtype;
  int64_t n = 0;
  int groups[4];
  for (int i = 0; i < q; ++i)
    for (int k = 0; k < q; ++k) n += aa::leaf_groups(law, q, i, k, groups, i < 64 ? p->adj[i] : 0);
  p->n_block_products = n;
  p->n_leaves = int64_t(q) * q;
  p->layout_version = layout1 ? 1 : 2;
  p->tile_override = -1;
  p->wg_per_cu = 0;
  p->persist_pol = -1;
  p->swiglu_persist = 0;
  // Tuning overrides, read once here so that a plan stays immutable.
  if (const char* t = getenv("AA_TILE")) {
    char* end = nullptr;
    long v = strtol(t, &end, 10);
    if (end != t && *end == '\0' && v >= 0) p->tile_override = int32_t(v);
  }
  if (const char* t = getenv("AA_WG_PER_CU")) {
    char* end = nullptr;
    long v = strtol(t, &end, 10);
    if (end != t && *end == '\0' && v > 0 && v <= 64) p->wg_per_cu = int32_t(v);
  }
  if (const char* t = getenv("AA_SWIGLU_PERSIST")) {
    if (t[0] == '1' && t[1] == '\0') p->swiglu_persist = 1;
  }
  if (const char* t = getenv("AA_PERSIST_POL")) {
    char* end = nullptr;
    long v = strtol(t, &end, 10);
    if (end != t && *end == '\0' && v >= 0 && v < 8) p->persist_pol = int32_t(v);
  }
  *out = p;
  return AA_OK;
}

}  // namespace

extern "C" {

aa_status_t aa_plan_create(aa_plan_t* out, aa_law_t law, int32_t q, int64_t d_in, int64_t d_out,
                           aa_type_kind_t type_kind, int64_t period, aa_dtype_t in_dtype,
                           aa_dtype_t out_dtype) {
  aa::clear_error();
  if (!out) return fail(AA_ERR_INVALID_ARG, "aa_plan_create: out is NULL");
  *out = nullptr;
  const int32_t law_raw = raw(law);
  if (law_raw == AA_LAW_DIGRAPH)
    return fail(AA_ERR_INVALID_ARG, "aa_plan_create: digraph plans are made by aa_plan_create_digraph");
  if (law_raw != AA_LAW_QQ && law_raw != AA_LAW_Q2XQ2)
    return fail(AA_ERR_INVALID_ARG, "aa_plan_create: unknown law");
  return create(out, static_cast<aa_law_t>(law_raw), q, nullptr, d_in, d_out, raw(type_kind), period, raw(in_dtype),
                raw(out_dtype));
}

aa_status_t aa_plan_create_digraph(aa_plan_t* out, int32_t q, const uint8_t* adjacency, int64_t d_in,
                                   int64_t d_out, aa_type_kind_t type_kind, int64_t period,
                                   aa_dtype_t in_dtype, aa_dtype_t out_dtype) {
  aa::clear_error();
  if (!out) return fail(AA_ERR_INVALID_ARG, "aa_plan_create_digraph: out is NULL");
  *out = nullptr;
  if (!adjacency) return fail(AA_ERR_INVALID_ARG, "aa_plan_create_digraph: adjacency is NULL");
  if (q > 64) return fail(AA_ERR_UNSUPPORTED, "aa_plan_create_digraph: q above 64");
  return create(out, AA_LAW_DIGRAPH, q, adjacency, d_in, d_out, raw(type_kind), period, raw(in_dtype),
                raw(out_dtype));
}

aa_status_t aa_plan_destroy(aa_plan_t plan) {
  aa::clear_error();
  delete plan;
  return AA_OK;
}

aa_status_t aa_packed_layout_version(aa_plan_t plan, int32_t* version) {
  aa::clear_error();
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_packed_layout_version: plan is NULL");
  if (!version) return fail(AA_ERR_INVALID_ARG, "aa_packed_layout_version: version is NULL");
  *version = plan->layout_version;
  return AA_OK;
}

aa_status_t aa_plan_info(aa_plan_t plan, int64_t* n_block_products, int64_t* n_leaves,
                         int64_t* packed_elems) {
  aa::clear_error();
  if (!plan) return fail(AA_ERR_INVALID_ARG, "aa_plan_info: plan is NULL");
  if (n_block_products) *n_block_products = plan->n_block_products;
  if (n_leaves) *n_leaves = plan->n_leaves;
  if (packed_elems) *packed_elems = plan->d_in * plan->d_out;
  return AA_OK;
}

}  // extern "C"
