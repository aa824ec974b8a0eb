// Stand-ins for the kernel launchers of libaa.so, for a host-only build of the
// plan code and the entry points under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Each records that it was reached and launches
// nothing; the driver checks that a call which fails validation never gets
// here and that a valid one does.
#include "aa_internal.h"

namespace aa {

int g_launches = 0;

aa_status_t launch_leaf_gemm(const aa_plan_s&, const LeafCall& c, hipStream_t) {
  ++g_launches;
  return c.M > 0 ? AA_OK : AA_ERR_INVALID_ARG;
}
aa_status_t launch_pack(const aa_plan_s&, const void*, void*, bool, hipStream_t) {
  ++g_launches;
  return AA_OK;
}
aa_status_t launch_decode(const aa_plan_s&, const void*, const void*, const void*, void*, int64_t n, int64_t,
                          const int32_t*, hipStream_t) {
  ++g_launches;
  return n > 0 ? AA_OK : AA_ERR_INVALID_ARG;
}
bool decode_swiglu_ok(const aa_plan_s& plan) { return plan.in_dtype == AA_BF16 && plan.b_in <= 256; }
size_t bwd_data_workspace_bytes(const aa_plan_s& plan, int64_t M) { return size_t(M) * size_t(plan.b_in) * 4; }
size_t bwd_weight_workspace_bytes(const aa_plan_s&, int64_t) { return 0; }
aa_status_t launch_bwd_data(const aa_plan_s&, const void*, const void*, void*, int64_t, int64_t, void*, hipStream_t) {
  ++g_launches;
  return AA_OK;
}
aa_status_t launch_bwd_weight(const aa_plan_s&, const void*, const void*, void*, int64_t, int64_t, void*,
                              hipStream_t) {
  ++g_launches;
  return AA_OK;
}
aa_status_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 44);
  return AA_OK;
}

}  // namespace aa
