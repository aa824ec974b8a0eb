// Drives every entry point of aa.h through its host checks, in a build whose
// kernel launchers are stand-ins (stub_launch.cpp) and whose host code runs
// under AddressSanitizer and UndefinedBehaviorSanitizer.  Exits non-zero on
// the first wrong status; the sanitizers abort on the first memory or
// undefined-behaviour error.  No HIP runtime call is made: device pointers are
// plain aligned addresses that nothing dereferences.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <thread>

#include "aa.h"

namespace aa {
extern int g_launches;
}

static int g_checks = 0;

static void expect(aa_status_t got, aa_status_t want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    fprintf(stderr, "line %d: %s: got %s, want %s (%s)\n", line, what, aa_status_string(got),
            aa_status_string(want), aa_last_error());
    exit(1);
  }
  if (want != AA_OK && aa_last_error()[0] == '\0') {
    fprintf(stderr, "line %d: %s: failure without a message\n", line, what);
    exit(1);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// A call that fails validation must reach no launcher.
#define EXPECT_NO_LAUNCH(call, want)   \
  do {                                 \
    const int before = aa::g_launches; \
    EXPECT(call, want);                \
    if (aa::g_launches != before) {    \
      fprintf(stderr, "line %d: %s launched after failing\n", __LINE__, #call); \
      exit(1);                         \
    }                                  \
  } while (0)

static void* P(uint64_t k) { return reinterpret_cast<void*>(k << 28); }   // disjoint, 16-byte aligned

int main() {
  aa_plan_t p = nullptr, up = nullptr, down = nullptr, g = nullptr;
  // ---- plan creation
  EXPECT(aa_plan_create(&p, AA_LAW_QQ, 32, 4096, 12288, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_OK);
  int64_t nb = 0, nl = 0, pe = 0;
  EXPECT(aa_plan_info(p, &nb, &nl, &pe), AA_OK);
  if (nb != 2 * 32 * 32 - 32 || nl != 32 * 32 || pe != int64_t(4096) * 12288) return 2;
  EXPECT(aa_plan_info(p, nullptr, nullptr, nullptr), AA_OK);
  int32_t ver = 0;
  EXPECT(aa_packed_layout_version(p, &ver), AA_OK);
  if (ver != 1) return 7;
  {
    aa_plan_t p2 = nullptr;
    EXPECT(aa_plan_create(&p2, AA_LAW_QQ, 256, 5120, 25600, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_OK);
    EXPECT(aa_packed_layout_version(p2, &ver), AA_OK);
    if (ver != 2) return 8;
    EXPECT(aa_project_fwd(p2, P(1), P(2), P(3), 32768, 0, nullptr, nullptr), AA_OK);
    EXPECT_NO_LAUNCH(aa_project_bwd_weight(p2, P(1), P(2), P(3), 64, 0, nullptr, nullptr, 0, nullptr),
                     AA_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(aa_decode_gemv(p2, P(1), P(2), P(3), 2, 0, static_cast<const int32_t*>(P(4)), nullptr),
                     AA_ERR_UNSUPPORTED);
    EXPECT(aa_plan_destroy(p2), AA_OK);
  }
  EXPECT(aa_packed_layout_version(p, nullptr), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_info(nullptr, &nb, &nl, &pe), AA_ERR_INVALID_ARG);
  aa_plan_t bad = p;
  EXPECT(aa_plan_create(nullptr, AA_LAW_QQ, 2, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 0, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  if (bad != nullptr) return 3;
  EXPECT(aa_plan_create(&bad, AA_LAW_Q2XQ2, 2, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 3, 64, 96, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_SHAPE);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 2, 36, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_UNSUPPORTED);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 2, 48, 64, AA_TYPES_EXPLICIT, 0, AA_BF16, AA_BF16), AA_ERR_UNSUPPORTED);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 4, 64, 64, AA_TYPES_POS_MOD, 6, AA_BF16, AA_BF16), AA_ERR_UNSUPPORTED);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 4, 64, 64, AA_TYPES_POS_MOD, -4, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 2, -64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 1 << 20, 1 << 24, 1 << 24, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16),
         AA_ERR_UNSUPPORTED);
  EXPECT(aa_plan_create(&bad, (aa_law_t)7, 2, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 2, 64, 64, (aa_type_kind_t)9, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_QQ, 2, 64, 64, AA_TYPES_POS_MOD, 0, (aa_dtype_t)5, AA_BF16), AA_ERR_INVALID_ARG);
  EXPECT(aa_plan_create(&bad, AA_LAW_DIGRAPH, 2, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
  // digraphs: the adjacency is read during the call only (a heap copy freed at once)
  {
    uint8_t* adj = static_cast<uint8_t*>(malloc(64 * 64));
    for (int i = 0; i < 64 * 64; ++i) adj[i] = uint8_t((i * 7) % 3 == 0);
    EXPECT(aa_plan_create_digraph(&g, 64, adj, 64 * 16, 64 * 32, AA_TYPES_POS_MOD, 0, AA_BF16, AA_F32), AA_OK);
    free(adj);
    uint8_t a2[4] = {0, 1, 0, 0};
    EXPECT(aa_plan_create_digraph(&bad, 65, a2, 65 * 16, 65 * 16, AA_TYPES_POS_MOD, 0, AA_BF16, AA_F32),
           AA_ERR_UNSUPPORTED);
    EXPECT(aa_plan_create_digraph(&bad, 2, nullptr, 32, 32, AA_TYPES_POS_MOD, 0, AA_BF16, AA_F32), AA_ERR_INVALID_ARG);
  }
  EXPECT(aa_plan_create(&up, AA_LAW_QQ, 32, 4096, 12288, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_OK);
  EXPECT(aa_plan_create(&down, AA_LAW_QQ, 32, 12288, 4096, AA_TYPES_POS_MOD, 0, AA_BF16, AA_F32), AA_OK);

  // ---- pack
  EXPECT_NO_LAUNCH(aa_pack_weights(nullptr, P(1), P(2), nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_pack_weights(p, P(1), reinterpret_cast<char*>(P(1)) + 16, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_unpack_weights(p, reinterpret_cast<char*>(P(1)) + 8, P(2), nullptr), AA_ERR_INVALID_ARG);
  EXPECT(aa_pack_weights(p, P(1), P(2), nullptr), AA_OK);
  EXPECT(aa_unpack_weights(p, P(2), P(1), nullptr), AA_OK);

  // ---- projection
  EXPECT_NO_LAUNCH(aa_project_fwd(p, nullptr, P(2), P(3), 8, 0, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(3), -1, 0, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(3), 8, -1, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(3), int64_t(1) << 31, 0, nullptr, nullptr), AA_ERR_UNSUPPORTED);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(3), 8, 0, static_cast<const int32_t*>(P(4)), nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(1), 8, 0, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_fwd(p, P(1), P(2), P(2), 8, 0, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT(aa_project_fwd(p, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr), AA_OK);
  EXPECT(aa_project_fwd(p, P(1), P(2), P(3), 2048, 5, nullptr, nullptr), AA_OK);

  // ---- SwiGLU, both forms
  EXPECT_NO_LAUNCH(aa_swiglu_ffn_fwd(up, p, P(1), P(2), P(3), P(4), P(5), P(6), 8, 0, nullptr, nullptr),
                   AA_ERR_SHAPE);
  EXPECT_NO_LAUNCH(aa_swiglu_ffn_fwd(up, down, P(1), P(2), P(3), P(4), P(1), P(6), 8, 0, nullptr, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_swiglu_ffn_fwd(up, down, P(1), P(2), P(3), P(4), nullptr, P(6), 8, 0, nullptr, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT(aa_swiglu_ffn_fwd(up, down, P(1), P(2), P(3), P(4), P(5), P(6), 2048, 0, nullptr, nullptr), AA_OK);
  EXPECT(aa_swiglu_ffn_fwd(up, down, P(1), P(2), P(3), P(4), P(5), P(6), 3, 7, nullptr, nullptr), AA_OK);
  EXPECT_NO_LAUNCH(aa_swiglu_ffn_fwd_noalloc(up, down, P(1), P(2), P(3), P(4), P(1), 8, 0, nullptr, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_swiglu_ffn_fwd_noalloc(up, down, P(1), P(2), P(3), P(4), P(6), 4096, 0, nullptr, nullptr),
                   AA_ERR_UNSUPPORTED);
  EXPECT(aa_swiglu_ffn_fwd_noalloc(up, down, P(1), P(2), P(3), P(4), P(6), 2048, 0, nullptr, nullptr), AA_OK);

  // ---- decode
  EXPECT_NO_LAUNCH(aa_decode_gemv(p, P(1), P(2), P(1), 4, 0, nullptr, nullptr), AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_decode_gemv(p, P(1), P(2), P(3), 4, 0, static_cast<const int32_t*>(
                                      reinterpret_cast<void*>(uintptr_t(P(4)) + 2)), nullptr), AA_ERR_INVALID_ARG);
  EXPECT(aa_decode_gemv(p, P(1), P(2), P(3), 4, 100, nullptr, nullptr), AA_OK);

  // ---- gradients
  size_t nd = 0, nw = 0;
  EXPECT(aa_project_bwd_workspace(p, 2048, &nd, &nw), AA_OK);
  EXPECT(aa_project_bwd_workspace(p, -1, &nd, &nw), AA_ERR_INVALID_ARG);
  EXPECT(aa_project_bwd_workspace(p, 2048, &nd, &nw), AA_OK);
  EXPECT_NO_LAUNCH(aa_project_bwd_data(p, P(1), P(2), P(3), 2048, 0, nullptr, P(4), nd - 1, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT_NO_LAUNCH(aa_project_bwd_data(p, P(1), P(2), P(3), 2048, 0, nullptr, P(3), nd, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT(aa_project_bwd_data(p, P(1), P(2), P(3), 2048, 0, nullptr, P(4), nd, nullptr), AA_OK);
  EXPECT_NO_LAUNCH(aa_project_bwd_weight(p, P(1), P(2), P(1), 2048, 0, nullptr, nullptr, 0, nullptr),
                   AA_ERR_INVALID_ARG);
  EXPECT(aa_project_bwd_weight(p, P(1), P(2), P(3), 2048, 0, nullptr, nullptr, 0, nullptr), AA_OK);
  EXPECT_NO_LAUNCH(aa_project_bwd_data(g, P(1), P(2), P(3), 64, 0, nullptr, P(4), 1 << 20, nullptr),
                   AA_ERR_UNSUPPORTED);

  // ---- events, strings, per-thread messages
  EXPECT(aa_set_kernel_events(nullptr, nullptr), AA_OK);
  for (int s = 0; s <= 5; ++s)
    if (aa_status_string(aa_status_t(s))[0] == '\0') return 4;
  aa_project_fwd(p, nullptr, P(2), P(3), 8, 0, nullptr, nullptr);
  char main_msg[256];
  snprintf(main_msg, sizeof main_msg, "%s", aa_last_error());
  std::thread t([&] {
    if (aa_last_error()[0] != '\0') exit(5);
    aa_plan_t tp = nullptr;
    EXPECT(aa_plan_create(&tp, AA_LAW_QQ, 0, 64, 64, AA_TYPES_POS_MOD, 0, AA_BF16, AA_BF16), AA_ERR_INVALID_ARG);
    aa_plan_destroy(tp);
  });
  t.join();
  if (strcmp(main_msg, aa_last_error()) != 0) return 6;

  EXPECT(aa_plan_destroy(p), AA_OK);
  EXPECT(aa_plan_destroy(up), AA_OK);
  EXPECT(aa_plan_destroy(down), AA_OK);
  EXPECT(aa_plan_destroy(g), AA_OK);
  EXPECT(aa_plan_destroy(nullptr), AA_OK);
  printf("host checks passed: %d\n", g_checks);
  return 0;
}
