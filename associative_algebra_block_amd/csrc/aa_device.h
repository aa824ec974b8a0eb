// Device-side building blocks shared by the kernel files of libaa.so: the
// bf16 MFMA fragment type, its loads, the multiply and the output stores, and
// the interaction table of the two laws.  Everything sits in an anonymous
// namespace, so each translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aa.h"

namespace aa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, workgroups dealt round-robin
constexpr int kWave = 64;

// ------------------------------------------------------------ fragments ---

// Loads that fall outside the operands (rows past a type's last row, k past
// the end of a block, pipeline steps past the last one) read from this
// all-zero buffer instead of branching around the load: the kernels stay
// branch-free between issuing a load and using it, so the compiler can keep
// several steps of loads in flight (counted waits instead of full drains).
// 64 lanes x 32 bytes covers an fp32 run of 8 values per lane.
__device__ __attribute__((aligned(256))) uint32_t g_zero_runs[64 * 8];

// Eight consecutive k values of one lane, in the input element type.
template <typename T> struct Run;
template <> struct Run<__bf16> {
  u32x4_t v;
  __device__ static Run zero() { Run r; r.v = u32x4_t{0u, 0u, 0u, 0u}; return r; }
  __device__ static Run load(const __bf16* p) {
    Run r;
    r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return r;
  }
  __device__ static Run load_cached(const __bf16* p) {
    Run r;
    r.v = *reinterpret_cast<const u32x4_t*>(p);
    return r;
  }
};
template <> struct Run<float> {
  u32x4_t lo, hi;
  __device__ static Run zero() { Run r; r.lo = u32x4_t{0u, 0u, 0u, 0u}; r.hi = r.lo; return r; }
  __device__ static Run load(const float* p) {
    Run r;
    r.lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    r.hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + 1);
    return r;
  }
  __device__ static Run load_cached(const float* p) {
    Run r;
    r.lo = reinterpret_cast<const u32x4_t*>(p)[0];
    r.hi = reinterpret_cast<const u32x4_t*>(p)[1];
    return r;
  }
};

// acc (16 n x 16 m) += A (16 n x 32 k) * B (32 k x 16 m).
__device__ inline f32x4_t mma(const Run<__bf16>& a, const Run<__bf16>& b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ inline f32x4_t mma(const Run<float>& a, const Run<float>& b, f32x4_t acc) {
  // Eight K=4 steps; step e pairs element e of every lane's run, so both
  // operands see the same k for each hardware k slot.
  const float* pa0 = reinterpret_cast<const float*>(&a.lo);
  const float* pa1 = reinterpret_cast<const float*>(&a.hi);
  const float* pb0 = reinterpret_cast<const float*>(&b.lo);
  const float* pb1 = reinterpret_cast<const float*>(&b.hi);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa0[e], pb0[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa1[e], pb1[e], acc, 0, 0, 0);
  return acc;
}

// Four consecutive outputs of one row.
__device__ inline void store4(__bf16* p, f32x4_t v) {
  bf16x4_t o;
  o[0] = (__bf16)v[0];
  o[1] = (__bf16)v[1];
  o[2] = (__bf16)v[2];
  o[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4_t*>(p) = o;
}
__device__ inline void store4(float* p, f32x4_t v) { *reinterpret_cast<f32x4_t*>(p) = v; }
// Streaming stores of outputs that are not read again by this kernel.
__device__ inline void store4_nt(__bf16* p, f32x4_t v) {
  bf16x4_t o;
  o[0] = (__bf16)v[0];
  o[1] = (__bf16)v[1];
  o[2] = (__bf16)v[2];
  o[3] = (__bf16)v[3];
  __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, o), reinterpret_cast<unsigned long long*>(p));
}
__device__ inline void store4_nt(float* p, f32x4_t v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p)); }

// silu(g) * u = g u / (1 + e^-g), with the hardware exponential and
// reciprocal (a few ulp of fp32; the correctly rounded division costs about
// ten instructions per output, which dominated the SwiGLU epilogues).
__device__ inline float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// Input groups of leaf (type i, output group k); returns their count (<= 4).
// For a digraph, adj_row has bit k set for the edges i -> k; a leaf of a
// non-edge has no groups (its outputs are zero).
__device__ inline int device_leaf_groups(int law, int i, int k, int* g, uint64_t adj_row = 0) {
  if (law == AA_LAW_DIGRAPH) {
    g[0] = i;
    g[1] = k;
    if (k == i) return 1;
    return (adj_row >> k) & 1 ? 2 : 0;
  }
  if (law == AA_LAW_QQ) {
    g[0] = i;
    g[1] = k;
    return i == k ? 1 : 2;
  }
  // Q2 x Q2: first factor from {a, a2}, second from {b, b2}; listed in the
  // order (a,b), (a,b2), (a2,b), (a2,b2) with repeats dropped.
  const int a = i >> 1, b = i & 1, a2 = k >> 1, b2 = k & 1;
  const bool da = a2 != a, db = b2 != b;
  g[0] = 2 * a + b;
  g[1] = db ? 2 * a + b2 : 2 * a2 + b;
  g[2] = 2 * a2 + b;
  g[3] = 2 * a2 + b2;
  if (db && !da) return 2;
  if (da && db) return 4;
  return da ? 2 : 1;
}

}  // namespace
}  // namespace aa
