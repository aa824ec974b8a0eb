// HIP kernel (gfx950) for the fused SwiGLU gate/up projection of leaves with
// many rows per row type, such as the pilot FFN of the agihunt.info review of
// "Change the Product, Keep the Parameters" (Q2 x Q2 law, width 768, SwiGLU
// width 1536, 3072 rows per type at batch 8 x context 1536).  There each leaf
// (type i, output group k) is a dense GEMM of a few thousand rows by K = 192
// times the leaf's 1, 2 or 4 input groups, and the work is bound by the matrix
// cores, not by HBM.  The operation is the row-typed projection
// h = silu(x * Wg) . (x * Wu), with a row of type i producing output group k
// from the table's input groups j of that leaf (x_j Wg_jk summed over them).
//
// Design.  One workgroup (four waves, two workgroups per CU) computes 128
// rows of one leaf by 128 outputs of its group (the gate and the up columns
// of them: 256 weight columns).  Per K stage of 32 (one 32-row slab of the
// packed layout) the workgroup copies the activation slab (128 rows x 64
// bytes) and the 16 weight strips' slabs (1 KiB each, stored as packed) from
// global memory straight into LDS (global_load_lds_dwordx4: no registers, no
// LDS store instructions); every wave then reads its operands from LDS.  Wave
// (wm, wn) computes rows 64 wm .. 64 wm + 63 against 32-column fragments of
// the gate and the up columns of outputs 64 wn .. 64 wn + 63 with
// v_mfma_f32_32x32x16_bf16: each operand value read from LDS feeds 32
// products, and a k16 step takes 8 MFMAs for 6 KiB of LDS reads.  Compared
// with 16 x 16 fragments and weights read by every wave from global memory,
// this halves the vector-memory instructions per flop.
//
// Pipeline.  Three stage buffers (72 KiB, two workgroups per CU): the copies
// of stage s + 2 go out before the products of stage s, whose buffer is
// s mod 3; each wave then waits for its own copies of stage s + 1 (vmcnt
// counts them in order, six per stage) and the workgroup meets at a barrier.
// No copies are issued past a tile's last stage.  Rows past the type's last
// row copy row 0 of the tile and are not stored.  One tile per workgroup:
// a persistent form that ran each workgroup's tiles back to back, copying the
// next tile's first stages during the current tile's last ones, measured
// slower (pilot gate/up 55.2 against 47.4 us).
//
// Layouts.  MFMA operands (lane l): the weight operand holds 8 consecutive k
// (k = 16 h + 8 (l / 32) of the stage) of output column l mod 32 of a
// fragment, the activation operand the same k of row l mod 32; result
// register r holds column 8 (r / 4) + 4 (l / 32) + r mod 4 of row l mod 32.
// In LDS, a weight strip's slab is 64 runs of 16 bytes, run (k / 8) * 16 + n
// holding rows 8 (k / 8) .. + 7 of column n, exactly as packed; activation
// rows are 64 bytes, their four 16-byte chunks XOR-swizzled by bits 2-3 of
// the row, so that the 16 rows a quarter-wave reads at one k fall on distinct
// banks.  Outputs go through LDS and leave as whole 128-byte lines (stores of
// 8 bytes per lane straight from the accumulators measured 96 against 49 us
// on the pilot FFN's gate/up).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aa_device.h"
#include "aa_internal.h"

namespace aa {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct Tile32Params {
  const __bf16* X;
  const unsigned char* W0;   // packed gate weight
  const unsigned char* W1;   // packed up weight
  void* Y;
  int64_t ldx;
  int64_t ldy;
  int64_t M;
  int64_t rows_per_type;     // block-row typing
  int32_t q;
  int32_t b_in;
  int32_t b_out;
  int32_t law;
  int32_t kind;              // position or block-row typing
  int32_t off_mod_q;
  int32_t mt_count;          // 128-row tiles per leaf (the largest type)
  int32_t nt_count;          // 128-output tiles per output group
};

__device__ inline f32x16_t mma32(u32x4_t a, u32x4_t b, f32x16_t acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc,
                                                 0, 0, 0);
}

constexpr int kT32Rows = 128;                      // rows per workgroup
constexpr int kT32Strips = 16;                     // 16-column weight strips per stage (8 gate, 8 up)
constexpr int kT32WBytes = kT32Strips * 1024;      // weight slabs of one stage
constexpr int kT32Buf = kT32WBytes + kT32Rows * 64;   // one stage buffer: 24 KiB
constexpr int kT32Lds = 3 * kT32Buf;                  // three stage buffers: two workgroups per CU

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst is the same for the whole wave).
__device__ inline void dma16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst), 16, 0, 0);
}

// One tile: 128 rows of row type i (one m-tile) by output columns nt * 128 ..
// of output group k.
struct T32Tile {
  int i, k, nt, n_stages, nrows;
  uint32_t gpack;          // Q2 x Q2: input group of segment s in bits 2s, 2s + 1
  int64_t first, stride;   // the tile's first row and the row step
};

// Tile `slot` of XCD `xcd`.  The (row type, m-tile) pairs, type-major, are
// split into 8 contiguous ranges; XCD x owns range x for every leaf of those
// rows, so that each XCD reads its own rows once and only the weights of the
// types it holds (about half a type per XCD for the pilot FFN: its L2 keeps
// that type's leaves and rows).  Its slots go leaf class by leaf class (most
// input groups first, so the longest tiles come first), then pair and
// n-tile.  Returns false past the XCD's slots and for tiles without rows.
__device__ inline bool t32_tile(const Tile32Params& p, int xcd, int slot, T32Tile& t) {
  const int q = p.q;
  const int pairs = q * p.mt_count;
  const int p0 = int(int64_t(xcd) * pairs / kNumXcd), p1 = int(int64_t(xcd + 1) * pairs / kNumXcd);
  const int per_class = (p1 - p0) * p.nt_count;
  if (slot >= q * per_class) return false;
  const int li = slot / per_class;
  const int rem = slot - li * per_class;
  const int pr = p0 + rem / p.nt_count;
  t.nt = rem - (rem / p.nt_count) * p.nt_count;
  t.i = pr / p.mt_count;
  const int mt = pr - t.i * p.mt_count;
  if (p.law == AA_LAW_QQ) t.k = li == q - 1 ? t.i : (li < t.i ? li : li + 1);   // two-group leaves first
  else t.k = t.i ^ (3 - li);   // Q2 x Q2: four input groups (i ^ k = 3), then two, then one
  int segs[4] = {0, 0, 0, 0};
  const int nseg = device_leaf_groups(p.law, t.i, t.k, segs);
  t.gpack = uint32_t(segs[0]) | (uint32_t(segs[1]) << 2) | (uint32_t(segs[2]) << 4) | (uint32_t(segs[3]) << 6);
  t.n_stages = nseg * (p.b_in / 32);
  int64_t count;
  if (p.kind == AA_TYPES_BLOCK_ROWS) {
    t.first = int64_t(t.i) * p.rows_per_type;
    t.stride = 1;
    count = p.rows_per_type;
  } else {
    int r0 = t.i - p.off_mod_q;
    if (r0 < 0) r0 += q;
    t.first = r0;
    t.stride = q;
    count = r0 < p.M ? (p.M - r0 + q - 1) / q : 0;
  }
  const int64_t m0 = int64_t(mt) * kT32Rows;
  t.nrows = m0 >= count ? 0 : int(count - m0 < kT32Rows ? count - m0 : kT32Rows);
  t.first += m0 * t.stride;
  return t.nrows > 0;
}

// Per-lane copy sources of a tile.  Weights: wave w copies the slabs of local
// strips 4 j + w (j = 0..3), 1 KiB each; local strips 0..7 are gate strips
// nt * 8 .., 8..15 the up strips of the same columns.  Activations: wave w
// copies row blocks 4 j + w (j = 0, 1) of 16 rows; in the 1 KiB block,
// 16-byte unit u holds chunk (u mod 4) ^ ((u / 16) mod 4) of row u / 4 (an XOR
// swizzle, so that 16 rows read at one k fall on distinct banks).
struct T32Src {
  const unsigned char* w[4];
  const __bf16* x[2];
};

__device__ inline void t32_sources(const Tile32Params& p, const T32Tile& t, int wave, int lane, T32Src& c) {
  const int nstrips = p.b_out / 16;
  const int64_t strip_bytes = int64_t(p.b_in) * 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * j + wave;
    int gs = t.nt * 8 + (s & 7);
    gs = gs < nstrips ? gs : nstrips - 1;
    c.w[j] = (s < 8 ? p.W0 : p.W1) + int64_t(gs) * strip_bytes + lane * 16;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (4 * j + wave) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    c.x[j] = p.X + (t.first + int64_t(r < t.nrows ? r : 0) * t.stride) * p.ldx + chunk * 8;
  }
}

// Copies stage st of tile t (32 rows of K: segment st / (b_in / 32), slab
// st mod (b_in / 32)) into the stage buffer at b: six copies per wave.
__device__ inline void t32_copy(const Tile32Params& p, const T32Tile& t, const T32Src& c, int st, unsigned char* b,
                                int wave) {
  const int spc = p.b_in / 32;
  const int s = st / spc, sl = st - s * spc;
  // input group of segment s without branches: Q_q has i then k, Q2 x Q2
  // up to four groups of two bits each
  const int grp = p.law == AA_LAW_QQ ? t.i + (t.k - t.i) * s : int((t.gpack >> (2 * s)) & 3u);
  const int64_t wofs = (int64_t(grp) * p.q + t.k) * (int64_t(p.b_in) * p.b_out * 2) + int64_t(sl) * 1024;
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(c.w[j] + wofs, b + (4 * j + wave) * 1024);
  const int64_t xofs = int64_t(grp) * p.b_in + sl * 32;
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(c.x[j] + xofs, b + kT32WBytes + (4 * j + wave) * 1024);
}

// The products of one stage from its buffer b.  Weight fragment f of wave
// (wm, wn) is local strips S(f) and S(f) + 1 (f = 0, 1 gate, f = 2, 3 up);
// activation fragment g is rows 64 wm + 32 g + (l mod 32), k half h: chunk
// 2 h + l / 32, swizzled.  All twelve operand reads are issued before the 16
// products (the scheduling barrier keeps the compiler from trading them back
// into one register and a wait per product pair).
__device__ inline void t32_compute(const unsigned char* b, int a_lane, const int (&b_lane)[2], int wn,
                                   f32x16_t (&acc)[4][2]) {
  u32x4_t av[2][4], bv[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int g = 0; g < 2; ++g) bv[h][g] = *reinterpret_cast<const u32x4_t*>(b + b_lane[h] + g * 32 * 64);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int strip = (f < 2 ? 0 : 8) + wn * 4 + 2 * (f & 1);
      av[h][f] = *reinterpret_cast<const u32x4_t*>(b + a_lane + strip * 1024 + h * 512);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[f][g] = mma32(av[h][f], bv[h][g], acc[f][g]);
}

// h = silu(gate) * up of tile t through the LDS region `region`, PASS rows
// at a time, then whole-line stores; ends with a barrier (the region is free
// again).
template <typename Tout, int PASS>
__device__ inline void t32_epilogue(const Tile32Params& p, const T32Tile& t, f32x16_t (&acc)[4][2],
                                    unsigned char* region, int tid, int lane, int wm, int wn) {
  // h in place of the gate accumulators (frees the up ones before the passes)
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][g][e] = silu_mul(acc[f][g][e], acc[f + 2][g][e]);
  constexpr int OP = 128 + 16 / int(sizeof(Tout));          // staged output row (elements)
  constexpr int VPR = 128 * int(sizeof(Tout)) / 16;          // 16-byte chunks per output row
  Tout* otile = reinterpret_cast<Tout*>(region);
  const int64_t col0 = int64_t(t.k) * p.b_out + int64_t(t.nt) * 128;
  const int ncols = p.b_out - t.nt * 128 < 128 ? p.b_out - t.nt * 128 : 128;
#pragma unroll
  for (int pass = 0; pass < kT32Rows / PASS; ++pass) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int row = 64 * wm + 32 * g + (lane & 31) - pass * PASS;   // row inside this pass
      const bool mine = PASS == kT32Rows || (PASS == 64 ? wm == pass : 2 * wm + g == pass);
      if (!mine) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t v{acc[f][g][4 * j], acc[f][g][4 * j + 1], acc[f][g][4 * j + 2], acc[f][g][4 * j + 3]};
          store4(otile + row * OP + wn * 64 + 32 * f + 8 * j + 4 * (lane >> 5), v);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int e0 = 0; e0 < PASS * VPR; e0 += 256) {
      const int e = e0 + tid;
      const int r = e / VPR, v = e - r * VPR;
      const int col = v * (16 / int(sizeof(Tout)));
      const int gr = pass * PASS + r;
      if (gr < t.nrows && col < ncols) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + r * OP + col);
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4_t*>(static_cast<Tout*>(p.Y) + (t.first + int64_t(gr) * t.stride) * p.ldy + col0 + col));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
  }
}

__device__ inline void t32_zero(f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][g][e] = 0.f;
}

__device__ inline void t32_lanes(int lane, int wm, int& a_lane, int (&b_lane)[2]) {
  a_lane = ((lane >> 4) & 1) * 1024 + (lane >> 5) * 256 + (lane & 15) * 16;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    b_lane[h] = kT32WBytes + (64 * wm + (lane & 31)) * 64 + (((2 * h + (lane >> 5)) ^ ((lane >> 2) & 3)) * 16);
}

// One tile per workgroup (the grid has every slot of every XCD).  Stage s of
// the tile lives in buffer s mod 3: the copies of stage s + 2 go out before
// the products of stage s, then each wave waits for its own copies of stage
// s + 1 (vmcnt(6): the six copies of stage s + 2 may stay in flight; vmcnt(0)
// when none were issued) and the workgroup meets at the barrier.
template <typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_tile32_swiglu_kernel(Tile32Params p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  const int tid = int(threadIdx.x);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  T32Tile t;
  if (!t32_tile(p, int(blockIdx.x % kNumXcd), int(blockIdx.x / kNumXcd), t)) return;
  T32Src src;
  t32_sources(p, t, wave, lane, src);
  int a_lane, b_lane[2];
  t32_lanes(lane, wm, a_lane, b_lane);
  f32x16_t acc[4][2];
  t32_zero(acc);

  t32_copy(p, t, src, 0, lds, wave);
  if (t.n_stages > 1) {
    t32_copy(p, t, src, 1, lds + kT32Buf, wave);
    __builtin_amdgcn_s_waitcnt(0x0f76);   // vmcnt(6): stage 0 landed
  } else {
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  }
  __builtin_amdgcn_s_barrier();
  int buf = 0;
  for (int st = 0; st < t.n_stages; ++st) {
    const bool more = st + 2 < t.n_stages;
    if (more) t32_copy(p, t, src, st + 2, lds + (buf == 0 ? 2 : buf - 1) * kT32Buf, wave);
    t32_compute(lds + buf * kT32Buf, a_lane, b_lane, wn, acc);
    if (more) __builtin_amdgcn_s_waitcnt(0x0f76);   // vmcnt(6): stage st + 1 landed
    else __builtin_amdgcn_s_waitcnt(0x0f70);        // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    buf = buf == 2 ? 0 : buf + 1;
  }
  // all three buffers are free: the whole tile in one pass when it fits
  constexpr int kWhole = kT32Rows * (128 + 16 / int(sizeof(Tout))) * int(sizeof(Tout));
  t32_epilogue<Tout, kWhole <= kT32Lds ? kT32Rows : 64>(p, t, acc, lds, tid, lane, wm, wn);
}

template <typename K>
void go_tile32(K kernel, const Tile32Params& p, dim3 grid, hipStream_t s) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kT32Lds);
  launch(kernel, grid, dim3{256, 1, 1}, uint32_t(kT32Lds), s, p);
}

}  // namespace

bool tile32_ok(const aa_plan_s& plan, const LeafCall& call, int64_t rows_max) {
  if (!call.swiglu || plan.in_dtype != AA_BF16 || plan.b_in % 32) return false;
  if (plan.type_kind != AA_TYPES_POS_MOD && plan.type_kind != AA_TYPES_BLOCK_ROWS) return false;
  if (plan.law != AA_LAW_QQ && plan.law != AA_LAW_Q2XQ2) return false;
  if (plan.tile_override == 500) return true;   // 501: the 16 x 16 tile kernel (tuning)
  return plan.tile_override < 0 && rows_max > 256;
}

aa_status_t launch_tile32(const aa_plan_s& plan, const LeafCall& call, int64_t rows_max, hipStream_t stream) {
  Tile32Params p{};
  p.X = static_cast<const __bf16*>(call.X);
  p.W0 = static_cast<const unsigned char*>(call.W0);
  p.W1 = static_cast<const unsigned char*>(call.W1);
  p.Y = call.Y;
  p.ldx = plan.d_in;
  p.ldy = plan.d_out;
  p.M = call.M;
  p.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? call.M / plan.q : 0;
  p.q = plan.q;
  p.b_in = int32_t(plan.b_in);
  p.b_out = int32_t(plan.b_out);
  p.law = plan.law;
  p.kind = plan.type_kind;
  p.off_mod_q = int32_t(call.pos_offset % plan.q);
  p.mt_count = int32_t((rows_max + kT32Rows - 1) / kT32Rows);
  p.nt_count = int32_t((plan.b_out + 127) / 128);
  if (p.mt_count < 1) return AA_OK;
  // slots of the XCD with the most (row type, m-tile) pairs
  const int64_t slots = int64_t(plan.q) * ((int64_t(plan.q) * p.mt_count + kNumXcd - 1) / kNumXcd) * p.nt_count;
  if (slots * kNumXcd > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_swiglu_ffn_fwd: too many tiles");
  const dim3 grid{uint32_t(slots * kNumXcd), 1, 1};
  if (plan.out_dtype == AA_F32) go_tile32(leaf_tile32_swiglu_kernel<float>, p, grid, stream);
  else go_tile32(leaf_tile32_swiglu_kernel<__bf16>, p, grid, stream);
  return after_launch(stream, "leaf_tile32(swiglu)");
}

}  // namespace aa
