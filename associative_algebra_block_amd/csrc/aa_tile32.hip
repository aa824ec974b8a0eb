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
// Pipeline.  NBUF stage buffers (3 by default, two workgroups per CU): the
// copies of stage s + NBUF - 1 go out before the products of stage s, whose
// buffer is s mod NBUF; each wave then waits for its own copies of stage s + 1
// (vmcnt counts them in order, six per stage) and the workgroup meets at a
// barrier.  No copies are issued past a tile's last stage.  Rows past the
// type's last row copy row 0 of the tile and are not stored.
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst is the same for the whole wave).
__device__ inline void dma16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst), 16, 0, 0);
}

// Waits until at most `pending` stages of this wave's copies (six each) are
// still in flight.
template <int NBUF>
__device__ inline void wait_copies(int pending) {
  static_assert(NBUF >= 3 && NBUF <= 6, "stage buffers");
  switch (pending) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;               // vmcnt(0)
    case 1: __builtin_amdgcn_s_waitcnt(0x0f76); break;               // vmcnt(6)
    case 2: __builtin_amdgcn_s_waitcnt(0x0f7c); break;               // vmcnt(12)
    case 3: __builtin_amdgcn_s_waitcnt(0x4f72); break;               // vmcnt(18)
    default: __builtin_amdgcn_s_waitcnt(0x4f78); break;              // vmcnt(24)
  }
}

template <int NBUF, typename Tout>
__global__ __launch_bounds__(256, NBUF <= 3 ? 2 : 1) void leaf_tile32_swiglu_kernel(Tile32Params p) {
  constexpr int kT32Lds = NBUF * kT32Buf;
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  const int tid = int(threadIdx.x);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = p.q;

  // ---- tile.  The (row type, m-tile) pairs, type-major, are split into 8
  // contiguous ranges; XCD x (blockIdx mod 8) owns range x for every leaf of
  // those rows, so that each XCD reads its own rows once and only the weights
  // of the types it holds (about half a type per XCD for the pilot FFN: its
  // L2 keeps that type's leaves and rows).  Its workgroups walk leaf class by
  // leaf class (most input groups first, so the longest tiles start first),
  // then pair and n-tile.
  const int xcd = int(blockIdx.x % kNumXcd), slot = int(blockIdx.x / kNumXcd);
  const int pairs = q * p.mt_count;
  const int p0 = int(int64_t(xcd) * pairs / kNumXcd), p1 = int(int64_t(xcd + 1) * pairs / kNumXcd);
  const int per_class = (p1 - p0) * p.nt_count;
  if (slot >= q * per_class) return;
  const int li = slot / per_class;
  const int rem = slot - li * per_class;
  const int pr = p0 + rem / p.nt_count;
  const int nt = rem - (rem / p.nt_count) * p.nt_count;
  const int i = pr / p.mt_count, mt = pr - i * p.mt_count;
  int k;
  if (p.law == AA_LAW_QQ) k = li == q - 1 ? i : (li < i ? li : li + 1);   // two-group leaves first
  else k = i ^ (3 - li);   // Q2 x Q2: four input groups (i ^ k = 3), then two, then one
  int segs[4] = {0, 0, 0, 0};
  const int nseg = device_leaf_groups(p.law, i, k, segs);
  // input group of segment s without branches: Q_q has i then k, Q2 x Q2
  // up to four groups of two bits each
  const bool qq = p.law == AA_LAW_QQ;
  const uint32_t gpack = uint32_t(segs[0]) | (uint32_t(segs[1]) << 2) | (uint32_t(segs[2]) << 4) | (uint32_t(segs[3]) << 6);
  const int spc = p.b_in / 32;   // stages per input group
  const int n_stages = nseg * spc;

  int64_t first, stride, count;
  if (p.kind == AA_TYPES_BLOCK_ROWS) {
    first = int64_t(i) * p.rows_per_type;
    stride = 1;
    count = p.rows_per_type;
  } else {
    int r0 = i - p.off_mod_q;
    if (r0 < 0) r0 += q;
    first = r0;
    stride = q;
    count = r0 < p.M ? (p.M - r0 + q - 1) / q : 0;
  }
  const int64_t m0 = int64_t(mt) * kT32Rows;
  const int nrows = m0 >= count ? 0 : int(count - m0 < kT32Rows ? count - m0 : kT32Rows);
  if (nrows <= 0) return;
  first += m0 * stride;

  // ---- copy geometry, fixed for the tile.  Weights: wave w copies the slabs
  // of local strips 4 j + w (j = 0..3), 1 KiB each; local strips 0..7 are
  // gate strips nt * 8 .., 8..15 the up strips of the same columns.
  // Activations: wave w copies row blocks 4 j + w (j = 0, 1) of 16 rows; in
  // the 1 KiB block, 16-byte unit u holds chunk (u mod 4) ^ ((u / 16) mod 4)
  // of row u / 4 (an XOR swizzle, so that 16 rows read at one k fall on
  // distinct banks).
  const int nstrips = p.b_out / 16;
  const int64_t strip_bytes = int64_t(p.b_in) * 32;
  const int64_t blk_bytes = int64_t(p.b_in) * p.b_out * 2;
  const unsigned char* wsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * j + wave;
    int gs = nt * 8 + (s & 7);
    gs = gs < nstrips ? gs : nstrips - 1;
    wsrc[j] = (s < 8 ? p.W0 : p.W1) + int64_t(gs) * strip_bytes + lane * 16;
  }
  const __bf16* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (4 * j + wave) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    xsrc[j] = p.X + (first + int64_t(r < nrows ? r : 0) * stride) * p.ldx + chunk * 8;
  }

  // ---- operand geometry: weight fragment f of this wave is local strips
  // S(f) and S(f) + 1 (f = 0, 1 gate, f = 2, 3 up); activation fragment g is
  // rows 64 wm + 32 g + (l mod 32), k half h: chunk 2 h + l / 32, swizzled.
  const int a_lane = ((lane >> 4) & 1) * 1024 + (lane >> 5) * 256 + (lane & 15) * 16;
  int b_lane[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    b_lane[h] = kT32WBytes + (64 * wm + (lane & 31)) * 64 + (((2 * h + (lane >> 5)) ^ ((lane >> 2) & 3)) * 16);

  auto copy_stage = [&](int st, int buf) __attribute__((always_inline)) {
    const int s = st / spc, c = st - s * spc;
    const int grp = qq ? i + (k - i) * s : int((gpack >> (2 * s)) & 3u);
    const int64_t wofs = (int64_t(grp) * q + k) * blk_bytes + int64_t(c) * 1024;
    unsigned char* b = lds + buf * kT32Buf;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(wsrc[j] + wofs, b + (4 * j + wave) * 1024);
    const int64_t xofs = int64_t(grp) * p.b_in + c * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(xsrc[j] + xofs, b + kT32WBytes + (4 * j + wave) * 1024);
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][g][e] = 0.f;
  // All twelve operand reads of a stage are issued before its 16 products
  // (the scheduling barrier keeps the compiler from trading them back into
  // one register and a wait per product pair).
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* b = lds + buf * kT32Buf;
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
  };

  // ---- pipeline: stage s lives in buffer s mod NBUF.  The copies of stage
  // s + NBUF - 1 go out before the products of stage s; the barrier after
  // them follows this wave's wait for its own copies of stage s + 1 (six per
  // stage; none are issued past the last stage, so the last waits drain all).
  const int pre = n_stages < NBUF - 1 ? n_stages : NBUF - 1;
  for (int s = 0; s < pre; ++s) copy_stage(s, s);
  wait_copies<NBUF>(pre - 1);
  __builtin_amdgcn_s_barrier();
  int buf = 0, nb = NBUF - 1;   // stage st's buffer, and stage st + NBUF - 1's
  for (int st = 0; st < n_stages; ++st) {
    if (st + NBUF - 1 < n_stages) copy_stage(st + NBUF - 1, nb);
    compute(buf);
    int pending = n_stages - 2 - st;
    pending = pending < NBUF - 2 ? pending : NBUF - 2;
    wait_copies<NBUF>(pending < 0 ? 0 : pending);
    __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    buf = buf == NBUF - 1 ? 0 : buf + 1;
    nb = nb == NBUF - 1 ? 0 : nb + 1;
  }

  // ---- epilogue: h = silu(gate) * up through LDS, half the rows per pass
  // when a whole tile does not fit (fp32 output), then whole-line stores.
  constexpr int OP = 128 + 16 / int(sizeof(Tout));          // staged output row (elements)
  constexpr int PASS_ROWS = kT32Rows * OP * int(sizeof(Tout)) <= kT32Lds ? kT32Rows : kT32Rows / 2;
  constexpr int VPR = 128 * int(sizeof(Tout)) / 16;          // 16-byte chunks per output row
  Tout* otile = reinterpret_cast<Tout*>(lds);
  const int64_t col0 = int64_t(k) * p.b_out + int64_t(nt) * 128;
  const int ncols = p.b_out - nt * 128 < 128 ? p.b_out - nt * 128 : 128;
#pragma unroll
  for (int pass = 0; pass < kT32Rows / PASS_ROWS; ++pass) {
    if (PASS_ROWS == kT32Rows || wm == pass) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc[f][g][4 * j + e], acc[f + 2][g][4 * j + e]);
            const int row = (PASS_ROWS == kT32Rows ? 64 * wm : 0) + 32 * g + (lane & 31);
            const int col = wn * 64 + 32 * f + 8 * j + 4 * (lane >> 5);
            store4(otile + row * OP + col, v);
          }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int e0 = 0; e0 < PASS_ROWS * VPR; e0 += 256) {
      const int e = e0 + tid;
      const int r = e / VPR, v = e - r * VPR;
      const int col = v * (16 / int(sizeof(Tout)));
      const int gr = pass * PASS_ROWS + r;
      if (gr < nrows && col < ncols) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + r * OP + col);
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4_t*>(static_cast<Tout*>(p.Y) + (first + int64_t(gr) * stride) * p.ldy + col0 + col));
      }
    }
    if (pass + 1 < kT32Rows / PASS_ROWS) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
    }
  }
}

template <int NBUF, typename Tout>
void go_tile32(const Tile32Params& p, dim3 grid, hipStream_t s) {
  auto kernel = leaf_tile32_swiglu_kernel<NBUF, Tout>;
  constexpr int lds = NBUF * kT32Buf;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  launch(kernel, grid, dim3{256, 1, 1}, uint32_t(lds), s, p);
}

}  // namespace

bool tile32_ok(const aa_plan_s& plan, const LeafCall& call, int64_t rows_max) {
  if (!call.swiglu || plan.in_dtype != AA_BF16 || plan.b_in % 32) return false;
  if (plan.type_kind != AA_TYPES_POS_MOD && plan.type_kind != AA_TYPES_BLOCK_ROWS) return false;
  if (plan.law != AA_LAW_QQ && plan.law != AA_LAW_Q2XQ2) return false;
  // 500: this kernel; 502, 503: four or six stage buffers (one workgroup per
  // CU); 501: the 16 x 16 tile kernel (tuning)
  if (plan.tile_override == 500 || plan.tile_override == 502 || plan.tile_override == 503) return true;
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
  const int64_t n_slots = int64_t(plan.q) * ((int64_t(plan.q) * p.mt_count + kNumXcd - 1) / kNumXcd) * p.nt_count;
  if (n_slots * kNumXcd > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_swiglu_ffn_fwd: too many tiles");
  const dim3 grid{uint32_t(n_slots * kNumXcd), 1, 1};
  const bool f32 = plan.out_dtype == AA_F32;
  if (plan.tile_override == 502) {
    if (f32) go_tile32<4, float>(p, grid, stream);
    else go_tile32<4, __bf16>(p, grid, stream);
  } else if (plan.tile_override == 503) {
    if (f32) go_tile32<6, float>(p, grid, stream);
    else go_tile32<6, __bf16>(p, grid, stream);
  } else {
    if (f32) go_tile32<3, float>(p, grid, stream);
    else go_tile32<3, __bf16>(p, grid, stream);
  }
  return after_launch(stream, "leaf_tile32(swiglu)");
}

}  // namespace aa
