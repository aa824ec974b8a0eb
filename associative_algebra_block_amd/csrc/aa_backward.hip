// Gradients of the row-typed projection (HIP, gfx950).
//
// The authors report a backward pass for the projection beside the forward
// one (agihunt.info review of "Change the Product, Keep the Parameters:
// Associative Algebra Layers for Transformers", paragraph on the kernel
// measurements: forward plus gradient on the Qwen3-30B-A3B expert shape).  It
// is the exact gradient of the bilinear map.  With T the interaction table
// (multiplication-table and pilot-law paragraphs) and tau(t) the type of row t
// (row-typing paragraph):
//   forward   Y[t, k]  = sum_j  X[t, j] W_jk        over (tau(t), j, k) in T
//   data      dX[t, j] = sum_k  dY[t, k] W_jk^T     over (tau(t), j, k) in T
//   weight    dW_jk    = sum_t  X[t, j]^T dY[t, k]  over (tau(t), j, k) in T
//
// Both gradients contract over an index the packed layout does not keep
// contiguous for the MFMA operands (the data gradient over the weight's
// columns, the weight gradient over tokens), so the operand that needs it is
// staged in LDS and read back with ds_read_b64_tr_b16, which transposes 16-bit
// elements across each group of 16 lanes: lane 4a + b receives element b of
// the 8-byte chunks addressed by lanes a, a + 4, a + 8 and a + 12 of its group.
// With a matrix stored k-major in LDS (its m index contiguous), lane r of group
// g addressing (k = 8g + r/4, m = m0 + 4 (r mod 4)) leaves lane (g, m0 + j)
// holding k = 8g .. 8g + 3 of row m0 + j; a second read at k + 4 completes the
// 8-element MFMA operand run.
//
// Data gradient.  Per row type i and input group j the sum runs over the
// output groups K(i, j) = {k : (i, j, k) in T}: under Q_q every k when j = i,
// only k = j otherwise (2q - 1 block products per type, as in the forward);
// under Q2 x Q2 one, two or four.  A work item is (type i, token tile, j, part
// of K(i, j)); long lists (Q_q's own group) are cut into parts of R blocks
// whose fp32 partial sums go to a workspace and are added by a second kernel.
// Under Q_q an item also carries the one-block leaves (i, k) of its range of
// k, which read the same dY blocks (so each is read once).  Per item the
// kernel computes dX^T = W_jk dY^T: the A operand (16 input
// features x 32 output features of W_jk) is a two-strip piece of the packed
// block copied to LDS as it is (the packed octets of 8 rows already hold the
// m index contiguous) and read transposed; the B operand is 16 bytes of a dY
// row, loaded straight from HBM.
//
// Weight gradient.  Under Q_q an off-diagonal block W_ik is reached only by
// rows of type i and a diagonal block W_kk by all rows, so the work items are
// (block (i, k), rows of type i) and (block (k, k), a token range of all
// rows); a workgroup computes a 128 x 128 tile of the block with its waves in
// a 2 x 2 arrangement, and the token ranges of a diagonal block leave fp32
// partial sums that a second kernel adds.  Under Q2 x Q2 a workgroup owns a
// column chunk of output group k and walks every row type i, adding
// X[rows, j]^T dY[rows, k] into the block (j, k) of each kept j; the four
// blocks of the column stay in registers to the end.  Both MFMA operands
// (X^T and dY, contracted over tokens) come from LDS tiles read transposed;
// the result lands in the packed layout directly (a lane holds four
// consecutive rows of one column, half of a packed run).
//
// Both kernels keep the forward kernels' pipeline discipline: NSET rotating
// register sets, loads of step e + NSET - 1 issued after step e's multiplies,
// void steps past the end reading one zero run (it stays in L1), whole rounds only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "aa_device.h"
#include "aa_internal.h"

namespace aa {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// One MFMA operand run from two transposing LDS reads (k and k + 4).
__device__ inline Run<__bf16> lds_run_tr(__bf16* p0, __bf16* p1) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p0));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p1));
  const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  Run<__bf16> r;
  r.v = u32x4_t{a[0], a[1], b[0], b[1]};
  return r;
}

// Rows of type i: first + s * stride for s < count (closed-form typings).
// The divisions are done once per kernel (TypeMap), not per pipeline step.
struct TypeRows {
  int64_t first, stride, count;
};
struct TypeMap {
  int kind, q, off_mod_q, m_mod_q;
  int64_t m_div_q, rows_per_type;
  __device__ TypeMap(int kind_, int q_, int off, int64_t M, int64_t rpt)
      : kind(kind_), q(q_), off_mod_q(off), m_mod_q(int(M % q_)), m_div_q(M / q_), rows_per_type(rpt) {}
  __device__ TypeRows rows(int i) const {
    TypeRows t;
    if (kind == AA_TYPES_BLOCK_ROWS) {
      t.first = int64_t(i) * rows_per_type;
      t.stride = 1;
      t.count = rows_per_type;
    } else {
      int r0 = i - off_mod_q;
      if (r0 < 0) r0 += q;
      t.first = r0;
      t.stride = q;
      t.count = m_div_q + (r0 < m_mod_q ? 1 : 0);   // rows r0 + s q below M
    }
    return t;
  }
};

// K(i, j): output groups k whose entry (i, j, k) is kept, ascending.
__device__ inline int klist_len(int law, int q, int i, int j) {
  if (law == AA_LAW_QQ) return j == i ? q : 1;
  const int a = i >> 1, b = i & 1, a1 = j >> 1, b1 = j & 1;
  return (a1 == a ? 2 : 1) * (b1 == b ? 2 : 1);
}
__device__ inline int klist_at(int law, int i, int j, int m) {
  if (law == AA_LAW_QQ) return j == i ? m : j;
  // Q2 x Q2: j = (a1, b1) is kept for k = (a2, b2) when a1 is a or a2 and b1
  // is b or b2, so a2 is free when a1 = a and must equal a1 otherwise.
  const int a = i >> 1, b = i & 1, a1 = j >> 1, b1 = j & 1;
  const int nb = b1 == b ? 2 : 1;
  const int a2 = a1 == a ? m / nb : a1;
  const int b2 = b1 == b ? m % nb : b1;
  return 2 * a2 + b2;
}

// ------------------------------------------------------- data gradient ---

struct BwdDataParams {
  const __bf16* dY;   // M x ldy
  const __bf16* W;    // packed
  void* dX;           // M x ldx (Tout)
  float* ws;          // split leaves: [part][M][b_in] fp32 partial sums
  int64_t M, ldy, ldx;
  int32_t q, b_in, b_out, law, kind, off_mod_q;
  int64_t rows_per_type;
  int32_t mt_count;   // token tiles per type
  int32_t R;          // blocks per part of a split leaf
  int32_t nb;         // block products per type: 2q - 1 (Q_q) or 9
  int32_t ksb;        // steps (KS strips) per block
  int32_t pair;       // Q_q items carry their one-block leaves (see DItem)
  int64_t units;      // q * mt_count * nb
};

// A work item: blocks kofs .. kofs + nblk - 1 of K(i, j) for token tile mt.
// Under Q_q an item also carries the one-block leaves (i, k) for the blocks k
// of its range other than i ("pairs"): dY[rows_i, k] feeds both W_ik (the
// own-group sum) and W_kk (input group k of the same rows), so it is read once.
struct DItem {
  int64_t gu;   // global index of its first unit
  int nu;       // units (block products) it covers
  int i, mt, j, p, kofs, nblk;
  bool split;   // K(i, j) has more than one part
};

// The item that contains global unit g.  Units are numbered type by type,
// then token tile.  Under Q_q a type's units come in groups p = 0, 1, ...:
// the blocks k in [pR, pR + R) of the own-group leaf and the one-block leaves
// of the same range, 2R units (one fewer when the range holds i).  With pairs
// one group is one item; without (wide blocks, whose two accumulator sets
// would not fit the registers) the part and each one-block leaf are items of
// their own, numbered side by side.  Under Q2 x Q2 the units follow input
// group j, then K(i, j).
__device__ inline DItem ditem_at(const BwdDataParams& P, int64_t g) {
  DItem it;
  // units < 2^31 (checked on the host), so 32-bit divisions
  const uint32_t tmi = uint32_t(g) / uint32_t(P.nb);
  const int u = int(uint32_t(g) - tmi * uint32_t(P.nb));
  it.i = int(tmi / uint32_t(P.mt_count));
  it.mt = int(tmi - uint32_t(it.i) * uint32_t(P.mt_count));
  const int64_t base = int64_t(tmi) * P.nb;
  if (P.law == AA_LAW_QQ) {
    const int q = P.q, R = P.R, i = it.i;
    const int np = (q + R - 1) / R;
    auto start = [&](int p) { return 2 * p * R - (i < p * R ? 1 : 0); };
    int p = u / (2 * R);
    if (p > np - 1) p = np - 1;
    if (u < start(p)) --p;
    else if (p + 1 < np && u >= start(p + 1)) ++p;
    const int sp = q - p * R < R ? q - p * R : R;
    const int o = u - start(p);
    if (P.pair || o < sp) {   // the group (pairs), or part p of the own-group leaf
      it.j = i;
      it.p = p;
      it.kofs = p * R;
      it.nblk = sp;
      it.split = q > R;
      it.gu = base + start(p);
      it.nu = P.pair ? 2 * sp - (i >= p * R && i < p * R + sp ? 1 : 0) : sp;
    } else {                  // without pairs: a one-block leaf of the range
      int j = p * R + (o - sp);
      if (i >= p * R && i < p * R + sp && j >= i) ++j;
      it.j = j;
      it.p = 0;
      it.kofs = 0;
      it.nblk = 1;
      it.split = false;
      it.gu = base + u;
      it.nu = 1;
    }
    return it;
  }
  int j = 0, start = 0;
  while (j < P.q - 1 && u >= start + klist_len(P.law, P.q, it.i, j)) {
    start += klist_len(P.law, P.q, it.i, j);
    ++j;
  }
  const int len = klist_len(P.law, P.q, it.i, j);
  it.j = j;
  it.p = (u - start) / P.R;
  it.kofs = it.p * P.R;
  it.nblk = len - it.kofs < P.R ? len - it.kofs : P.R;
  it.split = len > P.R;
  it.gu = base + start + it.kofs;
  it.nu = it.nblk;
  return it;
}

template <typename Tout, int NFI, int MF, int KS, int NSET, bool PAIR>
__global__ __launch_bounds__(256, 2) void bwd_data_kernel(BwdDataParams P) {
  constexpr int NTHR = 256;
  constexpr int TM = 64 * MF;
  constexpr int KH = KS / 2;                        // MFMA k-steps per step
  constexpr int NT = PAIR ? 2 : 1;                  // weight tiles per step
  constexpr int NWL = (32 * KS * NFI + NTHR - 1) / NTHR;   // 16-byte weight loads per thread
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int g = lane >> 4, r = lane & 15;
  const int b_in = P.b_in, q = P.q;
  const int nfi = b_in / 16;
  const int nstrips = P.b_out / 16;
  // LDS copy of a tile: the packed octets (8 rows x 16 columns, 256 bytes)
  // with 64 bytes of padding after each, so that the transposing reads of a
  // fragment's two octets fall on different banks.
  constexpr int OP = 160;                   // octet pitch in LDS (elements)
  const int strip_elems = 16 * b_in;        // in HBM
  const int lstrip = (b_in / 8) * OP;       // in LDS
  const int tile_elems = KS * lstrip;       // KS strips of b_in x 16
  const int tile_chunks = 2 * KS * b_in;    // 16-byte chunks of a tile
  int wofs[NWL];                            // LDS offset of this thread's chunks
#pragma unroll
  for (int c = 0; c < NWL; ++c) {
    const int ch = c * NTHR + int(threadIdx.x);
    const int st = ch / (2 * b_in), rr = ch - st * (2 * b_in);
    wofs[c] = st * lstrip + (rr >> 4) * OP + (rr & 15) * 8;
  }
  const int64_t blk = int64_t(b_in) * P.b_out;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  Tout* __restrict__ dX = static_cast<Tout*>(P.dX);

  const TypeMap tmap(P.kind, q, P.off_mod_q, P.M, P.rows_per_type);
  // ---- this workgroup's units: a contiguous share of its XCD's run
  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int64_t S8 = gridDim.x / kNumXcd;
  const int64_t xlo = P.units * xcd / kNumXcd, xhi = P.units * (xcd + 1) / kNumXcd;
  const int64_t lo = xlo + (xhi - xlo) * slot / S8, hi = xlo + (xhi - xlo) * (slot + 1) / S8;
  if (lo >= hi) return;
  DItem first = ditem_at(P, lo);
  if (first.gu < lo) first = ditem_at(P, first.gu + first.nu);
  if (first.gu >= hi) return;
  int n_steps = 0;
  for (DItem it = first;;) {
    n_steps += it.nblk * P.ksb;
    const int64_t nx = it.gu + it.nu;
    if (nx >= hi || nx >= P.units) break;
    it = ditem_at(P, nx);
  }

  struct Step {
    DItem it;
    int m, s;          // block of the item, k-step of the block
    bool live, last;   // last: the item's final step
    bool pair;         // PAIR: block k != i, whose W_kk product goes to dX[rows, k]
    bool blk_last;     // the block's final step
    TypeRows tr;
  };
  // Cursor of the next step to request.
  DItem cur_it = first;
  int cur_m = 0, cur_s = 0, issued = 0;
  auto setup = [&](Step& S) __attribute__((always_inline)) {
    S.live = issued < n_steps;
    S.it = cur_it;
    S.m = cur_m;
    S.s = cur_s;
    S.last = S.live && cur_m == cur_it.nblk - 1 && cur_s == P.ksb - 1;
    S.blk_last = S.live && cur_s == P.ksb - 1;
    S.pair = PAIR && cur_it.kofs + cur_m != cur_it.i;
    S.tr = tmap.rows(cur_it.i);
    if (S.live) {
      ++issued;
      if (++cur_s == P.ksb) {
        cur_s = 0;
        if (++cur_m == cur_it.nblk) {
          cur_m = 0;
          const int64_t nx = cur_it.gu + cur_it.nu;
          if (issued < n_steps) cur_it = ditem_at(P, nx);
        }
      }
    }
  };

  // ---- loads of one step: the weight tile (KS strips of block (j, k); past
  // the block's last strip, zeros) and each lane's dY runs.
  auto load = [&](const Step& S, u32x4_t (&wr)[NT][NWL], Run<__bf16> (&br)[KH][MF]) __attribute__((always_inline)) {
    const int k = klist_at(P.law, S.it.i, S.it.j, S.it.kofs + S.m);
    const int st0 = KS * S.s;
    const int ns = nstrips - st0 < KS ? nstrips - st0 : KS;
    const int nvalid = ns * 2 * b_in;   // valid 16-byte chunks
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // tile 1 (PAIR): W_kk, or W_ik again (from L2) when k = i
      const int jj = t == 1 && S.pair ? k : S.it.j;
      const __bf16* wt = P.W + (int64_t(jj) * q + k) * blk + int64_t(st0) * strip_elems;
#pragma unroll
      for (int c = 0; c < NWL; ++c) {
        const int ch = c * NTHR + int(threadIdx.x);
        const __bf16* src = S.live && ch < nvalid ? wt + ch * 8 : zero;   // a void step reads zeros (L1)
        wr[t][c] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      const bool kok = st0 + 2 * h + (g >> 1) < nstrips;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const int64_t tt = int64_t(S.it.mt) * TM + (wave * MF + mf) * 16 + r;
        const bool ok = S.live && kok && tt < S.tr.count;
        const __bf16* src =
            ok ? P.dY + (S.tr.first + tt * S.tr.stride) * P.ldy + int64_t(k) * P.b_out + st0 * 16 + h * 32 + g * 8
               : zero;
        br[h][mf] = Run<__bf16>::load_cached(src);
      }
    }
  };
  auto store_w = [&](const u32x4_t (&wr)[NT][NWL], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < NWL; ++c) {
        const int ch = c * NTHR + int(threadIdx.x);
        if (ch < tile_chunks) *reinterpret_cast<u32x4_t*>(lds + (buf * NT + t) * tile_elems + wofs[c]) = wr[t][c];
      }
  };

  // Per-lane offset of its transposing read inside a tile (see the header).
  const int lane_off = (g >> 1) * lstrip + (8 * (g & 1) + (r >> 2)) * 8 + ((r & 3) >> 1) * OP + (r & 1) * 4;
  f32x4_t acc[MF][NFI], acc2[PAIR ? MF : 1][PAIR ? NFI : 1];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int f = 0; f < NFI; ++f) acc[mf][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mf = 0; mf < (PAIR ? MF : 1); ++mf)
#pragma unroll
    for (int f = 0; f < (PAIR ? NFI : 1); ++f) acc2[mf][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Step& S, const Run<__bf16> (&br)[KH][MF], int buf) __attribute__((always_inline)) {
    if (!S.live) return;
    // No branch between the reads and the multiplies, so the reads of later
    // fragments overlap the multiplies of earlier ones.  Fragments past nfi
    // (NFI rounded up) re-read the last one and are never stored.
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      __bf16* t = lds + buf * NT * tile_elems + 2 * h * lstrip + lane_off;
#pragma unroll
      for (int f = 0; f < NFI; ++f) {
        const int fc = f < nfi ? f : nfi - 1;
        const Run<__bf16> a = lds_run_tr(t + fc * 2 * OP, t + fc * 2 * OP + 32);
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[mf][f] = mma(a, br[h][mf], acc[mf][f]);
      }
    }
    if (PAIR && S.pair) {
#pragma unroll
      for (int h = 0; h < KH; ++h) {
        __bf16* t = lds + (buf * NT + 1) * tile_elems + 2 * h * lstrip + lane_off;
#pragma unroll
        for (int f = 0; f < NFI; ++f) {
          const int fc = f < nfi ? f : nfi - 1;
          const Run<__bf16> a = lds_run_tr(t + fc * 2 * OP, t + fc * 2 * OP + 32);
#pragma unroll
          for (int mf = 0; mf < (PAIR ? MF : 1); ++mf)
            acc2[mf][f < (PAIR ? NFI : 1) ? f : 0] = mma(a, br[h][mf], acc2[mf][f < (PAIR ? NFI : 1) ? f : 0]);
        }
      }
      if (S.blk_last) {
        // block k complete: input group k of these rows
        const int k = S.it.kofs + S.m;
#pragma unroll
        for (int mf = 0; mf < (PAIR ? MF : 1); ++mf) {
          const int64_t tt = int64_t(S.it.mt) * TM + (wave * MF + mf) * 16 + r;
          if (tt < S.tr.count) {
            const int64_t row = S.tr.first + tt * S.tr.stride;
#pragma unroll
            for (int f = 0; f < (PAIR ? NFI : 1); ++f)
              if (f < nfi) store4(dX + row * P.ldx + int64_t(k) * b_in + f * 16 + 4 * g, acc2[mf][f]);
          }
#pragma unroll
          for (int f = 0; f < (PAIR ? NFI : 1); ++f) acc2[mf][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (!S.last) return;
    // lane (token r, g) holds input features f * 16 + 4g .. + 3 of its token
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int64_t tt = int64_t(S.it.mt) * TM + (wave * MF + mf) * 16 + r;
      if (tt < S.tr.count) {
        const int64_t row = S.tr.first + tt * S.tr.stride;
#pragma unroll
        for (int f = 0; f < NFI; ++f) {
          if (f < nfi) {
            if (S.it.split) store4(P.ws + (int64_t(S.it.p) * P.M + row) * b_in + f * 16 + 4 * g, acc[mf][f]);
            else store4(dX + row * P.ldx + int64_t(S.it.j) * b_in + f * 16 + 4 * g, acc[mf][f]);
          }
        }
      }
#pragma unroll
      for (int f = 0; f < NFI; ++f) acc[mf][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ---- software pipeline over NSET register sets
  u32x4_t wr[NSET][NT][NWL];
  Run<__bf16> br[NSET][KH][MF];
  Step S[NSET];
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) {
    setup(S[s]);
    load(S[s], wr[s], br[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rounds = (n_steps + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      const int buf = s & 1 ? 1 : 0;   // NSET is even, so set parity = step parity
      store_w(wr[s], buf);
      __syncthreads();
      compute(S[s], br[s], buf);
      const int sn = (s + NSET - 1) % NSET;
      setup(S[sn]);
      load(S[sn], wr[sn], br[sn]);
    }
  }
}

// Sum of n partial sums spaced `stride` floats apart, added in part order.
// The loads go out eight at a time before any add, so a thread waits for
// memory once per eight parts rather than once per part.
__device__ inline f32x4_t sum_parts(const float* src, int64_t stride, int n) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  int p = 0;
  for (; p + 8 <= n; p += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(src + int64_t(p + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; p < n; ++p) s += *reinterpret_cast<const f32x4_t*>(src + int64_t(p) * stride);
  return s;
}

// Sum the partial sums of the split leaves into dX: Q_q's own group, row by
// row (row t of type i gets input group i).
template <typename Tout>
__global__ __launch_bounds__(256) void bwd_data_reduce_kernel(BwdDataParams P, int nparts) {
  const int cpr = P.b_in / 4;
  const int64_t n = P.M * cpr;
  Tout* __restrict__ dX = static_cast<Tout*>(P.dX);
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = e / cpr;
    const int c = int(e - t * cpr) * 4;
    const int i = P.kind == AA_TYPES_BLOCK_ROWS ? int(t / P.rows_per_type) : int((P.off_mod_q + t) % P.q);
    const f32x4_t s = sum_parts(P.ws + t * P.b_in + c, P.M * P.b_in, nparts);
    store4(dX + t * P.ldx + int64_t(i) * P.b_in + c, s);
  }
}

// ----------------------------------------------------- weight gradient ---

struct BwdWeightParams {
  const __bf16* X;    // M x ldx
  const __bf16* dY;   // M x ldy
  void* dW;           // packed (Tout)
  float* ws;          // reduce kernel: [part][k][packed block] fp32 partial diagonal blocks
  int64_t M, ldx, ldy;
  int32_t q, b_in, b_out, law, kind, off_mod_q;
  int64_t rows_per_type;
  int32_t nchunks;    // column chunks of NC strips per output group
  int32_t ndin;       // row chunks of 64 NFW input features per block
  int32_t nparts;     // reduce kernel: partial sums per diagonal block
  int32_t ldsx, ldsy; // LDS row pitch (elements) of the X and dY tiles
};

// LDS row of token t in a 64-token tile: bits 2 and 3 swapped.  A transposing
// read takes tokens 8g + 0..3 for lane groups g = 0, 1 together; with a row
// pitch of an odd multiple of 32 bytes the swap puts those eight tokens on
// eight different 32-byte bank windows.
__device__ inline int tile_row(int t) { return t ^ ((((t >> 2) ^ (t >> 3)) & 1) * 12); }

// The Q2 x Q2 weight gradient: a workgroup owns a column chunk of output
// group k (and a chunk of input features) and walks every row type; the four
// blocks (j, k) of the column stay in four accumulator slots to the end.  A
// step is 64 tokens of one type i and one input group j (two MFMA k-steps).
template <typename Tout, int NFW, int NC, int NSET>
__global__ __launch_bounds__(256, 2) void bwd_weight_kernel(BwdWeightParams P) {
  constexpr int NTHR = 256;
  constexpr int TK = 64;                         // tokens per step
  constexpr int DIN = 64 * NFW;                  // input features per workgroup
  constexpr int NSLOT = 4;
  constexpr int XCPR = DIN / 8;                  // 16-byte chunks of an X tile row
  constexpr int NXL = TK * XCPR / NTHR;          // X loads per thread
  constexpr int NYL = (TK * 2 * NC + NTHR - 1) / NTHR;
  static_assert((TK * XCPR) % NTHR == 0, "X tile");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int g = lane >> 4, r = lane & 15;
  const int b_in = P.b_in, q = P.q;
  const int nstrips = P.b_out / 16;
  const int x_elems = TK * P.ldsx, y_elems = TK * P.ldsy;
  const int buf_elems = x_elems + y_elems;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  Tout* __restrict__ dW = static_cast<Tout*>(P.dW);
  const int64_t blk = int64_t(b_in) * P.b_out;

  // ---- item (output group k, column chunk c, row chunk dc); each XCD takes
  // a contiguous run, so one group's items share its L2
  const int64_t n_items = int64_t(q) * P.nchunks * P.ndin;
  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int64_t xlo = n_items * xcd / kNumXcd, xhi = n_items * (xcd + 1) / kNumXcd;
  int64_t item = xlo + slot;
  if (item >= xhi) return;
  const int dc = int(item % P.ndin);
  item /= P.ndin;
  const int c = int(item % P.nchunks);
  const int k = int(item / P.nchunks);
  const int col0 = c * NC * 16;   // first column of the chunk inside group k
  const int row0 = dc * DIN;      // first input feature of the chunk inside a block
  const TypeMap tmap(P.kind, q, P.off_mod_q, P.M, P.rows_per_type);

  // steps: every type, every 64-token chunk of it (at least one, so that the
  // step structure does not depend on empty types), every j with (i, j, k) in T
  auto chunks_of = [&](int i) __attribute__((always_inline)) {
    const int64_t n = tmap.rows(i).count;
    return n > 0 ? int((n + TK - 1) / TK) : 1;
  };
  int n_steps = 0;
  for (int i = 0; i < q; ++i) {
    int gl[4];
    n_steps += chunks_of(i) * device_leaf_groups(P.law, i, k, gl);
  }

  struct Step {
    int i, tc, j;
    bool live;
    TypeRows tr;
  };
  int cur_i = 0, cur_tc = 0, cur_jx = 0, issued = 0;
  auto setup = [&](Step& S) __attribute__((always_inline)) {
    S.live = issued < n_steps;
    int gl[4];
    const int ng = device_leaf_groups(P.law, cur_i, k, gl);
    const int nch = chunks_of(cur_i);
    S.i = cur_i;
    S.tc = cur_tc;
    S.j = gl[cur_jx];
    S.tr = tmap.rows(cur_i);
    if (S.live) {
      ++issued;
      if (++cur_jx == ng) {
        cur_jx = 0;
        if (++cur_tc == nch) {
          cur_tc = 0;
          if (issued < n_steps) ++cur_i;
        }
      }
    }
  };

  auto load = [&](const Step& S, u32x4_t (&xr)[NXL], u32x4_t (&yr)[NYL]) __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < NXL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / XCPR, cc = ch - tk * XCPR;
      const int64_t tt = int64_t(S.tc) * TK + tk;
      const bool ok = tt < S.tr.count && row0 + cc * 8 < b_in;
      const __bf16* src =
          ok ? P.X + (S.tr.first + tt * S.tr.stride) * P.ldx + int64_t(S.j) * b_in + row0 + cc * 8 : zero;
      xr[l] = *reinterpret_cast<const u32x4_t*>(src);
    }
#pragma unroll
    for (int l = 0; l < NYL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / (2 * NC), cc = ch - tk * (2 * NC);
      const int64_t tt = int64_t(S.tc) * TK + tk;
      const bool ok = ch < TK * 2 * NC && tt < S.tr.count && col0 + cc * 8 < P.b_out;
      const __bf16* src =
          ok ? P.dY + (S.tr.first + tt * S.tr.stride) * P.ldy + int64_t(k) * P.b_out + col0 + cc * 8 : zero;
      yr[l] = *reinterpret_cast<const u32x4_t*>(src);
    }
  };
  auto store_tiles = [&](const u32x4_t (&xr)[NXL], const u32x4_t (&yr)[NYL], int buf) __attribute__((always_inline)) {
    __bf16* base = lds + buf * buf_elems;
#pragma unroll
    for (int l = 0; l < NXL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / XCPR, cc = ch - tk * XCPR;
      *reinterpret_cast<u32x4_t*>(base + tile_row(tk) * P.ldsx + cc * 8) = xr[l];
    }
#pragma unroll
    for (int l = 0; l < NYL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / (2 * NC), cc = ch - tk * (2 * NC);
      if (ch < TK * 2 * NC) *reinterpret_cast<u32x4_t*>(base + x_elems + tile_row(tk) * P.ldsy + cc * 8) = yr[l];
    }
  };

  f32x4_t acc[NSLOT][NFW][NC];
#pragma unroll
  for (int s = 0; s < NSLOT; ++s)
#pragma unroll
    for (int a = 0; a < NFW; ++a)
#pragma unroll
      for (int b = 0; b < NC; ++b) acc[s][a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Transposing-read offsets: token 8g + r/4 (and + 4), features / columns
  // 4 (r mod 4), at the token's permuted row; a wave's row fragments past the
  // block re-read fragment 0 (never stored).
  const int trow = tile_row(8 * g + (r >> 2));   // = 16 (g / 2) + 4 (g mod 2) + r / 4; token + 4 is 8 rows on
  const int xoff = trow * P.ldsx + 4 * (r & 3);
  const int yoff = trow * P.ldsy + 4 * (r & 3);
  int fofs[NFW];
  bool fok[NFW];
#pragma unroll
  for (int a = 0; a < NFW; ++a) {
    const int f = wave + 4 * a;
    fok[a] = row0 + f * 16 < b_in;
    fofs[a] = fok[a] ? f * 16 : 0;
  }

  // Store slot sl as block (sl, k): lane (column r, g) holds rows 4g .. 4g+3
  // of each of its fragments, half of a packed run.
  auto flush = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < NFW; ++a) {
      if (fok[a]) {
        const int row = row0 + fofs[a] + 4 * g;
#pragma unroll
        for (int b = 0; b < NC; ++b) {
          const int st = c * NC + b;
          if (st < nstrips) {
            const int64_t o = int64_t(st) * (b_in * 16) + (row >> 3) * 128 + r * 8 + (row & 7);
            store4(dW + (int64_t(sl) * q + k) * blk + o, acc[sl][a][b]);
          }
        }
      }
    }
  };

  auto compute = [&](const Step& S, int buf) __attribute__((always_inline)) {
    if (!S.live) return;
    __bf16* base = lds + buf * buf_elems;
    Run<__bf16> bv[2][NC], av[2][NFW];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < NC; ++b) {
        __bf16* p = base + x_elems + yoff + 32 * h * P.ldsy + b * 16;
        bv[h][b] = lds_run_tr(p, p + 8 * P.ldsy);
      }
#pragma unroll
      for (int a = 0; a < NFW; ++a) {
        __bf16* p = base + xoff + 32 * h * P.ldsx + fofs[a];
        av[h][a] = lds_run_tr(p, p + 8 * P.ldsx);
      }
    }
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      if (S.j == sl) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int a = 0; a < NFW; ++a)
#pragma unroll
            for (int b = 0; b < NC; ++b) acc[sl][a][b] = mma(av[h][a], bv[h][b], acc[sl][a][b]);
      }
    }
  };

  u32x4_t xr[NSET][NXL], yr[NSET][NYL];
  Step S[NSET];
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) {
    setup(S[s]);
    load(S[s], xr[s], yr[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rounds = (n_steps + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      const int buf = s & 1;   // NSET is even, so set parity = step parity
      store_tiles(xr[s], yr[s], buf);
      __syncthreads();
      compute(S[s], buf);
      const int sn = (s + NSET - 1) % NSET;
      setup(S[sn]);
      load(S[sn], xr[sn], yr[sn]);
    }
  }
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) flush(sl);
}

// Q_q weight gradient by a walk over the row types.  A workgroup owns a
// 64-feature by 16 NC-column tile of output group k's blocks and walks every
// row type i.  The rows of type i reach two blocks of column group k: the
// diagonal W_kk through their input group k and W_ik through their own group
// i (for i = k the one leaf is W_kk's).  A step is 64 tokens of one type: the
// dY tile and both X tiles are staged once and multiplied into two
// accumulator slots.  The W_kk slot lives to the end of the walk; the W_ik
// slot is stored when type i's rows are done.  Each dY element is read once,
// each X element once per column chunk (the group's other chunks, on the
// same XCD, find it in L2), and no partial sums exist.
template <typename Tout, int NC, int NSET>
__global__ __launch_bounds__(256, 2) void bwd_weight_walk_kernel(BwdWeightParams P) {
  constexpr int NTHR = 256;
  constexpr int TK = 64;                              // tokens per step
  constexpr int XCPR = 8;                             // 16-byte chunks of a 64-feature X row
  constexpr int NXL = TK * XCPR / NTHR;               // loads per X tile and thread
  constexpr int NYL = (TK * 2 * NC + NTHR - 1) / NTHR;
  static_assert(NSET % 2 == 0, "set parity is the LDS buffer");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int g = lane >> 4, r = lane & 15;
  const int b_in = P.b_in, q = P.q;
  const int nstrips = P.b_out / 16;
  const int x_elems = TK * P.ldsx, y_elems = TK * P.ldsy;
  const int buf_elems = 2 * x_elems + y_elems;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  Tout* __restrict__ dW = static_cast<Tout*>(P.dW);
  const int64_t blk = int64_t(b_in) * P.b_out;

  // item (output group k, column chunk c, feature chunk dc); each XCD takes a
  // contiguous run, so one group's items share its L2
  const int64_t n_items = int64_t(q) * P.nchunks * P.ndin;
  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int64_t xlo = n_items * xcd / kNumXcd, xhi = n_items * (xcd + 1) / kNumXcd;
  int64_t item = xlo + slot;
  if (item >= xhi) return;
  const int dc = int(item % P.ndin);
  item /= P.ndin;
  const int c = int(item % P.nchunks);
  const int k = int(item / P.nchunks);
  const int col0 = c * NC * 16;   // first column of the chunk inside group k
  const int row0 = dc * 64;       // first input feature of the chunk inside a block
  const TypeMap tmap(P.kind, q, P.off_mod_q, P.M, P.rows_per_type);

  // steps: every type, every 64-token chunk of it (at least one, so that a
  // type without rows still stores its zero block)
  auto chunks_of = [&](int i) __attribute__((always_inline)) {
    const int64_t n = tmap.rows(i).count;
    return n > 0 ? int((n + TK - 1) / TK) : 1;
  };
  int n_steps = 0;
  for (int i = 0; i < q; ++i) n_steps += chunks_of(i);

  struct Step {
    int i, tc;
    bool live, last;   // last: type i's final chunk
    TypeRows tr;
  };
  int cur_i = 0, cur_tc = 0, issued = 0;
  auto setup = [&](Step& S) __attribute__((always_inline)) {
    S.live = issued < n_steps;
    const int nch = chunks_of(cur_i);
    S.i = cur_i;
    S.tc = cur_tc;
    S.last = S.live && cur_tc == nch - 1;
    S.tr = tmap.rows(cur_i);
    if (S.live) {
      ++issued;
      if (++cur_tc == nch) {
        cur_tc = 0;
        if (issued < n_steps) ++cur_i;
      }
    }
  };

  // a void step (past the walk) and the own-group tile of type k read zeros
  auto load = [&](const Step& S, u32x4_t (&xk)[NXL], u32x4_t (&xi)[NXL], u32x4_t (&yr)[NYL])
      __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < NXL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / XCPR, cc = ch - tk * XCPR;
      const int64_t tt = int64_t(S.tc) * TK + tk;
      const bool ok = S.live && tt < S.tr.count && row0 + cc * 8 < b_in;
      const __bf16* row = P.X + (S.tr.first + tt * S.tr.stride) * P.ldx + row0 + cc * 8;
      xk[l] = *reinterpret_cast<const u32x4_t*>(ok ? row + int64_t(k) * b_in : zero);
      xi[l] = *reinterpret_cast<const u32x4_t*>(ok && S.i != k ? row + int64_t(S.i) * b_in : zero);
    }
#pragma unroll
    for (int l = 0; l < NYL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / (2 * NC), cc = ch - tk * (2 * NC);
      const int64_t tt = int64_t(S.tc) * TK + tk;
      const bool ok = S.live && ch < TK * 2 * NC && tt < S.tr.count && col0 + cc * 8 < P.b_out;
      const __bf16* src =
          ok ? P.dY + (S.tr.first + tt * S.tr.stride) * P.ldy + int64_t(k) * P.b_out + col0 + cc * 8 : zero;
      yr[l] = *reinterpret_cast<const u32x4_t*>(src);
    }
  };
  auto store_tiles = [&](const u32x4_t (&xk)[NXL], const u32x4_t (&xi)[NXL], const u32x4_t (&yr)[NYL], int buf)
      __attribute__((always_inline)) {
    __bf16* base = lds + buf * buf_elems;
#pragma unroll
    for (int l = 0; l < NXL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / XCPR, cc = ch - tk * XCPR;
      *reinterpret_cast<u32x4_t*>(base + tile_row(tk) * P.ldsx + cc * 8) = xk[l];
      *reinterpret_cast<u32x4_t*>(base + x_elems + tile_row(tk) * P.ldsx + cc * 8) = xi[l];
    }
#pragma unroll
    for (int l = 0; l < NYL; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch / (2 * NC), cc = ch - tk * (2 * NC);
      if (ch < TK * 2 * NC) *reinterpret_cast<u32x4_t*>(base + 2 * x_elems + tile_row(tk) * P.ldsy + cc * 8) = yr[l];
    }
  };

  // slot 0: W_kk, slot 1: W_ik of the current type
  f32x4_t acc[2][NC];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int b = 0; b < NC; ++b) acc[sl][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Transposing-read offsets as in the Q2 x Q2 kernel above; wave w owns the
  // 16-feature fragment w of the chunk (a fragment past the block re-reads
  // fragment 0 and is never stored).
  const int trow = tile_row(8 * g + (r >> 2));
  const int xoff = trow * P.ldsx + 4 * (r & 3);
  const int yoff = trow * P.ldsy + 4 * (r & 3);
  const bool fok = row0 + wave * 16 < b_in;
  const int fofs = fok ? wave * 16 : 0;

  // Store slot sl as block (j, k): lane (column r, g) holds rows 4g .. 4g+3
  // of its fragment, half of a packed run.
  auto flush = [&](int sl, int j) __attribute__((always_inline)) {
    if (!fok) return;
    const int row = row0 + fofs + 4 * g;
#pragma unroll
    for (int b = 0; b < NC; ++b) {
      const int st = c * NC + b;
      if (st < nstrips) {
        const int64_t o = int64_t(st) * (b_in * 16) + (row >> 3) * 128 + r * 8 + (row & 7);
        store4(dW + (int64_t(j) * q + k) * blk + o, acc[sl][b]);
      }
    }
  };

  auto compute = [&](const Step& S, int buf) __attribute__((always_inline)) {
    if (!S.live) return;
    __bf16* base = lds + buf * buf_elems;
    Run<__bf16> bv[2][NC], ak[2], ai[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < NC; ++b) {
        __bf16* p = base + 2 * x_elems + yoff + 32 * h * P.ldsy + b * 16;
        bv[h][b] = lds_run_tr(p, p + 8 * P.ldsy);
      }
      __bf16* pk = base + xoff + 32 * h * P.ldsx + fofs;
      ak[h] = lds_run_tr(pk, pk + 8 * P.ldsx);
      __bf16* pi = pk + x_elems;
      ai[h] = lds_run_tr(pi, pi + 8 * P.ldsx);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NC; ++b) acc[0][b] = mma(ak[h], bv[h][b], acc[0][b]);
    if (S.i != k) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NC; ++b) acc[1][b] = mma(ai[h], bv[h][b], acc[1][b]);
      if (S.last) {
        flush(1, S.i);
#pragma unroll
        for (int b = 0; b < NC; ++b) acc[1][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  u32x4_t xk[NSET][NXL], xi[NSET][NXL], yr[NSET][NYL];
  Step S[NSET];
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) {
    setup(S[s]);
    load(S[s], xk[s], xi[s], yr[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rounds = (n_steps + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      const int buf = s & 1;   // NSET is even, so set parity = step parity
      store_tiles(xk[s], xi[s], yr[s], buf);
      __syncthreads();
      compute(S[s], buf);
      const int sn = (s + NSET - 1) % NSET;
      setup(S[sn]);
      load(S[sn], xk[sn], xi[sn], yr[sn]);
    }
  }
  flush(0, k);
}

// Add the parts' partial diagonal blocks (Q_q) into dW.
template <typename Tout>
__global__ __launch_bounds__(256) void bwd_weight_reduce_kernel(BwdWeightParams P) {
  const int64_t blk = int64_t(P.b_in) * P.b_out;
  const int64_t n4 = int64_t(P.q) * blk / 4;
  Tout* __restrict__ dW = static_cast<Tout*>(P.dW);
  for (int64_t e4 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e4 < n4; e4 += int64_t(gridDim.x) * blockDim.x) {
    const int64_t e = e4 * 4;
    const int64_t k = e / blk, o = e - k * blk;
    const f32x4_t s = sum_parts(P.ws + e, int64_t(P.q) * blk, P.nparts);
    store4(dW + (k * P.q + k) * blk + o, s);
  }
}

// ------------------------------------------- weight gradient, large tiles ---
//
// Q_q with input blocks of at most 128 features per chunk: a workgroup's
// output tile is 128 input features by 128 columns of one block, the four
// waves in a 2 x 2 arrangement (64 x 64 each), so that every 64-token step
// brings 16 KB of X and 16 KB of dY for 32 MFMAs per wave.  Work items:
//   off-diagonal block (i, k), i != k: the rows of type i (kept only there);
//   diagonal block (k, k): all rows, cut into P token ranges whose fp32
//   partial sums a second kernel adds when P > 1.
// Items are numbered by output group k (diagonal parts first), and every
// workgroup takes a contiguous, step-balanced range inside its XCD's run.

struct WTileParams {
  const __bf16* X;    // M x ldx
  const __bf16* dY;   // M x ldy
  void* dW;           // packed (Tout)
  float* ws;          // P > 1: [part][k][packed block] fp32 partial diagonal blocks
  int64_t M, ldx, ldy;
  int32_t q, b_in, b_out, kind, off_mod_q;
  int64_t rows_per_type;
  int32_t nch, ndc;   // 128-column chunks, 128-feature chunks of a block
  int32_t P, SB, SA;  // diagonal parts, steps per part, steps per off-diagonal item
  int64_t UB, Uk;     // units (steps) of the diagonal items of a group, of a group
  int64_t units;      // q * Uk
};

struct WItem {
  int64_t gu;
  int k, j, c, dc, part, nsteps;
  bool diag;
};

__device__ inline WItem witem_at(const WTileParams& P, int64_t g) {
  WItem it;
  const uint32_t kk = uint32_t(g / P.Uk);
  const int64_t u = g - int64_t(kk) * P.Uk;
  const int tiles = P.nch * P.ndc;
  it.k = int(kk);
  int tile;
  if (u < P.UB) {
    const int idx = int(u / P.SB);
    tile = idx / P.P;
    it.part = idx - tile * P.P;
    it.j = it.k;
    it.diag = true;
    it.nsteps = P.SB;
    it.gu = int64_t(kk) * P.Uk + int64_t(idx) * P.SB;
  } else {
    const int idx = int((u - P.UB) / P.SA);
    const int ii = idx / tiles;
    tile = idx - ii * tiles;
    it.j = ii < it.k ? ii : ii + 1;
    it.part = 0;
    it.diag = false;
    it.nsteps = P.SA;
    it.gu = int64_t(kk) * P.Uk + P.UB + int64_t(idx) * P.SA;
  }
  it.c = tile / P.ndc;
  it.dc = tile - it.c * P.ndc;
  return it;
}

template <typename Tout>
__global__ __launch_bounds__(256, 2) void bwd_weight_tile_kernel(WTileParams P) {
  constexpr int NTHR = 256, TK = 64, NSET = 2;
  constexpr int RP = 128;                 // LDS row pitch (elements): 256 bytes, chunks XOR-swizzled
  constexpr int TILE = TK * RP;           // elements of one staged tile
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __bf16* lds = reinterpret_cast<__bf16*>(smem);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int g = lane >> 4, r = lane & 15;
  const int dh = wave & 1, chh = wave >> 1;   // this wave's 64-feature and 64-column halves
  const int b_in = P.b_in, q = P.q;
  const int nstrips = P.b_out / 16;
  const int64_t blk = int64_t(b_in) * P.b_out;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  Tout* __restrict__ dW = static_cast<Tout*>(P.dW);
  const TypeMap tmap(P.kind, q, P.off_mod_q, P.M, P.rows_per_type);

  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int64_t S8 = gridDim.x / kNumXcd;
  const int64_t xlo = P.units * xcd / kNumXcd, xhi = P.units * (xcd + 1) / kNumXcd;
  const int64_t lo = xlo + (xhi - xlo) * slot / S8, hi = xlo + (xhi - xlo) * (slot + 1) / S8;
  if (lo >= hi) return;
  WItem first = witem_at(P, lo);
  if (first.gu < lo) first = witem_at(P, first.gu + first.nsteps);
  if (first.gu >= hi) return;
  int n_steps = 0;
  for (WItem it = first;;) {
    n_steps += it.nsteps;
    const int64_t nx = it.gu + it.nsteps;
    if (nx >= hi || nx >= P.units) break;
    it = witem_at(P, nx);
  }

  struct Step {
    WItem it;
    int st;
    bool live, last;
    TypeRows tr;       // the item's rows: type j's (off-diagonal) or all rows (diagonal)
  };
  WItem cur = first;
  int cur_st = 0, issued = 0;
  auto setup = [&](Step& S) __attribute__((always_inline)) {
    S.live = issued < n_steps;
    S.it = cur;
    S.st = cur_st;
    S.last = S.live && cur_st == cur.nsteps - 1;
    if (cur.diag) {
      S.tr.first = int64_t(cur.part) * P.SB * TK;
      S.tr.stride = 1;
      S.tr.count = P.M - S.tr.first;
    } else {
      S.tr = tmap.rows(cur.j);
    }
    if (S.live) {
      ++issued;
      if (++cur_st == cur.nsteps) {
        cur_st = 0;
        if (issued < n_steps) cur = witem_at(P, cur.gu + cur.nsteps);
      }
    }
  };

  // Thread t stages chunks t + 256 l (l < 4) of each tile: token ch / 16,
  // 16-byte chunk ch mod 16 of the row.
  auto load = [&](const Step& S, u32x4_t (&xr)[4], u32x4_t (&yr)[4]) __attribute__((always_inline)) {
    const int xw = b_in - S.it.dc * 128 < 128 ? b_in - S.it.dc * 128 : 128;
    const int yw = P.b_out - S.it.c * 128 < 128 ? P.b_out - S.it.c * 128 : 128;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int ch = l * NTHR + int(threadIdx.x);
      const int tk = ch >> 4, cc = ch & 15;
      const int64_t tt = int64_t(S.st) * TK + tk;
      const bool rok = S.live && tt < S.tr.count;   // a void step reads zeros (L1)
      const int64_t row = S.tr.first + tt * S.tr.stride;
      const __bf16* xs = rok && cc * 8 < xw ? P.X + row * P.ldx + int64_t(S.it.j) * b_in + S.it.dc * 128 + cc * 8 : zero;
      const __bf16* ys =
          rok && cc * 8 < yw ? P.dY + row * P.ldy + int64_t(S.it.k) * P.b_out + S.it.c * 128 + cc * 8 : zero;
      xr[l] = *reinterpret_cast<const u32x4_t*>(xs);
      yr[l] = *reinterpret_cast<const u32x4_t*>(ys);
    }
  };
  int sofs[4];   // LDS offset of the thread's chunks (row-permuted, XOR-swizzled)
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const int ch = l * NTHR + int(threadIdx.x);
    const int tk = ch >> 4, cc = ch & 15;
    const int R = tile_row(tk);
    sofs[l] = R * RP + (((cc >> 1) ^ (R & 7)) << 4) + (cc & 1) * 8;
  }
  auto store_tiles = [&](const u32x4_t (&xr)[4], const u32x4_t (&yr)[4], int buf) __attribute__((always_inline)) {
    __bf16* base = lds + buf * 2 * TILE;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      *reinterpret_cast<u32x4_t*>(base + sofs[l]) = xr[l];
      *reinterpret_cast<u32x4_t*>(base + TILE + sofs[l]) = yr[l];
    }
  };

  // Transposing reads: tokens 8g + r/4 (+ 4: 8 rows on) of k-step h (32 h
  // rows on), 4 consecutive features / columns at 4 (r mod 4) of 32-byte
  // chunk c32, which sits at c32 XOR (row mod 8).
  const int rbase = 16 * (g >> 1) + 4 * (g & 1) + (r >> 2);   // = tile_row(8g + r/4)
  const int rsw = rbase & 7;
  auto rd = [&](__bf16* tile, int h, int c32) __attribute__((always_inline)) {
    __bf16* p = tile + (32 * h + rbase) * RP + ((c32 ^ rsw) << 4) + 4 * (r & 3);
    return lds_run_tr(p, p + 8 * RP);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Step& S, int buf) __attribute__((always_inline)) {
    if (!S.live) return;
    __bf16* xt = lds + buf * 2 * TILE;
    __bf16* yt = xt + TILE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Run<__bf16> av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = rd(xt, h, 4 * dh + a);
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = rd(yt, h, 4 * chh + b);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mma(av[a], bv[b], acc[a][b]);
    }
    if (!S.last) return;
    // lane (column r, g) holds rows 4g .. 4g+3 of each fragment: half a packed run
    const bool partial = S.it.diag && P.P > 1;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = S.it.dc * 128 + 64 * dh + 16 * a + 4 * g;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int st = 8 * S.it.c + 4 * chh + b;
        if (row < b_in && st < nstrips) {
          const int64_t o = int64_t(st) * (b_in * 16) + (row >> 3) * 128 + r * 8 + (row & 7);
          if (partial) store4(P.ws + (int64_t(S.it.part) * q + S.it.k) * blk + o, acc[a][b]);
          else store4(dW + (int64_t(S.it.j) * q + S.it.k) * blk + o, acc[a][b]);
        }
        acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  u32x4_t xr[NSET][4], yr[NSET][4];
  Step S[NSET];
  setup(S[0]);
  load(S[0], xr[0], yr[0]);
  const int rounds = (n_steps + NSET - 1) / NSET;
  for (int rdn = 0; rdn < rounds; ++rdn) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      store_tiles(xr[s], yr[s], s);
      __syncthreads();
      const int sn = (s + 1) % NSET;
      setup(S[sn]);
      load(S[sn], xr[sn], yr[sn]);
      compute(S[s], s);
    }
  }
}

int lds_pitch(int cols) {
  // A pitch of 16 mod 64 elements (32 mod 128 bytes) puts the four tokens of
  // a transposing read's 16-lane group on disjoint banks.
  const int pad = ((16 - cols) % 64 + 64) % 64;
  return cols + pad;
}

int64_t max_rows_per_type(const aa_plan_s& plan, int64_t M) {
  if (plan.type_kind == AA_TYPES_BLOCK_ROWS) return M / plan.q;
  return (M + plan.q - 1) / plan.q;
}

// Work split of the large-tile weight gradient (Q_q): P token ranges of SB
// steps for each diagonal tile, chosen so that a diagonal part is about 1.5x
// the average work per workgroup (at most 8 parts).
struct TileSplit {
  int nch, ndc, P, SB, SA;
  int64_t UB, Uk, units;
};
TileSplit tile_split(const aa_plan_s& plan, int64_t M) {
  TileSplit t;
  t.nch = int((plan.b_out + 127) / 128);
  t.ndc = int((plan.b_in + 127) / 128);
  const int tiles = t.nch * t.ndc;
  const int64_t sbt = (M + 63) / 64 > 0 ? (M + 63) / 64 : 1;
  const int64_t rpt = max_rows_per_type(plan, M);
  t.SA = int((rpt + 63) / 64 > 0 ? (rpt + 63) / 64 : 1);
  const double avg = double(plan.q) * tiles * (double(sbt) + double(plan.q - 1) * t.SA) / 512.0;
  int P = int((double(sbt) + 1.5 * avg - 1.0) / (1.5 * avg > 1.0 ? 1.5 * avg : 1.0));
  P = P < 1 ? 1 : (P > 8 ? 8 : P);
  t.SB = int((sbt + P - 1) / P);
  t.P = int((sbt + t.SB - 1) / t.SB);
  t.UB = int64_t(tiles) * t.P * t.SB;
  t.Uk = t.UB + int64_t(plan.q - 1) * tiles * t.SA;
  t.units = int64_t(plan.q) * t.Uk;
  return t;
}


// Blocks per part of a split data-gradient leaf.  Q_q's own-group leaf has q
// blocks and every other leaf one.  Parts of R blocks keep work items within a
// factor R of each other; R follows the average work per workgroup (units /
// 512, between 2 and 4), so that small problems are not held up by a few long
// items.  Q2 x Q2 leaves (at most four blocks) are never split.
struct DataSplit {
  int mf, mt_count, R, nparts;
  int64_t units;
};
DataSplit data_split(const aa_plan_s& plan, int64_t M) {
  DataSplit d;
  const int nfi = int(plan.b_in / 16);
  const int64_t rpt = max_rows_per_type(plan, M);
  d.mf = (rpt > 64 && nfi <= 4) ? 2 : 1;
  d.mt_count = int((rpt + 64 * d.mf - 1) / (64 * d.mf));
  if (d.mt_count < 1) d.mt_count = 1;
  const int nb = plan.law == AA_LAW_QQ ? 2 * plan.q - 1 : 9;
  d.units = int64_t(plan.q) * d.mt_count * nb;
  // Q_q items with pairs cover about 2R units (a range of R own-group blocks
  // and the one-block leaves of the same range), without them R units
  const bool pair = plan.law == AA_LAW_QQ && nfi <= 8;
  const int64_t per = pair ? (d.units + 512) / 1024 : (d.units + 256) / 512;
  d.R = plan.law == AA_LAW_QQ ? int(per < 2 ? 2 : (per > 4 ? 4 : per)) : 4;
  const int len = plan.law == AA_LAW_QQ ? plan.q : 4;
  d.nparts = len > d.R ? (len + d.R - 1) / d.R : 1;
  return d;
}

// Work split of the Q2 x Q2 weight gradient: NFW row fragments per wave (64
// NFW input features per workgroup) and 2 strips per column chunk.
struct WeightShape {
  int nfw, nc, nchunks, ndin;
};
WeightShape weight_shape(const aa_plan_s& plan) {
  WeightShape s;
  const int nstrips = int(plan.b_out / 16);
  s.nc = 2;
  s.nchunks = (nstrips + s.nc - 1) / s.nc;
  const int64_t items2 = int64_t(plan.q) * s.nchunks * ((plan.b_in + 127) / 128);
  s.nfw = plan.b_in >= 128 && items2 >= 128 ? 2 : 1;
  s.ndin = int((plan.b_in + 64 * s.nfw - 1) / (64 * s.nfw));
  return s;
}

}  // namespace

size_t bwd_data_workspace_bytes(const aa_plan_s& plan, int64_t M) {
  const DataSplit d = data_split(plan, M);
  if (d.nparts == 1) return 0;
  return size_t(d.nparts) * size_t(M) * size_t(plan.b_in) * sizeof(float);
}

// Q_q weight gradients walk the row types (bwd_weight_walk_kernel) when the
// walk has a tile per CU or more (64 features x 64 columns of a group each),
// and otherwise split the diagonal blocks' rows over parts
// (bwd_weight_tile_kernel).  AA_TILE=630 / 631 force the walk / the parts.
constexpr int kWalkNC = 4;
bool weight_walk(const aa_plan_s& plan) {
  if (plan.law != AA_LAW_QQ) return false;
  if (plan.tile_override == 630) return true;
  if (plan.tile_override == 631) return false;
  const int64_t items = int64_t(plan.q) * ((plan.b_out + 16 * kWalkNC - 1) / (16 * kWalkNC)) * ((plan.b_in + 63) / 64);
  return items >= device_cu_count();
}

size_t bwd_weight_workspace_bytes(const aa_plan_s& plan, int64_t M) {
  if (plan.law != AA_LAW_QQ || weight_walk(plan)) return 0;
  const int parts = tile_split(plan, M).P;
  if (parts == 1) return 0;
  return size_t(parts) * size_t(plan.q) * size_t(plan.b_in) * size_t(plan.b_out) * sizeof(float);
}

aa_status_t launch_bwd_data(const aa_plan_s& plan, const void* dY, const void* W, void* dX, int64_t M,
                            int64_t pos_offset, void* ws, hipStream_t stream) {
  BwdDataParams P{};
  P.dY = static_cast<const __bf16*>(dY);
  P.W = static_cast<const __bf16*>(W);
  P.dX = dX;
  P.ws = static_cast<float*>(ws);
  P.M = M;
  P.ldy = plan.d_out;
  P.ldx = plan.d_in;
  P.q = plan.q;
  P.b_in = int32_t(plan.b_in);
  P.b_out = int32_t(plan.b_out);
  P.law = plan.law;
  P.kind = plan.type_kind;
  P.off_mod_q = int32_t(pos_offset % plan.q);
  P.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? M / plan.q : 0;
  const DataSplit dsp = data_split(plan, M);
  P.R = dsp.R;
  P.nb = plan.law == AA_LAW_QQ ? 2 * plan.q - 1 : 9;
  const int nfi = int(plan.b_in / 16);
  const bool pair = plan.law == AA_LAW_QQ && nfi <= 8;
  P.pair = pair ? 1 : 0;
  const int KS = !pair && nfi <= 8 ? 4 : 2;   // strips per step (Q_q steps carry two weight tiles)
  P.ksb = int32_t((plan.b_out / 16 + KS - 1) / KS);
  const int MF = dsp.mf;
  P.mt_count = dsp.mt_count;
  P.units = dsp.units;
  if (P.units >= (int64_t(1) << 31)) return fail(AA_ERR_UNSUPPORTED, "aa_project_bwd_data: too many rows per type");
  const size_t lds = size_t(2) * (pair ? 2 : 1) * KS * (plan.b_in / 8) * 160 * 2;
  int grid = device_cu_count() * 2;
  grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
  const bool f32 = plan.out_dtype == AA_F32;
  auto go = [&](auto nfi_c, auto mf_c, auto nset_c) {
    constexpr int NFIc = decltype(nfi_c)::value, MFc = decltype(mf_c)::value, NS = decltype(nset_c)::value;
    if constexpr (NFIc <= 8) {
      if (pair) {
        if (f32) launch((bwd_data_kernel<float, NFIc, MFc, 2, NS, true>), dim3(grid), dim3(256), lds, stream, P);
        else launch((bwd_data_kernel<__bf16, NFIc, MFc, 2, NS, true>), dim3(grid), dim3(256), lds, stream, P);
        return;
      }
    }
    constexpr int KSc = NFIc <= 8 ? 4 : 2;
    if (f32) launch((bwd_data_kernel<float, NFIc, MFc, KSc, NS, false>), dim3(grid), dim3(256), lds, stream, P);
    else launch((bwd_data_kernel<__bf16, NFIc, MFc, KSc, NS, false>), dim3(grid), dim3(256), lds, stream, P);
  };
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C4 = std::integral_constant<int, 4>;
  if (nfi <= 4) {
    if (MF == 2) go(C4{}, C2{}, C4{});
    else go(C4{}, C1{}, C4{});
  } else if (nfi <= 8) {
    go(std::integral_constant<int, 8>{}, C1{}, C4{});
  } else if (nfi <= 16) {
    go(std::integral_constant<int, 16>{}, C1{}, C2{});
  } else if (nfi <= 24) {
    go(std::integral_constant<int, 24>{}, C1{}, C2{});
  } else if (nfi <= 32) {
    go(std::integral_constant<int, 32>{}, C1{}, C2{});
  } else {
    return fail(AA_ERR_UNSUPPORTED, "aa_project_bwd_data: input blocks wider than 512 features");
  }
  aa_status_t st = after_launch(stream, "bwd_data");
  if (st != AA_OK) return st;
  if (dsp.nparts > 1) {
    const int nparts = dsp.nparts;
    const int64_t n = M * (plan.b_in / 4);
    const int blocks = int(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
    if (f32) launch((bwd_data_reduce_kernel<float>), dim3(blocks), dim3(256), 0, stream, P, nparts);
    else launch((bwd_data_reduce_kernel<__bf16>), dim3(blocks), dim3(256), 0, stream, P, nparts);
    st = after_launch(stream, "bwd_data_reduce");
  }
  return st;
}

aa_status_t launch_bwd_weight(const aa_plan_s& plan, const void* X, const void* dY, void* dW, int64_t M,
                              int64_t pos_offset, void* ws, hipStream_t stream) {
  const bool f32 = plan.out_dtype == AA_F32;
  if (weight_walk(plan)) {
    BwdWeightParams P{};
    P.X = static_cast<const __bf16*>(X);
    P.dY = static_cast<const __bf16*>(dY);
    P.dW = dW;
    P.M = M;
    P.ldx = plan.d_in;
    P.ldy = plan.d_out;
    P.q = plan.q;
    P.b_in = int32_t(plan.b_in);
    P.b_out = int32_t(plan.b_out);
    P.law = plan.law;
    P.kind = plan.type_kind;
    P.off_mod_q = int32_t(pos_offset % plan.q);
    P.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? M / plan.q : 0;
    P.nchunks = int((plan.b_out / 16 + kWalkNC - 1) / kWalkNC);
    P.ndin = int((plan.b_in + 63) / 64);
    P.ldsx = lds_pitch(64);
    P.ldsy = lds_pitch(16 * kWalkNC);
    const size_t lds = size_t(2) * 64 * (2 * P.ldsx + P.ldsy) * 2;
    const int64_t n_items = int64_t(plan.q) * P.nchunks * P.ndin;
    const int grid = int((n_items + kNumXcd - 1) / kNumXcd * kNumXcd);
    if (f32) launch((bwd_weight_walk_kernel<float, kWalkNC, 4>), dim3(grid), dim3(256), lds, stream, P);
    else launch((bwd_weight_walk_kernel<__bf16, kWalkNC, 4>), dim3(grid), dim3(256), lds, stream, P);
    return after_launch(stream, "bwd_weight_walk");
  }
  if (plan.law == AA_LAW_QQ) {
    const TileSplit ts = tile_split(plan, M);
    if (ts.units >= (int64_t(1) << 31)) return fail(AA_ERR_UNSUPPORTED, "aa_project_bwd_weight: too many rows");
    WTileParams T{};
    T.X = static_cast<const __bf16*>(X);
    T.dY = static_cast<const __bf16*>(dY);
    T.dW = dW;
    T.ws = static_cast<float*>(ws);
    T.M = M;
    T.ldx = plan.d_in;
    T.ldy = plan.d_out;
    T.q = plan.q;
    T.b_in = int32_t(plan.b_in);
    T.b_out = int32_t(plan.b_out);
    T.kind = plan.type_kind;
    T.off_mod_q = int32_t(pos_offset % plan.q);
    T.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? M / plan.q : 0;
    T.nch = ts.nch;
    T.ndc = ts.ndc;
    T.P = ts.P;
    T.SB = ts.SB;
    T.SA = ts.SA;
    T.UB = ts.UB;
    T.Uk = ts.Uk;
    T.units = ts.units;
    int grid = device_cu_count() * 2;
    grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
    const size_t lds = size_t(2) * 2 * 64 * 128 * 2;
    if (f32) launch((bwd_weight_tile_kernel<float>), dim3(grid), dim3(256), lds, stream, T);
    else launch((bwd_weight_tile_kernel<__bf16>), dim3(grid), dim3(256), lds, stream, T);
    aa_status_t st = after_launch(stream, "bwd_weight_tile");
    if (st != AA_OK || ts.P == 1) return st;
    BwdWeightParams R{};
    R.dW = dW;
    R.ws = static_cast<float*>(ws);
    R.q = plan.q;
    R.b_in = int32_t(plan.b_in);
    R.b_out = int32_t(plan.b_out);
    R.nparts = ts.P;
    const int64_t n4 = int64_t(plan.q) * plan.b_in * plan.b_out / 4;
    const int blocks = int(n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096);
    if (f32) launch((bwd_weight_reduce_kernel<float>), dim3(blocks), dim3(256), 0, stream, R);
    else launch((bwd_weight_reduce_kernel<__bf16>), dim3(blocks), dim3(256), 0, stream, R);
    return after_launch(stream, "bwd_weight_reduce");
  }
  const WeightShape sh = weight_shape(plan);
  BwdWeightParams P{};
  P.X = static_cast<const __bf16*>(X);
  P.dY = static_cast<const __bf16*>(dY);
  P.dW = dW;
  P.ws = static_cast<float*>(ws);
  P.M = M;
  P.ldx = plan.d_in;
  P.ldy = plan.d_out;
  P.q = plan.q;
  P.b_in = int32_t(plan.b_in);
  P.b_out = int32_t(plan.b_out);
  P.law = plan.law;
  P.kind = plan.type_kind;
  P.off_mod_q = int32_t(pos_offset % plan.q);
  P.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? M / plan.q : 0;
  P.nchunks = sh.nchunks;
  P.ndin = sh.ndin;
  P.ldsx = lds_pitch(64 * sh.nfw);
  P.ldsy = lds_pitch(16 * sh.nc);
  const size_t lds = size_t(2) * 64 * (P.ldsx + P.ldsy) * 2;
  const int64_t n_items = int64_t(plan.q) * sh.nchunks * sh.ndin;
  const int grid = int((n_items + kNumXcd - 1) / kNumXcd * kNumXcd);
  // four register sets (six measured slower: in-flight data beyond L2)
  if (sh.nfw == 2) {
    if (f32) launch((bwd_weight_kernel<float, 2, 2, 4>), dim3(grid), dim3(256), lds, stream, P);
    else launch((bwd_weight_kernel<__bf16, 2, 2, 4>), dim3(grid), dim3(256), lds, stream, P);
  } else {
    if (f32) launch((bwd_weight_kernel<float, 1, 2, 4>), dim3(grid), dim3(256), lds, stream, P);
    else launch((bwd_weight_kernel<__bf16, 1, 2, 4>), dim3(grid), dim3(256), lds, stream, P);
  }
  return after_launch(stream, "bwd_weight");
}

}  // namespace aa
