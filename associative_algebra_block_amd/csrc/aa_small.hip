// HIP kernels (gfx950) for plans whose weight blocks are narrower than the
// 16-wide MFMA fragment the main packed layout is built from: block sides
// b_in and b_out that are multiples of 4 but not both of 16, such as the
// Qwen3-32B FFN shape of the projection table in the agihunt.info review of
// "Change the Product, Keep the Parameters" (5120 -> 25600 features, q = 256:
// 20 x 100 blocks).  The operation is the same row-typed projection: a row of
// type i produces output group k as the sum over the table's input groups j
// of x_j W_jk (Q_q: j in {i, k}; a digraph: {i, k} for an edge i -> k, {i}
// for k = i, nothing otherwise).
//
// Packed layout version 2 (aa_pack_weights for such plans).  Blocks W_jk in
// row-major block order, each b_in * b_out elements.  Inside a block, runs of
// 4 elements: run (kq, n) holds rows 4 kq .. 4 kq + 3 of column n.  Columns
// are taken 16 at a time (a fragment); inside a fragment the runs go kq-major,
// then n.  The last fragment of a block may be narrower (b_out mod 16
// columns, same order).  The element count is exactly b_in * b_out.
//
// Formulation.  As in the main kernels, Y^T = W^T X^T with
// v_mfma_f32_16x16x32_bf16: each lane supplies 8 consecutive k of the A
// operand (weights) and of the B operand (activations).  The K axis of a leaf
// is the concatenation of its input groups, b_in each; since b_in is a
// multiple of 4, a lane's 8 k are two runs of 4 that may come from different
// input groups (blocks), so every lane loads its two 8-byte halves from its
// own addresses.  K past the leaf's end and columns past b_out read zeros.
//
// Work split.  A workgroup (4 waves) computes, for one row type i and one
// m-tile of 64 MF of its rows, a run of kc consecutive output groups, and NF
// of the blocks' 16-column fragments (blockIdx.y picks which, when a block
// has more fragments than one workgroup's registers hold); each
// wave owns MF 16-row fragments and walks the output groups, with the loads
// of the next output group in flight while it multiplies the current one
// (NSET = 2).  Outputs are stored straight from the accumulators: a lane holds
// 4 consecutive columns of one row.  Tiles are dealt so that each XCD runs a
// contiguous part of the (type, m-tile, output-group run) order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "aa_device.h"
#include "aa_internal.h"

namespace aa {
namespace {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct SmallParams {
  const __bf16* X;
  const __bf16* W0;
  const __bf16* W1;
  void* Y;
  int64_t M;
  int64_t ldx;
  int64_t ldy;
  int32_t q;
  int32_t b_in;
  int32_t b_out;
  int32_t law;
  int32_t kind;            // position or block-row typing
  int32_t off_mod_q;
  int64_t rows_per_type;   // block-row typing
  int32_t mt_count;        // m-tiles per row type
  int32_t kc;              // output groups per tile
  int32_t kchunks;         // tiles per (row type, m-tile)
  uint32_t n_tiles;
  uint64_t adj[64];        // digraph: bit k of adj[i] = edge i -> k
};

// Element offset of run (kq, n) inside a block of the version-2 layout.
__device__ __host__ inline int64_t v2_run(int b_in, int b_out, int kq, int n) {
  const int nfull = b_out >> 4;
  const int f = n >> 4;
  if (f < nfull) return int64_t(f) * 16 * b_in + kq * 64 + (n & 15) * 4;
  const int w = b_out - nfull * 16;
  return int64_t(nfull) * 16 * b_in + int64_t(kq) * 4 * w + (n - nfull * 16) * 4;
}

__device__ inline u32x2_t load8(const __bf16* p) { return *reinterpret_cast<const u32x2_t*>(p); }
__device__ inline Run<__bf16> join(u32x2_t lo, u32x2_t hi) {
  Run<__bf16> r;
  r.v = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  return r;
}

// Output store modes (tuning): 0 and 1 store each lane's four columns straight
// from the accumulators (nontemporal / cached); 2 and 3 first stage the
// wave's rows in LDS and store them as consecutive 4-column runs along each
// row (cached / nontemporal), so that one store instruction covers whole
// stretches of a few rows instead of 32-byte pieces of 16 rows.
template <int S, int NF, int MF, int NSET, bool SWIGLU, typename Tout, int STORE>
__global__ __launch_bounds__(256) void leaf_small_kernel(SmallParams p) {
  constexpr int NW = 4;
  constexpr int SROW = NF * 16 + 4;   // staged row stride (elements)
  __shared__ __attribute__((aligned(16))) Tout stage[STORE >= 2 ? NW * 16 * MF * SROW : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);

  // this workgroup's tile: XCD x (blockIdx mod 8) takes a contiguous run of
  // the tile order (row type, m-tile, run of output groups)
  const uint32_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  uint32_t t = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int chunk = int(t % uint32_t(p.kchunks));
  t /= uint32_t(p.kchunks);
  const int mt = int(t % uint32_t(p.mt_count));
  const int i = int(t / uint32_t(p.mt_count));
  const int f0 = int(blockIdx.y) * NF;   // this launch row's first 16-column fragment
  const int k0 = chunk * p.kc;
  const int k1 = k0 + p.kc < p.q ? k0 + p.kc : p.q;
  if (k0 >= k1) return;

  // rows of type i in closed form
  int64_t first, stride, count;
  if (p.kind == AA_TYPES_BLOCK_ROWS) {
    first = int64_t(i) * p.rows_per_type;
    stride = 1;
    count = p.rows_per_type;
  } else {
    int64_t r0 = int64_t(i) - p.off_mod_q;
    if (r0 < 0) r0 += p.q;
    first = r0;
    stride = p.q;
    count = r0 < p.M ? (p.M - r0 + p.q - 1) / p.q : 0;
  }
  int64_t xoff[MF], yoff[MF];
  bool rv[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int64_t r = (int64_t(mt) * NW * MF + wave * MF + mf) * 16 + l16;
    rv[mf] = r < count;
    const int64_t row = rv[mf] ? first + r * stride : 0;   // rows past the type's last re-read row 0
    xoff[mf] = row * p.ldx;
    yoff[mf] = row * p.ldy;
  }

  // K position of each of this lane's runs: step s, half h covers leaf k
  // 32 s + 8 g + 4 h .. + 3, which lies in input-group slot si at offset lk
  int si[S][2], lk[S][2];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 32 * s + 8 * g + 4 * h;
      si[s][h] = kk / p.b_in;
      lk[s][h] = kk - si[s][h] * p.b_in;
    }
  const uint64_t adj_row = p.law == AA_LAW_DIGRAPH ? p.adj[i] : 0;
  const int64_t blk_elems = int64_t(p.b_in) * p.b_out;

  struct Set {
    u32x2_t a0[S][NF][2], a1[S][NF][2], b[S][MF][2];
  };
  auto load = [&](int k, Set& st) __attribute__((always_inline)) {
    int sg[4] = {0, 0, 0, 0};
    const int nseg = device_leaf_groups(p.law, i, k, sg, adj_row);
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool kv = si[s][h] < nseg;
        const int seg = si[s][h] == 0 ? sg[0] : sg[1];
        const __bf16* wblk0 = p.W0 + (int64_t(seg) * p.q + k) * blk_elems;
        const __bf16* wblk1 = SWIGLU ? p.W1 + (int64_t(seg) * p.q + k) * blk_elems : nullptr;
        const int kq = lk[s][h] >> 2;
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
          st.b[s][mf][h] = load8(kv ? p.X + xoff[mf] + int64_t(seg) * p.b_in + lk[s][h] : zero);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int n = (f0 + f) * 16 + l16;
          const bool ok = kv && n < p.b_out;
          const int64_t o = ok ? v2_run(p.b_in, p.b_out, kq, n) : 0;
          st.a0[s][f][h] = load8(ok ? wblk0 + o : zero);
          if (SWIGLU) st.a1[s][f][h] = load8(ok ? wblk1 + o : zero);
        }
      }
  };
  auto compute_store = [&](int k, const Set& st, bool live) __attribute__((always_inline)) {
    f32x4_t acc0[NF][MF], acc1[NF][MF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        acc0[f][mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[f][mf] = acc0[f][mf];
      }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const Run<__bf16> xb = join(st.b[s][mf][0], st.b[s][mf][1]);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          acc0[f][mf] = mma(join(st.a0[s][f][0], st.a0[s][f][1]), xb, acc0[f][mf]);
          if (SWIGLU) acc1[f][mf] = mma(join(st.a1[s][f][0], st.a1[s][f][1]), xb, acc1[f][mf]);
        }
      }
    if (!live) return;
    Tout* Y = static_cast<Tout*>(p.Y);
    const int64_t col0 = int64_t(k) * p.b_out + f0 * 16;
    Tout* st_w = stage + wave * 16 * MF * SROW;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        f32x4_t v = acc0[f][mf];
        if (SWIGLU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[f][mf][e], acc1[f][mf][e]);
        }
        if constexpr (STORE >= 2) {
          store4(st_w + (mf * 16 + l16) * SROW + f * 16 + 4 * g, v);
        } else {
          // b_out is a multiple of 4: a lane's four columns are all in or all out
          if (rv[mf] && (f0 + f) * 16 + 4 * g < p.b_out) {
            if (STORE == 0) store4_nt(Y + yoff[mf] + col0 + f * 16 + 4 * g, v);
            else store4(Y + yoff[mf] + col0 + f * 16 + 4 * g, v);
          }
        }
      }
    if constexpr (STORE >= 2) {
      // this wave's staged rows back out as runs of 4 columns along each row
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
      const int ncol = p.b_out - f0 * 16 < NF * 16 ? p.b_out - f0 * 16 : NF * 16;
      const int cpr = ncol >> 2;
      const int total = 16 * MF * cpr;
      for (int e = lane; e < total; e += 64) {
        const int r = e / cpr, c = (e - r * cpr) * 4;
        const int64_t rr = (int64_t(mt) * NW * MF + wave * MF) * 16 + r;
        if (rr < count) {
          Tout* dst = Y + (first + rr * stride) * p.ldy + col0 + c;
          const Tout* src = st_w + r * SROW + c;
          if constexpr (sizeof(Tout) == 2) {
            const u32x2_t val = *reinterpret_cast<const u32x2_t*>(src);
            if (STORE == 3) __builtin_nontemporal_store(val, reinterpret_cast<u32x2_t*>(dst));
            else *reinterpret_cast<u32x2_t*>(dst) = val;
          } else {
            const u32x4_t val = *reinterpret_cast<const u32x4_t*>(src);
            if (STORE == 3) __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(dst));
            else *reinterpret_cast<u32x4_t*>(dst) = val;
          }
        }
      }
    }
  };

  // Output groups k0 .. k1 - 1, two per round with the next one's loads in
  // flight (NSET = 2); a step past k1 - 1 re-loads the last group and stores
  // nothing, so no load sits behind a branch.
  const int nk = k1 - k0;
  if (NSET == 1) {
    Set A;
    for (int u = 0; u < nk; ++u) {
      load(k0 + u, A);
      compute_store(k0 + u, A, true);
    }
  } else {
    Set A, B;
    load(k0, A);
    for (int u = 0; u < nk; u += 2) {
      load(k0 + u + 1 < k1 ? k0 + u + 1 : k1 - 1, B);
      compute_store(k0 + u, A, true);
      load(k0 + u + 2 < k1 ? k0 + u + 2 : k1 - 1, A);
      compute_store(k0 + u + 1, B, u + 1 < nk);
    }
  }
}

// ---- LDS-staged variant: plain projections whose leaves are at most 64 deep
// (b_in <= 32) with blocks of at most 4096 elements, e.g. the Qwen3-32B 20 x 100
// blocks.  The kernel above has every wave load all weight runs of a leaf for
// itself (16 KB of registers per wave and output group), which limits a CU to
// two workgroups and one output group of loads in flight each.  Here the four
// waves of a workgroup (one 16-row fragment each, 64 rows) share one copy of
// an output group's two weight blocks and activation segments: all 256
// threads load them (a few 16-byte runs each) two output groups ahead into
// registers and write them to one of two LDS stage buffers, and each wave
// reads its MFMA operands from there.  The type's own activation block is
// staged once per tile.  LDS per workgroup: two stages of 2 b_in b_out + 64
// b_in bf16 values, the own block (64 b_in), and each wave's output ring.
//
// Outputs leave in whole 128-byte lines.  A workgroup's output groups are
// consecutive, so its columns of a row form one stretch, written b_out
// columns per group.  Each wave keeps its 16 rows' unwritten columns in a
// ring of one line plus b_out columns, and after each group stores only the
// lines that are complete (after the run's last group, the rest): the memory
// side then sees no line written in two pieces at different times, which
// costs a read-modify-write of the line.  Runs of output groups are rounded
// so that they start on a line where the row length allows.
//
// What bounds it at the Qwen3-32B shape: the LDS traffic of the operands
// (each of the four waves reads both weight blocks of every group) and the
// store pattern (each wave keeps 16 rows a q apart in progress, a few
// hundred bytes per row per group), in about equal parts.
constexpr int kLdsTM = 64;

__host__ __device__ inline int ring_cols(int b_out, int out_bytes) { return 128 / out_bytes + b_out; }

struct LdsRegions {
  int w, xd, xo, out, total;   // byte offsets of the regions, total bytes
};
__host__ __device__ inline LdsRegions lds_regions(int b_in, int b_out, int out_bytes) {
  const int wb = 2 * b_in * b_out * 2, xb = kLdsTM * b_in * 2;
  LdsRegions r;
  r.w = 0;
  r.xd = 2 * wb;
  r.xo = r.xd + 2 * xb;
  r.out = (r.xo + xb + 15) / 16 * 16;
  r.total = r.out + 4 * 16 * ring_cols(b_out, out_bytes) * out_bytes;
  return r;
}

// WPT: 16-byte weight runs per thread and stage (two blocks of up to 1024 WPT
// bf16 values); XPT: 8-byte activation runs per thread and stage (64 rows of
// up to 32 k).
template <int S, int NF, int WPT, typename Tout>
__global__ __launch_bounds__(256, WPT == 4 ? 2 : 3) void leaf_small_lds_kernel(SmallParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int XPT = 2;
  constexpr int LE = 128 / int(sizeof(Tout));   // elements of a 128-byte line
  const int tid = int(threadIdx.x), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addresses, scalar buffer range
  const int g = lane >> 4, l16 = lane & 15;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  const LdsRegions R = lds_regions(p.b_in, p.b_out, int(sizeof(Tout)));

  const uint32_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  uint32_t t = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int chunk = int(t % uint32_t(p.kchunks));
  t /= uint32_t(p.kchunks);
  const int mt = int(t % uint32_t(p.mt_count));
  const int i = int(t / uint32_t(p.mt_count));
  const int k0 = chunk * p.kc;   // one launch row: NF 16 >= b_out
  const int k1 = k0 + p.kc < p.q ? k0 + p.kc : p.q;
  if (k0 >= k1) return;

  int64_t first, stride, count;
  if (p.kind == AA_TYPES_BLOCK_ROWS) {
    first = int64_t(i) * p.rows_per_type;
    stride = 1;
    count = p.rows_per_type;
  } else {
    int64_t r0 = int64_t(i) - p.off_mod_q;
    if (r0 < 0) r0 += p.q;
    first = r0;
    stride = p.q;
    count = r0 < p.M ? (p.M - r0 + p.q - 1) / p.q : 0;
  }
  const int64_t m0 = int64_t(mt) * kLdsTM;
  auto grow = [&](int r) -> int64_t { return m0 + r < count ? first + (m0 + r) * stride : 0; };

  const int blk_el = p.b_in * p.b_out;
  const int q4n = p.b_in >> 2;                    // 8-byte runs per activation row segment
  const int n_wc = blk_el * 4 / 16;               // 16-byte runs of the two blocks of a stage
  const int n_xr = kLdsTM * q4n;                  // 8-byte runs of a stage's activation segments
  const uint64_t adj_row = p.law == AA_LAW_DIGRAPH ? p.adj[i] : 0;

  // per-thread activation rows of the stage runs (fixed for the tile)
  int64_t xrow[XPT];
  int xq[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int r = tid + 256 * j;
    const int row = r < n_xr ? r / q4n : 0;
    xq[j] = r < n_xr ? r - row * q4n : 0;
    xrow[j] = grow(row) * p.ldx;
  }

  struct Set {
    u32x4_t w[WPT];
    u32x2_t x[XPT];
  };
  // Stage k: blocks (g0, k) and (g1, k) of the leaf's input groups (a diagonal
  // leaf, or a digraph leaf without an edge, re-reads valid blocks its zero
  // K masks out), and the rows' activation segment of group k.
  auto load = [&](int k, Set& st) __attribute__((always_inline)) {
    int sg[4] = {0, 0, 0, 0};
    const int nseg = device_leaf_groups(p.law, i, k, sg, adj_row);
    const int g0 = nseg > 0 ? sg[0] : i, g1 = nseg > 1 ? sg[1] : g0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int c = tid + 256 * j;
      const int e = c * 8;   // element offset in the stage (8 bf16 per run)
      const int slot2 = e >= blk_el ? 1 : 0;
      const __bf16* src = p.W0 + (int64_t(slot2 ? g1 : g0) * p.q + k) * blk_el + (e - slot2 * blk_el);
      st.w[j] = *reinterpret_cast<const u32x4_t*>(c < n_wc ? src : zero);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const __bf16* src = p.X + xrow[j] + int64_t(k) * p.b_in + 4 * xq[j];
      st.x[j] = *reinterpret_cast<const u32x2_t*>(tid + 256 * j < n_xr ? src : zero);
    }
  };
  auto store = [&](int buf, const Set& st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int c = tid + 256 * j;
      if (c < n_wc) *reinterpret_cast<u32x4_t*>(lds + R.w + buf * blk_el * 4 + c * 16) = st.w[j];
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int r = tid + 256 * j;
      if (r < n_xr) *reinterpret_cast<u32x2_t*>(lds + R.xd + buf * kLdsTM * p.b_in * 2 + r * 8) = st.x[j];
    }
  };

  // the type's own activation block, once per tile
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int r = tid + 256 * j;
    const __bf16* src = p.X + xrow[j] + int64_t(i) * p.b_in + 4 * xq[j];
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(r < n_xr ? src : zero);
    if (r < n_xr) *reinterpret_cast<u32x2_t*>(lds + R.xo + r * 8) = v;
  }

  // K position of this lane's runs (as in the kernel above)
  int si[S][2], lk[S][2];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 32 * s + 8 * g + 4 * h;
      si[s][h] = kk / p.b_in;
      lk[s][h] = kk - si[s][h] * p.b_in;
    }
  const int row_l = wave * 16 + l16;
  Tout* Y = static_cast<Tout*>(p.Y);
  const int RR = ring_cols(p.b_out, int(sizeof(Tout)));
  Tout* ring = reinterpret_cast<Tout*>(lds + R.out) + wave * 16 * RR;
  // column c of a row starts a line when (c + ph) is a multiple of LE (rows
  // whose length is a whole number of lines)
  const uint32_t ph = uint32_t((reinterpret_cast<uintptr_t>(p.Y) / sizeof(Tout)) % LE);
  uint32_t written = uint32_t(k0) * uint32_t(p.b_out);   // this wave's rows hold columns < written
  const int64_t wrow0 = m0 + wave * 16;       // this wave's first row of the tile
  const int64_t rows_left = count - wrow0;

  // Write out the complete lines of group k's columns and those before it
  // (after the run's last group, everything), as runs of 4 columns along
  // each row.
  auto flush = [&](int k, bool live) __attribute__((always_inline)) {
    const uint32_t c0 = uint32_t(k) * uint32_t(p.b_out);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's ring writes are done
    const uint32_t end = c0 + uint32_t(p.b_out);
    const uint32_t lb = (end + ph) / LE * LE;
    const uint32_t upto = !live ? written : k == k1 - 1 ? end : lb >= written + ph ? lb - ph : written;
    const int runs = int(upto - written) >> 2;
    const int wbase = int(written % uint32_t(RR));
    for (int e = lane; e < 16 * runs; e += 64) {
      const int r = e / runs, c = (e - r * runs) * 4;
      int slot = wbase + c;
      slot = slot >= RR ? slot - RR : slot;
      if (rows_left > r) {
        Tout* dst = Y + (first + (wrow0 + r) * stride) * p.ldy + written + c;
        const Tout* src = ring + r * RR + slot;
        if constexpr (sizeof(Tout) == 2) *reinterpret_cast<u32x2_t*>(dst) = *reinterpret_cast<const u32x2_t*>(src);
        else *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
    written = upto;
  };
  // Group k from LDS stage buf: the MFMA products, then the outputs into the ring.
  auto mma_to_ring = [&](int buf, int k, bool live) __attribute__((always_inline)) {
    int sg[4] = {0, 0, 0, 0};
    const int nseg = device_leaf_groups(p.law, i, k, sg, adj_row);
    f32x4_t acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const unsigned char* wl = lds + R.w + buf * blk_el * 4;
    const unsigned char* xd = lds + R.xd + buf * kLdsTM * p.b_in * 2;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      u32x2_t xb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool kv = si[s][h] < nseg;
        const unsigned char* base = si[s][h] == 0 ? lds + R.xo : xd;
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(base + (row_l * p.b_in + (kv ? lk[s][h] : 0)) * 2);
        xb[h] = kv ? v : u32x2_t{0u, 0u};
      }
      const Run<__bf16> xr = join(xb[0], xb[1]);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        u32x2_t a[2];
        const int n = f * 16 + l16;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = si[s][h] < nseg && n < p.b_out;
          const int64_t o = ok ? int64_t(si[s][h]) * blk_el + v2_run(p.b_in, p.b_out, lk[s][h] >> 2, n) : 0;
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(wl + o * 2);
          a[h] = ok ? v : u32x2_t{0u, 0u};
        }
        acc[f] = mma(join(a[0], a[1]), xr, acc[f]);
      }
    }
    // group k's columns c0 .. c0 + b_out - 1 into the ring (slot c mod RR; a
    // run of 4 never wraps, RR and c0 + n being multiples of 4)
    const uint32_t c0 = uint32_t(k) * uint32_t(p.b_out);
    const int base = int(c0 % uint32_t(RR));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = f * 16 + 4 * g;
      int slot = base + n;
      slot = slot >= RR ? slot - RR : slot;
      if (live && n < p.b_out) store4(ring + l16 * RR + slot, acc[f]);
    }
  };

  // Output groups k0 .. k1 - 1: stage u + 1 is in registers (loaded one
  // step earlier) and stage u + 2 being loaded while stage u is multiplied
  // from LDS; steps past k1 - 1 re-load the last group and store nothing.
  // A group's lines are stored after the barrier that follows its products,
  // so that the wait for the next stage's loads does not also wait for them.
  const int nk = k1 - k0;
  auto kat = [&](int u) { return k0 + (u < nk ? u : nk - 1); };
  Set A, B;
  load(kat(0), A);
  load(kat(1), B);
  store(0, A);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  for (int u = 0; u < nk; u += 2) {
    load(kat(u + 2), A);
    mma_to_ring(0, kat(u), true);
    store(1, B);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    flush(kat(u), true);
    load(kat(u + 3), B);
    mma_to_ring(1, kat(u + 1), u + 1 < nk);
    store(0, A);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    flush(kat(u + 1), u + 1 < nk);
  }
}

// ---- 32 x 32 fragments: the same staging for output blocks wider than 64
// columns (up to 128, e.g. the Qwen3-32B 20 x 100 blocks).  Measured at that
// shape, the kernel above spends about half its time on LDS operand traffic
// (each of its four waves reads both weight blocks of every group for 16
// rows), and its per-group vector arithmetic (addresses, masks, divisions)
// keeps the SIMDs busy more than half the time.  Here:
//   - The MFMA is v_mfma_f32_32x32x16_bf16: wave (rh, ch) of a 64-row tile
//     computes rows 32 rh .. 32 rh + 31 by columns 64 ch .. 64 ch + 63 (two
//     32-column fragments), so each weight value read from LDS feeds 32 rows.
//     Lane l of a fragment supplies 8 consecutive k (two runs of 4, k = 16 s +
//     8 (l / 32)) of column l mod 32 (weights) and of row l mod 32
//     (activations); register r of the result is column 8 (r / 4) + 4 (l / 32)
//     + r mod 4 of row l mod 32.
//   - Every LDS address a lane uses is fixed for the tile.  A stage's second
//     weight block is staged as zeros when the leaf has fewer input groups
//     (so no per-group masks), K positions past the leaf read a zero run, and
//     staging lanes without a run write to a dummy cell.
//   - The output ring is shared by the two column halves: it holds one line
//     plus two groups of columns per row, so that a wave may write group u + 1
//     while another still stores lines of group u.  After each group's
//     barrier wave w stores the complete lines of rows 16 w .. 16 w + 15, four
//     rows per store instruction with 16 lanes along each row, so that a store
//     covers whole lines.
// Loads run NSET - 1 groups ahead in register sets.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ inline f32x16_t mma32(const Run<__bf16>& a, const Run<__bf16>& b, f32x16_t acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                 acc, 0, 0, 0);
}

// Ring columns: one line plus two groups, padded to 4 times an odd number so
// that the 32 rows of a fragment's ring writes fall on distinct banks.
__host__ __device__ inline int ring32_cols(int b_out, int out_bytes) {
  int rr = (128 / out_bytes + 2 * b_out + 3) / 4 * 4;
  if ((rr / 4) % 2 == 0) rr += 4;
  return rr;
}
// LDS of the 32 x 32 fragment kernel (bytes): two weight stages, each of the
// two blocks followed by a 16-byte zero run; two activation stages; the own
// activation block; a 16-byte zero run and a 16-byte dummy cell; the ring.
struct T32Regions {
  int wst, xd, xo, zero, dummy, out, total;
};
__host__ __device__ inline T32Regions lds32_regions(int b_in, int b_out, int out_bytes) {
  const int xb = kLdsTM * b_in * 2;
  T32Regions r;
  r.wst = 2 * b_in * b_out * 2 + 16;   // stage stride; stage b starts at b * wst
  r.xd = 2 * r.wst;
  r.xo = r.xd + 2 * xb;
  r.zero = (r.xo + xb + 15) / 16 * 16;
  r.dummy = r.zero + 16;
  r.out = r.dummy + 16;
  r.total = r.out + kLdsTM * ring32_cols(b_out, out_bytes) * out_bytes;
  return r;
}

template <int KS, int WPT, int NSET, typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_small_t32_kernel(SmallParams p) {
  static_assert(NSET % 2 == 0, "set parity is the LDS buffer");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int XPT = 2;
  constexpr int LE = 128 / int(sizeof(Tout));   // elements of a 128-byte line
  constexpr int SZ = int(sizeof(Tout));
  const int tid = int(threadIdx.x), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave & 1, chh = wave >> 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const __bf16* zero = reinterpret_cast<const __bf16*>(g_zero_runs);
  const T32Regions R = lds32_regions(p.b_in, p.b_out, SZ);

  const uint32_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  uint32_t t = xcd * per + (xcd < rem ? xcd : rem) + slot;
  if (t >= p.n_tiles) return;
  const int chunk = int(t % uint32_t(p.kchunks));
  t /= uint32_t(p.kchunks);
  const int mt = int(t % uint32_t(p.mt_count));
  const int i = int(t / uint32_t(p.mt_count));
  const int k0 = chunk * p.kc;
  const int k1 = k0 + p.kc < p.q ? k0 + p.kc : p.q;
  if (k0 >= k1) return;

  int64_t first, stride, count;
  if (p.kind == AA_TYPES_BLOCK_ROWS) {
    first = int64_t(i) * p.rows_per_type;
    stride = 1;
    count = p.rows_per_type;
  } else {
    int64_t r0 = int64_t(i) - p.off_mod_q;
    if (r0 < 0) r0 += p.q;
    first = r0;
    stride = p.q;
    count = r0 < p.M ? (p.M - r0 + p.q - 1) / p.q : 0;
  }
  const int64_t m0 = int64_t(mt) * kLdsTM;
  auto grow = [&](int r) -> int64_t { return m0 + r < count ? first + (m0 + r) * stride : 0; };

  const int blk_el = p.b_in * p.b_out;
  const int q4n = p.b_in >> 2;
  const int n_wc = blk_el * 4 / 16;          // 16-byte runs of a stage's two blocks
  const int n_xr = kLdsTM * q4n;             // 8-byte runs of a stage's activation segments
  const uint64_t adj_row = p.law == AA_LAW_DIGRAPH ? p.adj[i] : 0;

  // ---- staging: each thread's runs, fixed for the tile
  int w_off[WPT], w_slot[WPT], w_dst[WPT];   // element offset in its block, block slot, LDS byte offset
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int c = tid + 256 * j;
    const int e = c * 8;
    w_slot[j] = c < n_wc ? (e >= blk_el ? 1 : 0) : 2;   // 2: no run
    w_off[j] = c < n_wc ? e - (e >= blk_el ? blk_el : 0) : 0;
    w_dst[j] = c < n_wc ? c * 16 : -1;
  }
  const __bf16* x_src[XPT];                  // the run's row and column inside an activation group
  int x_dst[XPT];                            // LDS byte offset inside an activation stage
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int r = tid + 256 * j;
    const int row = r < n_xr ? r / q4n : 0;
    const int xq = r < n_xr ? r - row * q4n : 0;
    x_src[j] = p.X + grow(row) * p.ldx + 4 * xq;
    x_dst[j] = r < n_xr ? r * 8 : -1;
  }

  struct Set {
    u32x4_t w[WPT];
    u32x2_t x[XPT];
  };
  // Group k: blocks (g0, k) and (g1, k) of the leaf's input groups, zeros for
  // a slot past the leaf's group count, and the rows' activation segment k.
  auto load = [&](int k, Set& st) __attribute__((always_inline)) {
    int sg[4] = {0, 0, 0, 0};
    const int nseg = __builtin_amdgcn_readfirstlane(device_leaf_groups(p.law, i, k, sg, adj_row));
    // block numbers are the same in every lane: keep their products scalar
    const int gb0 = __builtin_amdgcn_readfirstlane((nseg > 0 ? sg[0] : i) * p.q + k);
    const int gb1 = __builtin_amdgcn_readfirstlane((nseg > 1 ? sg[1] : i) * p.q + k);
    const __bf16* b0 = p.W0 + int64_t(gb0) * blk_el;
    const __bf16* b1 = p.W0 + int64_t(gb1) * blk_el;
    const int64_t xk = int64_t(__builtin_amdgcn_readfirstlane(k)) * p.b_in;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const __bf16* src = w_slot[j] < nseg ? (w_slot[j] == 0 ? b0 : b1) + w_off[j] : zero;
      st.w[j] = *reinterpret_cast<const u32x4_t*>(src);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const __bf16* src = x_dst[j] >= 0 ? x_src[j] + xk : zero;
      st.x[j] = *reinterpret_cast<const u32x2_t*>(src);
    }
  };
  auto store = [&](int buf, const Set& st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      *reinterpret_cast<u32x4_t*>(lds + (w_dst[j] >= 0 ? buf * R.wst + w_dst[j] : R.dummy)) = st.w[j];
#pragma unroll
    for (int j = 0; j < XPT; ++j)
      *reinterpret_cast<u32x2_t*>(lds + (x_dst[j] >= 0 ? R.xd + buf * kLdsTM * p.b_in * 2 + x_dst[j] : R.dummy)) =
          st.x[j];
  };

  // the zero runs (the weight stages' tails and the activation one) and the
  // type's own activation block, once per tile
  if (tid < 3)
    *reinterpret_cast<u32x4_t*>(lds + (tid < 2 ? tid * R.wst + 2 * blk_el * 2 : R.zero)) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(x_dst[j] >= 0 ? x_src[j] + int64_t(i) * p.b_in : zero);
    *reinterpret_cast<u32x2_t*>(lds + (x_dst[j] >= 0 ? R.xo + x_dst[j] : R.dummy)) = v;
  }

  // ---- operand addresses (LDS bytes), fixed for the tile: k-step s, half h
  // covers leaf k 16 s + 8 hi + 4 h .. + 3, in input-group slot si at offset lk.
  // Weights: relative to the stage; past the leaf's K (si >= 2) or past the
  // block's columns, the stage's zero tail.  Activations: per stage buffer
  // (slot 0: the own block, slot 1: the stage's segment, beyond: a zero run).
  int a_ofs[KS][2][2], b_ofs[2][KS][2];
  const int row_l = 32 * rh + l32;   // this lane's tile row (B operand and outputs)
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 16 * s + 8 * hi + 4 * h;
      const int si = kk / p.b_in, lk = kk - si * p.b_in;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = 64 * chh + 32 * f + l32;
        a_ofs[s][h][f] = si < 2 && n < p.b_out ? (si * blk_el + int(v2_run(p.b_in, p.b_out, lk >> 2, n))) * 2
                                               : 2 * blk_el * 2;
      }
      const int xo = (row_l * p.b_in + lk) * 2;
#pragma unroll
      for (int b = 0; b < 2; ++b)
        b_ofs[b][s][h] = si == 0 ? R.xo + xo : si == 1 ? R.xd + b * kLdsTM * p.b_in * 2 + xo : R.zero;
    }

  // ---- ring: this lane's row for its results; the 8 (fragment, register
  // quad) column offsets; the dummy cell for columns past the block
  const int RR = ring32_cols(p.b_out, SZ);
  const int ring_row = R.out + row_l * RR * SZ;
  int r_col[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) r_col[f][j] = 64 * chh + 32 * f + 8 * j + 4 * hi;

  // ---- stores: row group rg (0..3) of this wave's 16 rows is tile row
  // 16 wave + 4 rg + lane / 16; lane mod 16 picks the run along the row
  Tout* Y = static_cast<Tout*>(p.Y);
  const uint32_t ph = uint32_t((reinterpret_cast<uintptr_t>(p.Y) / sizeof(Tout)) % LE);
  uint32_t written = uint32_t(k0) * uint32_t(p.b_out);   // every row holds columns < written
  // ring slots of column `written` and of the next group's first column, kept
  // by addition (a division per group would cost more than the group's
  // address arithmetic)
  uint32_t wbase = written % uint32_t(RR), cbase = wbase;
  Tout* f_row[4];
  bool f_ok[4];
  int f_ring[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    const int tr = 16 * wave + 4 * rg + (lane >> 4);
    f_ok[rg] = m0 + tr < count;
    f_row[rg] = Y + (f_ok[rg] ? first + (m0 + tr) * stride : 0) * p.ldy;
    f_ring[rg] = R.out + tr * RR * SZ;
  }
  const int run_l = lane & 15;

  auto flush = [&](int k, bool live) __attribute__((always_inline)) {
    const uint32_t end = uint32_t(k) * uint32_t(p.b_out) + uint32_t(p.b_out);
    const uint32_t lb = (end + ph) / LE * LE;
    const uint32_t upto = !live ? written : k == k1 - 1 ? end : lb >= written + ph ? lb - ph : written;
    const int runs = int(upto - written) >> 2;
    for (int m = 0; m < runs; m += 16) {
      const int run = m + run_l;
      int sl = int(wbase) + 4 * run;
      sl = sl >= RR ? sl - RR : sl;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const unsigned char* src = lds + f_ring[rg] + sl * SZ;
        Tout* dst = f_row[rg] + written + 4 * run;
        if constexpr (SZ == 2) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(src);
          if (f_ok[rg] && run < runs) *reinterpret_cast<u32x2_t*>(dst) = v;
        } else {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
          if (f_ok[rg] && run < runs) *reinterpret_cast<u32x4_t*>(dst) = v;
        }
      }
    }
    wbase += upto - written;
    wbase = wbase >= uint32_t(RR) ? wbase - uint32_t(RR) : wbase;
    written = upto;
  };
  auto mma_to_ring = [&](int buf, int k, bool live) __attribute__((always_inline)) {
    f32x16_t acc[2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;
    const unsigned char* wl = lds + buf * R.wst;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Run<__bf16> xr = join(*reinterpret_cast<const u32x2_t*>(lds + b_ofs[buf][s][0]),
                                  *reinterpret_cast<const u32x2_t*>(lds + b_ofs[buf][s][1]));
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const Run<__bf16> ar = join(*reinterpret_cast<const u32x2_t*>(wl + a_ofs[s][0][f]),
                                    *reinterpret_cast<const u32x2_t*>(wl + a_ofs[s][1][f]));
        acc[f] = mma32(ar, xr, acc[f]);
      }
    }
    if (!live) return;
    const int base = int(cbase);
    cbase += uint32_t(p.b_out);
    cbase = cbase >= uint32_t(RR) ? cbase - uint32_t(RR) : cbase;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int sl = base + r_col[f][j];
        sl = sl >= RR ? sl - RR : sl;
        const int at = r_col[f][j] < p.b_out ? ring_row + sl * SZ : R.dummy;
        store4(reinterpret_cast<Tout*>(lds + at),
               f32x4_t{acc[f][4 * j], acc[f][4 * j + 1], acc[f][4 * j + 2], acc[f][4 * j + 3]});
      }
  };

  // Output groups k0 .. k1 - 1, NSET per round: stage v is in register set
  // v mod NSET from NSET - 1 steps before its products and in LDS buffer
  // v mod 2 from the barrier before them.  Steps past k1 - 1 re-load the
  // last group and store nothing.
  const int nk = k1 - k0;
  auto kat = [&](int u) { return k0 + (u < nk ? u : nk - 1); };
  Set S[NSET];
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) load(kat(s), S[s]);
  store(0, S[0]);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  for (int u = 0; u < nk; u += NSET) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      load(kat(u + s + NSET - 1), S[(s + NSET - 1) % NSET]);
      mma_to_ring(s & 1, kat(u + s), u + s < nk);
      store((s + 1) & 1, S[(s + 1) % NSET]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      flush(kat(u + s), u + s < nk);
    }
  }
}

// Thread c moves run c (4 elements) of the version-2 layout from or to the
// row-major weight.
template <typename T>
__global__ __launch_bounds__(256) void pack_v2_kernel(const T* __restrict__ src, T* __restrict__ dst, int32_t q,
                                                      int32_t b_in, int32_t b_out, int64_t d_out, int64_t n_runs,
                                                      bool unpack) {
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= n_runs) return;
  const int64_t runs_per_blk = int64_t(b_in) * b_out / 4;
  const int64_t blk = c / runs_per_blk;
  const int64_t w = c - blk * runs_per_blk;
  const int64_t j = blk / q, kb = blk % q;
  const int64_t nfull = b_out / 16, full_runs = nfull * 4 * b_in;
  int64_t kq, n;
  if (w < full_runs) {
    const int64_t f = w / (4 * b_in), r = w - f * 4 * b_in;
    kq = r / 16;
    n = f * 16 + r % 16;
  } else {
    const int64_t width = b_out - nfull * 16, r = w - full_runs;
    kq = r / width;
    n = nfull * 16 + r % width;
  }
  const int64_t row = j * b_in + 4 * kq, col = kb * b_out + n;
  if (!unpack) {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[c * 4 + e] = src[(row + e) * d_out + col];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(row + e) * d_out + col] = src[c * 4 + e];
  }
}

template <int S, int NF, int MF, int NSET, bool SW, int STORE>
void go_small_st(const SmallParams& p, bool fout, dim3 grid, hipStream_t s) {
  const dim3 block{256, 1, 1};
  if (fout) launch((leaf_small_kernel<S, NF, MF, NSET, SW, float, STORE>), grid, block, 0, s, p);
  else launch((leaf_small_kernel<S, NF, MF, NSET, SW, __bf16, STORE>), grid, block, 0, s, p);
}

// The store mode is a tuning override for the Qwen3-32B-shaped instance
// (600 + mode); every other instance uses the default mode.
constexpr int kSmallStoreDefault = 2;
template <int S, int NF, int MF, int NSET, bool SW>
void go_small(const SmallParams& p, bool fout, dim3 grid, hipStream_t s, int store) {
  if constexpr (S == 2 && NF == 8 && !SW) {
    switch (store) {
      case 0: return go_small_st<S, NF, MF, NSET, SW, 0>(p, fout, grid, s);
      case 1: return go_small_st<S, NF, MF, NSET, SW, 1>(p, fout, grid, s);
      case 3: return go_small_st<S, NF, MF, NSET, SW, 3>(p, fout, grid, s);
      default: break;
    }
  }
  go_small_st<S, NF, MF, NSET, SW, kSmallStoreDefault>(p, fout, grid, s);
}

// Instances: S k-steps of 32 (the leaf's K padded), NF fragments per
// workgroup.  The registers one lane holds grow with S NF (two loaded sets of
// S NF weight runs for the plain kernel, one set of both weights for the
// SwiGLU one), so S NF is kept at most 16 (plain) or 8 (SwiGLU) and wider
// blocks take several launch rows of fragments.
template <bool SW>
bool go_small_sn(int S, int NF, const SmallParams& p, bool fout, dim3 grid, hipStream_t s, int store) {
  constexpr int MF = SW ? 1 : 2, NSET = SW ? 1 : 2;
#define AA_SMALL(s_, n_)                                \
  if (S == s_ && NF == n_) {                            \
    go_small<s_, n_, MF, NSET, SW>(p, fout, grid, s, store);  \
    return true;                                        \
  }
  AA_SMALL(1, 1) AA_SMALL(1, 2) AA_SMALL(1, 4) AA_SMALL(1, 8)
  AA_SMALL(2, 1) AA_SMALL(2, 2) AA_SMALL(2, 4)
  AA_SMALL(4, 1) AA_SMALL(4, 2)
  AA_SMALL(8, 1)
  if constexpr (!SW) {
    AA_SMALL(2, 8) AA_SMALL(4, 4) AA_SMALL(8, 2)
  }
#undef AA_SMALL
  return false;
}

}  // namespace

namespace {

template <int S, int NF>
void go_small_lds(const SmallParams& p, bool fout, int wpt, dim3 grid, size_t lds, hipStream_t s) {
  const dim3 block{256, 1, 1};
  if (wpt <= 2) {
    if (fout) launch((leaf_small_lds_kernel<S, NF, 2, float>), grid, block, uint32_t(lds), s, p);
    else launch((leaf_small_lds_kernel<S, NF, 2, __bf16>), grid, block, uint32_t(lds), s, p);
  } else {
    if (fout) launch((leaf_small_lds_kernel<S, NF, 4, float>), grid, block, uint32_t(lds), s, p);
    else launch((leaf_small_lds_kernel<S, NF, 4, __bf16>), grid, block, uint32_t(lds), s, p);
  }
}

// Whether the LDS-staged kernel takes a plan: a plain projection, leaves of
// at most 64 k (b_in <= 32), two blocks per stage within 4 x 256 16-byte runs,
// and its LDS within the 64 KB a launch gets without an attribute.
int small_lds_nf(int64_t b_out) {
  const int nf = int((b_out + 15) / 16);
  return nf <= 2 ? 2 : nf <= 4 ? 4 : 8;
}
bool small_lds_ok(const aa_plan_s& plan, bool swiglu, bool fout) {
  if (swiglu || plan.b_in > 32 || plan.b_out > 128 || plan.b_in * plan.b_out > 4096) return false;
  return lds_regions(int(plan.b_in), int(plan.b_out), fout ? 4 : 2).total <= 65536;
}

template <typename K>
void go_t32_one(K kernel, const SmallParams& p, dim3 grid, size_t lds, hipStream_t s) {
  // beyond 64 KB (the one-workgroup-per-CU tuning mode) the launch needs the attribute
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(lds));
  launch(kernel, grid, dim3{256, 1, 1}, uint32_t(lds), s, p);
}
#ifndef AA_T32_NSET
#define AA_T32_NSET 4
#endif
template <int KS>
void go_small_t32(const SmallParams& p, bool fout, int wpt, dim3 grid, size_t lds, hipStream_t s) {
  constexpr int NS = AA_T32_NSET;
  if (wpt <= 2) {
    if (fout) go_t32_one(leaf_small_t32_kernel<KS, 2, NS, float>, p, grid, lds, s);
    else go_t32_one(leaf_small_t32_kernel<KS, 2, NS, __bf16>, p, grid, lds, s);
  } else {
    if (fout) go_t32_one(leaf_small_t32_kernel<KS, 4, NS, float>, p, grid, lds, s);
    else go_t32_one(leaf_small_t32_kernel<KS, 4, NS, __bf16>, p, grid, lds, s);
  }
}

// The 32 x 32 fragment kernel takes what the LDS-staged one does when the
// output blocks are wider than 64 columns (AA_TILE=611 keeps those on the
// 16 x 16 one).
bool small_t32_ok(const aa_plan_s& plan, bool swiglu, bool fout) {
  if (swiglu || plan.b_in > 32 || plan.b_out <= 64 || plan.b_out > 128 || plan.b_in * plan.b_out > 4096) return false;
  if (plan.tile_override == 611) return false;
  return lds32_regions(int(plan.b_in), int(plan.b_out), fout ? 4 : 2).total <= 65536;
}

// Runs of output groups that start on a 128-byte line: kc b_out columns a
// multiple of a line.
int32_t line_aligned_kc(int32_t kc, int64_t b_out, bool fout, int32_t q) {
  const int le = fout ? 32 : 64;
  int gcd = le, b = int(b_out);
  while (b) {
    const int t = gcd % b;
    gcd = b;
    b = t;
  }
  const int step = le / gcd;
  kc = (kc + step - 1) / step * step;
  return kc > q ? q : kc;
}

// The 32 x 32 fragment kernel: 64-row tiles, about four tiles per CU in all
// (AA_WG_PER_CU sets the count); AA_TILE=612 pads its LDS to hold the grid
// to one workgroup per CU.
aa_status_t launch_small_t32(const aa_plan_s& plan, SmallParams p, int64_t mi, bool fout, hipStream_t stream) {
  p.mt_count = int32_t((mi + kLdsTM - 1) / kLdsTM);
  const int64_t base = int64_t(plan.q) * p.mt_count;
  const int64_t want = int64_t(device_cu_count()) * (plan.wg_per_cu > 0 ? plan.wg_per_cu : 4);
  int64_t chunks = (want + base - 1) / base;
  if (chunks > plan.q) chunks = plan.q;
  p.kc = line_aligned_kc(int32_t((plan.q + chunks - 1) / chunks), plan.b_out, fout, plan.q);
  p.kchunks = int32_t((plan.q + p.kc - 1) / p.kc);
  const int64_t n_tiles = base * p.kchunks;
  if (n_tiles > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
  p.n_tiles = uint32_t(n_tiles);
  const int nseg_max = plan.q > 1 ? 2 : 1;
  const int KS = int((nseg_max * plan.b_in + 15) / 16);
  const int wpt = int((plan.b_in * plan.b_out / 4 + 255) / 256);
  const dim3 grid{uint32_t(n_tiles), 1, 1};
  size_t lds = size_t(lds32_regions(int(plan.b_in), int(plan.b_out), fout ? 4 : 2).total);
  if (plan.tile_override == 612) lds = lds < 90 * 1024 ? 90 * 1024 : lds;
  switch (KS) {
    case 1: go_small_t32<1>(p, fout, wpt, grid, lds, stream); break;
    case 2: go_small_t32<2>(p, fout, wpt, grid, lds, stream); break;
    case 3: go_small_t32<3>(p, fout, wpt, grid, lds, stream); break;
    default: go_small_t32<4>(p, fout, wpt, grid, lds, stream); break;
  }
  return after_launch(stream, "leaf_small_t32");
}

// The LDS-staged kernel: 64-row tiles, runs of output groups for about
// twelve workgroups per CU in all, fragments split over blockIdx.y by 8.
aa_status_t launch_small_lds(const aa_plan_s& plan, SmallParams p, int64_t mi, bool fout, hipStream_t stream) {
  p.mt_count = int32_t((mi + kLdsTM - 1) / kLdsTM);
  const int64_t base = int64_t(plan.q) * p.mt_count;
  const int64_t want = int64_t(device_cu_count()) * (plan.wg_per_cu > 0 ? plan.wg_per_cu : 12);
  int64_t chunks = (want + base - 1) / base;
  if (chunks > plan.q) chunks = plan.q;
  p.kc = line_aligned_kc(int32_t((plan.q + chunks - 1) / chunks), plan.b_out, fout, plan.q);
  p.kchunks = int32_t((plan.q + p.kc - 1) / p.kc);
  const int64_t n_tiles = base * p.kchunks;
  if (n_tiles > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
  p.n_tiles = uint32_t(n_tiles);
  const int S = plan.q > 1 && 2 * plan.b_in > 32 ? 2 : 1;
  const int nf = int((plan.b_out + 15) / 16);
  const int NF = small_lds_nf(plan.b_out);
  const int wpt = int((plan.b_in * plan.b_out / 4 + 255) / 256);
  const dim3 grid{uint32_t(n_tiles), uint32_t((nf + NF - 1) / NF), 1};
  const size_t lds = size_t(lds_regions(int(plan.b_in), int(plan.b_out), fout ? 4 : 2).total);
  if (S == 1) {
    if (NF == 2) go_small_lds<1, 2>(p, fout, wpt, grid, lds, stream);
    else if (NF == 4) go_small_lds<1, 4>(p, fout, wpt, grid, lds, stream);
    else go_small_lds<1, 8>(p, fout, wpt, grid, lds, stream);
  } else {
    if (NF == 2) go_small_lds<2, 2>(p, fout, wpt, grid, lds, stream);
    else if (NF == 4) go_small_lds<2, 4>(p, fout, wpt, grid, lds, stream);
    else go_small_lds<2, 8>(p, fout, wpt, grid, lds, stream);
  }
  return after_launch(stream, "leaf_small_lds");
}

}  // namespace

aa_status_t launch_small_gemm(const aa_plan_s& plan, const LeafCall& call, hipStream_t stream) {
  // plan creation admits layout-2 plans only in the shapes handled here
  if (!small_layout_ok(plan.law, plan.type_kind, plan.in_dtype, plan.b_in, plan.b_out))
    return fail(AA_ERR_UNSUPPORTED, "this plan's block shape has no kernel");
  SmallParams p{};
  p.X = static_cast<const __bf16*>(call.X);
  p.W0 = static_cast<const __bf16*>(call.W0);
  p.W1 = static_cast<const __bf16*>(call.W1);
  p.Y = call.Y;
  p.M = call.M;
  p.ldx = plan.d_in;
  p.ldy = plan.d_out;
  p.q = plan.q;
  p.b_in = int32_t(plan.b_in);
  p.b_out = int32_t(plan.b_out);
  p.law = plan.law;
  p.kind = plan.type_kind;
  p.off_mod_q = int32_t(call.pos_offset % plan.q);
  p.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? call.M / plan.q : 0;
  for (int r = 0; r < 64; ++r) p.adj[r] = plan.adj[r];
  const int mf = call.swiglu ? 1 : 2;
  const int64_t mi = plan.type_kind == AA_TYPES_BLOCK_ROWS ? call.M / plan.q : (call.M + plan.q - 1) / plan.q;
  p.mt_count = int32_t((mi + 64 * mf - 1) / (64 * mf));
  if (p.mt_count < 1) return AA_OK;
  // runs of output groups: enough tiles for about eight workgroups per CU
  const int64_t base = int64_t(plan.q) * p.mt_count;
  const int64_t want = int64_t(device_cu_count()) * 8;
  int64_t chunks = (want + base - 1) / base;
  if (chunks > plan.q) chunks = plan.q;
  p.kc = int32_t((plan.q + chunks - 1) / chunks);
  p.kchunks = int32_t((plan.q + p.kc - 1) / p.kc);
  const int64_t n_tiles = base * p.kchunks;
  if (n_tiles > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
  p.n_tiles = uint32_t(n_tiles);
  const int nseg_max = plan.q > 1 ? 2 : 1;
  const int steps = int((nseg_max * plan.b_in + 31) / 32);
  const int S = steps <= 1 ? 1 : steps <= 2 ? 2 : steps <= 4 ? 4 : 8;
  const int nf = int((plan.b_out + 15) / 16);
  const int budget = (call.swiglu ? 8 : 16) / S;
  int NF = 1;
  while (NF < nf && NF * 2 <= budget) NF *= 2;
  const dim3 grid{uint32_t(n_tiles), uint32_t((nf + NF - 1) / NF), 1};
  const bool fout = plan.out_dtype == AA_F32;
  const int store = plan.tile_override >= 600 && plan.tile_override < 604 ? plan.tile_override - 600
                                                                         : kSmallStoreDefault;
  // plain projections with leaves of at most 64 k and blocks of at most 4096
  // elements: the LDS-staged kernel (AA_TILE=610 forces the register kernel)
  if (small_t32_ok(plan, call.swiglu, fout) && plan.tile_override != 610 &&
      !(plan.tile_override >= 600 && plan.tile_override < 604))
    return launch_small_t32(plan, p, mi, fout, stream);
  if (small_lds_ok(plan, call.swiglu, fout) && plan.tile_override != 610 &&
      !(plan.tile_override >= 600 && plan.tile_override < 604))
    return launch_small_lds(plan, p, mi, fout, stream);
  const bool ok = call.swiglu ? go_small_sn<true>(S, NF, p, fout, grid, stream, store)
                              : go_small_sn<false>(S, NF, p, fout, grid, stream, store);
  if (!ok) return fail(AA_ERR_UNSUPPORTED, "this plan's block shape has no kernel");
  return after_launch(stream, call.swiglu ? "leaf_small(swiglu)" : "leaf_small");
}

aa_status_t launch_pack_v2(const aa_plan_s& plan, const void* src, void* dst, bool unpack, hipStream_t stream) {
  const int64_t n_runs = plan.d_in * plan.d_out / 4;
  if (n_runs == 0) return AA_OK;
  const dim3 block{256, 1, 1}, grid{uint32_t((n_runs + 255) / 256), 1, 1};
  // layout-2 plans take bf16 weights only
  launch(pack_v2_kernel<__bf16>, grid, block, 0, stream, static_cast<const __bf16*>(src),
         static_cast<__bf16*>(dst), plan.q, int32_t(plan.b_in), int32_t(plan.b_out), plan.d_out, n_runs, unpack);
  return after_launch(stream, unpack ? "unpack (layout 2)" : "pack (layout 2)");
}

}  // namespace aa
