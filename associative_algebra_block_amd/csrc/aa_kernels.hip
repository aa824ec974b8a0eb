// HIP kernels (gfx950) of libaa.so and their host launchers.
//
// What is computed (agihunt.info review of "Change the Product, Keep the
// Parameters: Associative Algebra Layers for Transformers"; paragraphs on the
// graph multiplication table, on row typing and on the pilot law): a row of
// type i produces output group k as the sum over the table's input groups j of
// x_j W_jk.  Under Q_q those groups are {i, k}; under the tensor square of Q2
// (q = 4) they are the 1, 2 or 4 groups (a', b') with a' in {a, a''} and b' in
// {b, b''}.  Each (type, output group) pair is one "leaf": a dense GEMM whose
// K dimension is the concatenation of its input groups, [x_i | x_k] times
// [W_ik ; W_kk], which is what the MFMA units are used for.
//
// Formulation.  The kernels compute the transposed leaf, Y^T = W^T X^T, with
// the bf16 MFMA v_mfma_f32_16x16x32_bf16: the A operand is a 16 (n) x 32 (k)
// fragment of W^T, the B operand a 32 (k) x 16 (m) fragment of X^T.  Both
// operands then hold 8 consecutive k per lane, so
//   - a weight fragment is one contiguous, fully coalesced 1 KiB read from the
//     block-packed layout (aa_pack_weights writes W in exactly this order), and
//   - an activation fragment is 16 B of one row of X,
// and the 16 x 16 accumulator holds 4 consecutive output columns of one row
// per lane, which are stored straight to row-major Y.  Weights stream from HBM
// directly into registers (no LDS round trip); the X rows of the tile are
// read per wave and shared through the L1/L2 caches.
//
// Work split.  One workgroup computes one tile of one leaf: TM rows of type i
// (strided rows of X under position typing, contiguous under block-row typing,
// a scanned list under explicit typing) by TN columns of output group k.
// Tiles are numbered so that each XCD's share of the grid is one contiguous
// run of output groups, which keeps the diagonal blocks W_kk that every row
// type reads resident in that XCD's L2; within the run, consecutive tiles
// share the row type, so the type's own activation block x_i stays hot too.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <string>
#include <type_traits>

#include "aa_device.h"
#include "aa_internal.h"

// Device memory of the allocation-free SwiGLU call (aa_swiglu_ffn_fwd_noalloc):
// its hidden activation H lives here instead of in a caller buffer.  Every
// GPU the library runs on holds its own copy from module load to process
// exit.  Host code never passes this name to a kernel (on the host it is only
// a stand-in); it uses the device address noalloc_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[aa::kNoAllocScratchBytes];

namespace aa {
namespace {

// ------------------------------------------------------------- leaf GEMM ---

struct LeafParams {
  const void* X;
  const void* W0;
  const void* W1;
  void* Y;
  int64_t M;
  int64_t ldx;
  int64_t ldy;
  int32_t q;
  int32_t b_in;
  int32_t b_out;
  int32_t law;
  int32_t kind;            // aa_type_kind_t
  int32_t off_mod_q;       // pos_offset mod q (position typing)
  int64_t rows_per_type;   // M / q (block-row typing)
  const int32_t* row_types;
  int32_t mt_count;        // m-tiles per leaf
  int32_t nt_count;        // n-tiles per leaf
  int32_t kc;              // output groups per tile-order chunk
  uint32_t n_tiles;
  int32_t cpr;             // streaming kernel: 16-byte LDS chunks per staged activation row
  uint64_t adj[64];        // general kernel, digraph law: bit k of adj[i] = edge i -> k
};

// Rows of type i, in order; fills rows[0..TM) for m-tile mt and returns how
// many are valid.  Position and block-row typing are closed-form.
template <int TM>
__device__ inline int tile_rows_closed_form(const LeafParams& p, int i, int mt, int32_t* rows) {
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
  const int64_t lo = int64_t(mt) * TM;
  const int n = lo >= count ? 0 : int(count - lo < TM ? count - lo : TM);
  for (int r = threadIdx.x; r < TM; r += blockDim.x)
    rows[r] = r < n ? int32_t(first + (lo + r) * stride) : -1;
  return n;
}

// XCD-aware tile numbering: XCD x (= blockIdx.x mod 8) receives a contiguous
// run of the tile order (output-group chunk, row type, output group in the
// chunk, m-tile, n-tile).
__device__ inline void decode_tile(const LeafParams& p, int& i, int& k, int& mt, int& nt) {
  const uint32_t bid = blockIdx.x;
  const uint32_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  uint32_t t = xcd * per + (xcd < rem ? xcd : rem) + slot;
  nt = int(t % uint32_t(p.nt_count));
  t /= uint32_t(p.nt_count);
  mt = int(t % uint32_t(p.mt_count));
  t /= uint32_t(p.mt_count);
  const int kk = int(t % uint32_t(p.kc));
  t /= uint32_t(p.kc);
  i = int(t % uint32_t(p.q));
  k = int(t / uint32_t(p.q)) * p.kc + kk;
}

template <typename Tin, typename Tout, int WN, int WM, int NF, int MF, bool SWIGLU, int STAGES>
__global__ __launch_bounds__(kWave * WN * WM) void leaf_gemm_kernel(LeafParams p) {
  constexpr int TN = WN * NF * 16;
  constexpr int TM = WM * MF * 16;
  __shared__ int32_t rows_lds[TM];
  __shared__ int32_t scan_state[2];

  int i, k, mt, nt;
  decode_tile(p, i, k, mt, nt);

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int wn = wave % WN, wm = wave / WN;
  const int g = lane >> 4;       // which 8-run of the 32-wide k slab
  const int l16 = lane & 15;

  int segs[4];
  const int nseg = device_leaf_groups(p.law, i, k, segs, p.law == AA_LAW_DIGRAPH ? p.adj[i] : 0);
  const int KF = (p.b_in + 31) / 32;
  const int nsteps = nseg * KF;

  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  const Tin* __restrict__ W0 = static_cast<const Tin*>(p.W0);
  const Tin* __restrict__ W1 = static_cast<const Tin*>(p.W1);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);
  const int64_t blk_elems = int64_t(p.b_in) * p.b_out;
  const int nfrag0 = nt * (TN / 16) + wn * NF;   // first 16-column strip of this wave

  // Explicit typing walks the type array; the others are one tile per group.
  int64_t scan_pos = 0;
  for (;;) {
    int nrows;
    if (p.kind != AA_TYPES_EXPLICIT) {
      nrows = tile_rows_closed_form<TM>(p, i, mt, rows_lds);
    } else {
      // Wave 0 collects the next TM rows whose type is i.
      if (wave == 0) {
        int count = 0;
        int64_t pos = scan_pos;
        while (count < TM && pos < p.M) {
          const int64_t r = pos + lane;
          const bool hit = r < p.M && p.row_types[r] == i;
          const uint64_t mask = __ballot(hit);
          const int total = __popcll(mask);
          const int take = total < TM - count ? total : TM - count;
          const int before = __popcll(mask & ((uint64_t(1) << lane) - 1));
          if (hit && before < take) rows_lds[count + before] = int32_t(r);
          if (take < total) {
            // stop after the take-th hit of this chunk
            uint64_t m = mask;
            for (int s = 0; s < take - 1; ++s) m &= m - 1;
            pos += __builtin_ctzll(m) + 1;
          } else {
            pos += kWave;
          }
          count += take;
        }
        for (int r = count + lane; r < TM; r += kWave) rows_lds[r] = -1;
        if (lane == 0) {
          scan_state[0] = count;
          scan_state[1] = int32_t(pos);  // M fits in int32 for explicit maps (checked on the host)
        }
      }
      __syncthreads();
      nrows = scan_state[0];
      scan_pos = scan_state[1];
    }
    __syncthreads();
    if (nrows == 0) return;

    // This lane's activation rows (B operand: column m = l16 of each m-fragment).
    const Tin* xrow[MF];
    bool rvalid[MF];
    int32_t rowid[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const int r = rows_lds[(wm * MF + f) * 16 + l16];
      rvalid[f] = r >= 0;
      rowid[f] = r;
      xrow[f] = X + int64_t(r >= 0 ? r : 0) * p.ldx;
    }
    bool nvalid[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) nvalid[f] = (nfrag0 + f) * 16 < p.b_out;

    f32x4_t acc0[NF][MF], acc1[NF][MF];
#pragma unroll
    for (int a = 0; a < NF; ++a)
#pragma unroll
      for (int b = 0; b < MF; ++b) {
        acc0[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

    Run<Tin> ra0[STAGES][NF], ra1[STAGES][NF], rb[STAGES][MF];

    const Tin* zrun = reinterpret_cast<const Tin*>(g_zero_runs) + lane * 8;
    auto load_step = [&](int s, Run<Tin>* a0, Run<Tin>* a1, Run<Tin>* b) {
      const int si = s / KF;
      const int kf = s - si * KF;
      const int seg = segs[si < nseg ? si : 0];
      const bool kval = (s < nsteps) && (kf * 32 + g * 8 < p.b_in);
      const int64_t wofs = (int64_t(seg) * p.q + k) * blk_elems + kf * 512 + lane * 8;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int64_t o = wofs + int64_t(nfrag0 + f) * 16 * p.b_in;
        const bool ok = kval && nvalid[f];
        a0[f] = Run<Tin>::load(ok ? W0 + o : zrun);
        if (SWIGLU) a1[f] = Run<Tin>::load(ok ? W1 + o : zrun);
      }
      const int xo = seg * p.b_in + kf * 32 + g * 8;
#pragma unroll
      for (int f = 0; f < MF; ++f) b[f] = Run<Tin>::load_cached((kval && rvalid[f]) ? xrow[f] + xo : zrun);
    };

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) load_step(st, ra0[st], ra1[st], rb[st]);

    for (int s0 = 0; s0 < nsteps; s0 += STAGES) {
#pragma unroll
      for (int u = 0; u < STAGES; ++u) {
        const int nx = (u + STAGES - 1) % STAGES;
        load_step(s0 + u + STAGES - 1, ra0[nx], ra1[nx], rb[nx]);
#pragma unroll
        for (int a = 0; a < NF; ++a)
#pragma unroll
          for (int b = 0; b < MF; ++b) {
            acc0[a][b] = mma(ra0[u][a], rb[u][b], acc0[a][b]);
            if (SWIGLU) acc1[a][b] = mma(ra1[u][a], rb[u][b], acc1[a][b]);
          }
      }
    }

    // Epilogue: lane holds Y[row(m = l16)][col .. col + 3] of each fragment.
    const int64_t col_base = int64_t(k) * p.b_out;
#pragma unroll
    for (int a = 0; a < NF; ++a) {
      if (!nvalid[a]) continue;
      const int col = (nfrag0 + a) * 16 + g * 4;
#pragma unroll
      for (int b = 0; b < MF; ++b) {
        if (!rvalid[b]) continue;
        f32x4_t v = acc0[a][b];
        if (SWIGLU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[a][b][e], acc1[a][b][e]);
        }
        store4(Y + int64_t(rowid[b]) * p.ldy + col_base + col, v);
      }
    }
    if (p.kind != AA_TYPES_EXPLICIT) return;
    __syncthreads();
  }
}


// ------------------------------------------------------ streaming leaf GEMM ---
//
// For the memory-bound shapes (few rows per type, every weight read once) the
// leaf's activation tile - TM rows by the whole concatenated K - is copied
// into LDS once per workgroup with direct global-to-LDS loads, and each wave
// streams its strips of the packed weight through two register buffers of CK
// k-slabs each: while one chunk of slabs is multiplied the next is in flight.
// A chunk never straddles two input groups, so all address arithmetic happens
// once per chunk and the k-slabs inside it are immediate offsets; the scalar
// unit, which the four SIMDs of a CU share, stays off the critical path.
//
// LDS layout of the activation tile: row r starts at byte r * (cpr + 1) * 16;
// its cpr 16-byte chunks hold the concatenated K (zero-padded), followed by
// one pad chunk.  With cpr a multiple of 16 the pad makes the 16 rows of a
// B-operand read fall into 16 distinct groups of four banks.
//
// Only bf16 inputs with closed-form row maps and b_in a multiple of 32 * CK
// take this path; the host falls back to the general kernel otherwise.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

template <int WN, int WM, int NF, int MF, int CK, int GC, bool DB, bool SWIGLU, typename Tout>
__global__ __launch_bounds__(kWave * WN * WM) void leaf_stream_kernel(LeafParams p) {
  using Tin = __bf16;
  constexpr int NWAVE = WN * WM;
  constexpr int TN = WN * NF * 16;
  constexpr int TM = WM * MF * 16;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int32_t rows_lds[TM];

  int i, k, mt, nt;
  decode_tile(p, i, k, mt, nt);
  const int nrows = tile_rows_closed_form<TM>(p, i, mt, rows_lds);
  __syncthreads();
  if (nrows == 0) return;

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int wn = wave % WN, wm = wave / WN;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  int segs[4];
  const int nseg = device_leaf_groups(p.law, i, k, segs);
  const int cps = p.b_in / 8;                 // 16-byte chunks of one segment row
  const int used = nseg * cps;
  const int rstride = p.cpr + 1;              // chunks per LDS row, pad included
  const int chunks_per_seg = p.b_in / (32 * CK);
  const int nchunks = nseg * chunks_per_seg;

  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);
  // 1. Activation tile -> LDS.  Wave-instruction j fills physical chunks
  //    [64 j, 64 j + 64); each lane fetches the logical chunk stored there.
  //    Lanes whose chunk is padding, lies past the leaf's K or belongs to a
  //    row past the type's last row do not load: those LDS bytes are never
  //    read into a kept output.
  {
    const int n_inst = (TM * rstride + 63) / 64;
    for (int j = wave; j < n_inst; j += NWAVE) {
      const int P = j * 64 + lane;
      const int r = P / rstride;
      const int c = P - r * rstride;
      if (r < nrows && c < used) {
        const int row = rows_lds[r];
        const int sg = c / cps;
        const Tin* src = X + int64_t(row) * p.ldx + segs[sg] * p.b_in + (c - sg * cps) * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)((lds_u8_t*)smem + j * 1024), 16, 0, 0);
      }
    }
  }

  // 2. Weight strips.  wl: this lane's byte offset inside a block (strip of
  //    its first n-fragment, its run in the slab).  Chunk c covers k-slabs
  //    [kf0, kf0 + CK) of segment c / chunks_per_seg.
  const int nfrag0 = nt * (TN / 16) + wn * NF;
  bool nvalid[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) nvalid[f] = (nfrag0 + f) * 16 < p.b_out;
  const int64_t blk_bytes = int64_t(p.b_in) * p.b_out * 2;
  const int64_t fstride = int64_t(16) * p.b_in * 2;        // bytes between 16-column strips
  const int64_t wl = int64_t(nfrag0) * fstride + lane * 16;
  const unsigned char* W0 = static_cast<const unsigned char*>(p.W0);
  const unsigned char* W1 = static_cast<const unsigned char*>(p.W1);

  auto chunk_ofs = [&](int c) -> int64_t {   // byte offset of chunk c's first slab, lane part excluded
    const int si = c / chunks_per_seg;
    const int kf0 = (c - si * chunks_per_seg) * CK;
    return (int64_t(segs[si]) * p.q + k) * blk_bytes + kf0 * 1024;
  };
  // Strips past the block's last column read the block's first strip instead
  // (their products are never stored), so every load hits real weight lines.
  int64_t fofs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) fofs[f] = (nvalid[f] ? int64_t(f) * fstride + wl : int64_t(lane) * 16);
  // A group is GC chunks; all of a group's weight loads are issued before
  // any of them is waited on, so each wave keeps GC * CK * NF KiB in flight
  // and a tile pays one memory latency per group, not one per chunk.  With
  // DB the next group is issued while the current one is multiplied.
  // The diagonal block W_kk is read by every row type, so it is loaded with
  // the default cache policy; the other blocks are read by one type only and
  // are streamed with the nontemporal hint so they do not evict it.
  auto load_group = [&](int g0, Run<Tin> (&a0)[GC][CK][NF], Run<Tin> (&a1)[GC][CK][NF]) {
#pragma unroll
    for (int gc = 0; gc < GC; ++gc) {
      const int c = g0 * GC + gc;
      if (c < nchunks) {
        const int64_t base = chunk_ofs(c);
        if (segs[c / chunks_per_seg] == k) {
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int kl = 0; kl < CK; ++kl) {
              const int64_t o = base + fofs[f] + kl * 1024;
              a0[gc][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W0 + o));
              if (SWIGLU) a1[gc][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W1 + o));
            }
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int kl = 0; kl < CK; ++kl) {
              const int64_t o = base + fofs[f] + kl * 1024;
              a0[gc][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W0 + o));
              if (SWIGLU) a1[gc][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W1 + o));
            }
        }
      }
    }
  };

  constexpr int NB = DB ? 2 : 1;
  Run<Tin> wb0[NB][GC][CK][NF], wb1[NB][GC][CK][NF];
  const int ngroups = (nchunks + GC - 1) / GC;
  load_group(0, wb0[0], wb1[0]);

  __syncthreads();   // activation tile resident (the wait covers every load above)

  f32x4_t acc0[NF][MF], acc1[NF][MF];
#pragma unroll
  for (int a = 0; a < NF; ++a)
#pragma unroll
    for (int b = 0; b < MF; ++b) {
      acc0[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc1[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // Byte offset in LDS of this lane's B-operand run for m-fragment b at k-slab 0.
  int xaddr[MF];
#pragma unroll
  for (int b = 0; b < MF; ++b) xaddr[b] = ((wm * MF + b) * 16 + l16) * rstride * 16 + g * 16;

  auto compute_chunk = [&](int c, Run<Tin> (&a0)[CK][NF], Run<Tin> (&a1)[CK][NF]) {
    const int si = c / chunks_per_seg;
    const int cofs = (si * cps + (c - si * chunks_per_seg) * CK * 4) * 16;   // chunk's first LDS column, bytes
#pragma unroll
    for (int kl = 0; kl < CK; ++kl) {
      Run<Tin> xb[MF];
#pragma unroll
      for (int b = 0; b < MF; ++b) xb[b].v = *reinterpret_cast<const u32x4_t*>(smem + xaddr[b] + cofs + kl * 64);
#pragma unroll
      for (int a = 0; a < NF; ++a)
#pragma unroll
        for (int b = 0; b < MF; ++b) {
          acc0[a][b] = mma(a0[kl][a], xb[b], acc0[a][b]);
          if (SWIGLU) acc1[a][b] = mma(a1[kl][a], xb[b], acc1[a][b]);
        }
    }
  };
  auto compute_group = [&](int g0, Run<Tin> (&a0)[GC][CK][NF], Run<Tin> (&a1)[GC][CK][NF]) {
#pragma unroll
    for (int gc = 0; gc < GC; ++gc) {
      const int c = g0 * GC + gc;
      if (c < nchunks) compute_chunk(c, a0[gc], a1[gc]);
    }
  };

  if (DB) {
    int g0 = 0;
    for (; g0 + 2 < ngroups; g0 += 2) {
      load_group(g0 + 1, wb0[NB - 1], wb1[NB - 1]);
      compute_group(g0, wb0[0], wb1[0]);
      load_group(g0 + 2, wb0[0], wb1[0]);
      compute_group(g0 + 1, wb0[NB - 1], wb1[NB - 1]);
    }
    if (g0 + 1 < ngroups) {
      load_group(g0 + 1, wb0[NB - 1], wb1[NB - 1]);
      compute_group(g0, wb0[0], wb1[0]);
      compute_group(g0 + 1, wb0[NB - 1], wb1[NB - 1]);
    } else {
      compute_group(g0, wb0[0], wb1[0]);
    }
  } else {
    compute_group(0, wb0[0], wb1[0]);
    for (int g0 = 1; g0 < ngroups; ++g0) {
      load_group(g0, wb0[0], wb1[0]);
      compute_group(g0, wb0[0], wb1[0]);
    }
  }

  // 3. Epilogue.  Lane holds Y[m = l16][n .. n + 3] of each fragment; the
  //    tile goes through LDS (row stride TN + 8 elements) so that the global
  //    stores are whole 16-byte runs along rows.
  __syncthreads();   // every wave is done reading the activation tile
  constexpr int OSTR = TN + 8;   // elements per LDS output row
  Tout* otile = reinterpret_cast<Tout*>(smem);
#pragma unroll
  for (int b = 0; b < MF; ++b) {
    const int m = (wm * MF + b) * 16 + l16;
#pragma unroll
    for (int a = 0; a < NF; ++a) {
      f32x4_t v = acc0[a][b];
      if (SWIGLU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[a][b][e], acc1[a][b][e]);
      }
      store4(otile + m * OSTR + (wn * NF + a) * 16 + g * 4, v);
    }
  }
  __syncthreads();
  constexpr int VPR = TN * int(sizeof(Tout)) / 16;   // 16-byte runs per tile row
  const int64_t col0 = int64_t(k) * p.b_out + int64_t(nt) * TN;
  const int ncols = p.b_out - nt * TN < TN ? p.b_out - nt * TN : TN;
  for (int e = threadIdx.x; e < TM * VPR; e += kWave * NWAVE) {
    const int r = e / VPR, v = e - r * VPR;
    const int col = v * (16 / int(sizeof(Tout)));
    if (r < nrows && col < ncols) {
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + r * OSTR + col);
      *reinterpret_cast<u32x4_t*>(Y + int64_t(rows_lds[r]) * p.ldy + col0 + col) = val;
    }
  }
}


// ----------------------------------------------- persistent streaming leaf GEMM ---
//
// The same leaf tiles as the streaming kernel above, but each workgroup walks
// a run of tiles and keeps the next tile's loads in flight while it
// multiplies, transposes and stores the current one.  The next tile's
// activation chunks and weight fragments are loaded into registers (the
// weights into the other of two register sets) right after the current
// tile's activations have been written to LDS; they are written to LDS only
// when the next tile starts.  All loads are ordinary register loads, so the
// compiler's wait counts stay exact, and barriers are plain s_barrier with
// LDS-only waits.
//
// Rows of a type are found in closed form in every lane (position or
// block-row typing).  One workgroup of four waves covers TN = 64 NF columns
// and TM = 16 MF rows; the grid is two workgroups per CU.

// Cache policy bits of the persistent kernel.  A block that only one tile
// reads is streamed past L2 with nontemporal accesses, so that the blocks
// several tiles share (the diagonal weight blocks W_kk, a type's own
// activation block x_i) stay resident.
constexpr int kPolWOwn = 1;   // own weight block W_ik: one m-tile per leaf
constexpr int kPolXOwn = 2;   // own activation block x_k: one n-tile per leaf
constexpr int kPolYNt = 4;    // outputs (written once)

template <int NF, int MF, int CK, int NCH, bool SWIGLU, int POL, typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_persist_kernel(LeafParams p) {
  using Tin = __bf16;
  constexpr int NWAVE = 4, NTHR = 256;
  constexpr int TN = NWAVE * NF * 16;
  constexpr int TM = MF * 16;
  constexpr int CPR = NCH * CK * 4;                 // 16-byte chunks of a staged row
  constexpr int RS = CPR + 1;                       // row stride in chunks (one pad chunk)
  constexpr int NXC = (TM * CPR + NTHR - 1) / NTHR; // activation chunks per thread per tile
  constexpr int OSTR = TN + 8;                      // staged output row stride (elements)
  constexpr int XBYTES = (TM * RS * 16 > TM * OSTR * int(sizeof(Tout))) ? TM * RS * 16 : TM * OSTR * int(sizeof(Tout));
  __shared__ __attribute__((aligned(1024))) unsigned char lds[XBYTES];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  // One weight chunk (CK 32-row slabs) spans exactly one input group: the
  // launcher only picks this kernel when b_in == 32 CK.
  const int64_t blk_bytes = int64_t(p.b_in) * p.b_out * 2;
  const int64_t fstride = int64_t(16) * p.b_in * 2;
  const unsigned char* W0 = static_cast<const unsigned char*>(p.W0);
  const unsigned char* W1 = static_cast<const unsigned char*>(p.W1);
  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);
  const bool qq = p.law == AA_LAW_QQ || p.law == AA_LAW_DIGRAPH;   // input groups i, then k

  // This workgroup's run of tiles: XCD x owns a contiguous run of the tile
  // order; its G8 workgroups take every G8-th tile of it.
  const uint32_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const uint32_t G8 = gridDim.x / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  const uint32_t run_begin = xcd * per + (xcd < rem ? xcd : rem);
  const uint32_t run_end = run_begin + per + (xcd < rem ? 1 : 0);

  struct Tile {
    int i, k, nt, nseg, nchunks, nrows;
    bool live;               // false: a step past the last tile (no stores)
    uint32_t gpack;          // Q2 x Q2: input group si in bits [2 si, 2 si + 2)
    int64_t first, stride;   // row of local row r = first + r * stride
  };
  // Input group si of a leaf by arithmetic only (Q_q: i then k).
  auto seg_of = [&](const Tile& T, int si) __attribute__((always_inline)) -> int {
    return qq ? (si == 0 ? T.i : T.k) : int((T.gpack >> (2 * si)) & 3u);
  };
  // rows of type i under position typing: M / q, plus one for the first
  // M mod q residues after the offset
  const int64_t m_div_q = p.M / p.q;
  const int m_mod_q = int(p.M - m_div_q * p.q);
  auto setup = [&](uint32_t t, Tile& T) __attribute__((always_inline)) {
    T.nt = int(t % uint32_t(p.nt_count));
    t /= uint32_t(p.nt_count);
    const int mt = int(t % uint32_t(p.mt_count));
    t /= uint32_t(p.mt_count);
    const int kk = int(t % uint32_t(p.kc));
    t /= uint32_t(p.kc);
    T.i = int(t % uint32_t(p.q));
    T.k = int(t / uint32_t(p.q)) * p.kc + kk;
    int sg[4] = {0, 0, 0, 0};
    T.nseg = device_leaf_groups(p.law, T.i, T.k, sg, p.law == AA_LAW_DIGRAPH ? p.adj[T.i] : 0);
    T.gpack = uint32_t(sg[0] & 3) | (uint32_t(sg[1] & 3) << 2) | (uint32_t(sg[2] & 3) << 4) | (uint32_t(sg[3] & 3) << 6);
    T.nchunks = T.nseg;
    int64_t count;
    if (p.kind == AA_TYPES_BLOCK_ROWS) {
      T.first = int64_t(T.i) * p.rows_per_type;
      T.stride = 1;
      count = p.rows_per_type;
    } else {
      int r0 = T.i - p.off_mod_q;
      if (r0 < 0) r0 += p.q;
      T.first = r0;
      T.stride = p.q;
      count = m_div_q + (r0 < m_mod_q ? 1 : 0);
    }
    const int64_t lo = int64_t(mt) * TM;
    T.nrows = lo >= count ? 0 : int(count - lo < TM ? count - lo : TM);
    T.first += lo * T.stride;
  };

  // Activation chunks, column-block major: the staged tile is NCH column
  // blocks of XCB chunks (the K of one weight chunk); logical chunk e is
  // block e / (TM XCB), row (e % (TM XCB)) / XCB, chunk e % XCB.  Thread t
  // holds e = t, t + 256, ...; since TM XCB is a multiple of 256, each load
  // instruction stays inside one column block and its cache policy is fixed
  // (under Q_q the last block is the own activation block x_k).  Lanes past
  // the tile's rows or K re-read a valid row (the tile's first, or row 0 of X
  // for an empty tile); those values land in LDS cells no kept output reads.
  constexpr int XCB = 4 * CK;                // = the chunks of one input group
  constexpr int JPB = TM * XCB / NTHR;       // loads per column block
  static_assert((TM * XCB) % NTHR == 0 && NXC == NCH * JPB, "staging layout");
  const int x_cc = int(threadIdx.x) % XCB, x_r0 = int(threadIdx.x) / XCB;
  auto load_x = [&](const Tile& T, Run<Tin> (&xr)[NXC]) __attribute__((always_inline)) {
    int64_t rowofs[JPB];
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) {
      const int r = jb * (NTHR / XCB) + x_r0;
      // a void step, and a digraph leaf with no input group (it stores
      // zeros), re-read row 0, which stays in L1, instead of fetching rows
      // nothing will use
      rowofs[jb] = (T.live && T.nrows > 0 && T.nchunks > 0 ? T.first + int64_t(r < T.nrows ? r : 0) * T.stride : 0) * p.ldx;
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // a void step reads the own group's first columns of row 0
      const int colofs = ch < T.nchunks ? seg_of(T, T.live ? ch : 0) * p.b_in + x_cc * 8 : 0;
#pragma unroll
      for (int jb = 0; jb < JPB; ++jb) {
        const Tin* src = X + rowofs[jb] + colofs;
        if ((POL & kPolXOwn) && ch == NCH - 1) xr[ch * JPB + jb] = Run<Tin>::load(src);
        else xr[ch * JPB + jb] = Run<Tin>::load_cached(src);
      }
    }
  };
  auto store_x = [&](const Run<Tin> (&xr)[NXC]) __attribute__((always_inline)) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int jb = 0; jb < JPB; ++jb) {
        const int r = jb * (NTHR / XCB) + x_r0;
        *reinterpret_cast<u32x4_t*>(lds + (r * RS + ch * XCB + x_cc) * 16) = xr[ch * JPB + jb].v;
      }
  };

  // Weight fragments of tile T.  The cache policy is fixed per chunk slot so
  // that no load sits in a branch: under Q_q chunk 0 is the row type's own
  // block W_ik, read by this type only (nontemporal under kPolWOwn, i.e. when
  // a leaf is a single m-tile; with several m-tiles the siblings reread it
  // from L2), and the last chunk is the diagonal block W_kk that every type
  // reads (default policy, stays in L2).  A diagonal leaf has a single chunk;
  // its second slot re-reads it.
  auto load_w = [&](const Tile& T, Run<Tin> (&a0)[NCH][CK][NF], Run<Tin> (&a1)[NCH][CK][NF]) __attribute__((always_inline)) {
    const int nfrag0 = T.nt * (TN / 16) + wave * NF;
    const int64_t wl = int64_t(nfrag0) * fstride + lane * 16;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int c = ch < T.nchunks ? ch : 0;
      // a void step, and a digraph leaf with no input group, address the
      // diagonal block W_kk (and re-read its first 1 KiB only, below)
      const int64_t base = (int64_t(T.live && T.nchunks > 0 ? seg_of(T, c) : T.k) * p.q + T.k) * blk_bytes;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int kl = 0; kl < CK; ++kl) {
          // (a void step, or no input group: every load re-reads the block's first 1 KiB)
          const int64_t o = !T.live || T.nchunks == 0 ? base + int64_t(lane) * 16
                                           : base + ((nfrag0 + f) * 16 < p.b_out ? wl + f * fstride : int64_t(lane) * 16) + kl * 1024;
          if ((POL & kPolWOwn) && ch == 0) {
            a0[ch][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W0 + o));
            if (SWIGLU) a1[ch][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W1 + o));
          } else {
            a0[ch][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W0 + o));
            if (SWIGLU) a1[ch][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W1 + o));
          }
        }
    }
  };

  auto compute_store = [&](const Tile& T, const Run<Tin> (&a0)[NCH][CK][NF], const Run<Tin> (&a1)[NCH][CK][NF]) __attribute__((always_inline)) {
    f32x4_t acc0[NF][MF], acc1[NF][MF];
#pragma unroll
    for (int a = 0; a < NF; ++a)
#pragma unroll
      for (int b = 0; b < MF; ++b) {
        acc0[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch < T.nchunks) {
        const int cofs = ch * XCB * 16;
#pragma unroll
        for (int kl = 0; kl < CK; ++kl) {
          Run<Tin> xv[MF];
#pragma unroll
          for (int b = 0; b < MF; ++b)
            xv[b].v = *reinterpret_cast<const u32x4_t*>(lds + (b * 16 + l16) * RS * 16 + g * 16 + cofs + kl * 64);
#pragma unroll
          for (int a = 0; a < NF; ++a)
#pragma unroll
            for (int b = 0; b < MF; ++b) {
              acc0[a][b] = mma(a0[ch][kl][a], xv[b], acc0[a][b]);
              if (SWIGLU) acc1[a][b] = mma(a1[ch][kl][a], xv[b], acc1[a][b]);
            }
        }
      }
    }
    // Every wave is done reading the activation tile: stage outputs in its place.
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    Tout* otile = reinterpret_cast<Tout*>(lds);
#pragma unroll
    for (int b = 0; b < MF; ++b)
#pragma unroll
      for (int a = 0; a < NF; ++a) {
        f32x4_t v = acc0[a][b];
        if (SWIGLU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[a][b][e], acc1[a][b][e]);
        }
        store4(otile + (b * 16 + l16) * OSTR + (wave * NF + a) * 16 + g * 4, v);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    constexpr int VPR = TN * int(sizeof(Tout)) / 16;
    const int64_t col0 = int64_t(T.k) * p.b_out + int64_t(T.nt) * TN;
    const int ncols = p.b_out - T.nt * TN < TN ? p.b_out - T.nt * TN : TN;
#pragma unroll
    for (int e0 = 0; e0 < TM * VPR; e0 += NTHR) {
      const int e = e0 + int(threadIdx.x);
      const int r = e / VPR, v = e - r * VPR;
      const int col = v * (16 / int(sizeof(Tout)));
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + (r < TM ? r : 0) * OSTR + col);
      if (T.live && e < TM * VPR && r < T.nrows && col < ncols) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Y + (T.first + int64_t(r) * T.stride) * p.ldy + col0 + col);
        if (POL & kPolYNt) __builtin_nontemporal_store(val, dst);
        else *dst = val;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // staged outputs read before the buffer is refilled
    __builtin_amdgcn_s_barrier();
  };

  Run<Tin> xr[NXC];
  Run<Tin> wa0[NCH][CK][NF], wa1[NCH][CK][NF], wb0[NCH][CK][NF], wb1[NCH][CK][NF];
  Tile TA, TB;
  const uint32_t t0 = run_begin + slot;
  if (t0 >= run_end) return;
  const int n_my = int((run_end - t0 + G8 - 1) / G8);
  const uint32_t t_last = t0 + uint32_t(n_my - 1) * G8;
  // Step u of this workgroup; steps past its last tile are void: all their
  // loads re-read one 1 KiB run and one activation row, which stay in L1,
  // and they store nothing.  No
  // load is ever skipped by a branch, and the loop exits only after whole
  // rounds of two steps, so every step sees the same queue of pending loads
  // and the waits before the multiplies never drain the prefetch.
  auto tile_at = [&](int u, Tile& T) __attribute__((always_inline)) {
    const bool live = u < n_my;
    setup(live ? t0 + uint32_t(u) * G8 : t_last, T);
    T.live = live;
  };
  tile_at(0, TA);
  load_x(TA, xr);
  load_w(TA, wa0, wa1);
  const int rounds = (n_my + 1) / 2;
  for (int rd = 0; rd < rounds; ++rd) {
    // TA: activations in xr, weights in wa
    store_x(xr);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    tile_at(2 * rd + 1, TB);
    load_x(TB, xr);
    load_w(TB, wb0, wb1);
    compute_store(TA, wa0, wa1);
    // TB: activations in xr, weights in wb
    store_x(xr);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    tile_at(2 * rd + 2, TA);
    load_x(TA, xr);
    load_w(TA, wa0, wa1);
    compute_store(TB, wb0, wb1);
  }
}

// ------------------------------------------------------------ job kernel ---
//
// Q_q leaves whose input groups are 32 CK wide, position or block-row typing.
// The work is split into jobs: a job is one TN-column strip nt of one output
// group k, over every row type i.  All leaves of a job share the diagonal
// block strip W_kk, which the workgroup copies to LDS once; per tile only the
// type's activation rows [x_i | x_k] and its own block strip W_ik stream in,
// into NSET rotating register sets, so that NSET - 1 tiles of loads are in
// flight while one tile is multiplied.  This raises the bytes in flight per
// CU, which is what bounds a streaming kernel on HBM.
//
// Grid: XCD x (blockIdx % 8) owns output groups [x gpx, (x + 1) gpx).  Each
// group gets wpg workgroups, dealt over its nt_count jobs; a job's workgroups
// split its q * mt_count tiles (type-major, then m-tile) into contiguous,
// balanced ranges.

struct JobParams {
  const void* X;
  const void* W0;
  const void* W1;
  void* Y;
  int64_t M;
  int64_t ldx;
  int64_t ldy;
  int32_t q;
  int32_t b_out;
  int32_t kind;            // aa_type_kind_t (position or block rows)
  int32_t off_mod_q;
  int64_t rows_per_type;   // block-row typing
  int32_t mt_count;
  int32_t nt_count;
  int32_t gpx;             // output groups per XCD
  int32_t wpg;             // workgroups per output group
};

template <int NF, int MF, int CK, int NSET, bool SWIGLU, int POL, typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_job_kernel(JobParams p) {
  using Tin = __bf16;
  constexpr int NTHR = 256;
  constexpr int TN = 4 * NF * 16;
  constexpr int TM = MF * 16;
  constexpr int BIN = 32 * CK;             // input group width
  constexpr int XCB = BIN / 8;             // 16-byte chunks of one group's row
  constexpr int RS = 2 * XCB + 1;          // staged activation row stride (chunks, one pad)
  constexpr int JPB = TM * XCB / NTHR;     // activation loads per thread per group
  static_assert((TM * XCB) % NTHR == 0, "activation tile");
  constexpr int NW = SWIGLU ? 2 : 1;
  constexpr int STRIP = BIN * 32;          // bytes of one 16-column strip of a block
  constexpr int WKK_BYTES = NW * (TN / 16) * STRIP;
  constexpr int OSTR = TN + 8;             // staged output row stride (elements)
  constexpr int XS_BYTES = TM * RS * 16 > TM * OSTR * int(sizeof(Tout)) ? TM * RS * 16 : TM * OSTR * int(sizeof(Tout));
  __shared__ __attribute__((aligned(1024))) unsigned char wkk[WKK_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char xs[XS_BYTES];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int q = p.q;
  const int nstrips = p.b_out / 16;
  const int64_t blk_bytes = int64_t(BIN) * p.b_out * 2;
  const unsigned char* W0 = static_cast<const unsigned char*>(p.W0);
  const unsigned char* W1 = static_cast<const unsigned char*>(p.W1);
  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);

  // ---- this workgroup's job and tile range
  const int xcd = int(blockIdx.x % kNumXcd), slot = int(blockIdx.x / kNumXcd);
  const int k = xcd * p.gpx + slot / p.wpg;
  const int r = slot % p.wpg;
  const int base = p.wpg / p.nt_count, extra = p.wpg % p.nt_count;
  int nt, w, s_job;
  if (r < extra * (base + 1)) {
    nt = r / (base + 1);
    w = r % (base + 1);
    s_job = base + 1;
  } else {
    const int r2 = r - extra * (base + 1);
    nt = extra + r2 / base;
    w = r2 % base;
    s_job = base;
  }
  // Tiles of the job are (type, m-tile) pairs, type-major.  When the job's
  // workgroups are a multiple of its m-tiles, each takes one m-tile over a
  // contiguous range of types, so the m-tiles of a type are multiplied at
  // the same time on different workgroups and its own weight strip W_ik
  // comes from HBM once (read one tile apart by one workgroup, it was often
  // evicted from L2 in between: the square product read 1.096x its
  // algorithmic bytes that way, 1.018x this way).  Otherwise each
  // takes a contiguous range of the (type, m-tile) order.  (Contiguous
  // ranges measure better than dealing the tiles in turn: with every
  // workgroup on the same row type at once, the traffic concentrates on one
  // row block of X, W and Y at a time.)
  const bool by_mt = p.mt_count > 1 && s_job % p.mt_count == 0;
  const int n_sub = by_mt ? s_job / p.mt_count : s_job;
  const int w_sub = by_mt ? w / p.mt_count : w;
  const int my_mt = by_mt ? w % p.mt_count : 0;
  const int tiles = by_mt ? q : q * p.mt_count;
  const int u_begin = int(int64_t(tiles) * w_sub / n_sub);
  const int u_end = int(int64_t(tiles) * (w_sub + 1) / n_sub);
  const int n_my = u_end - u_begin;
  if (n_my <= 0) return;

  // ---- the diagonal block strip W_kk (and the up projection's): requested
  // first, written to LDS after the first tiles have been requested
  constexpr int NCP = WKK_BYTES / (NTHR * 16);
  static_assert(WKK_BYTES % (NTHR * 16) == 0, "diagonal strip copy");
  u32x4_t wkk_tmp[NCP];
  {
    u32x4_t (&tmp)[NCP] = wkk_tmp;
#pragma unroll
    for (int j = 0; j < NCP; ++j) {
      const int e = (j * NTHR + int(threadIdx.x)) * 16;   // byte in wkk
      const int wsel = e / ((TN / 16) * STRIP);
      const int rem = e - wsel * (TN / 16) * STRIP;
      int sl = nt * (TN / 16) + rem / STRIP;
      sl = sl < nstrips ? sl : nstrips - 1;
      const int64_t src = (int64_t(k) * q + k) * blk_bytes + int64_t(sl) * STRIP + (rem % STRIP);
      tmp[j] = *reinterpret_cast<const u32x4_t*>((wsel ? W1 : W0) + src);
    }
  }
  // (the loads of the first tiles follow in the same order as in the steady
  // state, so the loop entry sees the same queue of pending loads)
  __builtin_amdgcn_sched_barrier(0);

  // ---- per-tile geometry (all wave-uniform)
  // A step past the workgroup's last tile is a "void" tile: no rows (so no
  // stores), type k (so only the first product runs), and its loads re-read
  // the job's diagonal strip, which is in bounds and resident in L2.  Steps
  // never branch around loads, so every step leaves the same queue of
  // pending loads and the waits stay exact.
  struct Tile {
    int i, nrows;
    bool valid;
    int64_t first, stride;
  };
  // rows of type i under position typing: M / q, plus one for the first
  // M mod q residues after the offset
  const int64_t m_div_q = p.M / q;
  const int m_mod_q = int(p.M - m_div_q * q);
  auto setup = [&](int u, Tile& T) __attribute__((always_inline)) {
    T.valid = u < n_my;
    const int ug = u_begin + (T.valid ? u : 0);
    T.i = by_mt || p.mt_count == 1 ? ug : ug / p.mt_count;
    const int mt = by_mt ? my_mt : ug - T.i * p.mt_count;
    int64_t count;
    if (p.kind == AA_TYPES_BLOCK_ROWS) {
      T.first = int64_t(T.i) * p.rows_per_type;
      T.stride = 1;
      count = p.rows_per_type;
    } else {
      int r0 = T.i - p.off_mod_q;
      if (r0 < 0) r0 += q;
      T.first = r0;
      T.stride = q;
      count = m_div_q + (r0 < m_mod_q ? 1 : 0);
    }
    const int64_t lo = int64_t(mt) * TM;
    T.nrows = lo >= count ? 0 : int(count - lo < TM ? count - lo : TM);
    T.first += lo * T.stride;
    if (!T.valid) {
      T.i = k;
      T.nrows = 0;
    }
  };

  // ---- loads of one tile into a register set.  Activations: chunk x_cc of
  // rows x_r0 + jb (NTHR / XCB), first of group i then of group k; rows past
  // the tile re-read its first row (or row 0 of X).  Own weight block: this
  // wave's NF strips of W_ik (strips past b_out re-read the last one).
  const int x_cc = int(threadIdx.x) % XCB, x_r0 = int(threadIdx.x) / XCB;
  // Addresses are a wave-uniform 64-bit base plus a 32-bit per-lane offset
  // (a tile spans TM rows of stride q, well inside 4 GiB).
  const int64_t wkk_base = (int64_t(k) * q + k) * blk_bytes;
  auto load = [&](const Tile& T, Run<Tin> (&xr)[2 * JPB], Run<Tin> (&wr)[CK][NF],
                  Run<Tin> (&wu)[CK][NF]) __attribute__((always_inline)) {
    const Tin* xt = X + (T.nrows > 0 ? T.first : 0) * p.ldx;
    const uint32_t rstep = uint32_t(T.stride * p.ldx);
    uint32_t rowofs[JPB];
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) {
      const int rr = jb * (NTHR / XCB) + x_r0;
      rowofs[jb] = uint32_t(rr < T.nrows ? rr : 0) * rstep + uint32_t(x_cc * 8);
    }
    const Tin* xv = reinterpret_cast<const Tin*>(W0 + wkk_base);
    const Tin* x0 = T.valid ? xt + T.i * BIN : xv;
    const Tin* x1 = T.valid ? xt + k * BIN : xv;
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) xr[jb] = Run<Tin>::load_cached(x0 + rowofs[jb]);
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) {
      if (POL & kPolXOwn) xr[JPB + jb] = Run<Tin>::load(x1 + rowofs[jb]);
      else xr[JPB + jb] = Run<Tin>::load_cached(x1 + rowofs[jb]);
    }
    const int64_t wb = (T.valid ? (int64_t(T.i) * q + k) * blk_bytes : wkk_base) + lane * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int sl = nt * (TN / 16) + wave * NF + f;
      sl = sl < nstrips ? sl : nstrips - 1;
#pragma unroll
      for (int kl = 0; kl < CK; ++kl) {
        const int64_t o = wb + int64_t(sl) * STRIP + kl * 1024;
        if (POL & kPolWOwn) {
          wr[kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W0 + o));
          if (SWIGLU) wu[kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W1 + o));
        } else {
          wr[kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W0 + o));
          if (SWIGLU) wu[kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W1 + o));
        }
      }
    }
  };
  auto store_x = [&](const Run<Tin> (&xr)[2 * JPB]) __attribute__((always_inline)) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int jb = 0; jb < JPB; ++jb) {
        const int rr = jb * (NTHR / XCB) + x_r0;
        *reinterpret_cast<u32x4_t*>(xs + (rr * RS + ch * XCB + x_cc) * 16) = xr[ch * JPB + jb].v;
      }
  };

  // ---- multiply one tile and store it
  constexpr int VPR = TN * int(sizeof(Tout)) / 16;   // 16-byte output vectors per row
  constexpr int NYV = (TM * VPR + NTHR - 1) / NTHR;     // per thread
  auto compute_store = [&](const Tile& T, const Run<Tin> (&wr)[CK][NF], const Run<Tin> (&wu)[CK][NF],
                           u32x4_t (&yv)[NYV]) __attribute__((always_inline)) {
    f32x4_t acc0[NF][MF], acc1[NF][MF];
#pragma unroll
    for (int a = 0; a < NF; ++a)
#pragma unroll
      for (int b = 0; b < MF; ++b) {
        acc0[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    // input group i times the own block W_ik (registers); a void step skips it
#pragma unroll
    for (int kl = 0; kl < CK; ++kl) {
      if (!T.valid) break;
      Run<Tin> xv[MF];
#pragma unroll
      for (int b = 0; b < MF; ++b)
        xv[b].v = *reinterpret_cast<const u32x4_t*>(xs + ((b * 16 + l16) * RS + kl * 4 + g) * 16);
#pragma unroll
      for (int a = 0; a < NF; ++a)
#pragma unroll
        for (int b = 0; b < MF; ++b) {
          acc0[a][b] = mma(wr[kl][a], xv[b], acc0[a][b]);
          if (SWIGLU) acc1[a][b] = mma(wu[kl][a], xv[b], acc1[a][b]);
        }
    }
    // input group k times the diagonal block W_kk (LDS); a diagonal leaf
    // (k == i) has only the first product
    if (T.i != k) {
#pragma unroll
      for (int kl = 0; kl < CK; ++kl) {
        Run<Tin> xv[MF], wk[NF], wk1[NF];
#pragma unroll
        for (int b = 0; b < MF; ++b)
          xv[b].v = *reinterpret_cast<const u32x4_t*>(xs + ((b * 16 + l16) * RS + XCB + kl * 4 + g) * 16);
#pragma unroll
        for (int a = 0; a < NF; ++a) {
          const int o = (wave * NF + a) * STRIP + kl * 1024 + lane * 16;
          wk[a].v = *reinterpret_cast<const u32x4_t*>(wkk + o);
          if (SWIGLU) wk1[a].v = *reinterpret_cast<const u32x4_t*>(wkk + (TN / 16) * STRIP + o);
        }
#pragma unroll
        for (int a = 0; a < NF; ++a)
#pragma unroll
          for (int b = 0; b < MF; ++b) {
            acc0[a][b] = mma(wk[a], xv[b], acc0[a][b]);
            if (SWIGLU) acc1[a][b] = mma(wk1[a], xv[b], acc1[a][b]);
          }
      }
    }
    // every wave is done reading the activation tile: stage outputs in its place
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    Tout* otile = reinterpret_cast<Tout*>(xs);
#pragma unroll
    for (int b = 0; b < MF; ++b)
#pragma unroll
      for (int a = 0; a < NF; ++a) {
        f32x4_t v = acc0[a][b];
        if (SWIGLU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[a][b][e], acc1[a][b][e]);
        }
        store4(otile + (b * 16 + l16) * OSTR + (wave * NF + a) * 16 + g * 4, v);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    const int64_t col0 = int64_t(k) * p.b_out + int64_t(nt) * TN;
    const int ncols = p.b_out - nt * TN < TN ? p.b_out - nt * TN : TN;
#pragma unroll
    for (int j = 0; j < NYV; ++j) {
      const int e = j * NTHR + int(threadIdx.x);
      const int rr = e / VPR, v = e - rr * VPR;
      const int col = v * (16 / int(sizeof(Tout)));
      yv[j] = *reinterpret_cast<const u32x4_t*>(otile + (rr < TM ? rr : 0) * OSTR + col);
      if (e < TM * VPR && rr < T.nrows && col < ncols) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Y + (T.first + int64_t(rr) * T.stride) * p.ldy + col0 + col);
        if (POL & kPolYNt) __builtin_nontemporal_store(yv[j], dst);
        else *dst = yv[j];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // staged outputs read before the buffer is refilled
    __builtin_amdgcn_s_barrier();
  };

  // ---- software pipeline over NSET register sets
  Run<Tin> xr[NSET][2 * JPB];
  Run<Tin> wr[NSET][CK][NF], wu[NSET][CK][NF];
  Tile T[NSET];
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) {
    setup(s, T[s]);
    load(T[s], xr[s], wr[s], wu[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < NCP; ++j)
    *reinterpret_cast<u32x4_t*>(wkk + (j * NTHR + int(threadIdx.x)) * 16) = wkk_tmp[j];
  // Per step: stage the activations of tile u, multiply, store its outputs,
  // then request tile u + NSET - 1.  The stores go out before the new loads
  // and their data registers stay live until those loads are issued: a
  // register that a pending store still reads is only reused once newer
  // loads exist, so waiting for the store never drains the loads in flight.
  // The loop runs whole rounds of NSET steps and exits only after the last
  // one, so the loop header is entered from one place with one queue.
  const int rounds = (n_my + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      const int u = rd * NSET + s;
      store_x(xr[s]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      u32x4_t yv[NYV];
      compute_store(T[s], wr[s], wu[s], yv);
      const int sn = (s + NSET - 1) % NSET;
      setup(u + NSET - 1, T[sn]);
      load(T[sn], xr[sn], wr[sn], wu[sn]);
#pragma unroll
      for (int j = 0; j < NYV; ++j) asm volatile("" ::"v"(yv[j]));
    }
  }
}

// ------------------------------------------------------- K-stream kernel ---
//
// Q_q leaves of any input-group width b_in = 32 CK cps, position or block-row
// typing.  A tile (type i, output group k, m-tile, n-tile) is multiplied in
// cps steps; step j covers K-chunk j of both input groups at once: slot 0 is
// x_i chunk j times W_ik chunk j, slot 1 is x_k chunk j times W_kk chunk j,
// so each slot's cache policy is fixed (own blocks streamed past L2, shared
// ones kept).  Steps are pipelined over NSET rotating register sets with the
// same discipline as the job kernel: loads of step e + NSET - 1 are issued
// after step e's multiplies and stores, the stored values stay live past
// them, void steps past the end re-read L2-resident data, and the loop exits
// only after whole rounds.  Tiles are numbered and dealt as in the persistent
// kernel (contiguous run of output groups per XCD, W_kk shared in its L2).

template <int NF, int MF, int CK, int NSET, bool SWIGLU, int POL, typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_kstream_kernel(LeafParams p) {
  using Tin = __bf16;
  constexpr int NTHR = 256;
  constexpr int TN = 4 * NF * 16;
  constexpr int TM = MF * 16;
  constexpr int XCB = 4 * CK;              // 16-byte chunks of one slot's row
  constexpr int RS = 2 * XCB + 1;          // staged activation row stride (chunks, one pad)
  constexpr int JPB = TM * XCB / NTHR;     // activation loads per thread per slot
  static_assert((TM * XCB) % NTHR == 0, "activation tile");
  constexpr int OSTR = TN + 8;
  constexpr int XS_BYTES = TM * RS * 16 > TM * OSTR * int(sizeof(Tout)) ? TM * RS * 16 : TM * OSTR * int(sizeof(Tout));
  __shared__ __attribute__((aligned(1024))) unsigned char xs[XS_BYTES];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int q = p.q;
  const int cps = p.b_in / (32 * CK);      // steps per tile
  const int nstrips = p.b_out / 16;
  const int strip_bytes = p.b_in * 32;
  const int64_t blk_bytes = int64_t(p.b_in) * p.b_out * 2;
  const unsigned char* W0 = static_cast<const unsigned char*>(p.W0);
  const unsigned char* W1 = static_cast<const unsigned char*>(p.W1);
  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);

  // ---- this workgroup's tiles: every G8-th tile of its XCD's run
  const uint32_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const uint32_t G8 = gridDim.x / kNumXcd;
  const uint32_t per = p.n_tiles / kNumXcd, rem = p.n_tiles % kNumXcd;
  const uint32_t run_begin = xcd * per + (xcd < rem ? xcd : rem);
  const uint32_t run_end = run_begin + per + (xcd < rem ? 1 : 0);
  const uint32_t t0 = run_begin + slot;
  if (t0 >= run_end) return;
  const int n_tiles_my = int((run_end - t0 + G8 - 1) / G8);
  const int n_steps = n_tiles_my * cps;
  const int64_t m_div_q = p.M / q;
  const int m_mod_q = int(p.M - m_div_q * q);

  struct Step {
    int i, k, nt, nrows, j;
    bool live, diag;
    int64_t first, stride;
  };
  // Step (u, j): tile u of this workgroup, K-chunk j.  Past the last step the
  // last tile is re-used with live = false.
  auto setup = [&](int u, int j, Step& S) __attribute__((always_inline)) {
    S.live = u < n_tiles_my;
    uint32_t t = t0 + uint32_t(S.live ? u : n_tiles_my - 1) * G8;
    S.j = S.live ? j : cps - 1;
    S.nt = int(t % uint32_t(p.nt_count));
    t /= uint32_t(p.nt_count);
    const int mt = int(t % uint32_t(p.mt_count));
    t /= uint32_t(p.mt_count);
    const int kk = int(t % uint32_t(p.kc));
    t /= uint32_t(p.kc);
    S.i = int(t % uint32_t(q));
    S.k = int(t / uint32_t(q)) * p.kc + kk;
    S.diag = S.i == S.k;
    int64_t count;
    if (p.kind == AA_TYPES_BLOCK_ROWS) {
      S.first = int64_t(S.i) * p.rows_per_type;
      S.stride = 1;
      count = p.rows_per_type;
    } else {
      int r0 = S.i - p.off_mod_q;
      if (r0 < 0) r0 += q;
      S.first = r0;
      S.stride = q;
      count = m_div_q + (r0 < m_mod_q ? 1 : 0);
    }
    const int64_t lo = int64_t(mt) * TM;
    S.nrows = lo >= count ? 0 : int(count - lo < TM ? count - lo : TM);
    S.first += lo * S.stride;
  };

  // ---- loads of one step.  Slot 0: x_i chunk j and W_ik chunk j; slot 1:
  // x_k chunk j and W_kk chunk j (a diagonal leaf re-reads the cached data of
  // slot 0; a void step re-reads one 1 KiB run and one row start).
  // Activations: chunk x_cc of rows x_r0 + jb (NTHR / XCB); rows past the
  // tile re-read its first row.
  const int x_cc = int(threadIdx.x) % XCB, x_r0 = int(threadIdx.x) / XCB;
  auto load = [&](const Step& S, Run<Tin> (&xr)[2 * JPB], Run<Tin> (&wr)[2][CK][NF],
                  Run<Tin> (&wu)[2][CK][NF]) __attribute__((always_inline)) {
    const Tin* xt = X + (S.nrows > 0 ? S.first : 0) * p.ldx;
    const uint32_t rstep = uint32_t(S.stride * p.ldx);
    uint32_t rowofs[JPB];
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) {
      const int rr = jb * (NTHR / XCB) + x_r0;
      // a void step reads the first columns of the tile's first row only
      rowofs[jb] = S.live ? uint32_t(rr < S.nrows ? rr : 0) * rstep + uint32_t(S.j * 32 * CK + x_cc * 8)
                          : uint32_t(x_cc * 8);
    }
    const Tin* x0 = xt + S.i * p.b_in;
    const Tin* x1 = (S.live && !S.diag) ? xt + S.k * p.b_in : x0;
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) xr[jb] = Run<Tin>::load_cached(x0 + rowofs[jb]);
#pragma unroll
    for (int jb = 0; jb < JPB; ++jb) {
      if (POL & kPolXOwn) xr[JPB + jb] = Run<Tin>::load(x1 + rowofs[jb]);
      else xr[JPB + jb] = Run<Tin>::load_cached(x1 + rowofs[jb]);
    }
    const int64_t kkb = (int64_t(S.k) * q + S.k) * blk_bytes;
    const int64_t b0 = S.live ? (int64_t(S.i) * q + S.k) * blk_bytes : kkb;
    const int64_t lo = int64_t(S.j) * CK * 1024 + lane * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int sl = S.nt * (TN / 16) + wave * NF + f;
      sl = sl < nstrips ? sl : nstrips - 1;
      const int64_t so = int64_t(sl) * strip_bytes + lo;
#pragma unroll
      for (int kl = 0; kl < CK; ++kl) {
        // a void step re-reads the first 1 KiB of W_kk, which stays in L1
        const int64_t o0 = S.live ? b0 + so + kl * 1024 : kkb + lane * 16;
        const int64_t o1 = S.live ? kkb + so + kl * 1024 : kkb + lane * 16;
        if (POL & kPolWOwn) {
          wr[0][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W0 + o0));
          if (SWIGLU) wu[0][kl][f] = Run<Tin>::load(reinterpret_cast<const Tin*>(W1 + o0));
        } else {
          wr[0][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W0 + o0));
          if (SWIGLU) wu[0][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W1 + o0));
        }
        wr[1][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W0 + o1));
        if (SWIGLU) wu[1][kl][f] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(W1 + o1));
      }
    }
  };
  auto store_x = [&](const Run<Tin> (&xr)[2 * JPB]) __attribute__((always_inline)) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int jb = 0; jb < JPB; ++jb) {
        const int rr = jb * (NTHR / XCB) + x_r0;
        *reinterpret_cast<u32x4_t*>(xs + (rr * RS + ch * XCB + x_cc) * 16) = xr[ch * JPB + jb].v;
      }
  };

  constexpr int VPR = TN * int(sizeof(Tout)) / 16;
  constexpr int NYV = (TM * VPR + NTHR - 1) / NTHR;
  f32x4_t acc0[NF][MF], acc1[NF][MF];
  // ---- multiply one step; on a tile's last step stage and store its outputs
  auto compute = [&](const Step& S, const Run<Tin> (&wr)[2][CK][NF], const Run<Tin> (&wu)[2][CK][NF],
                     u32x4_t (&yv)[NYV]) __attribute__((always_inline)) {
    if (S.j == 0) {
#pragma unroll
      for (int a = 0; a < NF; ++a)
#pragma unroll
        for (int b = 0; b < MF; ++b) {
          acc0[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc1[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl == 1 && S.diag) break;
#pragma unroll
      for (int kl = 0; kl < CK; ++kl) {
        Run<Tin> xv[MF];
#pragma unroll
        for (int b = 0; b < MF; ++b)
          xv[b].v = *reinterpret_cast<const u32x4_t*>(xs + ((b * 16 + l16) * RS + sl * XCB + kl * 4 + g) * 16);
#pragma unroll
        for (int a = 0; a < NF; ++a)
#pragma unroll
          for (int b = 0; b < MF; ++b) {
            acc0[a][b] = mma(wr[sl][kl][a], xv[b], acc0[a][b]);
            if (SWIGLU) acc1[a][b] = mma(wu[sl][kl][a], xv[b], acc1[a][b]);
          }
      }
    }
    // every wave is done reading the activation chunk before it is refilled
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (S.j == cps - 1) {
      Tout* otile = reinterpret_cast<Tout*>(xs);
#pragma unroll
      for (int b = 0; b < MF; ++b)
#pragma unroll
        for (int a = 0; a < NF; ++a) {
          f32x4_t v = acc0[a][b];
          if (SWIGLU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc0[a][b][e], acc1[a][b][e]);
          }
          store4(otile + (b * 16 + l16) * OSTR + (wave * NF + a) * 16 + g * 4, v);
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      const int64_t col0 = int64_t(S.k) * p.b_out + int64_t(S.nt) * TN;
      const int ncols = p.b_out - S.nt * TN < TN ? p.b_out - S.nt * TN : TN;
#pragma unroll
      for (int jj = 0; jj < NYV; ++jj) {
        const int e = jj * NTHR + int(threadIdx.x);
        const int rr = e / VPR, v = e - rr * VPR;
        const int col = v * (16 / int(sizeof(Tout)));
        yv[jj] = *reinterpret_cast<const u32x4_t*>(otile + (rr < TM ? rr : 0) * OSTR + col);
        if (S.live && e < TM * VPR && rr < S.nrows && col < ncols) {
          u32x4_t* dst = reinterpret_cast<u32x4_t*>(Y + (S.first + int64_t(rr) * S.stride) * p.ldy + col0 + col);
          if (POL & kPolYNt) __builtin_nontemporal_store(yv[jj], dst);
          else *dst = yv[jj];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // staged outputs read before the buffer is refilled
      __builtin_amdgcn_s_barrier();
    }
  };

  // ---- software pipeline over NSET register sets
  Run<Tin> xr[NSET][2 * JPB];
  Run<Tin> wr[NSET][2][CK][NF], wu[NSET][2][CK][NF];
  Step S[NSET];
  int lu = 0, lj = 0;   // the next step to request
  auto advance = [&]() __attribute__((always_inline)) {
    if (++lj == cps) {
      lj = 0;
      ++lu;
    }
  };
#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) {
    setup(lu, lj, S[s]);
    load(S[s], xr[s], wr[s], wu[s]);
    advance();
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rounds = (n_steps + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      store_x(xr[s]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
      u32x4_t yv[NYV];
#pragma unroll
      for (int jj = 0; jj < NYV; ++jj) yv[jj] = u32x4_t{0u, 0u, 0u, 0u};
      compute(S[s], wr[s], wu[s], yv);
      const int sn = (s + NSET - 1) % NSET;
      setup(lu, lj, S[sn]);
      load(S[sn], xr[sn], wr[sn], wu[sn]);
      advance();
#pragma unroll
      for (int jj = 0; jj < NYV; ++jj) asm volatile("" ::"v"(yv[jj]));
    }
  }
}

// --------------------------------------------------------- tile kernel ---
//
// Leaves with many rows per type (the pilot FFN: 3072 rows per type, Q2 x Q2)
// are real GEMMs and bound by the matrix cores, so this kernel uses large
// tiles: one workgroup of four waves computes TM = 128 rows of one leaf, each
// wave a 64-row half by four 16-column strips (4 x 4 MFMA tiles).  K runs over
// the leaf's input groups in stages of KC = 64 (two 32-row slabs).
//   - Weights go straight to registers: the packed layout stores every MFMA
//     A operand as one contiguous 1 KiB fragment, so each wave reads its own
//     eight fragments per stage with fully coalesced loads (the two waves of
//     a column half read the same fragments; the second read hits L2).
//   - Activations are shared by the waves of a row half: the stage (128 rows
//     x 128 bytes) is staged through LDS with a 16-byte pad per row.
// Keeping the weights out of LDS halves its traffic, which bounded the
// previous version.  The fused SwiGLU gate/up interleaves strips: each wave
// takes two gate strips and the same two up strips, so its accumulators hold
// g and u of the same outputs and the epilogue forms silu(g) u in registers;
// a workgroup then covers 64 output columns instead of 128, with the same
// register budget as the plain projection (two workgroups per CU).
// Stages are staged through NSET register sets: the loads of stage s + NSET -
// 1 are issued before the multiplies of stage s, the activations of stage s +
// 1 are written to the other LDS buffer after them, behind one barrier.
// Loads are never skipped (past the last stage they re-read it) and the loop
// runs whole rounds of NSET stages with the multiplies of void stages
// skipped, which keeps the compiler's waits exact.  Workgroups are numbered
// so that the leaves with the most input groups come first.  Outputs leave
// through LDS as 16-byte row stores.

template <bool SWIGLU, int NSET, typename Tout>
__global__ __launch_bounds__(256, 2) void leaf_tile_kernel(LeafParams p) {
  using Tin = __bf16;
  constexpr int TM = 128, KC = 64;
  constexpr int TN = SWIGLU ? 64 : 128;               // output columns per workgroup
  constexpr int XRS = KC * 2 + 16;                    // staged activation row (bytes)
  constexpr int XST = TM * XRS;                       // 18 KiB per stage
  constexpr int OSTR = TN + 8;
  constexpr int LDS_BYTES = 2 * XST > TM * OSTR * int(sizeof(Tout)) ? 2 * XST : TM * OSTR * int(sizeof(Tout));
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];

  const int tid = int(threadIdx.x);
  const int lane = tid % kWave, wave = tid / kWave;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;    // this wave's rows wm*64.., column half wn
  const int q = p.q;
  const int nstrips = p.b_out / 16;
  const int strip_bytes = p.b_in * 32;
  const int64_t blk_bytes = int64_t(p.b_in) * p.b_out * 2;
  const unsigned char* W0 = static_cast<const unsigned char*>(p.W0);
  const unsigned char* W1 = static_cast<const unsigned char*>(p.W1);
  const Tin* __restrict__ X = static_cast<const Tin*>(p.X);
  Tout* __restrict__ Y = static_cast<Tout*>(p.Y);

  // ---- tile, XCD-aware: XCD x (blockIdx % 8) owns the m-tiles mt = x, x + 8,
  // ... of every leaf, and its workgroups (blockIdx / 8, in dispatch order)
  // walk them leaf class by leaf class (most input groups first, so that the
  // long tiles start first), then row type, m-tile and n-tile.  An XCD thus
  // keeps re-reading its own activation m-tiles and the weight strips of a
  // few leaves from its L2; dealing the tiles over all XCDs in leaf order
  // had them re-read from beyond L2 (pilot FFN gate/up: L2 hit rate 54% ->
  // 81%, 62.3 -> 58.9 us; walking row type before leaf class reached 85% but
  // let long tiles start last, and the down projection lost 9 us).
  const int xcd = int(blockIdx.x % kNumXcd), slot = int(blockIdx.x / kNumXcd);
  const int mt_x = (p.mt_count - xcd + kNumXcd - 1) / kNumXcd;   // m-tiles of this XCD
  const int per_leaf = mt_x * p.nt_count;
  if (slot >= q * q * per_leaf) return;
  const int li = slot / (q * per_leaf);
  const int rem = slot - li * q * per_leaf;
  const int i = rem / per_leaf;
  const int rem2 = rem - i * per_leaf;
  const int mt = xcd + (rem2 / p.nt_count) * kNumXcd, nt = rem2 - (rem2 / p.nt_count) * p.nt_count;
  int k;
  if (p.law == AA_LAW_QQ) k = li == q - 1 ? i : (li < i ? li : li + 1);   // off-diagonal leaves first
  else k = i ^ (3 - li);   // Q2 x Q2: i ^ k = 3 (four groups), then 2 and 1 (two), then 0 (one)
  int segs[4] = {0, 0, 0, 0};
  const int nseg = device_leaf_groups(p.law, i, k, segs);
  const uint32_t gpack = uint32_t(segs[0]) | (uint32_t(segs[1]) << 2) | (uint32_t(segs[2]) << 4) | (uint32_t(segs[3]) << 6);
  const int cps = p.b_in / KC;                 // stages per input group
  const int n_stages = nseg * cps;

  // rows of this tile
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
  const int64_t m0 = int64_t(mt) * TM;
  const int nrows = m0 >= count ? 0 : int(count - m0 < TM ? count - m0 : TM);
  if (nrows <= 0) return;
  first += m0 * stride;

  // ---- per-thread load geometry (fixed for the whole K loop)
  // weights: this wave's strip a (0..3) of the tile; plain: strips
  // nt*8 + wn*4 + a of W0; SwiGLU: strips nt*4 + wn*2 + (a & 1) of W0 (a < 2,
  // gate) or W1 (a >= 2, up)
  int64_t wofs[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int sl = SWIGLU ? nt * 4 + wn * 2 + (a & 1) : nt * 8 + wn * 4 + a;
    sl = sl < nstrips ? sl : nstrips - 1;
    wofs[a] = int64_t(sl) * strip_bytes + lane * 16;
  }
  // activations: row r = j * 32 + tid / 8 (j = 0..3), 16-byte chunk tid % 8
  const Tin* xrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = j * 32 + tid / 8;
    xrow[j] = X + (first + int64_t(r < nrows ? r : 0) * stride) * p.ldx + (tid % 8) * 8;
  }

  Run<Tin> sw[NSET][KC / 32][4], sx[NSET][4];
  auto load_stage = [&](int st, Run<Tin> (&w)[KC / 32][4], Run<Tin> (&x)[4]) __attribute__((always_inline)) {
    st = st < n_stages ? st : n_stages - 1;
    const int s = st / cps, c = st - s * cps;
    const int grp = int((gpack >> (2 * s)) & 3u);
    const int gsel = p.law == AA_LAW_QQ ? (s == 0 ? i : k) : grp;
    const int64_t wb = (int64_t(gsel) * q + k) * blk_bytes + int64_t(c) * (KC / 32) * 1024;
#pragma unroll
    for (int sl = 0; sl < KC / 32; ++sl)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const unsigned char* wp = (SWIGLU && a >= 2) ? W1 : W0;
        w[sl][a] = Run<Tin>::load_cached(reinterpret_cast<const Tin*>(wp + wb + wofs[a] + sl * 1024));
      }
    const int xc = gsel * p.b_in + c * KC;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = Run<Tin>::load_cached(xrow[j] + xc);
  };
  auto store_stage = [&](int buf, const Run<Tin> (&x)[4]) __attribute__((always_inline)) {
    unsigned char* base = lds + buf * XST;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4_t*>(base + (j * 32 + tid / 8) * XRS + (tid % 8) * 16) = x[j].v;
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute_stage = [&](int buf, const Run<Tin> (&w)[KC / 32][4]) __attribute__((always_inline)) {
    const unsigned char* base = lds + buf * XST;
#pragma unroll
    for (int sl = 0; sl < KC / 32; ++sl) {
      Run<Tin> bv[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bv[b].v = *reinterpret_cast<const u32x4_t*>(base + (wm * 64 + b * 16 + l16) * XRS + (sl * 32 + g * 8) * 2);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mma(w[sl][a], bv[b], acc[a][b]);
    }
  };

#pragma unroll
  for (int s = 0; s < NSET - 1; ++s) load_stage(s, sw[s], sx[s]);
  store_stage(0, sx[0]);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  const int rounds = (n_stages + NSET - 1) / NSET;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      const int st = rd * NSET + s;
      const int sl = (s + NSET - 1) % NSET, sn = (s + 1) % NSET;
      load_stage(st + NSET - 1, sw[sl], sx[sl]);
      if (st < n_stages) compute_stage(st & 1, sw[s]);
      store_stage((st + 1) & 1, sx[sn]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_s_barrier();
    }
  }

  // ---- epilogue through LDS (both stage buffers are free after the barrier)
  Tout* otile = reinterpret_cast<Tout*>(lds);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (SWIGLU) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc[a][b][e], acc[a + 2][b][e]);
        store4(otile + (wm * 64 + b * 16 + l16) * OSTR + (wn * 2 + a) * 16 + g * 4, v);
      }
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4(otile + (wm * 64 + b * 16 + l16) * OSTR + (wn * 4 + a) * 16 + g * 4, acc[a][b]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  constexpr int VPR = TN * int(sizeof(Tout)) / 16;
  const int64_t col0 = int64_t(k) * p.b_out + int64_t(nt) * TN;
  const int ncols = p.b_out - nt * TN < TN ? p.b_out - nt * TN : TN;
#pragma unroll
  for (int e0 = 0; e0 < TM * VPR; e0 += 256) {
    const int e = e0 + tid;
    const int r = e / VPR, v = e - r * VPR;
    const int col = v * (16 / int(sizeof(Tout)));
    if (r < nrows && col < ncols) {
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(otile + r * OSTR + col);
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(Y + (first + int64_t(r) * stride) * p.ldy + col0 + col));
    }
  }
}

// --------------------------------------------------------------- decode ---

struct DecodeParams {
  const void* x;
  const void* W;
  const void* W1;   // SwiGLU: the up weight (W is the gate); else unused
  void* y;
  int64_t n;
  int64_t ldx;
  int64_t ldy;
  int32_t q;
  int32_t b_in;
  int32_t b_out;
  int32_t law;
  int32_t off_mod_q;
  const int32_t* row_types;
  int32_t nstrips;   // 16-column strips per output group
  int32_t nchunks;   // 64-column chunks per output group
};

// Decode: a workgroup computes a 64-column chunk of output group k for a
// group of TG tokens; wave w owns the chunk's w-th 16-column strip.  Every
// weight strip the wave needs - the diagonal block W_kk's strip, shared by
// the TG tokens, and for each token the strip of its own block W_ik - is
// requested before any is used, so a wave keeps (TG + 1) * KF KiB in flight.
// The tokens' activation segments are staged in LDS.  MFMA multiplies one
// 16 x 32 weight fragment by a 32 x 16 activation tile in which column j is
// token j's segment: all TG tokens at once for the diagonal block, and only
// token j's column (the others zero) for token j's own block.
template <typename Tin, typename Tout, int TG, int KF, bool SWIGLU = false>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  static_assert(TG <= 16, "one MFMA column per token");
  constexpr int NSEG = 3;                 // off-diagonal segments per token, at most (Q2 x Q2)
  __shared__ __attribute__((aligned(16))) Tin xs[TG][1 + NSEG][KF * 32];
  __shared__ int32_t tok_type[TG];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4, l16 = lane & 15;
  const int k = blockIdx.x / p.nchunks;
  const int strip = (blockIdx.x % p.nchunks) * 4 + wave;
  const int64_t tok0 = int64_t(blockIdx.y) * TG;
  const Tin* __restrict__ x = static_cast<const Tin*>(p.x);
  const Tin* __restrict__ W = static_cast<const Tin*>(p.W);
  const Tin* __restrict__ Wu = static_cast<const Tin*>(p.W1);
  Tout* __restrict__ y = static_cast<Tout*>(p.y);
  const int64_t blk = int64_t(p.b_in) * p.b_out;
  const bool strip_ok = strip < p.nstrips;
  const int64_t sofs = int64_t(strip_ok ? strip : 0) * 16 * p.b_in + lane * 8;   // strip + run, elements

  if (threadIdx.x < TG) {
    const int64_t r = tok0 + threadIdx.x;
    int ty = -1;
    if (r < p.n) {
      ty = p.row_types ? p.row_types[r] : int((p.off_mod_q + r) % p.q);
      if (ty < 0 || ty >= p.q) ty = -1;
    }
    tok_type[threadIdx.x] = ty;
  }
  __syncthreads();

  // Input groups of token j's leaf other than k (at most NSEG), by arithmetic.
  auto other_seg = [&](int ty, int s) -> int {
    if (p.law == AA_LAW_QQ) return (s == 0 && ty != k) ? ty : -1;
    int sg[4];
    const int ns = device_leaf_groups(p.law, ty, k, sg);
    int c = 0, out = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < ns && sg[e] != k) {
        if (c == s) out = sg[e];
        ++c;
      }
    return out;
  };

  // Stage the activation segments: xs[j][0] = x_j[group k], xs[j][1 + s] = x_j[other segment s].
  for (int e = threadIdx.x; e < TG * (1 + NSEG) * KF * 4; e += blockDim.x) {
    const int run = e % (KF * 4), slotseg = (e / (KF * 4)) % (1 + NSEG), j = e / (KF * 4 * (1 + NSEG));
    const int ty = tok_type[j];
    const int sg = ty < 0 ? -1 : (slotseg == 0 ? k : other_seg(ty, slotseg - 1));
    Run<Tin> v = Run<Tin>::zero();
    if (sg >= 0 && run * 8 < p.b_in) v = Run<Tin>::load_cached(x + (tok0 + j) * p.ldx + int64_t(sg) * p.b_in + run * 8);
    *reinterpret_cast<Run<Tin>*>(&xs[j][slotseg][run * 8]) = v;
  }

  // Weight strips: [0] the diagonal block's, [1 + j * NSEG + s] token j's segment s.
  // Absent strips (a token of type k, a missing token, a segment the law does
  // not use) re-read the diagonal strip, which is cached, and contribute
  // nothing because their activation column is zero.
  // In a half-width last slab (b_in an odd multiple of 16) the upper lane
  // groups have no weights; they re-read their strip's first run, and their
  // staged activations are zero.
  // With SWIGLU the same strips of the up weight are read too (u) and the
  // output is silu(gate) * up.
  constexpr int NW = 1 + TG;   // Q_q: one own block per token; Q2 x Q2 tokens loop below
  Run<Tin> w[NW][KF], u[SWIGLU ? NW : 1][KF];
  int kofs[KF];
#pragma unroll
  for (int kf = 0; kf < KF; ++kf) kofs[kf] = (kf * 32 + g * 8 < p.b_in) ? kf * 512 : 0;
  const int64_t odiag = (int64_t(k) * p.q + k) * blk + sofs;
#pragma unroll
  for (int kf = 0; kf < KF; ++kf) {
    w[0][kf] = Run<Tin>::load_cached(W + odiag + kofs[kf]);
    if (SWIGLU) u[0][kf] = Run<Tin>::load_cached(Wu + odiag + kofs[kf]);
  }
#pragma unroll
  for (int j = 0; j < TG; ++j) {
    const int ty = tok_type[j];
    const int sg = ty < 0 ? -1 : other_seg(ty, 0);
    const int64_t ob = sg >= 0 ? (int64_t(sg) * p.q + k) * blk + sofs : odiag;
#pragma unroll
    for (int kf = 0; kf < KF; ++kf) {
      w[1 + j][kf] = Run<Tin>::load(W + ob + kofs[kf]);
      if (SWIGLU) u[SWIGLU ? 1 + j : 0][kf] = Run<Tin>::load(Wu + ob + kofs[kf]);
    }
  }
  __syncthreads();   // staged activations visible

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const bool col_live = l16 < TG;
  // Diagonal block: column j = token j's segment k.
#pragma unroll
  for (int kf = 0; kf < KF; ++kf) {
    Run<Tin> b = Run<Tin>::zero();
    if (col_live) b = *reinterpret_cast<const Run<Tin>*>(&xs[col_live ? l16 : 0][0][kf * 32 + g * 8]);
    acc = mma(w[0][kf], b, acc);
    if (SWIGLU) acc1 = mma(u[0][kf], b, acc1);
  }
  // Own blocks: token j's column only.
#pragma unroll
  for (int j = 0; j < TG; ++j) {
#pragma unroll
    for (int kf = 0; kf < KF; ++kf) {
      Run<Tin> b = Run<Tin>::zero();
      if (l16 == j) b = *reinterpret_cast<const Run<Tin>*>(&xs[j][1][kf * 32 + g * 8]);
      acc = mma(w[1 + j][kf], b, acc);
      if (SWIGLU) acc1 = mma(u[SWIGLU ? 1 + j : 0][kf], b, acc1);
    }
  }
  // Q2 x Q2 tokens may have a second and third segment besides k.
  if (p.law != AA_LAW_QQ) {
    for (int j = 0; j < TG; ++j) {
      const int ty = tok_type[j];
      for (int s = 1; s < NSEG; ++s) {
        const int sg = ty < 0 ? -1 : other_seg(ty, s);
        if (sg < 0) continue;
        const int64_t ob = (int64_t(sg) * p.q + k) * blk + sofs;
        for (int kf = 0; kf < KF; ++kf) {
          Run<Tin> a = Run<Tin>::load(W + ob + kofs[kf]);
          Run<Tin> au = a;
          if (SWIGLU) au = Run<Tin>::load(Wu + ob + kofs[kf]);
          Run<Tin> b = Run<Tin>::zero();
          if (l16 == j) b = *reinterpret_cast<const Run<Tin>*>(&xs[j][1 + s][kf * 32 + g * 8]);
          acc = mma(a, b, acc);
          if (SWIGLU) acc1 = mma(au, b, acc1);
        }
      }
    }
  }
  if (SWIGLU) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = silu_mul(acc[e], acc1[e]);
  }
  // Lane holds y[token l16][strip cols g*4 .. g*4+3].
  if (col_live && strip_ok) {
    const int64_t r = tok0 + l16;
    if (r < p.n && tok_type[l16] >= 0) store4(y + r * p.ldy + int64_t(k) * p.b_out + strip * 16 + g * 4, acc);
  }
}

// Decode of one token per workgroup: a workgroup takes one 16-column strip
// of output group k for one token, and its four waves split the leaf's
// (input group, 32-row slab) pairs between them - a Q_q leaf has one or two
// input groups, a Q2 x Q2 leaf one, two or four ([review], multiplication-
// table and pilot-law paragraphs).  Every weight run a wave needs is requested
// before its first multiply, no wave waits on another's loads, and the grid
// has a workgroup per strip and token (the pilot's single-token gate/up: 96
// workgroups instead of 24 with a 64-column chunk per workgroup; the Qwen3-8B
// down projection: 256 instead of 64).  The waves' partial sums meet in LDS
// and are added in wave order.
template <typename Tout, int KF, int NSMAX, bool SWIGLU>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  using Tin = __bf16;
  constexpr int UPW = (NSMAX * KF + 3) / 4;   // (group, slab) units per wave
  __shared__ f32x4_t part[4][SWIGLU ? 2 : 1][kWave];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4, l16 = lane & 15;
  const int k = blockIdx.x / p.nstrips;
  const int strip = blockIdx.x % p.nstrips;
  const int64_t r = blockIdx.y;
  int ty = p.row_types ? p.row_types[r] : int((p.off_mod_q + r) % p.q);
  if (ty < 0 || ty >= p.q) return;   // a row the call leaves unwritten (whole workgroup)
  int sg[4];
  const int ns = device_leaf_groups(p.law, ty, k, sg);
  const Tin* __restrict__ W = static_cast<const Tin*>(p.W);
  const Tin* __restrict__ Wu = static_cast<const Tin*>(p.W1);
  const Tin* __restrict__ x = static_cast<const Tin*>(p.x);
  const int64_t blk = int64_t(p.b_in) * p.b_out;
  const int64_t sofs = int64_t(strip) * 16 * p.b_in + lane * 8;
  // Unit t of this wave is u = wave + 4 t: input group sg[u / KF], slab
  // u % KF.  Units past the leaf, slabs past b_in (KF rounded up) and the
  // upper half of a half-width last slab re-read a valid run and meet a zero
  // activation.
  Run<Tin> w[UPW], u[SWIGLU ? UPW : 1], b[UPW];
#pragma unroll
  for (int t = 0; t < UPW; ++t) {
    const int un = wave + 4 * t;
    const int s = un / KF, kf = un - s * KF;
    const bool live = s < ns && kf * 32 + g * 8 < p.b_in;
    const int j = s < ns ? sg[s] : k;
    const int64_t o = (int64_t(j) * p.q + k) * blk + sofs + (live ? kf * 512 : 0);
    w[t] = Run<Tin>::load(W + o);
    if (SWIGLU) u[t] = Run<Tin>::load(Wu + o);
    b[t] = Run<Tin>::zero();
    if (live && l16 == 0) b[t] = Run<Tin>::load_cached(x + r * p.ldx + int64_t(j) * p.b_in + kf * 32 + g * 8);
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < UPW; ++t) {
    acc = mma(w[t], b[t], acc);
    if (SWIGLU) acc1 = mma(u[t], b[t], acc1);
  }
  part[wave][0][lane] = acc;
  if (SWIGLU) part[wave][SWIGLU ? 1 : 0][lane] = acc1;
  __syncthreads();
  if (wave != 0 || l16 != 0) return;
  // lane (g, 0) holds the token's strip columns g*4 .. g*4+3
  f32x4_t sum = part[0][0][lane], sum1 = part[0][SWIGLU ? 1 : 0][lane];
#pragma unroll
  for (int v = 1; v < 4; ++v) {
    sum += part[v][0][lane];
    if (SWIGLU) sum1 += part[v][SWIGLU ? 1 : 0][lane];
  }
  if (SWIGLU) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] = silu_mul(sum[e], sum1[e]);
  }
  store4(static_cast<Tout*>(p.y) + r * p.ldy + int64_t(k) * p.b_out + strip * 16 + g * 4, sum);
}

// ----------------------------------------------------------------- pack ---

// Thread c moves one run of 8 elements: packed elements [8c, 8c + 8) from/to
// rows r .. r + 7 of one column of the row-major weight.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src, T* __restrict__ dst, int32_t q,
                                                   int32_t b_in, int32_t b_out, int64_t d_out,
                                                   int64_t n_runs, bool unpack) {
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= n_runs) return;
  const int64_t runs_per_blk = int64_t(b_in) * b_out / 8;
  const int64_t blk = c / runs_per_blk;
  const int64_t w = c - blk * runs_per_blk;
  const int64_t j = blk / q, kk = blk % q;
  const int64_t nt = w / (2 * b_in);          // a 16-column strip holds 2 * b_in runs
  const int64_t rr = w - nt * 2 * b_in;
  const int64_t kf = rr / 64, ln = rr % 64;   // slab and lane
  const int64_t row = j * b_in + kf * 32 + (ln >> 4) * 8;
  const int64_t col = kk * b_out + nt * 16 + (ln & 15);
  if (!unpack) {
    T v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[(row + e) * d_out + col];
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[c * 8 + e] = v[e];
  } else {
    T v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[c * 8 + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[(row + e) * d_out + col] = v[e];
  }
}

// ------------------------------------------------------------- variants ---

struct Variant {
  int id;
  int tn, tm, threads;
  // launches for each dtype pair
  void (*bb)(LeafParams, dim3, dim3, hipStream_t);   // bf16 -> bf16
  void (*bf)(LeafParams, dim3, dim3, hipStream_t);   // bf16 -> f32
  void (*ff)(LeafParams, dim3, dim3, hipStream_t);   // f32 -> f32
  void (*fb)(LeafParams, dim3, dim3, hipStream_t);   // f32 -> bf16
  void (*sbb)(LeafParams, dim3, dim3, hipStream_t);  // SwiGLU bf16 -> bf16
  void (*sbf)(LeafParams, dim3, dim3, hipStream_t);
  void (*sff)(LeafParams, dim3, dim3, hipStream_t);
  void (*sfb)(LeafParams, dim3, dim3, hipStream_t);
};

template <typename Tin, typename Tout, int WN, int WM, int NF, int MF, bool SW, int ST>
void launch_variant(LeafParams p, dim3 grid, dim3 block, hipStream_t s) {
  launch((leaf_gemm_kernel<Tin, Tout, WN, WM, NF, MF, SW, ST>), grid, block, 0, s, p);
}

#define AA_VARIANT(ID, WN, WM, NF, MF, ST)                                                        \
  Variant {                                                                                       \
    ID, WN * NF * 16, WM * MF * 16, kWave * WN * WM,                                              \
        launch_variant<__bf16, __bf16, WN, WM, NF, MF, false, ST>,                                \
        launch_variant<__bf16, float, WN, WM, NF, MF, false, ST>,                                 \
        launch_variant<float, float, WN, WM, NF, MF, false, ST>,                                  \
        launch_variant<float, __bf16, WN, WM, NF, MF, false, ST>,                                 \
        launch_variant<__bf16, __bf16, WN, WM, NF, MF, true, ST>,                                 \
        launch_variant<__bf16, float, WN, WM, NF, MF, true, ST>,                                  \
        launch_variant<float, float, WN, WM, NF, MF, true, ST>,                                   \
        launch_variant<float, __bf16, WN, WM, NF, MF, true, ST>                                   \
  }

const Variant kVariants[] = {
    AA_VARIANT(0, 4, 1, 2, 4, 4),   // TN 128, TM 64: few rows per type, wide blocks
    AA_VARIANT(1, 2, 2, 4, 4, 3),   // TN 128, TM 128
    AA_VARIANT(2, 1, 4, 3, 2, 4),   // TN 48,  TM 128: narrow output blocks
    AA_VARIANT(3, 2, 2, 1, 1, 4),   // TN 32,  TM 32: small problems
    AA_VARIANT(4, 4, 1, 1, 4, 4),   // TN 64,  TM 64
    AA_VARIANT(5, 4, 1, 2, 4, 2),   // TN 128, TM 64, two stages
    AA_VARIANT(6, 2, 2, 4, 4, 2),   // TN 128, TM 128, two stages
    AA_VARIANT(7, 4, 1, 6, 4, 2),   // TN 384, TM 64: one workgroup per Qwen3-8B leaf
    AA_VARIANT(8, 4, 1, 3, 4, 4),   // TN 192, TM 64
};
constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));

// Streaming variants (bf16 inputs, closed-form row maps).
struct StreamVariant {
  int id;
  int tn, tm, threads, ck;
  void (*plain_b)(LeafParams, dim3, dim3, size_t, hipStream_t);   // bf16 out
  void (*plain_f)(LeafParams, dim3, dim3, size_t, hipStream_t);   // f32 out
  void (*swi_b)(LeafParams, dim3, dim3, size_t, hipStream_t);
  void (*swi_f)(LeafParams, dim3, dim3, size_t, hipStream_t);
};

template <int WN, int WM, int NF, int MF, int CK, int GC, bool DB, bool SW, typename Tout>
void launch_stream(LeafParams p, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  launch((leaf_stream_kernel<WN, WM, NF, MF, CK, GC, DB, SW, Tout>), grid, block, lds, s, p);
}

// SwiGLU instances hold two weight streams, so they use half the group.
#define AA_STREAM(ID, WN, WM, NF, MF, CK, GC, DB, GCS)                                     \
  StreamVariant {                                                                          \
    ID, WN * NF * 16, WM * MF * 16, kWave * WN * WM, CK,                                   \
        launch_stream<WN, WM, NF, MF, CK, GC, DB, false, __bf16>,                          \
        launch_stream<WN, WM, NF, MF, CK, GC, DB, false, float>,                           \
        launch_stream<WN, WM, NF, MF, CK, GCS, DB, true, __bf16>,                          \
        launch_stream<WN, WM, NF, MF, CK, GCS, DB, true, float>                            \
  }

const StreamVariant kStream[] = {
    AA_STREAM(0, 4, 1, 2, 4, 4, 2, false, 1),   // TN 128, TM 64, 16 KiB in flight per wave
    AA_STREAM(1, 2, 2, 4, 4, 2, 2, false, 1),   // TN 128, TM 128
    AA_STREAM(2, 4, 1, 1, 4, 4, 2, false, 2),   // TN 64,  TM 64
    AA_STREAM(3, 4, 1, 2, 2, 4, 1, true, 1),    // TN 128, TM 32, double-buffered groups
    AA_STREAM(4, 3, 1, 1, 4, 4, 2, false, 2),   // TN 48,  TM 64: narrow output blocks
    AA_STREAM(5, 4, 1, 1, 4, 4, 1, true, 1),    // TN 64,  TM 64, double-buffered
    AA_STREAM(6, 3, 1, 1, 8, 4, 2, false, 1),   // TN 48,  TM 128
    AA_STREAM(7, 4, 1, 2, 4, 2, 2, true, 1),    // TN 128, TM 64, 2-slab chunks, double-buffered
    AA_STREAM(8, 8, 1, 1, 4, 4, 2, false, 2),   // TN 128, TM 64, 8 waves
};
constexpr int kNumStream = int(sizeof(kStream) / sizeof(kStream[0]));
constexpr size_t kStreamLdsMax = 64 * 1024;

// Persistent streaming variants (bf16 inputs, closed-form row maps, b_in a
// multiple of 32 * CK, at most NCH chunks per leaf).
typedef void (*LeafLaunch)(LeafParams, dim3, dim3, size_t, hipStream_t);
struct PersistVariant {
  int id;
  int tn, tm, ck, nch;
  // launchers indexed by the cache policy bits (kPol*)
  LeafLaunch plain_b[8], plain_f[8];
  LeafLaunch swi_b[8], swi_f[8];   // may be null
};

template <int NF, int MF, int CK, int NCH, bool SW, int POL, typename Tout>
void launch_persist(LeafParams p, dim3 grid, dim3 block, size_t, hipStream_t s) {
  launch((leaf_persist_kernel<NF, MF, CK, NCH, SW, POL, Tout>), grid, block, 0, s, p);
}

#define AA_PL(NF, MF, CK, NCH, SW, T)                                                            \
  {                                                                                              \
    launch_persist<NF, MF, CK, NCH, SW, 0, T>, launch_persist<NF, MF, CK, NCH, SW, 1, T>,       \
        launch_persist<NF, MF, CK, NCH, SW, 2, T>, launch_persist<NF, MF, CK, NCH, SW, 3, T>,   \
        launch_persist<NF, MF, CK, NCH, SW, 4, T>, launch_persist<NF, MF, CK, NCH, SW, 5, T>,   \
        launch_persist<NF, MF, CK, NCH, SW, 6, T>, launch_persist<NF, MF, CK, NCH, SW, 7, T>    \
  }
#define AA_PERSIST(ID, NF, MF, CK, NCH)                                                      \
  PersistVariant {                                                                           \
    ID, 4 * NF * 16, MF * 16, CK, NCH, AA_PL(NF, MF, CK, NCH, false, __bf16),                \
        AA_PL(NF, MF, CK, NCH, false, float), {}, {}                                           \
  }
#define AA_PERSIST_SW(ID, NF, MF, CK, NCH)                                                   \
  PersistVariant {                                                                           \
    ID, 4 * NF * 16, MF * 16, CK, NCH, AA_PL(NF, MF, CK, NCH, false, __bf16),                \
        AA_PL(NF, MF, CK, NCH, false, float), AA_PL(NF, MF, CK, NCH, true, __bf16),          \
        AA_PL(NF, MF, CK, NCH, true, float)                                                  \
  }

const PersistVariant kPersist[] = {
    AA_PERSIST(0, 2, 4, 4, 2),      // TN 128, TM 64: Q_q leaves with 128-wide input blocks
    AA_PERSIST_SW(1, 1, 4, 4, 2),   // TN 64,  TM 64 (also the SwiGLU gate/up instance)
    AA_PERSIST(2, 1, 4, 2, 2),      // TN 64,  TM 64: 64-wide input blocks (the Qwen3-1.7B shape)
};
constexpr int kNumPersist = int(sizeof(kPersist) / sizeof(kPersist[0]));

// Job-kernel variants (bf16 inputs, Q_q, closed-form row maps, b_in = 32 CK).
// Launchers are indexed by the two own-block policy bits; outputs are always
// stored nontemporally.
typedef void (*JobLaunch)(JobParams, dim3, dim3, hipStream_t);
struct JobVariant {
  int id;
  int tn, tm, ck;
  JobLaunch plain_b[4], plain_f[4];
  JobLaunch swi_b[4], swi_f[4];   // may be null
};

template <int NF, int MF, int CK, int NSET, bool SW, int POL, typename Tout>
void launch_job(JobParams p, dim3 grid, dim3 block, hipStream_t s) {
  launch((leaf_job_kernel<NF, MF, CK, NSET, SW, POL, Tout>), grid, block, 0, s, p);
}

#define AA_JL(NF, MF, CK, NSET, SW, T)                                                               \
  {                                                                                                  \
    launch_job<NF, MF, CK, NSET, SW, kPolYNt, T>, launch_job<NF, MF, CK, NSET, SW, kPolYNt | 1, T>, \
        launch_job<NF, MF, CK, NSET, SW, kPolYNt | 2, T>, launch_job<NF, MF, CK, NSET, SW, kPolYNt | 3, T> \
  }
#define AA_JOB(ID, NF, MF, CK, NSET)                                                               \
  JobVariant {                                                                                     \
    ID, 4 * NF * 16, MF * 16, CK, AA_JL(NF, MF, CK, NSET, false, __bf16),                          \
        AA_JL(NF, MF, CK, NSET, false, float), {}, {}                                              \
  }
#define AA_JOB_SW(ID, NF, MF, CK, NSET)                                                            \
  JobVariant {                                                                                     \
    ID, 4 * NF * 16, MF * 16, CK, AA_JL(NF, MF, CK, NSET, false, __bf16),                          \
        AA_JL(NF, MF, CK, NSET, false, float), AA_JL(NF, MF, CK, NSET, true, __bf16),              \
        AA_JL(NF, MF, CK, NSET, true, float)                                                       \
  }

const JobVariant kJob[] = {
    AA_JOB(0, 2, 4, 4, 3),      // TN 128, TM 64, two tiles in flight
    AA_JOB(1, 2, 2, 4, 4),      // TN 128, TM 32, three tiles in flight
    AA_JOB(3, 2, 4, 4, 2),      // TN 128, TM 64, one tile in flight
    AA_JOB_SW(2, 1, 4, 4, 3),   // TN 64,  TM 64 (also the SwiGLU gate/up instance)
    AA_JOB(4, 2, 2, 4, 3),      // TN 128, TM 32, two tiles in flight
    AA_JOB(5, 1, 4, 4, 4),      // TN 64,  TM 64, three tiles in flight
    AA_JOB(6, 3, 2, 4, 3),      // TN 192, TM 32, two tiles in flight
};
constexpr int kNumJob = int(sizeof(kJob) / sizeof(kJob[0]));

// K-stream variants (bf16 inputs, Q_q, closed-form row maps, b_in a multiple
// of 32 CK).  Launchers are indexed by the two own-block policy bits.
typedef void (*LeafLaunch2)(LeafParams, dim3, dim3, hipStream_t);
struct KStreamVariant {
  int id;
  int tn, tm, ck;
  int wpc;   // workgroups per CU (the VGPR budget allows three for the narrow ones)
  LeafLaunch2 plain_b[4], plain_f[4];
  LeafLaunch2 swi_b[4], swi_f[4];   // may be null
};

template <int NF, int MF, int CK, int NSET, bool SW, int POL, typename Tout>
void launch_kstream(LeafParams p, dim3 grid, dim3 block, hipStream_t s) {
  launch((leaf_kstream_kernel<NF, MF, CK, NSET, SW, POL, Tout>), grid, block, 0, s, p);
}

#define AA_KL(NF, MF, CK, NSET, SW, T)                                                                       \
  {                                                                                                          \
    launch_kstream<NF, MF, CK, NSET, SW, kPolYNt, T>, launch_kstream<NF, MF, CK, NSET, SW, kPolYNt | 1, T>, \
        launch_kstream<NF, MF, CK, NSET, SW, kPolYNt | 2, T>,                                                \
        launch_kstream<NF, MF, CK, NSET, SW, kPolYNt | 3, T>                                                 \
  }
#define AA_KS(ID, NF, MF, CK, NSET)                                                                        \
  KStreamVariant {                                                                                         \
    ID, 4 * NF * 16, MF * 16, CK, NF == 1 ? 3 : 2, AA_KL(NF, MF, CK, NSET, false, __bf16),              \
        AA_KL(NF, MF, CK, NSET, false, float), {}, {}                                                      \
  }
#define AA_KS_SW(ID, NF, MF, CK, NSET)                                                                     \
  KStreamVariant {                                                                                         \
    ID, 4 * NF * 16, MF * 16, CK, NF == 1 ? 3 : 2, AA_KL(NF, MF, CK, NSET, false, __bf16),              \
        AA_KL(NF, MF, CK, NSET, false, float), AA_KL(NF, MF, CK, NSET, true, __bf16),                      \
        AA_KL(NF, MF, CK, NSET, true, float)                                                               \
  }

const KStreamVariant kKStream[] = {
    AA_KS(0, 2, 4, 2, 3),      // TN 128, TM 64, 64-wide K chunks, two steps in flight
    AA_KS(1, 2, 4, 2, 4),      // TN 128, TM 64, three steps in flight
    AA_KS_SW(2, 1, 4, 2, 3),   // TN 64,  TM 64 (also a SwiGLU gate/up instance)
    AA_KS(3, 1, 4, 4, 3),      // TN 64,  TM 64, 128-wide K chunks (250 VGPRs: two per CU)
    AA_KS_SW(4, 1, 4, 2, 4),   // TN 64,  TM 64, three steps in flight
    AA_KS_SW(5, 2, 4, 2, 2),   // TN 128, TM 64, one step in flight
    AA_KS_SW(6, 2, 4, 1, 3),   // TN 128, TM 64, 32-wide K chunks, two steps in flight (SwiGLU gate/up)
};
constexpr int kNumKStream = int(sizeof(kKStream) / sizeof(kKStream[0]));

int64_t rows_per_type_max(const aa_plan_s& plan, int64_t M) {
  if (plan.type_kind == AA_TYPES_BLOCK_ROWS) return M / plan.q;
  return (M + plan.q - 1) / plan.q;
}

// 16-byte LDS chunks per staged activation row: the widest leaf's K padded
// to a multiple of 16 chunks.
int stream_cpr(const aa_plan_s& plan) {
  const int nseg_max = plan.law == AA_LAW_Q2XQ2 ? 4 : (plan.q > 1 ? 2 : 1);
  const int chunks = nseg_max * int(plan.b_in / 8);
  return (chunks + 15) / 16 * 16;
}

// LDS of a streaming launch: the activation tile, reused for the output tile.
size_t stream_lds_bytes(const aa_plan_s& plan, int v) {
  const size_t xt = size_t(kStream[v].tm) * (stream_cpr(plan) + 1) * 16;
  const size_t ot = size_t(kStream[v].tm) * (kStream[v].tn + 8) * (plan.out_dtype == AA_F32 ? 4 : 2);
  return xt > ot ? xt : ot;
}

// Streaming variant for this call, or -1 for the general kernel.
int choose_stream(const aa_plan_s& plan, int64_t M, bool swiglu) {
  if (plan.in_dtype != AA_BF16 || plan.type_kind == AA_TYPES_EXPLICIT || plan.law == AA_LAW_DIGRAPH) return -1;
  auto fits = [&](int v) {
    return stream_lds_bytes(plan, v) <= kStreamLdsMax && plan.b_in % (32 * kStream[v].ck) == 0;
  };
  if (plan.tile_override >= 100) {
    const int v = plan.tile_override - 100;
    return (v < kNumStream && fits(v)) ? v : -1;
  }
  if (plan.tile_override >= 0) return -1;
  const int64_t mi = rows_per_type_max(plan, M);
  // Many rows per type: the leaves are real GEMMs and the general kernel's
  // register tiling is the better fit.
  if (mi > 256) return -1;
  (void)swiglu;
  // Preference lists by output-block width; the first variant whose LDS tile
  // fits and whose chunk divides the input block wins.
  // (One output block of at most 64 columns takes the 64-wide tile even when
  // 48 would fit exactly: Qwen3-30B-A3B expert gate/up, 48-wide blocks, 8.4
  // against 9.3 us.)
  static const int wide[] = {0, 3, 7};
  static const int mid[] = {2, 3, 7};
  static const int narrow[] = {4, 2, 3};
  const bool narrow_fit = plan.b_out % 48 == 0 && plan.b_out % 64 && plan.b_out > 64;
  const int* pref = plan.b_out % 128 == 0 ? wide : (narrow_fit ? narrow : mid);
  for (int j = 0; j < 3; ++j)
    if (fits(pref[j])) return pref[j];
  return -1;
}

// Persistent variant for this call, or -1.
int choose_persist(const aa_plan_s& plan, int64_t M, bool swiglu) {
  if (plan.in_dtype != AA_BF16 || plan.type_kind == AA_TYPES_EXPLICIT) return -1;
  const int nseg_max = plan.law == AA_LAW_Q2XQ2 ? 4 : (plan.q > 1 ? 2 : 1);
  auto fits = [&](int v) {
    const PersistVariant& pv = kPersist[v];
    if (plan.b_in != 32 * pv.ck) return false;
    if (nseg_max > pv.nch) return false;
    return !swiglu || pv.swi_b[0] != nullptr;
  };
  if (plan.tile_override >= 200) {
    const int v = plan.tile_override - 200;
    return (v < kNumPersist && fits(v)) ? v : -1;
  }
  if (plan.tile_override >= 0) return -1;
  if (rows_per_type_max(plan, M) > 256) return -1;
  const int pref[] = {swiglu ? 1 : (plan.b_out % 128 == 0 ? 0 : 1), 1, 2};
  for (int v : pref) {
    if (!fits(v)) continue;
    // Below two tiles per workgroup there is nothing to pipeline, and the
    // streaming kernel does better (Qwen3-30B-A3B expert gate/up, 512 tiles:
    // SwiGLU FFN 19.2 against 22.6 us).  Digraph plans have no streaming
    // kernel.
    const PersistVariant& pv = kPersist[v];
    const int64_t tiles = int64_t(plan.q) * plan.q * ((rows_per_type_max(plan, M) + pv.tm - 1) / pv.tm) *
                          ((plan.b_out + pv.tn - 1) / pv.tn);
    if (plan.law != AA_LAW_DIGRAPH && tiles < 4 * int64_t(device_cu_count())) return -1;
    return v;
  }
  return -1;
}

int choose_variant(const aa_plan_s& plan, int64_t M) {
  if (plan.tile_override >= 0 && plan.tile_override < kNumVariants) return plan.tile_override;
  const int64_t mi = rows_per_type_max(plan, M);
  if (plan.b_out <= 32 || mi <= 32) return 3;
  if (plan.b_out <= 48) return 2;
  if (mi <= 64) return 0;
  // up to 128 rows per type each leaf is one m-tile, and two stages of
  // loads in flight do better than three (Qwen3-30B-A3B expert down
  // projection, 48-wide input blocks: 9.8 against 10.3 us)
  if (mi <= 128 && plan.in_dtype == AA_BF16) return 6;
  return 1;
}

}  // namespace

// Compute units of the current device (cached per calling thread, so calls
// from several host threads do not race on the cache).
int device_cu_count() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached_cus = cus;
    cached_dev = dev;
  }
  return cached_cus;
}

// ------------------------------------------------------------ launchers ---

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
aa_status_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AA_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(AA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return AA_OK;
}


aa_status_t after_launch(hipStream_t stream, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(AA_ERR_HIP, std::string(what) + ": launch failed: " + hipGetErrorString(e));
  static const bool debug = [] {
    const char* d = getenv("AA_DEBUG");
    return d && d[0] == '1';
  }();
  if (debug) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(AA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  }
  return AA_OK;
}

// Workgroup slots per XCD for the two-per-CU persistent kernels.
int slots_per_xcd() { return device_cu_count() * 2 / kNumXcd; }

// Job variant for this call, or -1.
int choose_job(const aa_plan_s& plan, int64_t M, bool swiglu) {
  if (plan.in_dtype != AA_BF16 || plan.law != AA_LAW_QQ) return -1;
  if (plan.type_kind != AA_TYPES_POS_MOD && plan.type_kind != AA_TYPES_BLOCK_ROWS) return -1;
  if (plan.q % kNumXcd) return -1;
  const int gpx = plan.q / kNumXcd;
  // activation offsets inside a tile are 32-bit: TM rows of stride q (or 1)
  const int64_t rstride = plan.type_kind == AA_TYPES_BLOCK_ROWS ? plan.d_in : int64_t(plan.q) * plan.d_in;
  auto fits = [&](int v) {
    const JobVariant& jv = kJob[v];
    if (plan.b_in != 32 * jv.ck) return false;
    if (rstride * jv.tm + plan.d_in >= (int64_t(1) << 32)) return false;
    if (swiglu && jv.swi_b[0] == nullptr) return false;
    const int64_t nt = (plan.b_out + jv.tn - 1) / jv.tn;
    return slots_per_xcd() / gpx >= nt;
  };
  if (plan.tile_override >= 300) {
    const int v = plan.tile_override - 300;
    return (v < kNumJob && fits(v)) ? v : -1;
  }
  if (plan.tile_override >= 0) return -1;
  if (rows_per_type_max(plan, M) > 256) return -1;
  const int v = swiglu ? 2 : 0;
  if (!fits(v)) return -1;
  // The job kernel pays a prologue per workgroup (its diagonal strip) and
  // balances a job's tiles over whole workgroups; it wins once every
  // workgroup has many tiles.  Fewer go to the persistent kernel.
  const JobVariant& jv = kJob[v];
  const int64_t mt = (rows_per_type_max(plan, M) + jv.tm - 1) / jv.tm;
  const int64_t nt = (plan.b_out + jv.tn - 1) / jv.tn;
  const int64_t tiles_per_wg = int64_t(plan.q) * plan.q * mt * nt / (int64_t(kNumXcd) * slots_per_xcd());
  return tiles_per_wg >= 16 ? v : -1;
}

// K-stream variant for this call, or -1.
int choose_kstream(const aa_plan_s& plan, int64_t M, bool swiglu) {
  if (plan.in_dtype != AA_BF16 || plan.law != AA_LAW_QQ) return -1;
  if (plan.type_kind != AA_TYPES_POS_MOD && plan.type_kind != AA_TYPES_BLOCK_ROWS) return -1;
  const int64_t rstride = plan.type_kind == AA_TYPES_BLOCK_ROWS ? plan.d_in : int64_t(plan.q) * plan.d_in;
  auto fits = [&](int v) {
    const KStreamVariant& kv = kKStream[v];
    if (plan.b_in % (32 * kv.ck)) return false;
    if (swiglu && kv.swi_b[0] == nullptr) return false;
    return rstride * kv.tm + plan.d_in < (int64_t(1) << 32);
  };
  if (plan.tile_override >= 400) {
    const int v = plan.tile_override - 400;
    return (v < kNumKStream && fits(v)) ? v : -1;
  }
  if (plan.tile_override >= 0) return -1;
  if (rows_per_type_max(plan, M) > 256) return -1;
  // 128-wide input groups go to the job and persistent kernels, and so do
  // plain projections with 64-wide ones when the persistent kernel has two
  // tiles per workgroup or more (the Qwen3-1.7B shape, 64 x 192 blocks: 15.9
  // against 19.0 us here); wider ones (a SwiGLU down projection) are
  // streamed in K chunks here.
  if (plan.b_in == 128) {
    // except the SwiGLU gate/up with 128-wide output tiles: 32-wide K chunks
    // keep two weight streams of 128-wide tiles within the register budget
    // (Qwen3-8B gate/up, weights streamed from HBM: 59.4 against 65.0 us on
    // the persistent kernel's 64-wide tiles)
    if (swiglu && !plan.swiglu_persist && plan.b_out % 128 == 0 && fits(6)) return 6;
    return -1;
  }
  if (plan.b_in == 64 && !swiglu && choose_persist(plan, M, false) >= 0) return -1;
  // 128-wide tiles when they divide the output groups (the Qwen3-8B down
  // projection: 39.4 vs 41.6 us for the 64-wide ones); 64-wide otherwise,
  // with three steps in flight (Qwen3-1.7B shape, 64 x 192 blocks: projection
  // 18.6 against 20.3 us with two, SwiGLU FFN 46.7 against 51.0 us)
  if (!swiglu && plan.b_out % 128 == 0 && fits(0)) return 0;
  return fits(4) ? 4 : (fits(2) ? 2 : -1);
}

// Large-tile kernels for leaves with many rows per type (override 500; 501
// keeps SwiGLU gate/up on the 16 x 16 tile kernel instead of the 32 x 32 one).
bool choose_tile(const aa_plan_s& plan, int64_t M) {
  if (plan.in_dtype != AA_BF16 || plan.law == AA_LAW_DIGRAPH) return false;
  if (plan.type_kind != AA_TYPES_POS_MOD && plan.type_kind != AA_TYPES_BLOCK_ROWS) return false;
  if (plan.b_in % 64) return false;
  if (plan.tile_override == 500 || plan.tile_override == 501) return true;
  if (plan.tile_override >= 0) return false;
  return rows_per_type_max(plan, M) > 256;
}

aa_status_t launch_leaf_gemm(const aa_plan_s& plan, const LeafCall& call, hipStream_t stream) {
  if (plan.layout_version == 2) return launch_small_gemm(plan, call, stream);
  if (tile32_ok(plan, call, rows_per_type_max(plan, call.M)))
    return launch_tile32(plan, call, rows_per_type_max(plan, call.M), stream);
  if (choose_tile(plan, call.M)) {
    LeafParams p{};
    p.X = call.X;
    p.W0 = call.W0;
    p.W1 = call.W1;
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
    const int64_t mi = rows_per_type_max(plan, call.M);
    p.mt_count = int32_t((mi + 127) / 128);
    const int tn = call.swiglu ? 64 : 128;   // output columns per workgroup
    p.nt_count = int32_t((plan.b_out + tn - 1) / tn);
    if (p.mt_count < 1) return AA_OK;
    // every XCD gets the same number of workgroups; those past its own tiles
    // (when the m-tiles do not divide by the XCDs) exit at once
    const int64_t n_slots = int64_t(plan.q) * plan.q * ((p.mt_count + kNumXcd - 1) / kNumXcd) * p.nt_count;
    if (n_slots * kNumXcd > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
    const dim3 grid{uint32_t(n_slots * kNumXcd), 1, 1}, block{256, 1, 1};
    const bool fout = plan.out_dtype == AA_F32;
    if (call.swiglu) {
      if (fout) launch((leaf_tile_kernel<true, 3, float>), grid, block, 0, stream, p);
      else launch((leaf_tile_kernel<true, 3, __bf16>), grid, block, 0, stream, p);
    } else {
      if (fout) launch((leaf_tile_kernel<false, 3, float>), grid, block, 0, stream, p);
      else launch((leaf_tile_kernel<false, 3, __bf16>), grid, block, 0, stream, p);
    }
    return after_launch(stream, call.swiglu ? "leaf_tile(swiglu)" : "leaf_tile");
  }
  const int kid = choose_kstream(plan, call.M, call.swiglu);
  if (kid >= 0) {
    const KStreamVariant& kv = kKStream[kid];
    LeafParams p{};
    p.X = call.X;
    p.W0 = call.W0;
    p.W1 = call.W1;
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
    const int64_t mi = rows_per_type_max(plan, call.M);
    p.mt_count = int32_t((mi + kv.tm - 1) / kv.tm);
    if (p.mt_count < 1) return AA_OK;
    p.nt_count = int32_t((plan.b_out + kv.tn - 1) / kv.tn);
    int kc = plan.q / kNumXcd;
    if (kc < 1) kc = 1;
    while (plan.q % kc) --kc;
    p.kc = kc;
    const int64_t n_tiles = int64_t(plan.q) * plan.q * p.mt_count * p.nt_count;
    if (n_tiles * (plan.b_in / (32 * kv.ck)) > int64_t(0x7fffffff))
      return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
    p.n_tiles = uint32_t(n_tiles);
    int64_t wgs = int64_t(device_cu_count()) * (plan.wg_per_cu > 0 ? plan.wg_per_cu : kv.wpc);
    const int64_t need = (n_tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (wgs > need) wgs = need;
    wgs = (wgs + kNumXcd - 1) / kNumXcd * kNumXcd;
    const dim3 grid{uint32_t(wgs), 1, 1}, block{256, 1, 1};
    int pol = (p.mt_count == 1 ? kPolWOwn : 0) | (p.nt_count == 1 ? kPolXOwn : 0);
    if (plan.persist_pol >= 0) pol = plan.persist_pol & 3;
    const bool fout = plan.out_dtype == AA_F32;
    auto fn = call.swiglu ? (fout ? kv.swi_f[pol] : kv.swi_b[pol]) : (fout ? kv.plain_f[pol] : kv.plain_b[pol]);
    fn(p, grid, block, stream);
    return after_launch(stream, call.swiglu ? "leaf_kstream(swiglu)" : "leaf_kstream");
  }
  const int jid = choose_job(plan, call.M, call.swiglu);
  if (jid >= 0) {
    const JobVariant& jv = kJob[jid];
    JobParams p{};
    p.X = call.X;
    p.W0 = call.W0;
    p.W1 = call.W1;
    p.Y = call.Y;
    p.M = call.M;
    p.ldx = plan.d_in;
    p.ldy = plan.d_out;
    p.q = plan.q;
    p.b_out = int32_t(plan.b_out);
    p.kind = plan.type_kind;
    p.off_mod_q = int32_t(call.pos_offset % plan.q);
    p.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? call.M / plan.q : 0;
    const int64_t mi = rows_per_type_max(plan, call.M);
    p.mt_count = int32_t((mi + jv.tm - 1) / jv.tm);
    if (p.mt_count < 1) return AA_OK;
    p.nt_count = int32_t((plan.b_out + jv.tn - 1) / jv.tn);
    p.gpx = plan.q / kNumXcd;
    p.wpg = slots_per_xcd() / p.gpx;
    if (plan.wg_per_cu > 0) {
      const int w = device_cu_count() * plan.wg_per_cu / kNumXcd / p.gpx;
      if (w >= p.nt_count) p.wpg = w;
    }
    if (int64_t(plan.q) * p.mt_count > int64_t(0x7fffffff))
      return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
    const dim3 grid{uint32_t(kNumXcd * p.gpx * p.wpg), 1, 1}, block{256, 1, 1};
    int pol = (p.mt_count == 1 ? kPolWOwn : 0) | (p.nt_count == 1 ? kPolXOwn : 0);
    if (plan.persist_pol >= 0) pol = plan.persist_pol & 3;
    const bool fout = plan.out_dtype == AA_F32;
    auto fn = call.swiglu ? (fout ? jv.swi_f[pol] : jv.swi_b[pol]) : (fout ? jv.plain_f[pol] : jv.plain_b[pol]);
    fn(p, grid, block, stream);
    return after_launch(stream, call.swiglu ? "leaf_job(swiglu)" : "leaf_job");
  }
  const int pid = choose_persist(plan, call.M, call.swiglu);
  if (pid >= 0) {
    const PersistVariant& pv = kPersist[pid];
    LeafParams p{};
    for (int r = 0; r < 64; ++r) p.adj[r] = plan.adj[r];
    p.X = call.X;
    p.W0 = call.W0;
    p.W1 = call.W1;
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
    const int64_t mi = rows_per_type_max(plan, call.M);
    p.mt_count = int32_t((mi + pv.tm - 1) / pv.tm);
    p.nt_count = int32_t((plan.b_out + pv.tn - 1) / pv.tn);
    int kc = plan.q / kNumXcd;
    if (kc < 1) kc = 1;
    while (plan.q % kc) --kc;
    p.kc = kc;
    const int64_t n_tiles = int64_t(plan.q) * plan.q * p.mt_count * p.nt_count;
    if (n_tiles > int64_t(0x7fffffff)) return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles");
    if (p.mt_count < 1) return AA_OK;
    p.n_tiles = uint32_t(n_tiles);
    int64_t wgs = int64_t(device_cu_count()) * (plan.wg_per_cu > 0 ? plan.wg_per_cu : 2);
    const int64_t need = (n_tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (wgs > need) wgs = need;
    wgs = (wgs + kNumXcd - 1) / kNumXcd * kNumXcd;
    const dim3 grid{uint32_t(wgs), 1, 1}, block{256, 1, 1};
    const bool fout = plan.out_dtype == AA_F32;
    int pol = (p.mt_count == 1 ? kPolWOwn : 0) | kPolYNt;
    // the last staged column block is the own activation block x_k when the
    // two input groups of a Q_q leaf fill the staged K exactly
    if (p.nt_count == 1 && plan.law != AA_LAW_Q2XQ2 && plan.q > 1 && pv.nch == 2) pol |= kPolXOwn;
    if (plan.persist_pol >= 0) pol = plan.persist_pol;
    auto fn = call.swiglu ? (fout ? pv.swi_f[pol] : pv.swi_b[pol]) : (fout ? pv.plain_f[pol] : pv.plain_b[pol]);
    fn(p, grid, block, 0, stream);
    return after_launch(stream, call.swiglu ? "leaf_persist(swiglu)" : "leaf_persist");
  }
  const int sid = choose_stream(plan, call.M, call.swiglu);
  const int vid = sid >= 0 ? 0 : choose_variant(plan, call.M);
  const Variant& v = kVariants[vid];
  const int tn = sid >= 0 ? kStream[sid].tn : v.tn;
  const int tm = sid >= 0 ? kStream[sid].tm : v.tm;
  const int threads = sid >= 0 ? kStream[sid].threads : v.threads;
  LeafParams p{};
  p.X = call.X;
  p.W0 = call.W0;
  p.W1 = call.W1;
  p.Y = call.Y;
  p.M = call.M;
  p.ldx = plan.d_in;
  p.ldy = plan.d_out;
  p.q = plan.q;
  p.b_in = int32_t(plan.b_in);
  p.b_out = int32_t(plan.b_out);
  p.law = plan.law;
  for (int r = 0; r < 64; ++r) p.adj[r] = plan.adj[r];
  p.kind = plan.type_kind;
  p.off_mod_q = int32_t(call.pos_offset % plan.q);
  p.rows_per_type = plan.type_kind == AA_TYPES_BLOCK_ROWS ? call.M / plan.q : 0;
  p.row_types = call.row_types;
  const int64_t mi = rows_per_type_max(plan, call.M);
  p.mt_count = plan.type_kind == AA_TYPES_EXPLICIT ? 1 : int32_t((mi + tm - 1) / tm);
  p.nt_count = int32_t((plan.b_out + tn - 1) / tn);
  p.cpr = stream_cpr(plan);
  int kc = plan.q / kNumXcd;
  if (kc < 1) kc = 1;
  while (plan.q % kc) --kc;
  p.kc = kc;
  const int64_t n_tiles = int64_t(plan.q) * plan.q * p.mt_count * p.nt_count;
  if (n_tiles > int64_t(0x7fffffff))
    return fail(AA_ERR_UNSUPPORTED, "aa_project_fwd: too many tiles for one launch");
  if (p.mt_count < 1) return AA_OK;
  p.n_tiles = uint32_t(n_tiles);
  const dim3 grid{uint32_t(n_tiles), 1, 1}, block{uint32_t(threads), 1, 1};
  const bool fin = plan.in_dtype == AA_F32, fout = plan.out_dtype == AA_F32;
  if (sid >= 0) {
    const StreamVariant& sv = kStream[sid];
    const size_t lds = stream_lds_bytes(plan, sid);
    auto fn = call.swiglu ? (fout ? sv.swi_f : sv.swi_b) : (fout ? sv.plain_f : sv.plain_b);
    fn(p, grid, block, lds, stream);
    return after_launch(stream, call.swiglu ? "leaf_stream(swiglu)" : "leaf_stream");
  }
  void (*fn)(LeafParams, dim3, dim3, hipStream_t);
  if (!call.swiglu) fn = fin ? (fout ? v.ff : v.fb) : (fout ? v.bf : v.bb);
  else fn = fin ? (fout ? v.sff : v.sfb) : (fout ? v.sbf : v.sbb);
  fn(p, grid, block, stream);
  return after_launch(stream, call.swiglu ? "leaf_gemm(swiglu)" : "leaf_gemm");
}

aa_status_t launch_pack(const aa_plan_s& plan, const void* src, void* dst, bool unpack, hipStream_t stream) {
  if (plan.layout_version == 2) return launch_pack_v2(plan, src, dst, unpack, stream);
  const int64_t n_runs = plan.d_in * plan.d_out / 8;
  if (n_runs == 0) return AA_OK;
  const dim3 block{256, 1, 1}, grid{uint32_t((n_runs + 255) / 256), 1, 1};
  if (plan.in_dtype == AA_BF16)
    launch(pack_kernel<__bf16>, grid, block, 0, stream, static_cast<const __bf16*>(src),
                       static_cast<__bf16*>(dst), plan.q, int32_t(plan.b_in), int32_t(plan.b_out), plan.d_out,
                       n_runs, unpack);
  else
    launch(pack_kernel<float>, grid, block, 0, stream, static_cast<const float*>(src),
                       static_cast<float*>(dst), plan.q, int32_t(plan.b_in), int32_t(plan.b_out), plan.d_out,
                       n_runs, unpack);
  return after_launch(stream, unpack ? "unpack" : "pack");
}

bool decode_swiglu_ok(const aa_plan_s& plan) {
  return plan.in_dtype == AA_BF16 && plan.b_in <= 256 && plan.law != AA_LAW_DIGRAPH && plan.layout_version == 1;
}

aa_status_t launch_decode(const aa_plan_s& plan, const void* x, const void* W, const void* W1, void* y,
                          int64_t n, int64_t pos_offset, const int32_t* row_types, hipStream_t stream) {
  // The decode of a digraph plan, and a decode of at least 2q position-typed
  // or 8q explicitly typed tokens, run as the row-typed projection of the new
  // rows (typed by position, or by the given types): the matrix-vector
  // kernel reads each token's own blocks once per token group, so its time
  // grows with the tokens, while the leaf kernels read every block once
  // (Qwen3-8B shape, by position: 32.7 against 29.9 us at 64 tokens, 441
  // against 32.7 us at 1024; explicit types: 154 against 77 us at 512, the
  // general kernel's ballot scan of the types costing more per token).
  //
  // Blocks wider than the matrix-vector kernels take (input blocks above 512
  // features; above 256 for the SwiGLU gate/up pair), and blocks of packed
  // layout 2, also run as the projection of the new rows, so that every plan
  // the leaf kernels accept decodes, whatever the token count.
  const bool too_wide = plan.b_in > 512 || (W1 != nullptr && !decode_swiglu_ok(plan)) || plan.layout_version != 1;
  if (plan.law == AA_LAW_DIGRAPH || too_wide || (W1 == nullptr && n >= (row_types ? 8 : 2) * int64_t(plan.q))) {
    aa_plan_s dp = plan;
    dp.type_kind = row_types ? AA_TYPES_EXPLICIT : AA_TYPES_POS_MOD;
    const LeafCall c{x, W, W1, y, n, pos_offset, row_types, W1 != nullptr};
    return launch_leaf_gemm(dp, c, stream);
  }
  DecodeParams p{};
  p.x = x;
  p.W = W;
  p.W1 = W1;
  p.y = y;
  p.n = n;
  p.ldx = plan.d_in;
  p.ldy = plan.d_out;
  p.q = plan.q;
  p.b_in = int32_t(plan.b_in);
  p.b_out = int32_t(plan.b_out);
  p.law = plan.law;
  p.off_mod_q = int32_t(pos_offset % plan.q);
  p.row_types = row_types;
  p.nstrips = int32_t(plan.b_out / 16);
  p.nchunks = (p.nstrips + 3) / 4;
  // KF k-slabs per input block; TG tokens per workgroup, fewer for wide
  // blocks so that (TG + 1) * KF weight runs fit the registers.
  const int kf = int((plan.b_in + 31) / 32);
  const bool fin = plan.in_dtype == AA_F32, fout = plan.out_dtype == AA_F32;
  // One token per workgroup (the waves splitting its leaf): every Q2 x Q2
  // decode, and Q_q generation (one token per call).
  const bool split = !fin && kf <= 12 && (plan.law == AA_LAW_Q2XQ2 || (plan.law == AA_LAW_QQ && n == 1));
  if (split) {
    const dim3 grid{uint32_t(plan.q * p.nstrips), uint32_t(n), 1}, block{256, 1, 1};
    auto go_split = [&](auto kf_c, auto ns_c) {
      constexpr int KFc = decltype(kf_c)::value, NSc = decltype(ns_c)::value;
      if (W1 != nullptr) {
        if (fout) launch((decode_split_kernel<float, KFc, NSc, true>), grid, block, 0, stream, p);
        else launch((decode_split_kernel<__bf16, KFc, NSc, true>), grid, block, 0, stream, p);
      } else {
        if (fout) launch((decode_split_kernel<float, KFc, NSc, false>), grid, block, 0, stream, p);
        else launch((decode_split_kernel<__bf16, KFc, NSc, false>), grid, block, 0, stream, p);
      }
    };
    auto by_kf = [&](auto ns_c) {
      if (kf <= 2) go_split(std::integral_constant<int, 2>{}, ns_c);
      else if (kf <= 4) go_split(std::integral_constant<int, 4>{}, ns_c);
      else if (kf <= 6) go_split(std::integral_constant<int, 6>{}, ns_c);
      else if (kf <= 8) go_split(std::integral_constant<int, 8>{}, ns_c);
      else go_split(std::integral_constant<int, 12>{}, ns_c);
    };
    if (plan.law == AA_LAW_Q2XQ2) by_kf(std::integral_constant<int, 4>{});
    else by_kf(std::integral_constant<int, 2>{});
    return after_launch(stream, W1 ? "decode_split(swiglu)" : "decode_split");
  }
  auto go = [&](auto tg_c, auto kf_c) {
    constexpr int TGc = decltype(tg_c)::value, KFc = decltype(kf_c)::value;
    const int64_t groups = (n + TGc - 1) / TGc;
    const dim3 block{256, 1, 1}, grid{uint32_t(plan.q * p.nchunks), uint32_t(groups), 1};
    if (groups > 65535) return false;
    if (W1 != nullptr) {   // SwiGLU gate/up (bf16 input; the caller checked KF <= 8)
      if constexpr (KFc <= 8) {
        if (fin) return false;
        if (fout) launch((decode_kernel<__bf16, float, TGc, KFc, true>), grid, block, 0, stream, p);
        else launch((decode_kernel<__bf16, __bf16, TGc, KFc, true>), grid, block, 0, stream, p);
        return true;
      } else {
        return false;
      }
    }
    if (fin && fout) launch((decode_kernel<float, float, TGc, KFc>), grid, block, 0, stream, p);
    else if (fin) launch((decode_kernel<float, __bf16, TGc, KFc>), grid, block, 0, stream, p);
    else if (fout) launch((decode_kernel<__bf16, float, TGc, KFc>), grid, block, 0, stream, p);
    else launch((decode_kernel<__bf16, __bf16, TGc, KFc>), grid, block, 0, stream, p);
    return true;
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  // A decode of one or two tokens (generation: one new position per call)
  // takes a group that size instead of leaving group slots empty.
  auto go_tg = [&](auto tg_max, auto kf_c) {
    constexpr int TGm = decltype(tg_max)::value;
    if (n == 1) return go(I1{}, kf_c);
    if (n == 2 && TGm >= 2) return go(I2{}, kf_c);
    if (TGm >= 4) return go(I4{}, kf_c);
    return go(std::integral_constant<int, TGm>{}, kf_c);
  };
  bool ok;
  switch (kf) {
    case 1: ok = go_tg(I4{}, std::integral_constant<int, 1>{}); break;
    case 2: ok = go_tg(I4{}, std::integral_constant<int, 2>{}); break;
    case 3: ok = go_tg(I4{}, std::integral_constant<int, 3>{}); break;
    case 4: ok = go_tg(I4{}, std::integral_constant<int, 4>{}); break;
    case 5: ok = go_tg(I2{}, std::integral_constant<int, 5>{}); break;
    case 6: ok = go_tg(I2{}, std::integral_constant<int, 6>{}); break;
    case 7: ok = go_tg(I2{}, std::integral_constant<int, 7>{}); break;
    case 8: ok = go_tg(I2{}, std::integral_constant<int, 8>{}); break;
    case 9: ok = go(I1{}, std::integral_constant<int, 9>{}); break;
    case 10: ok = go(I1{}, std::integral_constant<int, 10>{}); break;
    case 11: ok = go(I1{}, std::integral_constant<int, 11>{}); break;
    case 12: ok = go(I1{}, std::integral_constant<int, 12>{}); break;
    case 13: ok = go(I1{}, std::integral_constant<int, 13>{}); break;
    case 14: ok = go(I1{}, std::integral_constant<int, 14>{}); break;
    case 15: ok = go(I1{}, std::integral_constant<int, 15>{}); break;
    case 16: ok = go(I1{}, std::integral_constant<int, 16>{}); break;
    default:
      return fail(AA_ERR_UNSUPPORTED, "aa_decode_gemv: input block width d_in/q above 512");
  }
  if (!ok) return fail(AA_ERR_UNSUPPORTED, "aa_decode_gemv: too many tokens for one launch");
  return after_launch(stream, W1 ? "decode_gemv(swiglu)" : "decode_gemv");
}

}  // namespace aa
