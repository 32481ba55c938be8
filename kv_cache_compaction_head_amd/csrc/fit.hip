// Bias and value fits, in float64.
//
// "Fast KV Compaction via Attention Matching", section 2, algorithmic
// pipeline: the per-key bias is fitted by non-negative least squares on the
// attention mass of the original keys, then the values by ordinary least
// squares on the attention outputs given the kept keys and fitted bias.  With
// w = exp(beta):
//   bias:   min_{w >= 0} ||P_S w - 1||^2 + lam_w ||w - 1||^2
//   values: min_C ||X C - O||^2 + lam_v ||C - V_S||^2,  X = P_S diag(w) / r
// lam = ridge_rel * trace(Gram) / t pulls toward the prior (w = 1, C = V_S).
//
// Kernels (batched over heads; per-head sizes stay on the device, so nothing
// syncs with the host):
//   k_ps           P_S = exp(Q C_k^T - lse) on fp64 MFMA (16x16x4), with the
//                  partial column sums of each 64-query tile
//   k_atb          C = A^T B tiles on fp64 MFMA (the mass Gram, lower
//                  triangle), split-K with a fixed-order reduction
//   k_bias_lam, k_bias_prep   lam_w; H = M + lam_w I, c = P_S^T 1 + lam_w
//   k_nnls_sweep   block principal pivoting on the swept bias system
//   k_value_prep   X_F compacted at the front of each P_S row
//   k_atb2         the value Gram X_F^T X_F and X_F^T O in one launch
//   k_ridge_v, k_rhs_ridge   the value system's ridge
//   k_value_sweep  its solve by the same block sweeps
//   k_write_out    C_v and beta to the outputs.
// Keys whose multiplier is pinned at zero carry a factor 1e-30 in X; their
// coupling to the rest is ~1e-30 relative, so the value system is solved on
// the passive set only and those keys keep C_v = V (the ridge prior).
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace kvc {

constexpr int kTile = 64;   // fp64 output tile (4 waves x 32x32)
constexpr int kKC = 16;     // contraction rows staged per step
constexpr int kSB = 64;     // sweep step: pivots per step, band height

// ---------------------------------------------------------------------------
// 64x64 fp64 tile product on MFMA.  sA, sB: [kKC][kTile] in LDS, k-major.
// Wave w owns rows (w/2)*32.., cols (w%2)*32..: 2x2 MFMA 16x16 tiles.
// acc[ra][rb] element i of lane l -> row l/16 + 4*i, col l%16 of that tile (the
// f64 MFMA spreads a lane's four results over rows 4 apart, unlike the f32 forms).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_mma(const double* sA, const double* sB, f64x4 acc[2][2],
                                         int wave, int lane) {
  const int wy = wave >> 1, wx = wave & 1;
#pragma unroll
  for (int ks = 0; ks < kKC / 4; ++ks) {
    const int k = ks * 4 + (lane >> 4);
    double a[2], bb[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      a[r] = sA[k * kTile + wy * 32 + r * 16 + (lane & 15)];
      bb[r] = sB[k * kTile + wx * 32 + r * 16 + (lane & 15)];
    }
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[ra][rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ra], bb[rb], acc[ra][rb], 0, 0, 0);
  }
}

__device__ __forceinline__ int tile_row(int wave, int lane, int ra, int i) {
  return (wave >> 1) * 32 + ra * 16 + (lane >> 4) + 4 * i;
}
__device__ __forceinline__ int tile_col(int wave, int lane, int rb) {
  return (wave & 1) * 32 + rb * 16 + (lane & 15);
}

// Lower-triangular tile enumeration: bid -> (ty, tx), tx <= ty.
__device__ __forceinline__ void tri_decode(int bid, int& ty, int& tx) {
  int y = static_cast<int>((sqrtf(8.f * bid + 1.f) - 1.f) * 0.5f);
  while ((y + 1) * (y + 2) / 2 <= bid) ++y;
  while (y * (y + 1) / 2 > bid) --y;
  ty = y;
  tx = bid - y * (y + 1) / 2;
}

// ---------------------------------------------------------------------------
// P_S[b][i][a] = exp(q_i . k_{idx[a]} - lse_i), computed in fp64 and stored as
// Out (double for the fits; float for the whole-cache P of the greedy
// selection, where idx is null: every key, a = j).
// grid (ceil(n/64)*ceil(t/64), B).
// ---------------------------------------------------------------------------
template <class In, int D, class Out>
__global__ __launch_bounds__(256) void k_ps(const In* __restrict__ Q, const In* __restrict__ K,
                                            const int32_t* __restrict__ idx,
                                            const double* __restrict__ lse,
                                            Out* __restrict__ PS,
                                            double* __restrict__ colpart,
                                            const int32_t* __restrict__ tv, int n, int T, int t,
                                            int tiles_a, int qg) {
  // the whole 64 x D tiles of queries and (gathered) keys, staged once in the
  // input type with 16-byte loads and widened to fp64 as they leave LDS
  constexpr int VEC = 16 / sizeof(In), CPR = D / VEC, LDR = D + VEC;
  __shared__ __align__(16) In sQ[kTile * LDR], sK[kTile * LDR];
  const int b = blockIdx.y, ti = blockIdx.x / tiles_a, ta = blockIdx.x % tiles_a;
  const int i0 = ti * kTile, a0 = ta * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const In* Qb = Q + static_cast<size_t>(b / qg) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;
  const int32_t* ib = idx ? idx + static_cast<size_t>(b) * t : nullptr;
  const int tb = tv ? tv[b] : t;  // columns from tb on are zero (unused budget)
#pragma unroll
  for (int e = threadIdx.x; e < kTile * CPR; e += 256) {
    const int r = e / CPR, c = (e % CPR) * VEC;
    const int i = i0 + r, a = a0 + r;
    const uint4 qv = *reinterpret_cast<const uint4*>(Qb + static_cast<size_t>(i < n ? i : 0) * D + c);
    const uint4 kv = *reinterpret_cast<const uint4*>(
        Kb + static_cast<size_t>(a < tb ? (ib ? ib[a] : a) : 0) * D + c);
    *reinterpret_cast<uint4*>(&sQ[r * LDR + c]) = i < n ? qv : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&sK[r * LDR + c]) = a < tb ? kv : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  // fp64 MFMA 16x16x4 over the contraction, permuted so that in step kk of
  // group ks lane l supplies index 16 ks + 4 (l / 16) + kk: each lane reads
  // four consecutive values of a row at once
  const int wy = wave >> 1, wx = wave & 1, g = lane >> 4, l16 = lane & 15;
  f64x4 acc[2][2] = {};
#pragma unroll 2
  for (int ks = 0; ks < D / 16; ++ks) {
    const int k = 16 * ks + 4 * g;
    In av[2][4], bv[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        av[r][kk] = sQ[(wy * 32 + r * 16 + l16) * LDR + k + kk];
        bv[r][kk] = sK[(wx * 32 + r * 16 + l16) * LDR + k + kk];
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int ra = 0; ra < 2; ++ra)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[ra][rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(to_f64<In>(av[ra][kk]),
                                                             to_f64<In>(bv[rb][kk]), acc[ra][rb],
                                                             0, 0, 0);
  }
  double cs[2] = {0.0, 0.0};  // this lane's part of the tile's column sums
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + tile_row(wave, lane, ra, i), a = a0 + tile_col(wave, lane, rb);
        if (r < n && a < t) {
          const double v = a < tb ? exp(acc[ra][rb][i] - lse[static_cast<size_t>(b) * n + r]) : 0.0;
          PS[(static_cast<size_t>(b) * n + r) * t + a] = static_cast<Out>(v);
          cs[rb] += v;
        }
      }
  // column sums of the tile's 64 rows, in a fixed order, one partial per
  // (query tile, column): c = P_S^T 1 without reading P_S again
  if (colpart) {
    __shared__ double sCol[2][kTile];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      cs[rb] += __shfl_xor(cs[rb], 16);
      cs[rb] += __shfl_xor(cs[rb], 32);
      if (lane < 16) sCol[wave >> 1][(wave & 1) * 32 + rb * 16 + lane] = cs[rb];
    }
    __syncthreads();
    const int a = a0 + static_cast<int>(threadIdx.x);
    if (threadIdx.x < kTile && a < t)
      colpart[(static_cast<size_t>(b) * (gridDim.x / tiles_a) + ti) * t + a] =
          sCol[0][threadIdx.x] + sCol[1][threadIdx.x];
  }
}

// ---------------------------------------------------------------------------
// C[b][a][c] = sum_i A[b][i][ca(a)] * Bm[b][i][c]  for a < mA_b, c < mB_b.
// ca: optional per-head column map of A.  SYM: B = A, lower tiles only, and
// only the lower triangle is stored (every reader of the swept systems reads
// the lower triangle).  Each head has G workgroups.  Its split into row slices follows
// its own sizes (atb_shape), which only the device knows for the value fit's
// passive set: with ks > 1 workgroup g sums slice g / nt of tile g % nt into
// part[b][slice][tile][64*64] and k_atb_reduce adds the slices in order;
// with ks = 1 workgroup g computes tile g whole (G is at least every head's
// tile count).  The next
// 16-row chunk is fetched into registers while the MFMAs consume the current
// one.
// ---------------------------------------------------------------------------
struct AtbShape {
  int nt, ks, per;  // tiles, row slices, 16-row chunks per slice
};
constexpr int kAtbGrid = 2048;  // workgroups a product aims for, over all heads
__host__ __device__ inline AtbShape atb_shape(int mA, int mB, bool sym, int G, int cap_tiles,
                                              int nrows, int B) {
  const int ta = (mA + kTile - 1) / kTile, tb = (mB + kTile - 1) / kTile;
  const int nchunk = (nrows + kKC - 1) / kKC;
  AtbShape sh;
  sh.nt = sym ? ta * (ta + 1) / 2 : ta * tb;
  int ks = 1;
  if (sh.nt > 0) {
    ks = G / sh.nt;
    if (ks > kAtbGrid / (B * sh.nt)) ks = kAtbGrid / (B * sh.nt);  // enough work already
    if (ks > cap_tiles / sh.nt) ks = cap_tiles / sh.nt;  // partials of a head
    if (ks > 16) ks = 16;
    if (ks > nchunk / 4) ks = nchunk / 4;  // at least 4 chunks a slice
    if (ks < 1) ks = 1;
  }
  sh.ks = ks;
  sh.per = (nchunk + ks - 1) / ks;
  return sh;
}

__device__ __forceinline__ void atb_decode(bool sym, int tile, int tb, int& ty, int& tx) {
  if (sym) tri_decode(tile, ty, tx);
  else {
    ty = tile / tb;
    tx = tile % tb;
  }
}

// One 64 x 64 tile (a0, c0) over rows [k0, k1) into acc.  live: whether this
// wave's 32 x 32 quadrant holds entries that are needed (a wave whose
// quadrant is past the sizes or strictly above the diagonal still stages its
// share of the chunks, but issues no MFMAs).
template <class TB, bool SYM>
__device__ __forceinline__ void atb_tile(const double* __restrict__ Ab, int lda,
                                         const int32_t* __restrict__ ca,
                                         const TB* __restrict__ Bb, int ldb, int mA, int mB,
                                         int a0, int c0, int k0, int k1, double* sAt, double* sBt,
                                         f64x4 (&acc)[2][2], bool live = true) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // each thread stages one column of A and of B, rows r0, r0 + 4, ... of a
  // chunk; r0 is its wave's index, so each load is a uniform row address plus
  // a per-lane column offset
  constexpr int NE = kKC * kTile / 256, RS = 256 / kTile;
  const int r0 = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kTile);
  const int cl = static_cast<int>(threadIdx.x) % kTile;
  const int colA = a0 + cl < mA ? (ca ? ca[a0 + cl] : a0 + cl) : -1;
  const int colB = c0 + cl < mB ? (SYM ? (ca ? ca[c0 + cl] : c0 + cl) : c0 + cl) : -1;
  double va[NE], vb[NE];
  auto fetch = [&](int kbase) {
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int i = kbase + r0 + q * RS;
      const double* rowA = Ab + static_cast<size_t>(i) * lda;
      va[q] = (i < k1 && colA >= 0) ? rowA[colA] : 0.0;
      if (SYM)
        vb[q] = (i < k1 && colB >= 0) ? rowA[colB] : 0.0;
      else
        vb[q] = (i < k1 && colB >= 0)
                    ? static_cast<double>(Bb[static_cast<size_t>(i) * ldb + colB])
                    : 0.0;
    }
  };
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[ra][rb] = f64x4{0.0, 0.0, 0.0, 0.0};
  if (k0 < k1) fetch(k0);
  // (the loop is written out twice, with and without the MFMAs, so that the
  // accumulators carry no merge across a branch inside it)
  auto chunks = [&](auto mfma) {
    for (int k = k0; k < k1; k += kKC) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < NE; ++q) {
        const int e = threadIdx.x + q * 256;
        sAt[e] = va[q];
        sBt[e] = vb[q];
      }
      __syncthreads();
      if (k + kKC < k1) fetch(k + kKC);
      if constexpr (decltype(mfma)::value) tile_mma(sAt, sBt, acc, wave, lane);
    }
  };
  if (live) chunks(std::true_type{});
  else chunks(std::false_type{});
}

// One product of a launch: C = A^T B over heads (see k_atb).
template <class TB>
struct AtbArgs {
  const double* A;
  size_t sA;
  int lda;
  const int32_t* colA;
  size_t sColA;
  const TB* Bm;
  size_t sB;
  int ldb;
  double* C;
  size_t sC;
  int ldc, nrows;
  const int32_t* msz;
  int mA_const, mB_const;
  double* part;
  int G, cap_tiles;
};

// Workgroup bid (< B G) of product p.
template <class TB, bool SYM>
__device__ __forceinline__ void atb_block(const AtbArgs<TB>& p, int B, int bid, double* sAt,
                                          double* sBt) {
  const int G = p.G, b = bid / G, g = bid % G;
  const int mA = p.msz ? p.msz[b] : p.mA_const;
  const int mB = SYM ? mA : p.mB_const;
  const AtbShape sh = atb_shape(mA, mB, SYM, G, p.cap_tiles, p.nrows, B);
  if (g >= sh.nt * sh.ks && sh.ks > 1) return;
  const int tb = (mB + kTile - 1) / kTile;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const double* Ab = p.A + b * p.sA;
  const TB* Bb = p.Bm + b * p.sB;
  const int32_t* ca = p.colA ? p.colA + b * p.sColA : nullptr;
  // ks = 1: tile g over all rows, into C; else tile g % nt over row slice
  // g / nt, into the partials (G is at least the tile count of every head)
  const bool whole = sh.ks == 1;
  const int split = whole ? 0 : g / sh.nt, tile = whole ? g : g % sh.nt;
  if (tile >= sh.nt) return;
  const int k0 = whole ? 0 : split * sh.per * kKC;
  const int k1 = whole ? p.nrows : min(p.nrows, (split + 1) * sh.per * kKC);
  double* Cb = p.C + b * p.sC;
  f64x4 acc[2][2];
  int ty, tx;
  atb_decode(SYM, tile, tb, ty, tx);
  const int a0 = ty * kTile, c0 = tx * kTile;
  // this wave's quadrant: wanted unless past the sizes or (symmetric)
  // strictly above the diagonal
  const int qa = a0 + (wave >> 1) * 32, qc = c0 + (wave & 1) * 32;
  const bool live = qa < mA && qc < mB && !(SYM && qa < qc);
  atb_tile<TB, SYM>(Ab, p.lda, ca, Bb, p.ldb, mA, mB, a0, c0, k0, k1, sAt, sBt, acc, live);
  if (!live) return;
  double* P =
      p.part + (static_cast<size_t>(b) * p.cap_tiles + split * sh.nt + tile) * (kTile * kTile);
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = tile_row(wave, lane, ra, i), cc = tile_col(wave, lane, rb);
        const int r = a0 + rr, c = c0 + cc;
        if (!whole) {
          P[rr * kTile + cc] = acc[ra][rb][i];
        } else if (r < mA && c < mB && !(SYM && r < c)) {
          Cb[static_cast<size_t>(r) * p.ldc + c] = acc[ra][rb][i];
        }
      }
}

template <class TB, bool SYM>
__global__ __launch_bounds__(256) void k_atb(AtbArgs<TB> p, int B) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  atb_block<TB, SYM>(p, B, blockIdx.x, sAt, sBt);
}

// Two independent products in one launch (the value system's Gram and its
// right-hand side): the first B G1 workgroups take the first, the rest the
// second, so neither launch's tail waits on its own.
template <class TB1, bool S1, class TB2, bool S2>
__global__ __launch_bounds__(256) void k_atb2(AtbArgs<TB1> p1, AtbArgs<TB2> p2, int B) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  const int n1 = B * p1.G;
  if (static_cast<int>(blockIdx.x) < n1) atb_block<TB1, S1>(p1, B, blockIdx.x, sAt, sBt);
  else atb_block<TB2, S2>(p2, B, blockIdx.x - n1, sAt, sBt);
}

// Sum a head's row slices of each tile in order and store (the lower
// triangle of a symmetric product); nothing to do for heads computed whole.
// grid (tiles that may split * 16, B), block 256: one element per thread.
template <class TB, bool SYM>
__device__ __forceinline__ void atb_reduce_block(const AtbArgs<TB>& p, int B, int b, int bx) {
  const int tile = bx >> 4;
  const int mA = p.msz ? p.msz[b] : p.mA_const;
  const int mB = SYM ? mA : p.mB_const;
  const AtbShape sh = atb_shape(mA, mB, SYM, p.G, p.cap_tiles, p.nrows, B);
  if (sh.ks == 1 || tile >= sh.nt) return;
  int ty, tx;
  atb_decode(SYM, tile, (mB + kTile - 1) / kTile, ty, tx);
  const int a0 = ty * kTile, c0 = tx * kTile;
  double* Cb = p.C + b * p.sC;
  const double* P = p.part + (static_cast<size_t>(b) * p.cap_tiles + tile) * (kTile * kTile);
  const int e = (bx & 15) * 256 + threadIdx.x;
  const int r = a0 + e / kTile, c = c0 + e % kTile;
  if (SYM && r < c) return;
  double v = 0.0;
  for (int sp = 0; sp < sh.ks; ++sp) v += P[static_cast<size_t>(sp) * sh.nt * kTile * kTile + e];
  if (r < mA && c < mB) Cb[static_cast<size_t>(r) * p.ldc + c] = v;
}

template <class TB, bool SYM>
__global__ __launch_bounds__(256) void k_atb_reduce(AtbArgs<TB> p) {
  atb_reduce_block<TB, SYM>(p, gridDim.y, blockIdx.y, blockIdx.x);
}

// The reductions of k_atb2's two products: x blocks [0, r1) the first.
template <class TB1, bool S1, class TB2, bool S2>
__global__ __launch_bounds__(256) void k_atb_reduce2(AtbArgs<TB1> p1, AtbArgs<TB2> p2, int r1) {
  if (static_cast<int>(blockIdx.x) < r1) atb_reduce_block<TB1, S1>(p1, gridDim.y, blockIdx.y, blockIdx.x);
  else atb_reduce_block<TB2, S2>(p2, gridDim.y, blockIdx.y, blockIdx.x - r1);
}

// Block-wide sum (blockDim 256..1024), deterministic tree order.
__device__ double block_sum(double v, double* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < nw; ++w) s += sh[w];
  __syncthreads();
  return s;
}

__device__ double block_max(double v, double* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  double s = -INFINITY;
  for (int w = 0; w < nw; ++w) s = fmax(s, sh[w]);
  __syncthreads();
  return s;
}

__device__ int block_count(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < nw; ++w) s += sh[w];
  __syncthreads();
  return s;
}

// Bias system of head b in its sweep matrix (right-hand side in row 0,
// variables from row 64; see the sweep engine below): the Gram M = P_S^T P_S
// is already in the variable block.  k_bias_lam: lam_w = ridge * tr(M) / t,
// and the scale tr(M) / t beside it for a raised ridge (grid (B), block
// 1024).  k_bias_prep, one wave per row a: c_a = (P_S^T 1)_a from the
// partial column sums k_ps writes per 64-query tile (lanes 0..3 each add a
// quarter of the tiles in order, then the quarters are added in order; c is
// kept for a raised ridge), lam_w added to the diagonal, c_a + lam_w stored in
// column 0 and columns 1..63 (unused right-hand-side slots) cleared (grid
// (ceil(t/16), B), block 1024); its threads also clear the team barrier words
// of the pivoting launch that follows.
__global__ __launch_bounds__(1024) void k_bias_lam(const double* __restrict__ S, size_t sS, int ld,
                                                   double* __restrict__ lam,
                                                   const int32_t* __restrict__ tv, int t_str,
                                                   double ridge) {
  __shared__ double sh[16];
  const int b = blockIdx.x;
  const int t = tv ? tv[b] : t_str;
  const double* Sb = S + b * sS;
  double tr = 0.0;
  for (int a = threadIdx.x; a < t; a += blockDim.x)
    tr += Sb[static_cast<size_t>(kSB + a) * ld + kSB + a];
  tr = block_sum(tr, sh);
  if (threadIdx.x == 0) {
    lam[2 * b] = ridge * tr / t;
    lam[2 * b + 1] = tr / t;
  }
}
// Every thread of the grid clears its share of the nbar team barrier words.
__device__ __forceinline__ void clear_bar(unsigned* __restrict__ bar, int nbar) {
  const size_t nt = static_cast<size_t>(gridDim.x) * gridDim.y * blockDim.x;
  for (size_t i = (static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x +
                  threadIdx.x;
       i < static_cast<size_t>(nbar); i += nt)
    bar[i] = 0u;
}
__global__ __launch_bounds__(1024) void k_bias_prep(double* __restrict__ S, size_t sS, int ld,
                                                    const double* __restrict__ part, int nslab,
                                                    double* __restrict__ colsum,
                                                    const double* __restrict__ lam,
                                                    const int32_t* __restrict__ tv, int t_str,
                                                    unsigned* __restrict__ bar, int nbar) {
  clear_bar(bar, nbar);
  const int b = blockIdx.y;
  const int t = tv ? tv[b] : t_str;
  const double lw = lam[2 * b];
  const int lane = threadIdx.x & 63, a = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (a >= t) return;
  const int per = (nslab + 3) / 4, k0 = min(nslab, lane * per), k1 = min(nslab, k0 + per);
  double qs = 0.0;
  if (lane < 4)
    for (int k = k0; k < k1; ++k) qs += part[(static_cast<size_t>(b) * nslab + k) * t_str + a];
  const double q1 = __shfl(qs, 1), q2 = __shfl(qs, 2), q3 = __shfl(qs, 3);
  const double c = ((qs + q1) + q2) + q3;  // lane 0's value is the one used
  if (lane == 0) colsum[static_cast<size_t>(b) * t_str + a] = c;
  double* row = S + b * sS + static_cast<size_t>(kSB + a) * ld;
  row[lane] = lane == 0 ? c + lw : 0.0;
  if (lane == 0) row[kSB + a] += lw;
}

// Teams.  The iterative parts of the fits (the NNLS pivoting rounds and the
// value system's sweeps) run in launches whose grid is no larger than what
// the device holds at once (occupancy times compute units), so on a device
// not busy with other long-running work every workgroup is resident: each
// head gets a team of g workgroups synchronised by team_sync, a barrier
// through per-member flags in global memory.  (Plain launches: a
// cooperative launch would add nothing these barriers use, and under a
// profiler a process that had made one crashed in the HIP runtime's exit
// handler.)
//
// Placement and coherence: workgroups are dispatched round-robin over the
// XCDs, so with nteams a multiple of 8, team = blockIdx mod nteams keeps a
// team on one XCD, sharing one L2.  At start every member records its
// hardware XCC id.  If a team's members all match, its barrier only has every
// wave wait for its stores (which write through the CU's L1 into the shared
// L2) and, after the wait, invalidates the CU's L1 so later loads see the
// other members' data.  Otherwise the team falls back to agent-scope fences
// (L2 write-back and invalidate), which are correct for any placement.  The
// few control words (sizes, tolerances, pivoting state) are always read and
// written with agent-scope atomics.
//
// Every wait is bounded by the constant-rate wall clock (the bound is a kernel
// argument, 20 s unless the host sets another); a wait that runs out raises a
// flag that turns every later wait into a no-op and flags the heads, so no
// workgroup can spin forever.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;  // round-robin dispatch period

// bulk data: ordinary accesses (made coherent by team_sync)
__device__ __forceinline__ double ldc(const double* p) { return *p; }
__device__ __forceinline__ int ldc(const int32_t* p) { return *p; }
__device__ __forceinline__ void stc(double* p, double v) { *p = v; }
__device__ __forceinline__ void stc(int32_t* p, int v) { *p = v; }
// control words: agent-scope atomics
__device__ __forceinline__ double lda(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int lda(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sta(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sta(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Team {
  int rank, size;
  unsigned* flag0;  // rank 0's arrival flag; rank r's is fstride * r words on
  unsigned* mine;   // this workgroup's arrival flag
  int fstride;      // words between consecutive ranks' flags
  unsigned* tickets;  // the team's tile-task counter
  unsigned tbase;     // its value at the start of the current step's tile phase
  unsigned* ready;    // number of lookahead factors the team's lookahead member has published
  unsigned pubs;      // ... that this member has seen published
  unsigned gen;
  int* err;
  bool fast;
  uint64_t spin;  // bound on each wait, in ticks of the 100 MHz wall clock
};

__device__ __forceinline__ int hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xf;  // HW_REG_XCC_ID[3:0]
}

// A barrier is an arrival (after its stores, the workgroup writes the number
// of barriers it has reached into its own flag, a 64-byte slot) and a wait
// (wave 0 reads every member's flag, one lane per member, until all have
// reached this barrier).  One flag per member instead of one shared counter:
// no atomic read-modify-writes queue on one address, and a single vector load
// per poll sees every member.  team_sync does both; a member that needs
// nothing the others produce before the barrier may arrive, keep working, and
// wait later (team_wait before its next arrival: flags only grow, so a member
// already at the next barrier still counts as arrived at this one).
__device__ __forceinline__ void team_arrive(Team& tm) {
  if (tm.size == 1) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!tm.fast) __threadfence();
    __hip_atomic_store(tm.mine, tm.gen + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void team_wait(Team& tm) {
  if (tm.size == 1) {
    __syncthreads();
    return;
  }
  if (threadIdx.x < 64) {
    const unsigned target = tm.gen + 1;
    const int lane = threadIdx.x;
    const uint64_t t0 = wall_clock64();
    unsigned spins = 0;
    for (;;) {
      bool in = true;
      for (int r = lane; r < tm.size; r += 64)
        in &= __hip_atomic_load(tm.flag0 + static_cast<size_t>(r) * tm.fstride, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT) >= target;
      if (__all(in)) break;
      // the time-out on every poll (a scalar clock read); the error flag every
      // 32 polls: it is another memory round trip that would otherwise delay
      // seeing the last arrival
      if (wall_clock64() - t0 > tm.spin) {
        if (lane == 0) atomicOr(tm.err, 1);
        break;
      }
      if ((++spins & 31u) == 0 &&
          __hip_atomic_load(tm.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      if (tm.fast) asm volatile("buffer_inv sc1" ::: "memory");
      else __threadfence();
    }
  }
  tm.gen++;
  __syncthreads();
}

__device__ __forceinline__ void team_sync(Team& tm) {
  team_arrive(tm);
  team_wait(tm);
}

// Arrival at the next two barriers at once (the flag counts both), for a
// member that writes nothing the others read between them; it then waits
// for each of the two in turn.
__device__ __forceinline__ void team_arrive2(Team& tm) {
  if (tm.size == 1) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!tm.fast) __threadfence();
    __hip_atomic_store(tm.mine, tm.gen + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ unsigned* uniform(unsigned* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u >> 32));
  return reinterpret_cast<unsigned*>((static_cast<unsigned long long>(hi) << 32) | lo);
}
__device__ __forceinline__ Team uniform_team(const Team& t) {
  Team u;
  u.rank = __builtin_amdgcn_readfirstlane(t.rank);
  u.size = __builtin_amdgcn_readfirstlane(t.size);
  u.flag0 = uniform(t.flag0);
  u.mine = uniform(t.mine);
  u.fstride = __builtin_amdgcn_readfirstlane(t.fstride);
  u.tickets = uniform(t.tickets);
  u.tbase = __builtin_amdgcn_readfirstlane(t.tbase);
  u.ready = uniform(t.ready);
  u.pubs = __builtin_amdgcn_readfirstlane(t.pubs);
  u.gen = __builtin_amdgcn_readfirstlane(t.gen);
  u.err = reinterpret_cast<int*>(uniform(reinterpret_cast<unsigned*>(t.err)));
  u.fast = __builtin_amdgcn_readfirstlane(static_cast<int>(t.fast)) != 0;
  u.spin = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(t.spin >> 32))) << 32) |
           __builtin_amdgcn_readfirstlane(static_cast<unsigned>(t.spin));
  return u;
}

// Draws the next number from the team's ticket counter: lane 0 holds it once
// the atomic returns, and ticket_value gives it to the whole wave (only
// there does the wave wait for the atomic).
__device__ __forceinline__ unsigned draw_ticket(const Team& tm) {
  unsigned v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(tm.tickets, 1u);
  return v;
}
__device__ __forceinline__ unsigned ticket_value(unsigned drawn) {
  return __builtin_amdgcn_readfirstlane(drawn);
}

// Team of this workgroup from the XCD-aligned mapping, then one agent-fenced
// barrier to compare the members' XCC ids (fast barrier if they all match).
__device__ void team_setup(Team& tm, int& team, int& nteams, unsigned* bar, int* err, int* xcc,
                           int tx, uint64_t spin) {
  nteams = kXcds * tx;
  team = static_cast<int>(blockIdx.x % nteams);
  tm.rank = static_cast<int>(blockIdx.x / nteams);
  tm.size = static_cast<int>(gridDim.x / nteams);
  tm.fstride = kFlagStride * nteams;
  tm.flag0 = bar + static_cast<size_t>(team) * kFlagStride;
  tm.mine = bar + static_cast<size_t>(blockIdx.x) * kFlagStride;
  tm.tickets = bar + kTicketOffset + static_cast<size_t>(team) * kFlagStride;
  tm.tbase = 0;
  tm.ready = bar + kReadyOffset + static_cast<size_t>(team) * kFlagStride;
  tm.pubs = 0;
  tm.gen = 0;
  tm.err = err;
  tm.fast = false;
  tm.spin = spin;
  if (tm.size == 1) return;
  __shared__ int s_ok;
  if (threadIdx.x == 0) sta(&xcc[blockIdx.x], hw_xcc_id());
  team_sync(tm);
  if (threadIdx.x == 0) {
    const int mine = lda(&xcc[blockIdx.x]);
    int ok = 1;
    for (int r = 0; r < tm.size; ++r) ok &= lda(&xcc[team + r * nteams]) == mine;
    s_ok = ok;
  }
  __syncthreads();
  tm.fast = s_ok != 0;
}

constexpr int kMaxTeamT = 4096;            // largest t (variables of a sweep matrix)
constexpr int kMaxRows = kMaxTeamT + 128;  // rows of a sweep matrix (right-hand sides first)
// Team kernels run 256 threads per workgroup (4 waves, one 32 x 32 quadrant
// of a 64 x 64 tile each).
constexpr int kTeamThreads = 256;

// ---------------------------------------------------------------------------
// Block sweep engine.
//
// Both fits solve symmetric systems with the sweep operator (Goodnight 1979),
// applied to up to 64 variables at a time.  For a symmetric A and an index
// set F, sweeping F gives
//     [ -A_FF^-1           A_FF^-1 A_FG              ]
//     [  A_GF A_FF^-1      A_GG - A_GF A_FF^-1 A_FG  ].
// Sweeping a set P whose members are partly in F (swept back out, sign
// s = -1) and partly outside it (s = +1) is one rank-|P| update: with
// B = A_PP^-1, U = A[:, P] and V = U B,
//     A_ij -= V_i . U_j  (i, j not in P),   A_iP = V_iP s,   A_PP = -s B s.
// The generic part is applied in factored form: with A_PP = L D L^T (L unit
// lower, D the pivots, signs s), U B U^T = W D^-1 W^T for W = U L^-T, whose
// terms are bounded by the diagonal as in a Cholesky update; U B U^T formed
// through an explicit B loses everything when the pivot block is
// ill-conditioned.  The pivot rows and columns are written from V and B
// directly (folded into the update they would come out as differences of
// terms of order 1 and of order |B|).
//
// A head's matrix is the lower triangle of S (leading dimension ld): rows
// [0, r_al) are the right-hand sides (n_rhs of them), rows [r_al, r_al +
// n_var) the variables.  Right-hand sides are never swept, so once F is swept
// their columns hold A_FF^-1 b_F on F and b_G - A_GF A_FF^-1 b_F on G: the
// passive-set solution and minus the gradient elsewhere (all the NNLS
// pivoting rule reads), or the value fit's G^-1 R.
//
// One step (pivot set P, k <= 64) by a team:
//   A. the members hold L^-1 and 1/D of the pivot block A_PP = L D L^T,
//      either from the previous step's lookahead member (see sweep_step) or
//      by gathering A_PP and factoring it in LDS (small_ldl: 16-pivot
//      diagonal sweeps, panels on fp64 MFMA; the pivot blocks are
//      quasi-definite, so each pivot is nonzero with the sign s_q), and form
//      B = L^-T D^-1 L^-1 on MFMA.  They split the 32-row halves of the
//      64-row bands, gather U = A[rows, P] for theirs, form W = U L^-T and
//      V = U B on fp64 MFMA and stage both in global memory;
//   -- team barrier --
//   B. the members' waves take tile tasks of the lower triangle by ticket
//      and update them in place, A -= W D^-1 W^T on fp64 MFMA off the pivots
//      (phase A copied every pivot column, so no tile is read by another
//      member here);
//   -- team barrier --
// ---------------------------------------------------------------------------

struct __align__(16) SweepSmem {
  double pp[kSB][kSB + 1];         // pivot block, then its inverse B
  double li[kSB][kSB + 1];         // L^-1 (unit lower; identity past k)
  double rD[kSB];                  // 1 / D (0 past k)
  double sV[kSB][17];              // LDL scratch: a 16 x 17 block per wave
  double sgn[kSB];                 // s_q
  double dg[kSB];                  // pivot q's variable before any sweep (0: none)
  int piv[kSB];                    // matrix row of pivot q
  double sgn2[kSB];                // the next step's pivots (lookahead)
  int piv2[kSB];
  double u0[kSB];                  // one right-hand side: A[0, P] before the step
  double w0d[kSB];                 // ... its W row times 1/D
  double v0[kSB];                  // ... and its V row
  int16_t list[kMaxTeamT];         // NNLS: variables exchanged this round
  int16_t pos[kMaxRows];           // matrix row -> pivot slot, -1 if not a pivot
  uint8_t inF[kMaxTeamT];   // NNLS: passive set
  double red[16];
  int ired[16];
  int scan[16];
};
// The team kernels' LDS, at file scope so that the (non-inlined) helpers
// address it as LDS rather than through generic pointers.
__shared__ SweepSmem g_sw;

// Global-memory doubles: the helpers below are not inlined into the kernels,
// so their pointers must say which address space they point into, or every
// access becomes a generic (flat) one that the compiler has to order against
// LDS traffic.
typedef __attribute__((address_space(1))) double gdouble;

struct SweepMat {
  gdouble* S;      // lower triangle, ld x ld
  gdouble* U;      // [rows][64] W = A[:, P] L^-T of the step
  gdouble* V;      // [rows][64] A[:, P] B
  gdouble* stage;  // [kStage] L^-1 (at kSB*kSB) and 1/D (at 2*kSB*kSB) of the next step
  int ld, r_al, n_rhs, n_var;
  // the variables' diagonal before any sweep (the relative pivot test), or
  // null: sign test only
  const gdouble* dg0;
};
constexpr int kStage = kSweepStage;
static_assert(kSweepStage == 2 * kSB * kSB + kSB, "staging layout");
__device__ __forceinline__ gdouble* gptr(double* p) { return (gdouble*)p; }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ gdouble* uniform(gdouble* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u >> 32));
  return reinterpret_cast<gdouble*>((static_cast<unsigned long long>(hi) << 32) | lo);
}
__device__ __forceinline__ SweepMat uniform_mat(const SweepMat& m) {
  return SweepMat{uniform(m.S),     uniform(m.U),    uniform(m.V),     uniform(m.stage),
                  uniform(m.ld),    uniform(m.r_al), uniform(m.n_rhs), uniform(m.n_var),
                  uniform(const_cast<gdouble*>(m.dg0))};
}

__device__ __forceinline__ size_t s_idx(const SweepMat& M, int i, int j) {
  return i >= j ? static_cast<size_t>(i) * M.ld + j : static_cast<size_t>(j) * M.ld + i;
}
__device__ __forceinline__ double s_at(const SweepMat& M, int i, int j) { return M.S[s_idx(M, i, j)]; }
// A(i, j) if ok, else 0: the load is issued unconditionally (from element 0
// when !ok), so a batch of these stays one batch of loads instead of a chain
// of branches that each wait for their load.
__device__ __forceinline__ double s_at_or0(const SweepMat& M, bool ok, int i, int j) {
  const double v = M.S[ok ? s_idx(M, i, j) : 0];
  return ok ? v : 0.0;
}
__device__ __forceinline__ bool s_active(const SweepMat& M, int s) {
  return s < M.n_rhs || (s >= M.r_al && s < M.r_al + M.n_var);
}


__device__ double wg_max(double v) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sm.red[wave] = v;
  __syncthreads();
  double s = -INFINITY;
#pragma unroll
  for (int w = 0; w < kTeamThreads / 64; ++w) s = fmax(s, sm.red[w]);
  return s;
}

__device__ int wg_imax(int v) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sm.ired[wave] = v;
  __syncthreads();
  int s = -1;
#pragma unroll
  for (int w = 0; w < kTeamThreads / 64; ++w) s = max(s, sm.ired[w]);
  return s;
}

// Order-preserving append: every thread with f set gets slot base + (number
// of set flags in lower threads); returns base + total.  *slot = its slot.
__device__ int wg_append(bool f, int base, int* slot) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(f);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) sm.scan[wave] = __popcll(m);
  __syncthreads();
  int off = base, tot = base;
#pragma unroll
  for (int w = 0; w < kTeamThreads / 64; ++w) {
    const int c = sm.scan[w];
    off += w < wave ? c : 0;
    tot += c;
  }
  *slot = off + below;
  return tot;
}

// The pivot block sm.pp[0:k][0:k] = A_PP = L D L^T (small_ldl; sm.pp is
// overwritten) gives sm.li = L^-1 (identity past k) and sm.rD = 1/D (0 past
// k); small_b then forms B = A_PP^-1 = L^-T D^-1 L^-1 on fp64 MFMA.  The
// factorization is blocked by 16 pivots; a diagonal block is swept pivot by
// pivot (Gauss-Jordan), and before sweep p its pivot row holds
// -L_bb^-1[p][j] at the swept columns j < p and the pivot on the diagonal.
// Inverting the pivot block by a blocked sweep instead would form its
// off-diagonal parts through explicit inverses of the 16 x 16 blocks and lose
// them when those are ill-conditioned.  A pivot without the sign s_p is
// replaced by s_p (the system is not numerically definite); small_ldl's
// return value, meaningful in wave 0, says whether that happened.
// The wave's index in the workgroup as a wave-uniform value: the compiler
// cannot tell that threadIdx.x / 64 is the same across a wave, and would
// otherwise treat every branch and address derived from it as divergent.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Lane src's value of v, for the whole wave (two 32-bit lane reads).
__device__ __forceinline__ double rdlane(double v, int src) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(u), src);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(u >> 32), src);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// 1/d by Newton-Raphson from the hardware estimate (about 2^-24 relative;
// two steps, each squaring the relative error: within an ulp or so of the
// rounded quotient).  The pivot chain waits on this reciprocal at every
// pivot; the IEEE division sequence is twice as long.
__device__ __forceinline__ double recip(double d) {
  double r = __builtin_amdgcn_rcp(d);
  double e = fma(-d, r, 1.0);
  r = fma(r, e, r);
  e = fma(-d, r, 1.0);
  return fma(r, e, r);
}

// Sweep of a 16 x 16 diagonal block by the 16 lanes of each 16-lane row of a
// wave: lane c holds column c of the block, a[r] = A[o + r][o + c] (the
// four rows of lanes compute the same thing; the first one stores).  The
// pivot row is then lane-local (A[M][c] = a[M]); the pivot column A[r][M]
// comes from lane M through a DPP row broadcast fused into the update FMA
// (v_fmac_f64 with row_newbcast on its first source), so a row update costs
// one FMA and no separate data movement.
//
// Pivot M, with d = A[M][M] and s, thr its sign and threshold:
//   ok  = d s > thr (a failed pivot is replaced by s, so 1/s = s)
//   r   = 1/d (hardware estimate + two Newton-Raphson steps)
//   be  = -A[M][c] r off the pivot lane, 0 on it
//   a[i] += A[i][M] be for every row i != M;
// the pivot row becomes A[M][c] r (tm), -1 on the pivot lane.  Instead of
// rewriting the pivot column by 1/d, the pivot lane records r as its column
// scale sc (be = 0 leaves its rows as they are): a swept column's stored
// values are its true values over sc, and the updates of later pivots need
// no correction (the scale of the pivot column is still 1 when it is swept,
// and a lane's own scale cancels out of its update); only the L^-1 record
// reads true values.  lcol[M] records row M of the block's L^-1 at column c
// (-A[M][c] at the swept columns c < M, 1 at c = M, 0 after).
//
// The chain from one pivot to the next is d -> ok -> r -> be -> the update
// of row M + 1 (the next pivot's row).  Each pivot's block therefore updates
// rows M + 1 and M + 2 at once and leaves its other 13 rows to the next
// block, whose instructions interleave them with its own dependent chain
// (the waves issue in order, so independent work has to sit between the
// dependent steps to hide their latency).  Hand-scheduled asm, with the
// wait states the hardware asks for: two between a VALU write of a register
// and its read through DPP (the s_nop 1 that opens each block covers
// whatever the compiler placed between blocks; inside a block the deferred
// row of M + 3 comes first, ahead of the next block's update of that row),
// one between the reciprocal estimate and its first use.  ok is the same in
// every lane (d, s and thr are), so the substitution of s for d is a move
// under an exec mask built from it; `bad` collects the lanes of failed
// pivots.
struct DiagTmp {
  double x, y, r, tm, be, bp, sg, thr;
  unsigned long long sv, bad;
};
// sgl, thrl: lane c's own pivot's sign and threshold (broadcast from lane M
// inside block M); nn: 0 on the pivot lane, -1 elsewhere
template <int M>
__device__ __forceinline__ void diag_blk(double (&a)[16], DiagTmp& z, double sgl, double thrl,
                                         double nn);
template <> __device__ __forceinline__ void diag_blk<0>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a0] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a0], %[nn]\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "s_nop 0\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_mul_f64 %[tm], %[a0], %[r]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[be] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[be] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<1>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a1] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a1], %[nn]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a1], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[be] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[be] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<2>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a2] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a2], %[nn]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a2], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[be] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[be] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<3>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a3] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a3], %[nn]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a3], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[be] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[be] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<4>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a4] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a4], %[nn]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a4], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[be] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[be] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<5>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a5] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a5], %[nn]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a5], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[be] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[be] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<6>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a6] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a6], %[nn]\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a6], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[be] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[be] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<7>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a7] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a7], %[nn]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a7], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[be] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[be] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<8>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a8] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a8], %[nn]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a8], %[r]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[be] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[be] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<9>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a9] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a9], %[nn]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a9], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[be] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[be] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<10>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a10] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a10], %[nn]\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a10], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[be] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[be] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<11>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a11] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a11], %[nn]\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a11], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[be] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[be] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<12>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a12] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a12], %[nn]\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a12], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[be] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[be] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<13>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a13] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a13], %[nn]\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a13], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[be] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[be] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<14>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a14] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a14], %[nn]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a14], %[r]\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[be] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<15>(double (&a)[16], DiagTmp& z, double sgl,
                                                      double thrl, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a15] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[sg], %[sgl] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b64_dpp %[thr], %[thrl] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a15], %[nn]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[x], %[y], %[sg]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_cmp_lt_f64_e32 vcc, %[thr], %[x]\n"
      "v_mov_b64_e32 %[x], %[sg]\n"
      "s_and_saveexec_b64 %[sv], vcc\n"
      "v_mov_b64_e32 %[x], %[y]\n"
      "s_mov_b64 exec, %[sv]\n"
      "s_andn2_b64 %[sv], %[sv], vcc\n"
      "s_or_b64 %[bad], %[bad], %[sv]\n"
      "v_rcp_f64_e32 %[r], %[x]\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[y], -%[x], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[y], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[tm], %[a15], %[r]\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [tm] "=&v"(z.tm), [be] "=&v"(z.be),
        [sg] "=&v"(z.sg), [thr] "=&v"(z.thr), [sv] "=&s"(z.sv), [bad] "+s"(z.bad)
      : [bp] "v"(z.bp), [sgl] "v"(sgl), [thrl] "v"(thrl), [nn] "v"(nn)
      : "vcc");
}
template <> __device__ __forceinline__ void diag_blk<16>(double (&a)[16], DiagTmp& z, double, double,
                                                       double) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15])
      : [bp] "v"(z.bp));
}


// The same sweep without the pivot test on the chain (the common case):
// d goes straight to the reciprocal, and the test runs once at the end on
// each pivot's recorded reciprocal (diag_sweep).  A failed pivot leaves
// non-finite or meaningless values here, and the block is swept again by
// diag_blk, which substitutes s for d.
template <int M>
__device__ __forceinline__ void diag_fast(double (&a)[16], DiagTmp& z, double nn);
template <> __device__ __forceinline__ void diag_fast<0>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a0] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a0], %[nn]\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "s_nop 0\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[be] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[be] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<1>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a1] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a1], %[nn]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[be] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[be] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<2>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a2] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a2], %[nn]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[be] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[be] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<3>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a3] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a3], %[nn]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[be] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[be] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<4>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a4] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a4], %[nn]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[be] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[be] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<5>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a5] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a5], %[nn]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[be] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[be] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<6>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a6] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a6], %[nn]\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[be] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[be] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<7>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a7] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a7], %[nn]\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[be] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[be] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<8>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a8] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a8], %[nn]\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[be] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[be] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<9>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a9] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a9], %[nn]\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[be] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[be] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<10>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a10] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a10], %[nn]\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[be] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[be] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<11>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a11] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a11], %[nn]\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[be] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[be] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<12>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a12] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a12], %[nn]\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[be] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[be] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<13>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a13] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a13], %[nn]\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[be] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[be] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<14>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a14] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a14], %[nn]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a15], %[a15], %[be] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<15>(double (&a)[16], DiagTmp& z, double nn) {
  asm volatile(
      "s_nop 1\n"
      "v_mov_b64_dpp %[y], %[a15] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[a15], %[nn]\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_rcp_f64_e32 %[r], %[y]\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[x], -%[y], %[r], 1.0\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fma_f64 %[r], %[r], %[x], %[r]\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f64 %[be], %[be], %[r]\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),
        [x] "=&v"(z.x), [y] "=&v"(z.y), [r] "=&v"(z.r), [be] "=&v"(z.be)
      : [bp] "v"(z.bp), [nn] "v"(nn));
}
template <> __device__ __forceinline__ void diag_fast<16>(double (&a)[16], DiagTmp& z, double) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %[a0], %[a0], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a1], %[a1], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a2], %[a2], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a3], %[a3], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a4], %[a4], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a5], %[a5], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a6], %[a6], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a7], %[a7], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a8], %[a8], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a9], %[a9], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a10], %[a10], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a11], %[a11], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a12], %[a12], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a13], %[a13], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %[a14], %[a14], %[bp] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]), [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]), [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15])
      : [bp] "v"(z.bp));
}

// Threshold of a pivot's test d s > thr: a variable swept in (s = +1) needs
// d > kPivotRel * dg, dg its diagonal before any sweep (d / dg is the squared
// sine of the angle between its column and the span of the variables already
// swept: a smaller ratio means the column is numerically in that span; with
// no dg only d > 0 is asked); a variable swept out (s = -1) needs d < 0; an
// identity row past the block passes (d = 1, s = 1, thr = 0).
constexpr double kPivotRel = 1e-12;

template <int M>
__device__ __forceinline__ void diag_pivot(double (&a)[16], double (&lcol)[16], DiagTmp& z,
                                           double sgl, double thrl, int c, double& sc) {
  const bool piv = c == M;
  const double rowm = a[M];
  diag_blk<M>(a, z, sgl, thrl, piv ? 0.0 : -1.0);
  lcol[M] = c < M ? -(rowm * sc) : (piv ? 1.0 : 0.0);
  a[M] = piv ? -1.0 : z.tm;
  if (piv) sc = z.r;
  z.bp = z.be;
}
template <int... Ms>
__device__ __forceinline__ void diag_pivots(std::integer_sequence<int, Ms...>, double (&a)[16],
                                            double (&lcol)[16], DiagTmp& z, double sgl,
                                            double thrl, int c, double& sc) {
  (diag_pivot<Ms>(a, lcol, z, sgl, thrl, c, sc), ...);
}
template <int M>
__device__ __forceinline__ void diag_pivot_fast(double (&a)[16], double (&lcol)[16], DiagTmp& z,
                                                int c, double& sc) {
  const bool piv = c == M;
  const double rowm = a[M];
  diag_fast<M>(a, z, piv ? 0.0 : -1.0);
  lcol[M] = c < M ? -(rowm * sc) : (piv ? 1.0 : 0.0);
  a[M] = piv ? -1.0 : -z.be;  // off the pivot lane be = -A[M][c] r
  if (piv) sc = z.r;
  z.bp = z.be;
}
template <int... Ms>
__device__ __forceinline__ void diag_pivots_fast(std::integer_sequence<int, Ms...>,
                                                 double (&a)[16], double (&lcol)[16], DiagTmp& z,
                                                 int c, double& sc) {
  (diag_pivot_fast<Ms>(a, lcol, z, c, sc), ...);
}
// Diagonal block at o: its L^-1 into the diagonal block of sm.li (upper part
// zero), 1/D into sm.rD[o..o+15].  Run by one wave.  The fast sweep first;
// its pivots are then tested on their reciprocals r (d s > thr is r s > 0
// and r s thr < 1; a NaN or infinite r fails), and only if one fails is the
// block swept again with the test and substitution on the chain.
__device__ __forceinline__ bool diag_sweep(int o, int k) {
  SweepSmem& sm = g_sw;
  const int c = threadIdx.x & 15;
  double a[16], lcol[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = sm.pp[o + r][o + c];
  const bool in = o + c < k;
  const double sgl = in ? sm.sgn[o + c] : 1.0;
  const double thrl = in && sgl > 0.0 ? kPivotRel * sm.dg[o + c] : 0.0;
  double sc = 1.0;  // after the sweep: 1/D of pivot c
  DiagTmp z{};
  diag_pivots_fast(std::make_integer_sequence<int, 16>{}, a, lcol, z, c, sc);
  diag_fast<16>(a, z, 0.0);
  const double rs = sc * sgl;
  const bool ok = rs > 0.0 && rs * thrl < 1.0;
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = sm.pp[o + r][o + c];
    sc = 1.0;
    z = DiagTmp{};
    diag_pivots(std::make_integer_sequence<int, 16>{}, a, lcol, z, sgl, thrl, c, sc);
    diag_blk<16>(a, z, 0.0, 0.0, 0.0);
  }
  if ((threadIdx.x & 63) < 16) {
    sm.rD[o + c] = sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.li[o + r][o + c] = lcol[r];
  }
  return z.bad != 0;
}

// Blocked LDL^T helpers, one wave each, fp64 MFMA 16x16x4 (lane l supplies
// row l % 16, contraction index l / 16; results at rows l / 16 + 4 i).
// W_rj = A[r][j] L_jj^-T, parked transposed above the diagonal of sm.li:
// li[16 j + q][16 r + i] = W_rj[i][q] (that region is cleared at the end).
__device__ __forceinline__ void ldl_panel(int r, int j) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15, o = 16 * j;
  f64x4 w4 = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int m = 4 * ks + g16;
    w4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.pp[16 * r + l16][o + m], sm.li[o + l16][o + m], w4,
                                              0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) sm.li[o + l16][16 * r + g16 + 4 * x] = w4[x];
}
// A[r][c] -= W_rj D_j^-1 W_cj^T (a trailing block of step j)
__device__ __forceinline__ void ldl_trail(int r, int c, int j) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15, o = 16 * j;
  f64x4 u4 = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int q = o + 4 * ks + g16;
    u4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.li[q][16 * r + l16] * sm.rD[q],
                                              sm.li[q][16 * c + l16], u4, 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) sm.pp[16 * r + g16 + 4 * x][16 * c + l16] -= u4[x];
}
// (L^-1)[j][c] = -L_jj^-1 sum_{m=c}^{j-1} L[j][m] (L^-1)[m][c], with
// L[j][m] = W_jm D_m^-1; tmp is this wave's 16 x 17 LDS scratch.
__device__ __forceinline__ void ldl_linv(int j, int c, double (*tmp)[17]) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15, o = 16 * j;
  f64x4 t4 = {};
  for (int m = c; m < j; ++m)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int q = 16 * m + 4 * ks + g16;
      t4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.li[q][o + l16] * sm.rD[q],
                                                sm.li[q][16 * c + l16], t4, 0, 0, 0);
    }
#pragma unroll
  for (int x = 0; x < 4; ++x) tmp[g16 + 4 * x][l16] = t4[x];
  f64x4 r4 = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kk = 4 * ks + g16;
    r4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.li[o + l16][o + kk], tmp[kk][l16], r4, 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) sm.li[o + g16 + 4 * x][16 * c + l16] = -r4[x];
}

// Blocked L D L^T of the pivot block by the workgroup, two barriers per
// 16-pivot block j: first the panels W_rj (r > j) on every wave; then wave 0
// updates diagonal block j + 1 and sweeps it (the chain the next block
// waits for), while waves 1-3 update the other trailing blocks of step j and
// form the L^-1 blocks of block row j.
__device__ __forceinline__ bool small_ldl(int k) {
  SweepSmem& sm = g_sw;
  const int tid = threadIdx.x, wave = wave_id();
  const int nb = (k + 15) >> 4;
  double(*tmp)[17] = reinterpret_cast<double(*)[17]>(&sm.sV[16 * wave][0]);
  bool bad = false;
  if (wave == 0) bad = diag_sweep(0, k);
  for (int j = 0; j < nb; ++j) {
    __syncthreads();  // diagonal block j swept; every update of the steps before j done
    for (int r = j + 1, item = 0; r < nb; ++r, ++item)
      if (item % 4 == wave) ldl_panel(r, j);
    __syncthreads();  // the panels of step j parked
    if (wave == 0) {
      if (j + 1 < nb) {
        ldl_trail(j + 1, j + 1, j);
        bad |= diag_sweep(16 * (j + 1), k);
      }
    } else {
      int item = 0;
      for (int r = j + 1; r < nb; ++r)
        for (int c = j + 1; c <= r; ++c) {
          if (r == j + 1 && c == j + 1) continue;
          if (item++ % 3 == wave - 1) ldl_trail(r, c, j);
        }
      for (int c = 0; c < j; ++c)
        if (item++ % 3 == wave - 1) ldl_linv(j, c, tmp);
    }
  }
  __syncthreads();
  // 16 x 16 blocks of sm.li: the parked panels (above the diagonal) cleared,
  // blocks past the factored ones set to the identity (no pivots there);
  // wave w takes block row w
  {
    const int lane = tid & 63, g16 = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      if (wave < nb && bj <= wave) continue;  // written by the factorization
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 16 * wave + g16 + 4 * x, c = 16 * bj + l16;
        sm.li[r][c] = r == c ? 1.0 : 0.0;
      }
    }
  }
  if (tid >= k && tid < kSB) sm.rD[tid] = 0.0;
  __syncthreads();
  return bad;
}

// sm.pp <- B = L^-T D^-1 L^-1 from sm.li and sm.rD (identity and 0 past k).
__device__ __forceinline__ void small_b(int k) {
  SweepSmem& sm = g_sw;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1, g16 = lane >> 4, l16 = lane & 15;
  f64x4 acc[2][2] = {};
  // L^-1 is lower triangular: rows m below this wave's quadrant contribute nothing
  for (int ks = max(wr, wc) * 8; ks < (k + 3) / 4; ++ks) {
    const int m = 4 * ks + g16;
    const double rdm = sm.rD[m];
    double av[2], bv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      av[x] = sm.li[m][wr * 32 + x * 16 + l16] * rdm;
      bv[x] = sm.li[m][wc * 32 + x * 16 + l16];
    }
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[ra][rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ra], bv[rb], acc[ra][rb], 0, 0, 0);
  }
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wr * 32 + ra * 16 + g16 + 4 * i, col = wc * 32 + rb * 16 + l16;
        sm.pp[row][col] = (row < k && col < k) ? acc[ra][rb][i] : 0.0;
      }
  __syncthreads();
}

// Phase A for one half of a 64-row band (matrix rows band*64 + 32*half ..,
// 16 per wave pair): U = A[rows, P] gathered from the lower triangle, W =
// U L^-T and V = U B on MFMA, stored to M.U / M.V.  Half bands, so that the
// members share the bands evenly when there are fewer bands than members.
// The contraction index is permuted so that each lane's 16 values of a row
// are contiguous: in MFMA step kk, lane l supplies q = 16*(l/16) + kk.
__device__ __forceinline__ void v_band(const SweepMat& M, int band, int half, int k) {
  SweepSmem& sm = g_sw;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wr = wave >> 1, wc = wave & 1, g16 = lane >> 4, l16 = lane & 15;
  const int s0 = band * kSB + 32 * half + 16 * wr;
  double u[16];
  {
    const int s = s0 + l16;
    const bool act = s_active(M, s);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int q = g16 * 16 + kk;
      const bool ok = act && q < k;
      u[kk] = s_at_or0(M, ok, s, ok ? sm.piv[q] : 0);
    }
  }
  f64x4 acc[2] = {}, accw[2] = {};
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const int q = g16 * 16 + kk;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int c = wc * 32 + rb * 16 + l16;
      acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(u[kk], sm.pp[q][c], acc[rb], 0, 0, 0);
      accw[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(u[kk], sm.li[c][q], accw[rb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t s = static_cast<size_t>(s0 + g16 + 4 * i);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int c = wc * 32 + rb * 16 + l16;
      M.V[s * kSB + c] = acc[rb][i];
      M.U[s * kSB + c] = accw[rb][i];
    }
  }
}

// Phase B, one wave per 64 x 64 tile, no barriers: the wave streams the
// contraction in eight chunks of 8 (the next chunk's operands in flight while
// the current one's MFMAs run), accumulating all sixteen 16 x 16 blocks, then
// loads the tile's current values (32 rows at a time, one batch each) and
// stores the update.  Entries off the pivots get T -= W_I D^-1 W_J^T; pivot
// columns V_iq s_q, pivot rows V_jq s_q and the pivot block -s_q s_q' B[q][q']
// are written directly.  In MFMA step kk of chunk c, lane l supplies
// contraction index q = 8 c + 2 (l/16) + kk, so each lane reads 2 contiguous
// values per row.
// A wave's part of a tile: NRA x NRB blocks of 16 x 16 starting at block
// (ro, co) of tile (I, J) (the whole tile, a half or a quadrant).
template <int NRA, int NRB>
__device__ __forceinline__ void wave_tile_chunk(const SweepMat& M, int I, int J, int ro, int co,
                                                int c, double (&a)[NRA][2], double (&b)[NRB][2]) {
  const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int x = 0; x < NRA; ++x) {
    const gdouble* pa =
        M.U + static_cast<size_t>(I * kSB + 16 * (ro + x) + l16) * kSB + 8 * c + 2 * g16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) a[x][kk] = pa[kk];
  }
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    const gdouble* pb =
        M.U + static_cast<size_t>(J * kSB + 16 * (co + x) + l16) * kSB + 8 * c + 2 * g16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) b[x][kk] = pb[kk];
  }
}

template <int NRA, int NRB>
__device__ __forceinline__ void wave_tile_mfma(int c, bool diag, int ro, int co,
                                               const double (&a)[NRA][2],
                                               const double (&b)[NRB][2],
                                               f64x4 (&acc)[NRA][NRB]) {
  const int lane = threadIdx.x & 63, g16 = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const double rdq = g_sw.rD[8 * c + 2 * g16 + kk];
#pragma unroll
    for (int ra = 0; ra < NRA; ++ra) {
      const double av = a[ra][kk] * rdq;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        if (!diag || co + rb <= ro + ra)
          acc[ra][rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, b[rb][kk], acc[ra][rb], 0, 0, 0);
    }
  }
}

template <int NRA, int NRB>
__device__ __forceinline__ void wave_tile(const SweepMat& M, int I, int J, int ro, int co,
                                          int nch) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, g16 = lane >> 4, l16 = lane & 15;
  const bool diag = I == J;
  if (diag && co > ro + NRA - 1) return;  // strictly upper part of a diagonal tile
  f64x4 acc[NRA][NRB];
#pragma unroll
  for (int ra = 0; ra < NRA; ++ra)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[ra][rb] = f64x4{0.0, 0.0, 0.0, 0.0};
  // When every row of the part (or every column) is a pivot or inactive, no
  // entry takes the W D^-1 W^T update (pivot entries come from V and the
  // pivot block; inactive rows and columns of W are zero), so the
  // contraction is skipped.  The value fit's pivot blocks are whole bands.
  bool rfree = true, cfree = true;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int c = J * kSB + 16 * (co + rb) + l16;
    cfree &= sm.pos[c] >= 0 || !s_active(M, c);
  }
#pragma unroll
  for (int ra = 0; ra < NRA; ++ra)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = I * kSB + 16 * (ro + ra) + g16 + 4 * i;
      rfree &= sm.pos[r] >= 0 || !s_active(M, r);
    }
  if (!__all(rfree) && !__all(cfree)) {
    // the next chunk's loads are issued ahead of the current chunk's MFMAs;
    // the scheduling barriers keep the compiler from sinking them below
    // (it would, to shorten register live ranges, and every chunk would then
    // wait a whole L2 round trip)
    // (only the first nch chunks: W and 1/D are zero past the step's k
    // pivots)
    // (a full step's eight chunks unrolled, fewer in a loop over pairs)
    double a0[NRA][2], b0[NRB][2], a1[NRA][2], b1[NRB][2];
    wave_tile_chunk<NRA, NRB>(M, I, J, ro, co, 0, a0, b0);
    if (nch >= 8) {
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        wave_tile_chunk<NRA, NRB>(M, I, J, ro, co, c + 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        wave_tile_mfma<NRA, NRB>(c, diag, ro, co, a0, b0, acc);
        if (c + 2 < 8) wave_tile_chunk<NRA, NRB>(M, I, J, ro, co, c + 2, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        wave_tile_mfma<NRA, NRB>(c + 1, diag, ro, co, a1, b1, acc);
      }
    } else {
      const int nc = (nch + 1) & ~1;  // whole pairs of chunks
#pragma unroll 1
      for (int c = 0; c < nc; c += 2) {
        wave_tile_chunk<NRA, NRB>(M, I, J, ro, co, c + 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        wave_tile_mfma<NRA, NRB>(c, diag, ro, co, a0, b0, acc);
        if (c + 2 < nc) wave_tile_chunk<NRA, NRB>(M, I, J, ro, co, c + 2, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        wave_tile_mfma<NRA, NRB>(c + 1, diag, ro, co, a1, b1, acc);
      }
    }
  }
  // pivot slots of this part's rows and columns (sm.pos is -1 off the
  // pivots, inactive rows and columns included)
  int pc[NRB], pr[NRA][4];
  bool touch = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    pc[rb] = sm.pos[J * kSB + 16 * (co + rb) + l16];
    touch |= pc[rb] >= 0;
  }
#pragma unroll
  for (int ra = 0; ra < NRA; ++ra)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[ra][i] = sm.pos[I * kSB + 16 * (ro + ra) + g16 + 4 * i];
      touch |= pr[ra][i] >= 0;
    }
  if (!__any(touch)) {
    // no pivot row or column here: every entry takes T -= W_I D^-1 W_J^T.
    // Entries of a row sit 16 doubles apart (immediate offsets from one row
    // pointer).  Blocks strictly above the diagonal of a diagonal tile are
    // skipped; inside a diagonal 16 x 16 block the upper entries are written
    // too (their update is the mirror image and only the lower triangle is
    // ever read).
#pragma unroll
    for (int rh = 0; rh < NRA; rh += 2) {
      double x[2][NRB][4];
      gdouble* row[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = I * kSB + 16 * (ro + rh + h) + g16 + 4 * i;
          row[h][i] = M.S + static_cast<size_t>(r) * M.ld + J * kSB + 16 * co + l16;
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            if (!diag || co + rb <= ro + rh + h) x[h][rb][i] = row[h][i][16 * rb];
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            if (!diag || co + rb <= ro + rh + h) row[h][i][16 * rb] = x[h][rb][i] - acc[rh + h][rb][i];
    }
    return;
  }
#pragma unroll
  for (int rh = 0; rh < NRA; rh += 2) {
    // current values (or the V entries that replace them), one batch of loads
    double x[2][NRB][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = I * kSB + 16 * (ro + rh + h) + g16 + 4 * i;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int c = J * kSB + 16 * (co + rb) + l16;
          const int q = pr[rh + h][i], qc = pc[rb];
          const gdouble* src = qc >= 0 ? M.V + (static_cast<size_t>(r) * kSB + qc)
                             : q >= 0  ? M.V + (static_cast<size_t>(c) * kSB + q)
                                       : M.S + (static_cast<size_t>(r) * M.ld + c);
          x[h][rb][i] = *src;
        }
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = I * kSB + 16 * (ro + rh + h) + g16 + 4 * i;
          const int c = J * kSB + 16 * (co + rb) + l16;
          if (diag && r < c) continue;
          const int q = pr[rh + h][i], qc = pc[rb];
          double v;
          if (q >= 0 && qc >= 0) v = -sm.sgn[q] * sm.sgn[qc] * sm.pp[q][qc];
          else if (qc >= 0) v = sm.sgn[qc] * x[h][rb][i];
          else if (q >= 0) v = sm.sgn[q] * x[h][rb][i];
          else v = x[h][rb][i] - acc[rh + h][rb][i];
          M.S[static_cast<size_t>(r) * M.ld + c] = v;
        }
  }
}

// Active tiles of a step in row-major order: variable band Iv (0..nvb-1) has
// nrb right-hand-side tiles, then, unless Iv < skip, variable tiles c0..Iv;
// bands below c0 have none (c0 > 0: forward elimination, see sweep_step).
struct TileWalk {
  int Iv, j, nrb, skip, vb0, c0;
  __device__ int count(int iv) const {
    return iv < c0 ? 0 : nrb + (iv >= skip ? iv + 1 - c0 : 0);
  }
  __device__ void seek(int a) {
    Iv = 0;
    while (a >= count(Iv)) {
      a -= count(Iv);
      ++Iv;
    }
    j = a;
  }
  __device__ void next() {
    if (++j >= count(Iv)) {
      ++Iv;
      j = 0;
    }
  }
  __device__ int I() const { return vb0 + Iv; }
  __device__ int J() const { return j < nrb ? j : vb0 + c0 + j - nrb; }
};

// One sweep step over the k pivots in sm.piv / sm.sgn / sm.pos, by the team.
// Tiles whose row band is a variable band below skip_below (and whose column
// is a variable band) are left alone: the value fit never reads them again.
// c0 > 0 (the value fit's forward elimination, pivots in band c0 = skip_below
// swept in order): no band below c0 is touched at all, and variable tiles
// start at column band c0.  Bands already swept then keep the values of
// their own step: right-hand sides (A_PP^-1 b_P) and, below them, pivot
// columns (A_iP A_PP^-1); sweep_backsub turns those into the solution.
//
// Lookahead: when the next step's kn pivots are already known (sm.piv2,
// sm.sgn2) and the team has more than one member, its last member does no
// tiles; it takes the next pivot block from S before this step's update,
// applies the update to it from the staged W rows (A' = A - W D^-1 W^T; the
// two pivot sets are disjoint), factors it and publishes L^-1 and 1/D in
// M.stage, which the next step loads instead of factoring (pre = true); the
// members that build bands and tiles form B from them.
// One right-hand side (the bias system): its column is updated outside the
// tile tasks.  Every member forms the right-hand-side row's W and V from
// U_0 = A[0, P] (gathered before the step's first barrier, so before any
// member writes column 0) and the step's factors, then updates column 0 of
// the rows of its own half bands (the ones whose W rows it staged): a pivot
// row takes s_q V_0q, any other row A_r0 - W_r D^-1 W_0^T, eight lanes a row,
// each over eight pivots, added by a fixed butterfly.
__device__ __forceinline__ void rhs_col0(const SweepMat& M, int k, int first, int nhalf,
                                         int stride) {
  SweepSmem& sm = g_sw;
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid < kSB) {
    double w = 0.0, v = 0.0;
    for (int q = 0; q < k; ++q) {
      const double u = sm.u0[q];
      w = fma(u, sm.li[tid][q], w);
      v = fma(u, sm.pp[q][tid], v);
    }
    sm.w0d[tid] = tid < k ? w * sm.rD[tid] : 0.0;
    sm.v0[tid] = v;
  }
  __syncthreads();
  const int part = tid & 7;
  for (int bi = first; bi < nhalf; bi += stride) {
    const int r = M.r_al + 32 * bi + (tid >> 3);
    const bool act = r < M.r_al + M.n_var;
    const int q = act ? sm.pos[r] : -1;
    double d = 0.0;
    if (act && q < 0) {
      const gdouble* wr = M.U + static_cast<size_t>(r) * kSB + 8 * part;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fma(wr[i], sm.w0d[8 * part + i], d);
    }
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    d += __shfl_xor(d, 4);
    if (act && part == 0) {
      gdouble* a0 = M.S + static_cast<size_t>(r) * M.ld;
      *a0 = q >= 0 ? sm.sgn[q] * sm.v0[q] : *a0 - d;
    }
  }
}

// Returns whether a pivot of this step had the wrong sign (a lookahead
// member flags its own into *status).
__device__ __forceinline__ bool sweep_step(const SweepMat& M, Team& tm, int k, int skip_below,
                                           int kn, bool pre, int c0) {
  SweepSmem& sm = g_sw;
  const int trank = tm.rank, tsize = tm.size;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const bool la = kn > 0 && tsize > 1;
  const bool me_la = la && trank == tsize - 1;
  bool bad = false;
  // pre: the previous step's lookahead member (the last rank) factored this
  // pivot block; it kept L^-1 and 1/D in its LDS, and in a single-XCD team the
  // others fetched them at the end of the previous step (below)
  if (pre) {
    if (trank != tsize - 1 && !tm.fast) {
      for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
        const int r = e >> 6, c = e & 63;
        sm.li[r][c] = M.stage[kSB * kSB + e];
      }
      if (tid < kSB) sm.rD[tid] = M.stage[2 * kSB * kSB + tid];
      __syncthreads();
    }
  } else {
    for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
      const int a = e >> 6, c = e & 63;
      const bool in = a < k && c < k;
      const double v = s_at_or0(M, in, in ? sm.piv[a] : 0, in ? sm.piv[c] : 0);
      sm.pp[a][c] = in ? v : (a == c ? 1.0 : 0.0);
    }
    if (tid < kSB) sm.dg[tid] = tid < k && M.dg0 ? M.dg0[sm.piv[tid] - M.r_al] : 0.0;
    __syncthreads();
    bad = small_ldl(k);
  }
  const int nrb = (M.n_rhs + kSB - 1) / kSB, nvb = (M.n_var + kSB - 1) / kSB;
  const int vb0 = M.r_al / kSB;
  const int vmembers = la ? tsize - 1 : tsize;
  // One right-hand side (the bias system): its column can be updated by
  // rhs_col0 instead of by tile tasks, and then each diagonal tile taken as
  // one task.  Used when that lets every tile task of the step go to a wave
  // of its own and the usual split (right-hand-side tasks, half tiles) does
  // not: the step then waits for one task per wave instead of two.
  bool fused = false;
  if (M.r_al == kSB && M.n_rhs == 1 && c0 == 0 && skip_below == 0 && tsize > 1) {
    const int tv = nvb * (nvb + 1) / 2, nwv = vmembers * (kTeamThreads / 64);
    const int tu = tv + nvb, pu = 2 * tu <= nwv ? 4 : (tu < nwv ? 2 : 1);
    const bool half = 2 * tv > nwv && tv < nwv;
    fused = half && 2 * tv - nvb <= nwv && nvb + tv * pu > nwv;
  }
  double u0r = 0.0;  // A[0, P] for rhs_col0, gathered before any column-0 write
  if (fused && !me_la && tid < k) u0r = M.S[static_cast<size_t>(sm.piv[tid]) * M.ld];
  // B (for V = U B and the pivot block) only where the bands and tiles are
  // built: the lookahead member needs L^-1 and D alone
  if (!me_la) small_b(k);
  if (!me_la) {
    // (the bands of the right-hand sides and of variable bands c0 on; with
    // one right-hand side, the variable bands alone)
    const int rb0 = fused ? 0 : nrb;
    for (int bi = trank; bi < 2 * (rb0 + nvb - c0); bi += vmembers) {
      const int b = bi >> 1;
      v_band(M, b < rb0 ? b : vb0 + c0 + b - rb0, bi & 1, k);
    }
    if (fused && tid < kSB) sm.u0[tid] = u0r;
  } else {
    // the next pivot block after this step's update, A' = A[P', P'] -
    // W' D^-1 W'^T with W' = A[P', P] L^-T, taken from S before any member
    // updates it and formed in LDS while the others build the bands
    const int wr = wave >> 1, wc = wave & 1, g16 = lane >> 4, l16 = lane & 15;
    double ua[2][16], app[kSB * kSB / kTeamThreads];
    // both gathers at once: A[P', P] for W' and A[P', P'] for the block
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ra = wr * 32 + x * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int q = g16 * 16 + kk;
        const bool ok = ra < kn && q < k;
        ua[x][kk] = s_at_or0(M, ok, ok ? sm.piv2[ra] : 0, ok ? sm.piv[q] : 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i) {
      const int e = tid + i * kTeamThreads, a = e >> 6, c = e & 63;
      const bool in = a < kn && c < kn;
      app[i] = s_at_or0(M, in, in ? sm.piv2[a] : 0, in ? sm.piv2[c] : 0);
    }
    // all the lookahead member reads from S is in registers once these loads
    // land (the arrival waits for them): count it in at the first barrier now
    // and form the block while the others update the tiles.  In a single-XCD
    // team it also arrives at the closing barrier now: it writes nothing the
    // tiles read, and the workers take its factors by the ready count, so the
    // step closes when the tiles are done; elsewhere the others read the
    // staged factors after the closing barrier, so it arrives there after
    // publishing
    if (tm.fast) team_arrive2(tm);
    else team_arrive(tm);
    f64x4 wa[2][2] = {};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int q = g16 * 16 + kk;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const double l = sm.li[wc * 32 + y * 16 + l16][q];
#pragma unroll
        for (int x = 0; x < 2; ++x)
          wa[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(ua[x][kk], l, wa[x][y], 0, 0, 0);
      }
    }
    __syncthreads();  // B and L^-1 of this step are no longer read here
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i) {
      const int e = tid + i * kTeamThreads, a = e >> 6, c = e & 63;
      const bool in = a < kn && c < kn;
      sm.pp[a][c] = in ? app[i] : (a == c ? 1.0 : 0.0);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.li[wr * 32 + x * 16 + g16 + 4 * i][wc * 32 + y * 16 + l16] = wa[x][y][i];
    __syncthreads();
    f64x4 acc[2][2] = {};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int q = g16 * 16 + kk;
      const double rdq = sm.rD[q];
      double av[2], bv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        av[x] = sm.li[wr * 32 + x * 16 + l16][q] * rdq;
        bv[x] = sm.li[wc * 32 + x * 16 + l16][q];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wr * 32 + x * 16 + g16 + 4 * i, col = wc * 32 + y * 16 + l16;
          if (row < kn && col < kn) sm.pp[row][col] -= acc[x][y][i];
        }
  }
  int total = 0;
  for (int iv = c0; iv < nvb; ++iv)
    total += (fused ? 0 : nrb) + (iv >= skip_below ? iv + 1 - c0 : 0);
  const int workers = la ? tsize - 1 : tsize;
  const int nw = workers * (kTeamThreads / 64);
  const int parts = 2 * total <= nw ? 4 : (total < nw ? 2 : 1);
  // With at most 16 right-hand sides (and not one alone, see rhs_col0), a
  // right-hand-side tile is one task over its first 16 columns (the others
  // are inactive: zero and never updated), ahead of the variable tiles.
  const bool narrow = !fused && nrb == 1 && M.n_rhs <= 16;
  const int rtasks = narrow ? nvb : 0;
  // With one right-hand side and half tiles, a diagonal tile is one task (its
  // lower ten 16 x 16 blocks; as two halves it was three and seven blocks,
  // each half paying a task's loads and stores): band iv has tasks
  // iv^2 .. iv^2 + 2 iv, the last its diagonal tile.
  const bool dsingle = fused && parts == 2;
  const int tasks = narrow    ? rtasks + (total - nvb) * parts
                    : dsingle ? 2 * total - nvb
                              : total * parts;
  const int nch = (k + 7) / 8;  // contraction chunks of 8 that hold pivots
  if (me_la) {
    // the lookahead member arrived at the first barrier after its gathers;
    // it factors the next block and waits for that barrier only before the
    // next
    if (tid < kSB) {
      sm.sgn[tid] = sm.sgn2[tid];
      sm.dg[tid] = tid < kn && M.dg0 ? M.dg0[sm.piv2[tid] - M.r_al] : 0.0;
    }
    __syncthreads();
    const bool bad2 = small_ldl(kn);
    for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
      const int r = e >> 6, c = e & 63;
      M.stage[kSB * kSB + e] = sm.li[r][c];
    }
    if (tid < kSB) M.stage[2 * kSB * kSB + tid] = sm.rD[tid];
    bad |= bad2;
    // the factors are out: raise the team's ready count (after every wave's
    // stores have landed)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      if (!tm.fast) __threadfence();
      __hip_atomic_store(tm.ready, tm.pubs + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    team_wait(tm);
  } else {
    // Tile tasks (the active tiles, or their halves or quarters when there
    // are fewer tiles than waves) are handed out by ticket: each wave of the
    // tile workers draws task numbers from the team's counter, the next one
    // while it works on the current, until a number runs past the step's
    // tasks.  Waves that draw cheap tiles (no pivot rows or columns) take
    // more of them.  Each wave overshoots exactly once, so every member
    // advances the step's base by tasks + waves without reading the counter.
    team_arrive(tm);
    unsigned pend = draw_ticket(tm);  // the previous step's draws all ended before its barrier
    team_wait(tm);
    const unsigned base = uniform(static_cast<int>(tm.tbase)), end = base + tasks;
    unsigned tk = ticket_value(pend);
    while (tk < end) {
      pend = draw_ticket(tm);
      if (tk >= base) {  // (always, unless a timed-out barrier let the members drift apart)
        const int a = static_cast<int>(tk - base);
        if (a < rtasks) {
          wave_tile<4, 1>(M, vb0 + a, 0, 0, 0, nch);
        } else if (dsingle) {
          int iv = static_cast<int>(sqrtf(static_cast<float>(a)));
          while (iv * iv > a) --iv;
          while ((iv + 1) * (iv + 1) <= a) ++iv;
          const int r = a - iv * iv;
          if (r == 2 * iv) wave_tile<4, 4>(M, vb0 + iv, vb0 + iv, 0, 0, nch);
          else wave_tile<2, 4>(M, vb0 + iv, vb0 + (r >> 1), 2 * (r & 1), 0, nch);
        } else {
          const int av = a - rtasks, part = av % parts;
          TileWalk w{0, 0, (narrow || fused) ? 0 : nrb, skip_below, vb0, c0};
          w.seek(av / parts);
          if (parts == 1) wave_tile<4, 4>(M, w.I(), w.J(), 0, 0, nch);
          else if (parts == 2) wave_tile<2, 4>(M, w.I(), w.J(), 2 * part, 0, nch);
          else wave_tile<2, 2>(M, w.I(), w.J(), 2 * (part >> 1), 2 * (part & 1), nch);
        }
      }
      tk = ticket_value(pend);
    }
    if (fused) rhs_col0(M, k, trank, 2 * nvb, vmembers);
  }
  tm.tbase += tasks + nw;
  // A tile worker arrives at the closing barrier as soon as its tiles are
  // done.  In a single-XCD team it then fetches the next step's L^-1 and 1/D
  // as soon as the lookahead member has published them (L1-bypassing loads,
  // since the same staging area was read a step ago), while the barrier
  // completes.
  const bool fetch = la && !me_la && tm.fast;
  if (!me_la) team_arrive(tm);  // every wave of this member is past its tiles
  if (fetch) {
    if (tid == 0) {
      const uint64_t t0 = wall_clock64();
      unsigned spins = 0;
      while (__hip_atomic_load(tm.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tm.pubs + 1) {
        if (wall_clock64() - t0 > tm.spin) {
          atomicOr(tm.err, 1);
          break;
        }
        if ((++spins & 31u) == 0 &&
            __hip_atomic_load(tm.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
          break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    double nli[kSB * kSB / kTeamThreads], nrd = 0.0;
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i)
      nli[i] = __hip_atomic_load(&M.stage[kSB * kSB + tid + i * kTeamThreads], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    if (tid < kSB)
      nrd = __hip_atomic_load(&M.stage[2 * kSB * kSB + tid], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    // this step's L^-1 and 1/D are no longer read (every wave is past its tiles)
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i) {
      const int e = tid + i * kTeamThreads;
      sm.li[e >> 6][e & 63] = nli[i];
    }
    if (tid < kSB) sm.rD[tid] = nrd;
  }
  if (me_la && !tm.fast) team_arrive(tm);
  team_wait(tm);
  if (la) tm.pubs += 1;
  return bad;
}

// One step as a call (the NNLS rounds): the team and the matrix are copied
// into registers for the step (the caller's copy lives in scratch, and every
// scratch access is a vector memory operation whose wait also waits for all
// older loads and stores).
__device__ __noinline__ bool sweep_step_call(const SweepMat M_arg, Team& team_ref, int k_arg,
                                             int skip_arg, int kn_arg, bool pre_arg) {
  // every argument is the same in all lanes; a called function receives them
  // in vector registers, so say so, or every branch and address derived from
  // them is compiled as divergent (exec-masked)
  const SweepMat M = uniform_mat(M_arg);
  Team tm = uniform_team(team_ref);
  const bool bad = sweep_step(M, tm, uniform(k_arg), uniform(skip_arg), uniform(kn_arg),
                              uniform(static_cast<int>(pre_arg)) != 0, 0);
  team_ref.gen = tm.gen;
  team_ref.tbase = tm.tbase;
  team_ref.pubs = tm.pubs;
  return bad;
}

// Back substitution after the forward elimination (sweep_step with c0 > 0)
// of the value system's n variables: band k's right-hand sides hold
// Y_k = A_kk^-1 b_k and band j > k's pivot columns of band k hold
// L_jk = A_jk A_kk^-1 (the blocks as they stood at step k), so the solution
// is X_k = Y_k - sum_{j > k} L_jk^T X_j.  Taken band by band from the last:
// once X_j is final, every (band k < j, right-hand-side tile) of it is a
// workgroup task (the team's workgroups take them in turn), with a team
// barrier between bands.
__device__ __forceinline__ void wg_backsub(const SweepMat& M, int J, int K, int r) {
  SweepSmem& sm = g_sw;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int g16 = lane >> 4, l16 = lane & 15, wr = wave >> 1, wc = wave & 1;
  // L_JK (rows b of band J, columns a of band K) into pp, X_J's tile r into
  // li; rows past the variables and columns past the right-hand sides are 0
  __syncthreads();  // the previous task's reads of pp and li are done
#pragma unroll 4
  for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
    const int b = e >> 6, x = e & 63;
    const int row = J * kSB + b, col = r * kSB + x;
    const bool ok = s_active(M, row);
    const gdouble* p = M.S + static_cast<size_t>(ok ? row : 0) * M.ld;
    const double l = p[ok ? K * kSB + x : 0], xv = p[ok && col < M.n_rhs ? col : 0];
    sm.pp[b][x] = ok ? l : 0.0;
    sm.li[b][x] = ok && col < M.n_rhs ? xv : 0.0;
  }
  __syncthreads();
  // each wave a 32 x 32 quadrant of the 64 x 64 update L_JK^T X_J
  f64x4 acc[2][2] = {};
#pragma unroll
  for (int c = 0; c < kSB / 4; ++c) {
    const int b = 4 * c + g16;
    double av[2], bv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      av[x] = sm.pp[b][wr * 32 + x * 16 + l16];
      bv[x] = sm.li[b][wc * 32 + x * 16 + l16];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = K * kSB + wr * 32 + x * 16 + g16 + 4 * i;
        const int col = r * kSB + wc * 32 + y * 16 + l16;
        if (s_active(M, row) && col < M.n_rhs)
          M.S[static_cast<size_t>(row) * M.ld + col] -= acc[x][y][i];
      }
}

// Whether the value system of n variables and d right-hand sides is solved
// by forward elimination and back substitution rather than the whole sweep.
// The elimination skips the swept bands' tiles, but the back substitution
// adds a team barrier per band: it pays when a team of one workgroup does
// all tiles itself, or when the first step's tiles fill the team's waves
// (4 a member) at least twice over.
__device__ __forceinline__ bool value_elim(int n, int d, int tsize, bool full) {
  const int nvb = (n + kSB - 1) / kSB, nrb = (d + kSB - 1) / kSB;
  if (full || nvb < 2) return false;
  return tsize == 1 || nvb * nrb + nvb * (nvb + 1) / 2 > 8 * tsize;
}

__device__ __forceinline__ void sweep_backsub(const SweepMat& M, Team& tm, int n) {
  const int nvb = (n + kSB - 1) / kSB, nrb = (M.n_rhs + kSB - 1) / kSB;
  const int vb0 = M.r_al / kSB;
  for (int j = nvb - 1; j >= 1; --j) {
    for (int a = tm.rank; a < j * nrb; a += tm.size) wg_backsub(M, vb0 + j, vb0 + a / nrb, a % nrb);
    team_sync(tm);
  }
}

// The value system's n variables (rows r_al .. r_al + n - 1), swept in 64 at
// a time, as one call: the per-step call costs more here than the register
// pressure of the loop around the inlined step.  Unless `full`, no tile of a
// swept band is updated again: either its variable tiles alone are left (the
// solution needs none of them), or (value_elim) the bands are eliminated
// forward and the solution taken by back substitution, about half the tile
// work of the sweep.  With `full` the whole sweep runs and the variable
// block ends as -(G + lam I)^-1, which the refinement steps apply.
__device__ __noinline__ bool sweep_run(const SweepMat M_arg, Team& team_ref, int n_arg,
                                       int full_arg) {
  SweepSmem& sm = g_sw;
  const SweepMat M = uniform_mat(M_arg);
  const int n = uniform(n_arg);
  const bool full = uniform(full_arg) != 0;
  Team tm = uniform_team(team_ref);
  const int tid = threadIdx.x;
  const bool elim = value_elim(n, M.n_rhs, tm.size, full);
  bool bad = false;
  for (int s0 = 0; s0 < n; s0 += kSB) {
    const int k = min(kSB, n - s0);
    const int kn = min(kSB, n - s0 - k);
    if (tid < k) {
      sm.piv[tid] = M.r_al + s0 + tid;
      sm.sgn[tid] = 1.0;
      sm.pos[M.r_al + s0 + tid] = static_cast<int16_t>(tid);
    }
    if (tid < kn) {
      sm.piv2[tid] = M.r_al + s0 + k + tid;
      sm.sgn2[tid] = 1.0;
    }
    __syncthreads();
    bad |= sweep_step(M, tm, k, full ? 0 : s0 / kSB, kn, s0 > 0 && tm.size > 1,
                      elim ? s0 / kSB : 0);
    if (tid < k) sm.pos[M.r_al + s0 + tid] = -1;
    __syncthreads();
  }
  if (elim) sweep_backsub(M, tm, n);
  team_ref.gen = tm.gen;
  team_ref.tbase = tm.tbase;
  team_ref.pubs = tm.pubs;
  return bad;
}

__device__ __forceinline__ double sweep_flops(int k, int n) {
  const double kd = k, nd = n;
  return kd * nd * nd + 2.0 * nd * kd * kd + kd * kd * kd;
}

// ---------------------------------------------------------------------------
// NNLS by block principal pivoting (Judice & Pires 1994; Kim & Park 2011) on
// the swept system [H c; c^T .] of each head, one team per head.  Start from
// the empty passive set (x = 0, gradient -c); each round reads x_F and the
// gradient from the right-hand-side column, exchanges every infeasible
// variable while the infeasible count keeps falling (three more tries after
// it stops), else only the one with the largest index, and sweeps the
// exchanged variables in or out.  Stops at the KKT point or after max_iters
// exchanges (status bit 2, w = max(x, 0)).  Every member runs the rule on the
// same data, so the rule needs no barrier.  Output: w, and the passive list
// (support of w) for the value fit.
//
// A failed pivot (H_FF not numerically positive definite: a pivot of the
// wrong sign or zero) restarts the head with the ridge raised tenfold, at
// most three times: relative ridge max(10^e ridge, 10^(e-1) 1e-9) at the
// e-th raise, so that ridge 0 (the plain NNLS) also recovers.  The team
// rebuilds H = P_S^T P_S + lam I and c = P_S^T 1 + lam from P_S and the
// column sums (the sweeps overwrote them).  The raises are recorded in the
// status word (KVC_STATUS_RIDGE_RAISED and the count in bits 8-9); bit 1
// stays set only if the last attempt still failed.  The relative ridge in
// use is left in lam[2b+1] for the value fit.
// ---------------------------------------------------------------------------

// Rebuild head b's bias system for relative ridge `rel`: the Gram tiles of
// the lower triangle are dealt round-robin over the team's members (one
// 64 x 64 fp64 MFMA tile product over all n rows each, staged through the
// pivot-block LDS, which no sweep uses meanwhile); lam_w = rel tr(H)/t with
// tr(H)/t from lam[2b+1]; column 0 of the variable rows = c + lam_w and
// columns 1..15 cleared.
__device__ __noinline__ void rebuild_bias(const SweepMat M, const Team tm,
                                          const double* __restrict__ PSb, int t_str, int n,
                                          int t, const double* __restrict__ cb, double lw) {
  SweepSmem& sm = g_sw;
  double* sAt = &sm.pp[0][0];
  double* sBt = sAt + kKC * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tt = (t + kTile - 1) / kTile, ntl = tt * (tt + 1) / 2;
  for (int tile = tm.rank; tile < ntl; tile += tm.size) {
    int ty, tx;
    tri_decode(tile, ty, tx);
    const int a0 = ty * kTile, c0 = tx * kTile;
    f64x4 acc[2][2];
    atb_tile<double, true>(PSb, t_str, nullptr, PSb, t_str, t, t, a0, c0, 0, n, sAt, sBt, acc);
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = a0 + tile_row(wave, lane, ra, i), c = c0 + tile_col(wave, lane, rb);
          if (r < t && c < t)
            M.S[static_cast<size_t>(kSB + r) * M.ld + kSB + c] =
                acc[ra][rb][i] + (r == c ? lw : 0.0);
        }
  }
  for (int e = tm.rank * kTeamThreads + threadIdx.x; e < t * 16; e += tm.size * kTeamThreads) {
    const int r = e >> 4, c = e & 15;
    M.S[static_cast<size_t>(kSB + r) * M.ld + c] = c == 0 ? cb[r] + lw : 0.0;
  }
}

__global__ __launch_bounds__(256) void k_nnls_sweep(
    double* __restrict__ S, size_t sS, int ld, double* __restrict__ Ub, double* __restrict__ Vb,
    size_t sUV, double* __restrict__ stage, double* __restrict__ wv, int32_t* __restrict__ Fidx,
    int32_t* __restrict__ inv,
    int32_t* __restrict__ msz, int32_t* __restrict__ status, unsigned* __restrict__ bar,
    int* __restrict__ err, int* __restrict__ xcc, double* __restrict__ flops,
    const int32_t* __restrict__ tv, int B, int t_str, int max_iters, int tx, uint64_t spin,
    const double* __restrict__ PS, int n, const double* __restrict__ cvec,
    double* __restrict__ lam, double ridge) {
  SweepSmem& sm = g_sw;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx, spin);
  const int tid = threadIdx.x;
  for (int s = tid; s < kMaxRows; s += kTeamThreads) sm.pos[s] = -1;
  constexpr int NV = kMaxTeamT / kTeamThreads;
  for (int b = team; b < B; b += nteams) {
    const int t = tv ? tv[b] : t_str;
    // the diagonals before any sweep sit in the head's w output until w is
    // written at the end
    double* dg0 = wv + static_cast<size_t>(b) * t_str;
    const SweepMat M{gptr(S + b * sS), gptr(Ub + b * sUV), gptr(Vb + b * sUV),
                     gptr(stage + static_cast<size_t>(b) * kStage), ld, kSB, 1, t, gptr(dg0)};
    // the head's failure flag: the first word of its staging area, which
    // the steps do not use (they stage at kSB*kSB and after)
    unsigned long long* fail =
        reinterpret_cast<unsigned long long*>(stage + static_cast<size_t>(b) * kStage);
    double fl = 0.0, rel = ridge, floor_rel = 1e-9;
    int done = 0, raises = 0;
    bool failed = false;
    double val[NV];
    for (;;) {
      // one attempt; the flag is cleared before this member's first step,
      // so before any member can raise it (every step has a team barrier)
      if (tm.rank == 0 && tid == 0)
        __hip_atomic_store(fail, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int j = tid; j < t; j += kTeamThreads) sm.inF[j] = 0;
      double cm = 0.0, hm = 0.0;
      for (int j = tid; j < t; j += kTeamThreads) {
        const gdouble* row = M.S + static_cast<size_t>(kSB + j) * ld;
        cm = fmax(cm, fabs(row[0]));
        hm = fmax(hm, row[kSB + j]);
        dg0[j] = row[kSB + j];  // every member stores the same values
      }
      const double scale = fmax(wg_max(cm), wg_max(hm));
      int N = t + 1, bud = 3;
      bool bad = false;
      done = 0;
      for (int it = 0;; ++it) {
        double xm = 0.0;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          const int j = tid + q * kTeamThreads;
          const double v = M.S[static_cast<size_t>(kSB + (j < t ? j : 0)) * ld];
          val[q] = j < t ? v : 0.0;
          if (j < t && sm.inF[j]) xm = fmax(xm, fabs(val[q]));
        }
        const double tol = 1e-13 * scale * fmax(1.0, wg_max(xm));
        int nv = 0, vmax = -1, slot;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          const int j = tid + q * kTeamThreads;
          bool f = false;
          if (j < t) f = sm.inF[j] ? val[q] < 0.0 : val[q] > tol;
          if (q * kTeamThreads < t) {
            nv = wg_append(f, nv, &slot);
            if (f) {
              sm.list[slot] = static_cast<int16_t>(j);
              vmax = j;
            }
          }
        }
        if (nv == 0) {
          done = 1;
          break;
        }
        if (it >= max_iters) {
          done = 2;
          break;
        }
        int nflip = nv;
        if (nv < N) {
          N = nv;
          bud = 3;
        } else if (bud >= 1) {
          --bud;
        } else {
          vmax = wg_imax(vmax);
          __syncthreads();
          if (tid == 0) sm.list[0] = static_cast<int16_t>(vmax);
          nflip = 1;
        }
        __syncthreads();
        for (int s0 = 0; s0 < nflip; s0 += kSB) {
          const int k = min(kSB, nflip - s0);
          const int kn = min(kSB, nflip - s0 - k);
          if (tid < k) {
            const int j = sm.list[s0 + tid];
            sm.piv[tid] = kSB + j;
            sm.sgn[tid] = sm.inF[j] ? -1.0 : 1.0;
            sm.pos[kSB + j] = static_cast<int16_t>(tid);
          }
          if (tid < kn) {
            const int j = sm.list[s0 + k + tid];
            sm.piv2[tid] = kSB + j;
            sm.sgn2[tid] = sm.inF[j] ? -1.0 : 1.0;
          }
          __syncthreads();
          bad |= sweep_step_call(M, tm, k, 0, kn, s0 > 0 && tm.size > 1);
          if (tid < k) {
            const int j = sm.list[s0 + tid];
            sm.inF[j] ^= 1;
            sm.pos[kSB + j] = -1;
          }
          __syncthreads();
          fl += sweep_flops(k, t + 1);
        }
      }
      // the team's verdict: any member's failed pivot
      if (bad && tid == 0) atomicOr(fail, 1ull);
      team_sync(tm);
      failed = __hip_atomic_load(fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      if (!failed || raises == 3) break;
      ++raises;
      rel = fmax(rel * 10.0, floor_rel);
      floor_rel *= 10.0;
      rebuild_bias(M, tm, PS + static_cast<size_t>(b) * n * t_str, t_str, n, t,
                   cvec + static_cast<size_t>(b) * t_str, rel * lam[2 * b + 1]);
      team_sync(tm);
    }
    if (tm.rank == 0) {
      double* w = wv + static_cast<size_t>(b) * t_str;
      int32_t* Fb = Fidx + static_cast<size_t>(b) * t_str;
      int32_t* ib = inv + static_cast<size_t>(b) * t_str;
      int m = 0, slot;
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int j = tid + q * kTeamThreads;
        double x = 0.0;
        if (j < t) {
          x = sm.inF[j] ? val[q] : 0.0;
          if (done == 2) x = fmax(x, 0.0);
          w[j] = x;
        }
        if (q * kTeamThreads < t) {
          const bool f = j < t && x > 0.0;
          m = wg_append(f, m, &slot);
          if (j < t) {
            ib[j] = f ? slot : -1;
            if (f) Fb[slot] = j;
          }
        }
      }
      for (int j = t + tid; j < t_str; j += kTeamThreads) {
        w[j] = 0.0;
        ib[j] = -1;
      }
      if (tid == 0) {
        msz[b] = m;
        flops[2 * b] = fl;
        if (raises > 0) lam[2 * b] = rel * lam[2 * b + 1];
        lam[2 * b + 1] = rel;  // the value fit's relative ridge
        if (status) {
          if (done == 2) atomicOr(&status[b], 2);
          if (failed) atomicOr(&status[b], 1);
          if (raises > 0) atomicOr(&status[b], 64 | (raises << 8));
        }
      }
    }
    team_sync(tm);
  }
  if (tm.rank == 0 && tid == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    for (int b = team; b < B; b += nteams) atomicOr(&status[b], 8);
}

// Value system [G R; R^T .] (G = X_F^T X_F + lam_v I of order m = msz[b], R =
// X_F^T O + lam_v V_F with D columns, right-hand sides in rows [0, r_al)):
// sweep the m variables in bands of 64; afterwards rows r_al + a hold C_v[a].
__global__ __launch_bounds__(256) void k_value_sweep(
    double* __restrict__ S, size_t sS, int ld, int r_al, double* __restrict__ Ub,
    double* __restrict__ Vb, size_t sUV, double* __restrict__ stage, const int32_t* __restrict__ msz,
    int32_t* __restrict__ status, unsigned* __restrict__ bar, int* __restrict__ err,
    int* __restrict__ xcc, double* __restrict__ flops, int B, int D, int tx, uint64_t spin,
    int full) {
  SweepSmem& sm = g_sw;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx, spin);
  const int tid = threadIdx.x;
  for (int s = tid; s < kMaxRows; s += kTeamThreads) sm.pos[s] = -1;
  for (int b = team; b < B; b += nteams) {
    const int m = msz[b];
    const SweepMat M{gptr(S + b * sS), gptr(Ub + b * sUV), gptr(Vb + b * sUV),
                     gptr(stage + static_cast<size_t>(b) * kStage), ld, r_al, D, m, nullptr};
    const bool bad = sweep_run(M, tm, m, full);
    if (tm.rank == 0 && tid == 0) {
      // a sweep (what it counts is the whole sweep's work either way); or
      // the elimination over the part not yet swept and the back
      // substitution (each band's rows against all bands above it)
      const bool elim = value_elim(m, D, tm.size, full != 0);
      double fl = 0.0;
      for (int s0 = 0; s0 < m; s0 += kSB) {
        const int k = min(kSB, m - s0);
        fl += elim ? sweep_flops(k, m - s0 + D) + 2.0 * s0 * k * D : sweep_flops(k, m + D);
      }
      flops[2 * b + 1] = fl;
    }
    // every member reports the failed pivots it saw (the lookahead member,
    // the last rank, factors the blocks after the first)
    if (bad && tid == 0 && status) atomicOr(&status[b], 1);
  }
  if (tm.rank == 0 && tid == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    for (int b = team; b < B; b += nteams) atomicOr(&status[b], 8);
}

// r_i = sum_a P_S[i][a] w'_a, X = P_S diag(w') / r, w' = max(w, 1e-30); the
// passive columns X_F are written compacted to the front of each row (column
// inv[a] for passive a; the row stride stays t), so the value system's
// products read them contiguously.  One wave per row: it sums the row (lane
// partials, then a butterfly), then reads it again and writes the passive
// entries.  The rewrite is in place and safe: passive a goes to slot
// inv[a] <= a, and the wave reads positions [a0, a0 + 64) of a pass before it
// writes any slot of that pass (all below a0 + 64), so no position is read
// after it has been written.  grid (ceil(n/4), B), block 256.
__global__ __launch_bounds__(256) void k_value_prep(double* __restrict__ PS,
                                                    const double* __restrict__ wv,
                                                    const int32_t* __restrict__ inv, int n,
                                                    int t) {
  const int b = blockIdx.y, i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= n) return;
  double* row = PS + (static_cast<size_t>(b) * n + i) * t;
  const double* w = wv + static_cast<size_t>(b) * t;
  const int32_t* ib = inv + static_cast<size_t>(b) * t;
  double s = 0.0;
  for (int a = lane; a < t; a += 64) s += row[a] * fmax(w[a], 1e-30);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  const double rs = 1.0 / s;
  for (int a0 = 0; a0 < t; a0 += 64) {
    const int a = a0 + lane;
    const double v = a < t ? row[a] * fmax(w[a], 1e-30) : 0.0;
    const int slot = a < t ? ib[a] : -1;
    if (slot >= 0) row[slot] = v * rs;
  }
}

// lam_v = ridge * trace(G) / t with the head's relative ridge (lam[2b+1], left
// there by the NNLS: the caller's, or the raised one); G += lam_v I (G at Gb,
// order msz, stride ld); lam[2b+1] = lam_v.  grid (B), block 256.
__global__ void k_ridge_v(double* __restrict__ Gb, size_t sS, int ld,
                          const int32_t* __restrict__ msz, double* __restrict__ lam,
                          const int32_t* __restrict__ tv, int t_str) {
  __shared__ double sh[16];
  const int b = blockIdx.x, m = msz[b];
  const int t = tv ? tv[b] : t_str;
  const double rel = lam[2 * b + 1];  // read by every thread before thread 0 rewrites it
  double* G = Gb + b * sS;
  double tr = 0.0;
  for (int a = threadIdx.x; a < m; a += blockDim.x) tr += G[static_cast<size_t>(a) * ld + a];
  tr = block_sum(tr, sh);
  const double lv = rel * tr / t;
  for (int a = threadIdx.x; a < m; a += blockDim.x) G[static_cast<size_t>(a) * ld + a] += lv;
  if (threadIdx.x == 0) lam[2 * b + 1] = lv;
}

// R[a][c] += lam_v * V[idx[F[a]]][c]  (R at Rb, stride ld); the grid's
// threads also clear the team barrier words of the value sweep that follows.
// grid (ceil(t*D/256), B).
template <class In>
__global__ void k_rhs_ridge(double* __restrict__ Rb, size_t sS, int ld, const In* __restrict__ V,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ Fidx,
                            const int32_t* __restrict__ msz, const double* __restrict__ lam,
                            int T, int t, int D, unsigned* __restrict__ bar, int nbar) {
  clear_bar(bar, nbar);
  const int b = blockIdx.y, m = msz[b];
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= m) return;
  const int j = idx[static_cast<size_t>(b) * t + Fidx[static_cast<size_t>(b) * t + a]];
  Rb[b * sS + static_cast<size_t>(a) * ld + c] +=
      lam[2 * b + 1] * to_f64<In>(V[(static_cast<size_t>(b) * T + j) * D + c]);
}

// out_V[b][a][c] = fitted value (row inv[a] of C at Cb, stride ld) for passive
// keys, the V row (the prior) for keys whose multiplier is zero, as float32 or
// as the bfloat16 rounding of that float32 value; out_bias = log(max(w,
// 1e-30)).  grid (ceil(t*D/256), B).
template <class In, class OutT>
__global__ void k_write_out(const double* __restrict__ Cb, size_t sS, int ld,
                            const In* __restrict__ V, const int32_t* __restrict__ idx,
                            const int32_t* __restrict__ inv, const double* __restrict__ wv,
                            OutT* __restrict__ out_V, float* __restrict__ out_bias, int T, int t,
                            int D) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= t) return;
  const int p = inv[static_cast<size_t>(b) * t + a];
  const int j = idx[static_cast<size_t>(b) * t + a];  // -1: slot past this head's budget
  float v = 0.f;
  if (p >= 0) v = static_cast<float>(Cb[b * sS + static_cast<size_t>(p) * ld + c]);
  else if (j >= 0) v = to_f32<In>(V[(static_cast<size_t>(b) * T + j) * D + c]);
  out_V[(static_cast<size_t>(b) * t + a) * D + c] = from_f32<OutT>(v);
  if (c == 0)
    out_bias[static_cast<size_t>(b) * t + a] =
        j >= 0 ? static_cast<float>(log(fmax(wv[static_cast<size_t>(b) * t + a], 1e-30)))
               : -INFINITY;
}

// ---------------------------------------------------------------------------
// Refinement of the value fit (corrected semi-normal equations).  With C the
// solution of the swept normal equations, one step is
//   E = O - X_F C,   Y = X_F^T E - lam_v (C - V_F),   C <- C + (G + lam_v I)^-1 Y,
// the gradient of the regularised least squares at C mapped through the
// inverse the full sweep left in the variable block: a residual taken
// against O itself, so rounding in the normal equations (whose condition is
// that of X_F squared) is corrected instead of repeated.  Y's first term is a
// k_atb product; the other two products are small fp64 tiles, 64 x 64 outputs
// per workgroup, 4 x 4 per thread, the contraction staged 16 at a time.
// ---------------------------------------------------------------------------
constexpr int kRK = 16;  // contraction values staged per chunk

// E[b][i][c] = O[b][i][c] - sum_{a < m} X[i][a] C[a][c]; X in PS (row stride
// t, passive columns first), C the value system's solution rows (stride ld).
// grid (ceil(n/64), D/64, B), block 256.
template <int D>
__global__ __launch_bounds__(256) void k_csne_resid(const double* __restrict__ PS,
                                                    const double* __restrict__ Cb, size_t sS,
                                                    int ld, const float* __restrict__ O,
                                                    const int32_t* __restrict__ msz,
                                                    double* __restrict__ E, int n, int t) {
  __shared__ double sA[kTile][kRK + 1], sB[kRK][kTile];
  const int b = blockIdx.z, m = msz[b], i0 = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const double* X = PS + static_cast<size_t>(b) * n * t;
  const double* C = Cb + b * sS;
  double acc[4][4] = {};
  for (int a0 = 0; a0 < m; a0 += kRK) {
    for (int e = tid; e < kTile * kRK; e += 256) {
      const int r = e / kRK, k = e % kRK, i = i0 + r, a = a0 + k;
      sA[r][k] = (i < n && a < m) ? X[static_cast<size_t>(i) * t + a] : 0.0;
    }
    for (int e = tid; e < kRK * kTile; e += 256) {
      const int k = e / kTile, c = e % kTile, a = a0 + k;
      sB[k][c] = a < m ? C[static_cast<size_t>(a) * ld + c0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRK; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(sA[4 * ty + r][k], sB[k][4 * tx + c], acc[r][c]);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * ty + r;
    if (i >= n) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const size_t o = (static_cast<size_t>(b) * n + i) * D + c0 + 4 * tx + c;
      E[o] = static_cast<double>(O[o]) - acc[r][c];
    }
  }
}

// Cn[b][a][c] = C[a][c] + sum_{a' < m} Ginv[a][a'] Y[a'][c] for a < m, with
// Ginv = -(the swept variable block, lower triangle read symmetrically) and
// Y = XtE - lam_v (C - V_F).  grid (ceil(t/64), D/64, B), block 256.
template <class In, int D>
__global__ __launch_bounds__(256) void k_csne_update(
    const double* __restrict__ Cb, const double* __restrict__ Gb, size_t sS, int ld,
    const double* __restrict__ XtE, const In* __restrict__ V, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ Fidx, const int32_t* __restrict__ msz,
    const double* __restrict__ lam, double* __restrict__ Cn, int T, int t) {
  __shared__ double sA[kTile][kRK + 1], sB[kRK][kTile];
  const int b = blockIdx.z, m = msz[b], a0t = blockIdx.x * kTile, c0 = blockIdx.y * kTile;
  if (a0t >= m) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const double* C = Cb + b * sS;
  const double* G = Gb + b * sS;
  const double lv = lam[2 * b + 1];
  double acc[4][4] = {};
  for (int q0 = 0; q0 < m; q0 += kRK) {
    for (int e = tid; e < kTile * kRK; e += 256) {
      const int r = e / kRK, k = e % kRK, a = a0t + r, q = q0 + k;
      const int hi = a > q ? a : q, lo = a > q ? q : a;
      sA[r][k] = (a < m && q < m) ? -G[static_cast<size_t>(hi) * ld + lo] : 0.0;
    }
    for (int e = tid; e < kRK * kTile; e += 256) {
      const int k = e / kTile, c = e % kTile, q = q0 + k;
      double y = 0.0;
      if (q < m) {
        const int j = idx[static_cast<size_t>(b) * t + Fidx[static_cast<size_t>(b) * t + q]];
        const double vs = to_f64<In>(V[(static_cast<size_t>(b) * T + j) * D + c0 + c]);
        y = XtE[(static_cast<size_t>(b) * t + q) * D + c0 + c] -
            lv * (C[static_cast<size_t>(q) * ld + c0 + c] - vs);
      }
      sB[k][c] = y;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRK; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(sA[4 * ty + r][k], sB[k][4 * tx + c], acc[r][c]);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a = a0t + 4 * ty + r;
    if (a >= m) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cc = c0 + 4 * tx + c;
      Cn[(static_cast<size_t>(b) * t + a) * D + cc] = C[static_cast<size_t>(a) * ld + cc] + acc[r][c];
    }
  }
}

// C[a][c] = Cn[b][a][c] for a < m.  grid (ceil(t*D/256), B).
__global__ void k_csne_copy(double* __restrict__ Cb, size_t sS, int ld,
                            const double* __restrict__ Cn, const int32_t* __restrict__ msz, int t,
                            int D) {
  const int b = blockIdx.y, m = msz[b];
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= m) return;
  Cb[b * sS + static_cast<size_t>(a) * ld + c] = Cn[(static_cast<size_t>(b) * t + a) * D + c];
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------

// Workgroups of a team kernel the current device holds at once (cached).
static int coop_capacity(const void* func) {
  static int cache[2][64] = {};
  const int which = func == reinterpret_cast<const void*>(&k_nnls_sweep) ? 0 : 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[which][dev] == 0) {
    int nb = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, func, kTeamThreads, 0) != hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[which][dev] = nb * cus < kMaxTeamGrid ? nb * cus : kMaxTeamGrid;
  }
  return cache[which][dev];
}

// Team shape: nteams = 8*tx teams (a multiple of the XCD count, so each team
// stays on one XCD), g members each: no more than the tiles of a sweep step,
// no more than the device holds.  Returns the grid size.
static int team_shape(int B, int tiles, int cap, int& tx) {
  tiles = tiles < 1 ? 1 : tiles;
  tx = (B + kXcds - 1) / kXcds;
  if (kXcds * tx > cap) tx = cap / kXcds > 0 ? cap / kXcds : 1;
  const int nteams = kXcds * tx;
  int g = cap / nteams < tiles ? cap / nteams : tiles;
  if (g < 1) g = 1;
  return g * nteams;
}

// A^T B over heads: G workgroups a head (~`target` in all, at least one a
// tile of the largest product); each head's split-K follows its own sizes.
template <class TB, bool SYM>
static AtbArgs<TB> atb_args(const double* A, size_t sA, int lda, const int32_t* colA,
                            size_t sColA, const TB* Bm, size_t sB, int ldb, double* C, size_t sC,
                            int ldc, int nrows, const int32_t* msz, int mA, int mB, double* part,
                            size_t part_cap, int B, int target) {
  const int ta = (mA + kTile - 1) / kTile, tb = (mB + kTile - 1) / kTile;
  const int ntiles = SYM ? ta * (ta + 1) / 2 : ta * tb;
  int G = (target + B - 1) / B;
  if (G > 16 * ntiles) G = 16 * ntiles;
  if (G < ntiles) G = ntiles;
  // odd, so that consecutive heads start on different XCDs (workgroups go
  // round-robin over 8) and their busy workgroups spread evenly
  G |= 1;
  const size_t ct = part_cap / (static_cast<size_t>(B) * kTile * kTile);
  const int cap_tiles = ct > (1u << 20) ? (1 << 20) : static_cast<int>(ct);
  return AtbArgs<TB>{A,  sA,  lda,   colA,  sColA, Bm, sB, ldb, C,        sC,
                     ldc, nrows, msz, mA, mB,   part, G,  cap_tiles};
}

// x blocks of the product's split-K reduction (0: no head splits).
template <class TB, bool SYM>
static int atb_reduce_x(const AtbArgs<TB>& p, int B) {
  const int ta = (p.mA_const + kTile - 1) / kTile, tb = (p.mB_const + kTile - 1) / kTile;
  const int ntiles = SYM ? ta * (ta + 1) / 2 : ta * tb;
  if (ntiles == 0 || B == 0) return 0;
  // sizes known here (no per-head column count): nothing to reduce when no
  // head splits
  if (!p.msz && atb_shape(p.mA_const, p.mB_const, SYM, p.G, p.cap_tiles, p.nrows, B).ks == 1)
    return 0;
  // a head splits only with fewer than kAtbGrid / (2 B) tiles
  int rt = kAtbGrid / (2 * B);
  if (rt > ntiles) rt = ntiles;
  return rt < 1 ? 0 : rt * 16;
}

template <class TB, bool SYM>
static void launch_atb(const double* A, size_t sA, int lda, const int32_t* colA, size_t sColA,
                       const TB* Bm, size_t sB, int ldb, double* C, size_t sC, int ldc, int nrows,
                       const int32_t* msz, int mA, int mB, double* part, size_t part_cap, int B,
                       hipStream_t st) {
  const int ta = (mA + kTile - 1) / kTile, tb = (mB + kTile - 1) / kTile;
  if ((SYM ? ta * (ta + 1) / 2 : ta * tb) == 0 || B == 0) return;
  const AtbArgs<TB> p = atb_args<TB, SYM>(A, sA, lda, colA, sColA, Bm, sB, ldb, C, sC, ldc, nrows,
                                          msz, mA, mB, part, part_cap, B, kAtbGrid);
  hipLaunchKernelGGL((k_atb<TB, SYM>), dim3(B * p.G), dim3(256), 0, st, p, B);
  const int rx = atb_reduce_x<TB, SYM>(p, B);
  if (rx > 0) hipLaunchKernelGGL((k_atb_reduce<TB, SYM>), dim3(rx, B), dim3(256), 0, st, p);
}

// Two products in one launch (and one reduction launch), each aiming at half
// the usual grid and taking half of the partials buffer.
template <class TB1, bool S1, class TB2, bool S2>
static void launch_atb2(const AtbArgs<TB1>& p1, const AtbArgs<TB2>& p2, int B, hipStream_t st) {
  hipLaunchKernelGGL((k_atb2<TB1, S1, TB2, S2>), dim3(B * (p1.G + p2.G)), dim3(256), 0, st, p1,
                     p2, B);
  const int r1 = atb_reduce_x<TB1, S1>(p1, B), r2 = atb_reduce_x<TB2, S2>(p2, B);
  if (r1 + r2 > 0)
    hipLaunchKernelGGL((k_atb_reduce2<TB1, S1, TB2, S2>), dim3(r1 + r2, B), dim3(256), 0, st, p1,
                       p2, r1);
}

int sweep_ld(int t, int D) {
  return (t + kSB - 1) / kSB * kSB + (D + kSB - 1) / kSB * kSB;
}

template <class In, int D>
hipError_t launch_fit(const void* Qv, const void* Kv, const void* Vv, const double* lse,
                      const float* O, const int32_t* idx, FitBufs fb, float* out_bias,
                      void* out_V, bool v_bf16, int32_t* status, int B, int n, int T, int t,
                      double ridge, int max_iters, int qg, hipStream_t st) {
  const In* Q = static_cast<const In*>(Qv);
  const In* K = static_cast<const In*>(Kv);
  const In* V = static_cast<const In*>(Vv);
  const int tt = (t + kTile - 1) / kTile, tn = (n + kTile - 1) / kTile;
  int ld = sweep_ld(t, D);
  size_t sS = static_cast<size_t>(ld) * ld, sUV = static_cast<size_t>(ld) * kSB;
  constexpr int rv = (D + kSB - 1) / kSB * kSB;  // right-hand-side rows of the value system
  const size_t sPS = static_cast<size_t>(n) * t;
  // P_S, M = P_S^T P_S (into the bias system's variable block), column sums
  prof_mark(3, false, st);
  hipLaunchKernelGGL((k_ps<In, D, double>), dim3(tn * tt, B), dim3(256), 0, st, Q, K, idx, lse, fb.PS,
                     fb.colpart, fb.tv, n, T, t, tt, qg);
  prof_mark(3, true, st);
  prof_mark(4, false, st);
  launch_atb<double, true>(fb.PS, sPS, t, nullptr, 0, fb.PS, sPS, t,
                           fb.S + static_cast<size_t>(kSB) * ld + kSB, sS, ld, n, fb.tv, t, t,
                           fb.part, fb.part_cap, B, st);
  prof_mark(4, true, st);
  hipLaunchKernelGGL(k_bias_lam, dim3(B), dim3(1024), 0, st, fb.S, sS, ld, fb.lam, fb.tv, t,
                     ridge);
  hipLaunchKernelGGL(k_bias_prep, dim3((t + 15) / 16, B), dim3(1024), 0, st, fb.S, sS, ld,
                     fb.colpart, tn, fb.cvec, fb.lam, fb.tv, t, fb.bar, kBarWords);
  // pivoting rounds: one launch, a team per head
  prof_mark(5, false, st);
  int cap = coop_capacity(reinterpret_cast<const void*>(&k_nnls_sweep));
  if (cap <= 0) return hipErrorLaunchFailure;
  int tx;
  const int nvb = (t + kSB - 1) / kSB;
  int grid = team_shape(B, nvb + nvb * (nvb + 1) / 2, cap, tx);
  hipError_t e;
  int* err = reinterpret_cast<int*>(fb.bar + kBarWords - 1);
  const int32_t* tvp = fb.tv;
  {
    const double* psp = fb.PS;
    const double* cvp = fb.cvec;
    void* args[] = {&fb.S,   &sS,      &ld,        &fb.U,   &fb.V,  &sUV,     &fb.stage, &fb.wv,
                    &fb.Fidx, &fb.inv, &fb.msz,    &status, &fb.bar, &err,    &fb.xcc,
                    &fb.flops, &tvp,   &B,        &t,         &max_iters, &tx, &fb.wait_ticks,
                    &psp,     &n,      &cvp,      &fb.lam,   &ridge};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&k_nnls_sweep), dim3(grid),
                        dim3(kTeamThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  prof_mark(5, true, st);
  // value fit on the passive set: G = X_F^T X_F + lam_v I, R = X_F^T O + lam_v V_F
  prof_mark(6, false, st);
  hipLaunchKernelGGL(k_value_prep, dim3((n + 3) / 4, B), dim3(256), 0, st, fb.PS, fb.wv, fb.inv, n,
                     t);
  double* G0 = fb.S + static_cast<size_t>(rv) * ld + rv;
  double* R0 = fb.S + static_cast<size_t>(rv) * ld;
  prof_mark(11, false, st);
  {
    // G = X_F^T X_F and X_F^T O side by side
    const size_t half = fb.part_cap / 2;
    const AtbArgs<double> pg = atb_args<double, true>(fb.PS, sPS, t, nullptr, 0, fb.PS, sPS, t, G0,
                                                      sS, ld, n, fb.msz, t, t, fb.part, half, B,
                                                      kAtbGrid / 2);
    const AtbArgs<float> pr = atb_args<float, false>(
        fb.PS, sPS, t, nullptr, 0, O, static_cast<size_t>(n) * D, D, R0, sS, ld, n, fb.msz, t, D,
        fb.part + half, half, B, kAtbGrid / 2);
    launch_atb2<double, true, float, false>(pg, pr, B, st);
  }
  prof_mark(11, true, st);
  hipLaunchKernelGGL(k_ridge_v, dim3(B), dim3(256), 0, st, G0, sS, ld, fb.msz, fb.lam, fb.tv, t);
  hipLaunchKernelGGL((k_rhs_ridge<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, R0, sS,
                     ld, V, idx, fb.Fidx, fb.msz, fb.lam, T, t, D, fb.bar, kBarWords);
  cap = coop_capacity(reinterpret_cast<const void*>(&k_value_sweep));
  if (cap <= 0) return hipErrorLaunchFailure;
  constexpr int nrb = rv / kSB;
  grid = team_shape(B, nvb * nrb + nvb * (nvb + 1) / 2, cap, tx);
  prof_mark(12, false, st);
  {
    int r_al = rv, Dv = D, full = fb.refine > 0 ? 1 : 0;
    const int32_t* ms = fb.msz;
    void* args[] = {&fb.S,   &sS,     &ld,  &r_al,   &fb.U,     &fb.V, &sUV, &fb.stage,
                    &ms,     &status, &fb.bar, &err, &fb.xcc, &fb.flops, &B,  &Dv,
                    &tx,     &fb.wait_ticks, &full};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&k_value_sweep), dim3(grid),
                        dim3(kTeamThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  prof_mark(12, true, st);
  for (int step = 0; step < fb.refine; ++step) {
    hipLaunchKernelGGL((k_csne_resid<D>), dim3((n + kTile - 1) / kTile, D / kTile, B), dim3(256),
                       0, st, fb.PS, R0, sS, ld, O, fb.msz, fb.E, n, t);
    launch_atb<double, false>(fb.PS, sPS, t, nullptr, 0, fb.E, static_cast<size_t>(n) * D, D,
                              fb.Rp, static_cast<size_t>(t) * D, D, n, fb.msz, t, D, fb.part,
                              fb.part_cap, B, st);
    hipLaunchKernelGGL((k_csne_update<In, D>), dim3(tt, D / kTile, B), dim3(256), 0, st, R0, G0,
                       sS, ld, fb.Rp, V, idx, fb.Fidx, fb.msz, fb.lam, fb.Cn, T, t);
    hipLaunchKernelGGL(k_csne_copy, dim3((t * D + 255) / 256, B), dim3(256), 0, st, R0, sS, ld,
                       fb.Cn, fb.msz, t, D);
  }
  if (v_bf16)
    hipLaunchKernelGGL((k_write_out<In, bf16_t>), dim3((t * D + 255) / 256, B), dim3(256), 0, st,
                       R0, sS, ld, V, idx, fb.inv, fb.wv, static_cast<bf16_t*>(out_V), out_bias, T,
                       t, D);
  else
    hipLaunchKernelGGL((k_write_out<In, float>), dim3((t * D + 255) / 256, B), dim3(256), 0, st,
                       R0, sS, ld, V, idx, fb.inv, fb.wv, static_cast<float*>(out_V), out_bias, T,
                       t, D);
  prof_mark(6, true, st);
  return hipGetLastError();
}

// P [B][n][T] float32 of every key (the dictionary of the greedy selection).
template <class In, int D>
hipError_t launch_probs_all(const void* Q, const void* K, const double* lse, float* P, int B,
                            int n, int T, int qg, hipStream_t st) {
  const int tt = (T + kTile - 1) / kTile, tn = (n + kTile - 1) / kTile;
  hipLaunchKernelGGL((k_ps<In, D, float>), dim3(tn * tt, B), dim3(256), 0, st,
                     static_cast<const In*>(Q), static_cast<const In*>(K), nullptr, lse, P,
                     nullptr, nullptr, n, T, T, tt, qg);
  return hipGetLastError();
}

#define KVC_INST_FIT(In, D)                                                                   \
  template hipError_t launch_fit<In, D>(const void*, const void*, const void*, const double*, \
                                        const float*, const int32_t*, FitBufs, float*, void*,  \
                                        bool, int32_t*, int, int, int, int, double, int, int, \
                                        hipStream_t);
#define KVC_INST_PROBS(In, D)                                                          \
  template hipError_t launch_probs_all<In, D>(const void*, const void*, const double*, \
                                              float*, int, int, int, int, hipStream_t);
KVC_INST_PROBS(bf16_t, 128)
KVC_INST_PROBS(bf16_t, 64)
KVC_INST_PROBS(float, 128)
KVC_INST_PROBS(float, 64)
KVC_INST_FIT(bf16_t, 128)
KVC_INST_FIT(bf16_t, 64)
KVC_INST_FIT(float, 128)
KVC_INST_FIT(float, 64)

}  // namespace kvc
