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
//   k_atb          C = A^T B tiles on fp64 MFMA (Grams, X^T O), split-K
//   k_bias_lam, k_bias_prep   lam_w; H = M + lam_w I, c = P_S^T 1 + lam_w
//   k_nnls_sweep   block principal pivoting on the swept bias system
//   k_value_prep, k_ridge_v, k_rhs_ridge   the value system
//   k_value_sweep  its solve by the same block sweeps
//   k_write_out    C_v and beta to the outputs.
// Keys whose multiplier is pinned at zero carry a factor 1e-30 in X; their
// coupling to the rest is ~1e-30 relative, so the value system is solved on
// the passive set only and those keys keep C_v = V (the ridge prior).
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
// ca: optional per-head column map of A.  SYM: B = A, lower tiles only,
// mirrored.  Each head has G workgroups.  Its split into row slices follows
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

// One 64 x 64 tile (a0, c0) over rows [k0, k1) into acc.
template <class TB, bool SYM>
__device__ __forceinline__ void atb_tile(const double* __restrict__ Ab, int lda,
                                         const int32_t* __restrict__ ca,
                                         const TB* __restrict__ Bb, int ldb, int mA, int mB,
                                         int a0, int c0, int k0, int k1, double* sAt, double* sBt,
                                         f64x4 (&acc)[2][2]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int NE = kKC * kTile / 256;
  int colA_r[NE], colB_r[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int r = (threadIdx.x + q * 256) % kTile;
    const int a = a0 + r, c = c0 + r;
    colA_r[q] = a < mA ? (ca ? ca[a] : a) : -1;
    colB_r[q] = c < mB ? (SYM ? (ca ? ca[c] : c) : c) : -1;
  }
  double va[NE], vb[NE];
  auto fetch = [&](int kbase) {
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int e = threadIdx.x + q * 256, i = kbase + e / kTile;
      va[q] = (i < k1 && colA_r[q] >= 0) ? Ab[static_cast<size_t>(i) * lda + colA_r[q]] : 0.0;
      if (SYM)
        vb[q] = (i < k1 && colB_r[q] >= 0) ? Ab[static_cast<size_t>(i) * lda + colB_r[q]] : 0.0;
      else
        vb[q] = (i < k1 && colB_r[q] >= 0)
                    ? static_cast<double>(Bb[static_cast<size_t>(i) * ldb + colB_r[q]])
                    : 0.0;
    }
  };
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[ra][rb] = f64x4{0.0, 0.0, 0.0, 0.0};
  if (k0 < k1) fetch(k0);
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
    tile_mma(sAt, sBt, acc, wave, lane);
  }
}

template <class TB, bool SYM>
__global__ __launch_bounds__(256) void k_atb(const double* __restrict__ A, size_t sA, int lda,
                                             const int32_t* __restrict__ colA, size_t sColA,
                                             const TB* __restrict__ Bm, size_t sB, int ldb,
                                             double* __restrict__ C, size_t sC, int ldc,
                                             int nrows, const int32_t* __restrict__ msz,
                                             int mA_const, int mB_const,
                                             double* __restrict__ part, int G, int cap_tiles) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int mA = msz ? msz[b] : mA_const;
  const int mB = SYM ? mA : mB_const;
  const AtbShape sh = atb_shape(mA, mB, SYM, G, cap_tiles, nrows, gridDim.x / G);
  if (g >= sh.nt * sh.ks && sh.ks > 1) return;
  const int tb = (mB + kTile - 1) / kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double* Ab = A + b * sA;
  const TB* Bb = Bm + b * sB;
  const int32_t* ca = colA ? colA + b * sColA : nullptr;
  // ks = 1: tile g over all rows, into C; else tile g % nt over row slice
  // g / nt, into the partials (G is at least the tile count of every head)
  const bool whole = sh.ks == 1;
  const int split = whole ? 0 : g / sh.nt, tile = whole ? g : g % sh.nt;
  if (tile >= sh.nt) return;
  const int k0 = whole ? 0 : split * sh.per * kKC;
  const int k1 = whole ? nrows : min(nrows, (split + 1) * sh.per * kKC);
  double* Cb = C + b * sC;
  f64x4 acc[2][2];
  {
    int ty, tx;
    atb_decode(SYM, tile, tb, ty, tx);
    const int a0 = ty * kTile, c0 = tx * kTile;
    atb_tile<TB, SYM>(Ab, lda, ca, Bb, ldb, mA, mB, a0, c0, k0, k1, sAt, sBt, acc);
    double* P = part + (static_cast<size_t>(b) * cap_tiles + split * sh.nt + tile) * (kTile * kTile);
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
          } else if (r < mA && c < mB) {
            Cb[static_cast<size_t>(r) * ldc + c] = acc[ra][rb][i];
            if (SYM && tx != ty) Cb[static_cast<size_t>(c) * ldc + r] = acc[ra][rb][i];
          }
        }
  }
}

// Sum a head's row slices of each tile in order and store (mirrored for
// symmetric products); nothing to do for heads computed whole.  grid
// (tiles that may split * 16, B), block 256: one element per thread.
template <bool SYM>
__global__ __launch_bounds__(256) void k_atb_reduce(const double* __restrict__ part,
                                                    double* __restrict__ C, size_t sC, int ldc,
                                                    const int32_t* __restrict__ msz, int mA_const,
                                                    int mB_const, int nrows, int G,
                                                    int cap_tiles) {
  const int b = blockIdx.y, tile = blockIdx.x >> 4;
  const int mA = msz ? msz[b] : mA_const;
  const int mB = SYM ? mA : mB_const;
  const AtbShape sh = atb_shape(mA, mB, SYM, G, cap_tiles, nrows, gridDim.y);
  if (sh.ks == 1 || tile >= sh.nt) return;
  int ty, tx;
  atb_decode(SYM, tile, (mB + kTile - 1) / kTile, ty, tx);
  const int a0 = ty * kTile, c0 = tx * kTile;
  double* Cb = C + b * sC;
  const double* P = part + (static_cast<size_t>(b) * cap_tiles + tile) * (kTile * kTile);
  const int e = (blockIdx.x & 15) * 256 + threadIdx.x;
  const int r = a0 + e / kTile, c = c0 + e % kTile;
  double v = 0.0;
  for (int sp = 0; sp < sh.ks; ++sp) v += P[static_cast<size_t>(sp) * sh.nt * kTile * kTile + e];
  if (r < mA && c < mB) {
    Cb[static_cast<size_t>(r) * ldc + c] = v;
    if (SYM && tx != ty) Cb[static_cast<size_t>(c) * ldc + r] = v;
  }
}

// c = P_S^T 1 from the partial column sums k_ps writes per 64-query tile:
// four threads per column each add a quarter of the tiles in order, then the
// quarters are added in order.  grid (ceil(t/64), B), block 256.
__global__ __launch_bounds__(256) void k_colsum_final(const double* __restrict__ part,
                                                      double* __restrict__ out, int nslab, int t) {
  __shared__ double sh[4][64];
  const int b = blockIdx.y, col = threadIdx.x & 63, qt = threadIdx.x >> 6;
  const int a = blockIdx.x * 64 + col;
  const int per = (nslab + 3) / 4, k0 = qt * per, k1 = min(nslab, k0 + per);
  double s = 0.0;
  if (a < t)
    for (int k = k0; k < k1; ++k) s += part[(static_cast<size_t>(b) * nslab + k) * t + a];
  sh[qt][col] = s;
  __syncthreads();
  if (qt == 0 && a < t) out[static_cast<size_t>(b) * t + a] = ((sh[0][col] + sh[1][col]) + sh[2][col]) + sh[3][col];
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
// is already in the variable block.  k_bias_lam: lam_w = ridge * tr(M) / t
// (grid (B), block 1024).  k_bias_prep then adds lam_w to the diagonal,
// stores c = P_S^T 1 + lam_w in column 0 of the variable rows and clears
// columns 1..63 (unused right-hand-side slots), one wave per row (grid
// (ceil(t/16), B), block 1024).
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
  if (threadIdx.x == 0) lam[2 * b] = ridge * tr / t;
}
__global__ __launch_bounds__(1024) void k_bias_prep(double* __restrict__ S, size_t sS, int ld,
                                                    const double* __restrict__ colsum,
                                                    const double* __restrict__ lam,
                                                    const int32_t* __restrict__ tv, int t_str) {
  const int b = blockIdx.y;
  const int t = tv ? tv[b] : t_str;
  const double lw = lam[2 * b];
  const int lane = threadIdx.x & 63, a = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (a >= t) return;
  double* row = S + b * sS + static_cast<size_t>(kSB + a) * ld;
  row[lane] = lane == 0 ? colsum[static_cast<size_t>(b) * t_str + a] + lw : 0.0;
  if (lane == 0) row[kSB + a] += lw;
}

// Teams.  The iterative parts of the fits (the NNLS pivoting rounds and the
// value system's sweeps) run in cooperative launches:
// each head gets a team of g co-resident workgroups synchronised by
// team_sync, a barrier through per-member flags in global memory.
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
// Every wait is bounded by the constant-rate wall clock; a wait that runs out
// raises a flag that turns every later wait into a no-op and flags the heads,
// so no workgroup can spin forever.
// ---------------------------------------------------------------------------
constexpr uint64_t kSpinTicks = 2000000000ull;  // 20 s at the 100 MHz wall clock
constexpr int kXcds = 8;                        // round-robin dispatch period

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
      // the time-out and the error flag every 32 polls: each is another round
      // trip that would otherwise delay seeing the last arrival
      if ((++spins & 31u) == 0) {
        if (__hip_atomic_load(tm.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        if (wall_clock64() - t0 > kSpinTicks) {
          if (lane == 0) atomicOr(tm.err, 1);
          break;
        }
      }
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
                           int tx) {
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
  double sW[kSB][17];              // small inverse: panel of a 16-pivot block,
  double sV[kSB][17];              // and L[b, <b] L^-1[<b, <b] (16 x 48)
  double sLb[2][16][17];           // L^-1 of a 16 x 16 diagonal block (two in flight)
  double mbc[16];
  double sgn[kSB];                 // s_q
  int piv[kSB];                    // matrix row of pivot q
  double sgn2[kSB];                // the next step's pivots (lookahead)
  int piv2[kSB];
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
                  uniform(m.ld),    uniform(m.r_al), uniform(m.n_rhs), uniform(m.n_var)};
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
// pivot, and before sweep p its pivot row holds -L_bb^-1[p][j] at the swept
// columns j < p and the pivot on the diagonal.  Inverting the pivot block by
// a blocked sweep instead would form its off-diagonal parts through explicit
// inverses of the 16 x 16 blocks and lose them when those are
// ill-conditioned.  A pivot without the sign s_p is replaced by s_p (the
// system is not numerically definite); small_ldl's return value, meaningful
// in wave 0, says whether that happened.
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

// Wave 0 sweeps the 16 x 16 diagonal block at o of sm.pp.  Lane (g, c) =
// (lane / 16, lane % 16) holds rows 4g .. 4g+3 of column c.  For pivot m the
// pivot column's entries of a lane's rows come from lane m of its 16-lane row
// (DPP row broadcast), and the pivot row's entry of its column from row group
// m / 4 (two lane-half swaps); the pivot itself is read from its lane.
// Records -L^-1 of the block (the pivot rows at their turn) into sL and 1/D
// into sm.rD[o..o+15].  Returns whether a pivot lacked its sign (replaced by
// the sign).
template <int N>
__device__ __forceinline__ double row_bcast(double v) {  // lane N of each 16-lane row
  const unsigned long long u = __double_as_longlong(v);
  // every lane is written (all rows and banks enabled), so no old value
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x150 + N, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), 0x150 + N, 0xF, 0xF, true);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo)));
}
template <int G>
__device__ __forceinline__ unsigned group_bcast32(unsigned x) {  // 16-lane row G to all four
  const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);  // rows (0,0,2,2) / (1,1,3,3)
  const unsigned w = (G & 1) ? s16[1] : s16[0];
  const auto s32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);  // halves (lo,lo) / (hi,hi)
  return (G >> 1) ? s32[1] : s32[0];
}
template <int G>
__device__ __forceinline__ double group_bcast(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = group_bcast32<G>(static_cast<unsigned>(u));
  const unsigned hi = group_bcast32<G>(static_cast<unsigned>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
// 1/d by Newton-Raphson from the hardware estimate (two steps, each squaring
// the relative error: within an ulp or so of the rounded quotient).  The
// pivot chain waits on this reciprocal at every pivot; the IEEE division
// sequence is twice as long.
__device__ __forceinline__ double recip(double d) {
  double r = __builtin_amdgcn_rcp(d);
  double e = fma(-d, r, 1.0);
  r = fma(r, e, r);
  e = fma(-d, r, 1.0);
  return fma(r, e, r);
}
template <int M>
__device__ __forceinline__ void diag_pivot(double (&a)[4], int g, int c, int o, int k,
                                           double (*sL)[17], double& myrd, bool& bad) {
  constexpr int GM = M >> 2, IM = M & 3;
  SweepSmem& sm = g_sw;
  double colm[4];  // A[4g + i][m]
#pragma unroll
  for (int i = 0; i < 4; ++i) colm[i] = row_bcast<M>(a[i]);
  const double rowm = group_bcast<GM>(a[IM]);  // A[m][c]
  const double sg = o + M < k ? sm.sgn[o + M] : 1.0;
  const double d = rdlane(a[IM], 16 * GM + M);
  // a pivot without its sign is replaced by the sign (1/s = s); the test
  // runs beside the reciprocal instead of ahead of it
  const bool ok = d * sg > 0.0;
  bad |= !ok;
  const double rd = ok ? recip(d) : sg;
  // the four row groups write the same values (no branch on the pivot chain)
  sL[M][c] = c < M ? -rowm : (c == M ? 1.0 : 0.0);
  const bool piv = c == M;
  if (piv) myrd = rd;
  const double tm = rowm * rd;  // row m of this column, scaled
  // off the pivot row: the pivot column scales by 1/D, the others lose
  // A[r][m] * A[m][c] / D (a * 1 and colm * 0 are exact)
  const double al = piv ? rd : 1.0, be = piv ? 0.0 : -tm;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double nv = fma(colm[i], be, a[i] * al);
    a[i] = (i == IM && g == GM) ? (piv ? -rd : tm) : nv;
  }
}
template <int... Ms>
__device__ __forceinline__ void diag_pivots(std::integer_sequence<int, Ms...>, double (&a)[4], int g,
                                            int c, int o, int k, double (*sL)[17], double& myrd,
                                            bool& bad) {
  (diag_pivot<Ms>(a, g, c, o, k, sL, myrd, bad), ...);
}
__device__ __forceinline__ bool diag_sweep(int o, int k, double (*sL)[17]) {
  SweepSmem& sm = g_sw;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  bool bad = false;
  double a[4], myrd = 0.0;  // lane c keeps 1/D of pivot c
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = sm.pp[o + 4 * g + i][o + c];
  diag_pivots(std::make_integer_sequence<int, 16>{}, a, g, c, o, k, sL, myrd, bad);
  if (g == 0) sm.rD[o + c] = myrd;
  return bad;
}

// Pipelined blocked L D L^T of the pivot block (16-pivot blocks b): wave 0
// runs the chain the next block waits for -- the sweep of diagonal block b,
// then block b+1's panel rows W = A[b+1, b] L_bb^-T and its diagonal update
// A[b+1, b+1] -= W D_b^-1 W^T -- while waves 1-3 do the rest of block b:
// rows b of L^-1 (-L_bb^-1 L[b, <b] L^-1[<b, <b]), the diagonal block of
// L^-1, the trailing lower blocks other than (b+1, b+1), and the panel L[>b+1,
// b] = W D_b^-1.  Each bulk wave forms the panel rows it needs itself, so one
// workgroup barrier per block suffices; L is parked above the diagonal of
// sm.li, transposed (L[r][c] at li[c][r]), and cleared at the end.
__device__ __forceinline__ bool small_ldl(int k) {
  SweepSmem& sm = g_sw;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int g16 = lane >> 4, l16 = lane & 15;
  bool bad = false;
  const int nb = (k + 15) >> 4, kb = 16 * nb;
  for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
    const int r = e >> 6, c = e & 63;
    if (r >= kb || c >= r) sm.li[r][c] = r == c ? 1.0 : 0.0;
  }
  if (wave == 0) bad = diag_sweep(0, k, sm.sLb[0]);
  for (int j = 0; j < nb; ++j) {
    const int o = 16 * j, o2 = o + 16;
    __syncthreads();  // block j swept, the bulk work of block j - 1 done
    double(*sL)[17] = sm.sLb[j & 1];
    if (wave == 0) {
      if (j + 1 < nb) {
        // W = A[b+1, b] L_bb^-T (W[i][q] = sum_m A[o2+i][o+m] sL[q][m]) and
        // then A[b+1, b+1] -= W D^-1 W^T, each four fp64 MFMAs
        f64x4 w4 = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int m = 4 * ks + g16;
          w4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.pp[o2 + l16][o + m], sL[l16][m], w4, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = g16 + 4 * x;  // W[i][l16]
          sm.sW[i][l16] = w4[x];
          sm.li[o + l16][o2 + i] = w4[x] * sm.rD[o + l16];  // L[o2 + i][o + l16], parked
        }
        f64x4 d4 = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int q = 4 * ks + g16;
          d4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.sW[l16][q] * sm.rD[o + q], sm.sW[l16][q], d4,
                                                    0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) sm.pp[o2 + g16 + 4 * x][o2 + l16] -= d4[x];
        bad |= diag_sweep(o2, k, sm.sLb[(j + 1) & 1]);
      }
    } else {
      const int w = wave - 1;
      if (w < j) {  // rows o..o+15 of L^-1, columns 16w..16w+15
        const int jb = 16 * w;
        double* T = &sm.sV[0][0];
        f64x4 t4 = {};
        for (int i0 = jb; i0 < o; i0 += 4) {
          const int i = i0 + g16;
          t4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.li[i][o + l16], sm.li[i][jb + l16], t4, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) T[(g16 + 4 * x) * 48 + jb + l16] = t4[x];
        f64x4 u4 = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int m2 = 4 * ks + g16;
          u4 = __builtin_amdgcn_mfma_f64_16x16x4f64(sL[l16][m2], T[m2 * 48 + jb + l16], u4, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) sm.li[o + g16 + 4 * x][jb + l16] = -u4[x];
      }
      for (int e = tid - 64; e < 256; e += 192) {
        const int m = e >> 4, jj = e & 15;
        if (jj < m) sm.li[o + m][o + jj] = sL[m][jj];
      }
      // trailing lower blocks (r, c), r >= c > j, but (j + 1, j + 1)
      int idx = 0;
      for (int r = j + 1; r < nb; ++r)
        for (int c = j + 1; c <= r; ++c) {
          if (r == j + 1 && c == j + 1) continue;
          if (idx++ % 3 != w) continue;
          f64x4 acc = {};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int q = 4 * ks + g16;
            double wa = 0.0, wb = 0.0;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const double lq = sL[q][m];
              wa = fma(sm.pp[16 * r + l16][o + m], lq, wa);
              wb = fma(sm.pp[16 * c + l16][o + m], lq, wb);
            }
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(wa * sm.rD[o + q], wb, acc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.pp[16 * r + g16 + 4 * i][16 * c + l16] -= acc[i];
        }
      // the panel of L for rows past block j + 1, parked
      for (int e = tid - 64; e < (kb - o2 - 16) * 16; e += 192) {
        const int row = o2 + 16 + (e >> 4), q = e & 15;
        double w2 = 0.0;
#pragma unroll
        for (int m = 0; m < 16; ++m) w2 = fma(sm.pp[row][o + m], sL[q][m], w2);
        sm.li[o + q][row] = w2 * sm.rD[o + q];
      }
    }
  }
  __syncthreads();
  // clear the parked L; past k: identity rows and columns of L^-1, no pivot
  for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
    const int r = e >> 6, c = e & 63;
    if (c > r) sm.li[r][c] = 0.0;
    else if (r >= k || c >= k) sm.li[r][c] = r == c ? 1.0 : 0.0;
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
// nrb right-hand-side tiles, then, unless Iv < skip, variable tiles 0..Iv.
struct TileWalk {
  int Iv, j, nrb, skip, vb0;
  __device__ int count(int iv) const { return nrb + (iv >= skip ? iv + 1 : 0); }
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
  __device__ int J() const { return j < nrb ? j : vb0 + j - nrb; }
};

// One sweep step over the k pivots in sm.piv / sm.sgn / sm.pos, by the team.
// Tiles whose row band is a variable band below skip_below (and whose column
// is a variable band) are left alone: the value fit never reads them again.
//
// Lookahead: when the next step's kn pivots are already known (sm.piv2,
// sm.sgn2) and the team has more than one member, its last member does no
// tiles; it takes the next pivot block from S before this step's update,
// applies the update to it from the staged W rows (A' = A - W D^-1 W^T; the
// two pivot sets are disjoint), factors it and publishes L^-1 and 1/D in
// M.stage, which the next step loads instead of factoring (pre = true); the
// members that build bands and tiles form B from them.
// Returns whether a pivot of this step had the wrong sign (a lookahead
// member flags its own into *status).
__device__ __noinline__ bool sweep_step(const SweepMat M_arg, Team& team_ref, int k_arg,
                                        int skip_arg, int kn_arg, bool pre_arg, int32_t* status) {
  SweepSmem& sm = g_sw;
  // every argument is the same in all lanes; a called function receives them
  // in vector registers, so say so, or every branch and address derived from
  // them is compiled as divergent (exec-masked)
  const SweepMat M = uniform_mat(M_arg);
  const int k = uniform(k_arg), skip_below = uniform(skip_arg), kn = uniform(kn_arg);
  const bool pre = uniform(static_cast<int>(pre_arg)) != 0;
  // the team in registers for the step: the caller's copy lives in scratch,
  // and every scratch access is a vector memory operation whose wait also
  // waits for all older loads and stores (the ticket atomic, a tile's stores)
  Team tm = uniform_team(team_ref);
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
    __syncthreads();
    bad = small_ldl(k);
  }
  const int nrb = (M.n_rhs + kSB - 1) / kSB, nvb = (M.n_var + kSB - 1) / kSB;
  const int vb0 = M.r_al / kSB;
  const int vmembers = la ? tsize - 1 : tsize;
  // B (for V = U B and the pivot block) only where the bands and tiles are
  // built: the lookahead member needs L^-1 and D alone
  if (!me_la) small_b(k);
  if (!me_la) {
    for (int bi = trank; bi < 2 * (nrb + nvb); bi += vmembers) {
      const int b = bi >> 1;
      v_band(M, b < nrb ? b : vb0 + b - nrb, bi & 1, k);
    }
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
    // and form the block while the others update the tiles
    team_arrive(tm);
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
  for (int iv = 0; iv < nvb; ++iv) total += nrb + (iv >= skip_below ? iv + 1 : 0);
  const int workers = la ? tsize - 1 : tsize;
  const int nw = workers * (kTeamThreads / 64);
  const int parts = 2 * total <= nw ? 4 : (total < nw ? 2 : 1);
  // With at most 16 right-hand sides (the bias system has one), a
  // right-hand-side tile is one task over its first 16 columns (the others
  // are inactive: zero and never updated), ahead of the variable tiles.
  const bool narrow = nrb == 1 && M.n_rhs <= 16;
  const int rtasks = narrow ? nvb : 0;
  const int tasks = narrow ? rtasks + (total - nvb) * parts : total * parts;
  const int nch = (k + 7) / 8;  // contraction chunks of 8 that hold pivots
  if (me_la) {
    // the lookahead member arrived at the first barrier after its gathers;
    // it factors the next block and waits for that barrier only before the
    // next
    if (tid < kSB) sm.sgn[tid] = sm.sgn2[tid];
    __syncthreads();
    const bool bad2 = small_ldl(kn);
    for (int e = tid; e < kSB * kSB; e += kTeamThreads) {
      const int r = e >> 6, c = e & 63;
      M.stage[kSB * kSB + e] = sm.li[r][c];
    }
    if (tid < kSB) M.stage[2 * kSB * kSB + tid] = sm.rD[tid];
    if (bad2 && tid == 0 && status) atomicOr(status, 1);
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
        } else {
          const int av = a - rtasks, part = av % parts;
          TileWalk w{0, 0, narrow ? 0 : nrb, skip_below, vb0};
          w.seek(av / parts);
          if (parts == 1) wave_tile<4, 4>(M, w.I(), w.J(), 0, 0, nch);
          else if (parts == 2) wave_tile<2, 4>(M, w.I(), w.J(), 2 * part, 0, nch);
          else wave_tile<2, 2>(M, w.I(), w.J(), 2 * (part >> 1), 2 * (part & 1), nch);
        }
      }
      tk = ticket_value(pend);
    }
  }
  tm.tbase += tasks + nw;
  // A worker of a single-XCD team fetches the next step's L^-1 and 1/D as
  // soon as the lookahead member has published them (normally before the
  // worker's last tile is done), into registers while the closing barrier
  // completes; L1-bypassing loads, since the same staging area was read a
  // step ago.
  const bool fetch = la && !me_la && tm.fast;
  double nli[kSB * kSB / kTeamThreads], nrd = 0.0;
  if (fetch) {
    if (tid == 0) {
      const uint64_t t0 = wall_clock64();
      unsigned spins = 0;
      while (__hip_atomic_load(tm.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tm.pubs + 1) {
        if ((++spins & 31u) == 0) {
          if (__hip_atomic_load(tm.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
          if (wall_clock64() - t0 > kSpinTicks) {
            atomicOr(tm.err, 1);
            break;
          }
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i)
      nli[i] = __hip_atomic_load(&M.stage[kSB * kSB + tid + i * kTeamThreads], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    if (tid < kSB)
      nrd = __hip_atomic_load(&M.stage[2 * kSB * kSB + tid], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
  }
  team_sync(tm);
  if (fetch) {  // this step's 1/D is no longer read: every wave is past its tiles
#pragma unroll
    for (int i = 0; i < kSB * kSB / kTeamThreads; ++i) {
      const int e = tid + i * kTeamThreads;
      sm.li[e >> 6][e & 63] = nli[i];
    }
    if (tid < kSB) sm.rD[tid] = nrd;
    __syncthreads();
  }
  if (la) tm.pubs += 1;
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
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_nnls_sweep(
    double* __restrict__ S, size_t sS, int ld, double* __restrict__ Ub, double* __restrict__ Vb,
    size_t sUV, double* __restrict__ stage, double* __restrict__ wv, int32_t* __restrict__ Fidx,
    int32_t* __restrict__ inv,
    int32_t* __restrict__ msz, int32_t* __restrict__ status, unsigned* __restrict__ bar,
    int* __restrict__ err, int* __restrict__ xcc, double* __restrict__ flops,
    const int32_t* __restrict__ tv, int B, int t_str, int max_iters, int tx) {
  SweepSmem& sm = g_sw;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx);
  const int tid = threadIdx.x;
  for (int s = tid; s < kMaxRows; s += kTeamThreads) sm.pos[s] = -1;
  constexpr int NV = kMaxTeamT / kTeamThreads;
  for (int b = team; b < B; b += nteams) {
    const int t = tv ? tv[b] : t_str;
    const SweepMat M{gptr(S + b * sS), gptr(Ub + b * sUV), gptr(Vb + b * sUV),
                     gptr(stage + static_cast<size_t>(b) * kStage), ld, kSB, 1, t};
    for (int j = tid; j < t; j += kTeamThreads) sm.inF[j] = 0;
    double cm = 0.0, hm = 0.0;
    for (int j = tid; j < t; j += kTeamThreads) {
      const gdouble* row = M.S + static_cast<size_t>(kSB + j) * ld;
      cm = fmax(cm, fabs(row[0]));
      hm = fmax(hm, row[kSB + j]);
    }
    const double scale = fmax(wg_max(cm), wg_max(hm));
    int N = t + 1, bud = 3, done = 0;
    bool bad = false;
    double fl = 0.0;
    double val[NV];
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
        bad |= sweep_step(M, tm, k, 0, kn, s0 > 0 && tm.size > 1, status ? status + b : nullptr);
        if (tid < k) {
          const int j = sm.list[s0 + tid];
          sm.inF[j] ^= 1;
          sm.pos[kSB + j] = -1;
        }
        __syncthreads();
        fl += sweep_flops(k, t + 1);
      }
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
        if (status) {
          if (done == 2) atomicOr(&status[b], 2);
          if (bad) atomicOr(&status[b], 1);
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
    int* __restrict__ xcc, double* __restrict__ flops, int B, int D, int tx) {
  SweepSmem& sm = g_sw;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx);
  const int tid = threadIdx.x;
  for (int s = tid; s < kMaxRows; s += kTeamThreads) sm.pos[s] = -1;
  for (int b = team; b < B; b += nteams) {
    const int m = msz[b];
    const SweepMat M{gptr(S + b * sS), gptr(Ub + b * sUV), gptr(Vb + b * sUV),
                     gptr(stage + static_cast<size_t>(b) * kStage), ld, r_al, D, m};
    bool bad = false;
    for (int s0 = 0; s0 < m; s0 += kSB) {
      const int k = min(kSB, m - s0);
      const int kn = min(kSB, m - s0 - k);
      if (tid < k) {
        sm.piv[tid] = r_al + s0 + tid;
        sm.sgn[tid] = 1.0;
        sm.pos[r_al + s0 + tid] = static_cast<int16_t>(tid);
      }
      if (tid < kn) {
        sm.piv2[tid] = r_al + s0 + k + tid;
        sm.sgn2[tid] = 1.0;
      }
      __syncthreads();
      bad |= sweep_step(M, tm, k, s0 / kSB, kn, s0 > 0 && tm.size > 1,
                        status ? status + b : nullptr);
      if (tid < k) sm.pos[r_al + s0 + tid] = -1;
      __syncthreads();
    }
    if (tm.rank == 0 && tid == 0) {
      double fl = 0.0;
      for (int s0 = 0; s0 < m; s0 += kSB) fl += sweep_flops(min(kSB, m - s0), m + D);
      flops[2 * b + 1] = fl;
      if (bad && status) atomicOr(&status[b], 1);
    }
  }
  if (tm.rank == 0 && tid == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    for (int b = team; b < B; b += nteams) atomicOr(&status[b], 8);
}

// r_i = sum_a P_S[i][a] w'_a, X = P_S diag(w') / r, w' = max(w, 1e-30); the
// passive columns X_F are written compacted to the front of each row (column
// inv[a] for passive a; the row stride stays t), so the value system's
// products read them contiguously.  The whole row is read before any of it
// is written (block_sum's barrier), which makes the in-place rewrite safe.
// grid (n, B), block 256.
__global__ __launch_bounds__(256) void k_value_prep(double* __restrict__ PS,
                                                    const double* __restrict__ wv,
                                                    const int32_t* __restrict__ inv, int n,
                                                    int t) {
  constexpr int NV = kMaxTeamT / 256;
  __shared__ double sh[16];
  const int b = blockIdx.y, i = blockIdx.x;
  double* row = PS + (static_cast<size_t>(b) * n + i) * t;
  const double* w = wv + static_cast<size_t>(b) * t;
  const int32_t* ib = inv + static_cast<size_t>(b) * t;
  double v[NV];
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int a = threadIdx.x + q * 256;
    v[q] = a < t ? row[a] * fmax(w[a], 1e-30) : 0.0;
    s += v[q];
  }
  s = block_sum(s, sh);
  const double rs = 1.0 / s;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int a = threadIdx.x + q * 256;
    if (a < t) {
      const int slot = ib[a];
      if (slot >= 0) row[slot] = v[q] * rs;
    }
  }
}

// lam_v = ridge * trace(G) / t; G += lam_v I (G at Gb, order msz, stride ld).
// grid (B), block 256.
__global__ void k_ridge_v(double* __restrict__ Gb, size_t sS, int ld,
                          const int32_t* __restrict__ msz, double* __restrict__ lam,
                          const int32_t* __restrict__ tv, int t_str, double ridge) {
  __shared__ double sh[16];
  const int b = blockIdx.x, m = msz[b];
  const int t = tv ? tv[b] : t_str;
  double* G = Gb + b * sS;
  double tr = 0.0;
  for (int a = threadIdx.x; a < m; a += blockDim.x) tr += G[static_cast<size_t>(a) * ld + a];
  tr = block_sum(tr, sh);
  const double lv = ridge * tr / t;
  for (int a = threadIdx.x; a < m; a += blockDim.x) G[static_cast<size_t>(a) * ld + a] += lv;
  if (threadIdx.x == 0) lam[2 * b + 1] = lv;
}

// R[a][c] += lam_v * V[idx[F[a]]][c]  (R at Rb, stride ld).  grid (ceil(t*D/256), B).
template <class In>
__global__ void k_rhs_ridge(double* __restrict__ Rb, size_t sS, int ld, const In* __restrict__ V,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ Fidx,
                            const int32_t* __restrict__ msz, const double* __restrict__ lam,
                            int T, int t, int D) {
  const int b = blockIdx.y, m = msz[b];
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= m) return;
  const int j = idx[static_cast<size_t>(b) * t + Fidx[static_cast<size_t>(b) * t + a]];
  Rb[b * sS + static_cast<size_t>(a) * ld + c] +=
      lam[2 * b + 1] * to_f64<In>(V[(static_cast<size_t>(b) * T + j) * D + c]);
}

// out_V[b][a][c] = fitted value (row inv[a] of C at Cb, stride ld) for passive
// keys, the V row (the prior) for keys whose multiplier is zero;
// out_bias = log(max(w, 1e-30)).  grid (ceil(t*D/256), B).
template <class In>
__global__ void k_write_out(const double* __restrict__ Cb, size_t sS, int ld,
                            const In* __restrict__ V, const int32_t* __restrict__ idx,
                            const int32_t* __restrict__ inv, const double* __restrict__ wv,
                            float* __restrict__ out_V, float* __restrict__ out_bias, int T, int t,
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
  out_V[(static_cast<size_t>(b) * t + a) * D + c] = v;
  if (c == 0)
    out_bias[static_cast<size_t>(b) * t + a] =
        j >= 0 ? static_cast<float>(log(fmax(wv[static_cast<size_t>(b) * t + a], 1e-30)))
               : -INFINITY;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------

// Co-resident workgroups of a team kernel on the current device (cached).
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

// A^T B over heads: G workgroups a head (~2048 in all, at least one a tile
// of the largest product); each head's split-K follows its own sizes.
template <class TB, bool SYM>
static void launch_atb(const double* A, size_t sA, int lda, const int32_t* colA, size_t sColA,
                       const TB* Bm, size_t sB, int ldb, double* C, size_t sC, int ldc, int nrows,
                       const int32_t* msz, int mA, int mB, double* part, size_t part_cap, int B,
                       hipStream_t st) {
  const int ta = (mA + kTile - 1) / kTile, tb = (mB + kTile - 1) / kTile;
  const int ntiles = SYM ? ta * (ta + 1) / 2 : ta * tb;
  if (ntiles == 0 || B == 0) return;
  int G = (kAtbGrid + B - 1) / B;
  if (G > 16 * ntiles) G = 16 * ntiles;
  if (G < ntiles) G = ntiles;
  // odd, so that consecutive heads start on different XCDs (workgroups go
  // round-robin over 8) and their busy workgroups spread evenly
  G |= 1;
  const size_t ct = part_cap / (static_cast<size_t>(B) * kTile * kTile);
  const int cap_tiles = ct > (1u << 20) ? (1 << 20) : static_cast<int>(ct);
  hipLaunchKernelGGL((k_atb<TB, SYM>), dim3(B * G), dim3(256), 0, st, A, sA, lda, colA, sColA, Bm,
                     sB, ldb, C, sC, ldc, nrows, msz, mA, mB, part, G, cap_tiles);
  // sizes known here (no per-head column count): skip the reduction when no
  // head splits
  if (!msz && atb_shape(mA, mB, SYM, G, cap_tiles, nrows, B).ks == 1) return;
  // a head splits only with fewer than kAtbGrid / (2 B) tiles
  int rt = kAtbGrid / (2 * B);
  if (rt > ntiles) rt = ntiles;
  if (rt < 1) return;
  hipLaunchKernelGGL((k_atb_reduce<SYM>), dim3(rt * 16, B), dim3(256), 0, st, part, C, sC, ldc,
                     msz, mA, mB, nrows, G, cap_tiles);
}

int sweep_ld(int t, int D) {
  return (t + kSB - 1) / kSB * kSB + (D + kSB - 1) / kSB * kSB;
}

template <class In, int D>
hipError_t launch_fit(const void* Qv, const void* Kv, const void* Vv, const double* lse,
                      const float* O, const int32_t* idx, FitBufs fb, float* out_bias,
                      float* out_V, int32_t* status, int B, int n, int T, int t, double ridge,
                      int max_iters, int qg, hipStream_t st) {
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
  hipLaunchKernelGGL(k_colsum_final, dim3((t + 63) / 64, B), dim3(256), 0, st, fb.colpart,
                     fb.cvec, tn, t);
  hipLaunchKernelGGL(k_bias_lam, dim3(B), dim3(1024), 0, st, fb.S, sS, ld, fb.lam, fb.tv, t,
                     ridge);
  hipLaunchKernelGGL(k_bias_prep, dim3((t + 15) / 16, B), dim3(1024), 0, st, fb.S, sS, ld, fb.cvec,
                     fb.lam, fb.tv, t);
  // pivoting rounds: one cooperative launch, a team per head
  prof_mark(5, false, st);
  int cap = coop_capacity(reinterpret_cast<const void*>(&k_nnls_sweep));
  if (cap <= 0) return hipErrorLaunchFailure;
  int tx;
  const int nvb = (t + kSB - 1) / kSB;
  int grid = team_shape(B, nvb + nvb * (nvb + 1) / 2, cap, tx);
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(fb.bar), 0, kBarWords, st);
  if (e != hipSuccess) return e;
  int* err = reinterpret_cast<int*>(fb.bar + kBarWords - 1);
  const int32_t* tvp = fb.tv;
  {
    void* args[] = {&fb.S,   &sS,      &ld,        &fb.U,   &fb.V,  &sUV,     &fb.stage, &fb.wv,
                    &fb.Fidx, &fb.inv, &fb.msz,    &status, &fb.bar, &err,    &fb.xcc,
                    &fb.flops, &tvp,   &B,        &t,         &max_iters, &tx};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_nnls_sweep), dim3(grid),
                                   dim3(kTeamThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  prof_mark(5, true, st);
  // value fit on the passive set: G = X_F^T X_F + lam_v I, R = X_F^T O + lam_v V_F
  prof_mark(6, false, st);
  hipLaunchKernelGGL(k_value_prep, dim3(n, B), dim3(256), 0, st, fb.PS, fb.wv, fb.inv, n, t);
  double* G0 = fb.S + static_cast<size_t>(rv) * ld + rv;
  double* R0 = fb.S + static_cast<size_t>(rv) * ld;
  launch_atb<double, true>(fb.PS, sPS, t, nullptr, 0, fb.PS, sPS, t, G0, sS, ld, n, fb.msz, t, t,
                           fb.part, fb.part_cap, B, st);
  hipLaunchKernelGGL(k_ridge_v, dim3(B), dim3(256), 0, st, G0, sS, ld, fb.msz, fb.lam, fb.tv, t,
                     ridge);
  launch_atb<float, false>(fb.PS, sPS, t, nullptr, 0, O, static_cast<size_t>(n) * D, D, R0, sS, ld,
                           n, fb.msz, t, D, fb.part, fb.part_cap, B, st);
  hipLaunchKernelGGL((k_rhs_ridge<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, R0, sS,
                     ld, V, idx, fb.Fidx, fb.msz, fb.lam, T, t, D);
  cap = coop_capacity(reinterpret_cast<const void*>(&k_value_sweep));
  if (cap <= 0) return hipErrorLaunchFailure;
  constexpr int nrb = rv / kSB;
  grid = team_shape(B, nvb * nrb + nvb * (nvb + 1) / 2, cap, tx);
  e = launch_fill_i32(reinterpret_cast<int32_t*>(fb.bar), 0, kBarWords, st);
  if (e != hipSuccess) return e;
  {
    int r_al = rv, Dv = D;
    const int32_t* ms = fb.msz;
    void* args[] = {&fb.S, &sS,     &ld,  &r_al, &fb.U,     &fb.V, &sUV, &fb.stage, &ms,
                    &status, &fb.bar, &err, &fb.xcc, &fb.flops, &B,    &Dv,  &tx};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_value_sweep), dim3(grid),
                                   dim3(kTeamThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_write_out<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, R0, sS,
                     ld, V, idx, fb.inv, fb.wv, out_V, out_bias, T, t, D);
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
                                        const float*, const int32_t*, FitBufs, float*, float*, \
                                        int32_t*, int, int, int, int, double, int, int,      \
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
