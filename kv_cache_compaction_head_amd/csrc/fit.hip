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
// Kernels (one per step, all batched over heads, per-head sizes read on the
// device so nothing syncs with the host):
//   k_ps          P_S = exp(Q C_k^T - lse) on fp64 MFMA (16x16x4)
//   k_atb         C = A^T B tiles on fp64 MFMA (Grams, X^T O)
//   k_bias_prep   lam_w, H = M + lam_w I, c = P_S^T 1 + lam_w, pivoting state
//   k_bpp_index / k_gather_sub / k_bpp_update   block principal pivoting
//                 (Judice & Pires 1994; Kim & Park 2011): solve on the passive
//                 set, exchange every infeasible variable, fall back to single
//                 exchanges (largest index) when the infeasible count stops
//                 shrinking.  The passive-set system is solved by
//   k_potrf_first / k_trsm_panel / k_syrk_update   right-looking blocked
//                 Cholesky, 64 wide
//   k_chol_solve  forward + back substitution, one wave per right-hand side
//   k_value_prep, k_ridge_v, k_rhs_ridge, k_write_out   value fit plumbing.
// Keys whose multiplier is pinned at zero carry a factor 1e-30 in X; their
// coupling to the rest is ~1e-30 relative, so the value system is solved on
// the passive set only and those keys keep C_v = V (the ridge prior).
#include "common.h"
#include "launch.h"

namespace kvc {

constexpr int kTile = 64;   // fp64 output tile (4 waves x 32x32)
constexpr int kKC = 16;     // contraction rows staged per step
constexpr int kNB = 64;     // Cholesky panel width

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
// P_S[b][i][a] = exp(q_i . k_{idx[a]} - lse_i), fp64.  grid (ceil(n/64)*ceil(t/64), B).
// ---------------------------------------------------------------------------
template <class In, int D>
__global__ __launch_bounds__(256) void k_ps(const In* __restrict__ Q, const In* __restrict__ K,
                                            const int32_t* __restrict__ idx,
                                            const float* __restrict__ lse,
                                            double* __restrict__ PS, int n, int T, int t,
                                            int tiles_a) {
  __shared__ double sA[kKC * kTile], sB[kKC * kTile];
  const int b = blockIdx.y, ti = blockIdx.x / tiles_a, ta = blockIdx.x % tiles_a;
  const int i0 = ti * kTile, a0 = ta * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const In* Qb = Q + static_cast<size_t>(b) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;
  const int32_t* ib = idx + static_cast<size_t>(b) * t;
  f64x4 acc[2][2] = {};
  for (int c0 = 0; c0 < D; c0 += kKC) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKC * kTile; e += 256) {
      const int r = e / kKC, c = e % kKC;  // r: tile row, c: contraction index
      const int i = i0 + r, a = a0 + r;
      sA[c * kTile + r] = i < n ? to_f64<In>(Qb[static_cast<size_t>(i) * D + c0 + c]) : 0.0;
      sB[c * kTile + r] = a < t ? to_f64<In>(Kb[static_cast<size_t>(ib[a]) * D + c0 + c]) : 0.0;
    }
    __syncthreads();
    tile_mma(sA, sB, acc, wave, lane);
  }
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + tile_row(wave, lane, ra, i), a = a0 + tile_col(wave, lane, rb);
        if (r < n && a < t)
          PS[(static_cast<size_t>(b) * n + r) * t + a] =
              exp(acc[ra][rb][i] - static_cast<double>(lse[static_cast<size_t>(b) * n + r]));
      }
}

// ---------------------------------------------------------------------------
// C[b][a][c] = sum_i A[b][i][ca(a)] * Bm[b][i][cb(c)]  for a < mA_b, c < mB_b.
// ca/cb: optional per-head column index maps.  SYM: B = A, lower tiles only,
// mirrored.  grid (tiles, B).
// ---------------------------------------------------------------------------
template <class TB, bool SYM>
__global__ __launch_bounds__(256) void k_atb(const double* __restrict__ A, size_t sA, int lda,
                                             const int32_t* __restrict__ colA, size_t sColA,
                                             const TB* __restrict__ Bm, size_t sB, int ldb,
                                             double* __restrict__ C, size_t sC, int ldc,
                                             int nrows, const int32_t* __restrict__ msz,
                                             int mA_const, int mB_const, int tiles_x) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  const int b = blockIdx.y;
  const int mA = msz ? msz[b] : mA_const;
  const int mB = SYM ? mA : mB_const;
  int ty, tx;
  if (SYM) tri_decode(blockIdx.x, ty, tx);
  else {
    ty = blockIdx.x / tiles_x;
    tx = blockIdx.x % tiles_x;
  }
  const int a0 = ty * kTile, c0 = tx * kTile;
  if (a0 >= mA || c0 >= mB) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double* Ab = A + b * sA;
  const TB* Bb = Bm + b * sB;
  const int32_t* ca = colA ? colA + b * sColA : nullptr;
  f64x4 acc[2][2] = {};
  for (int k0 = 0; k0 < nrows; k0 += kKC) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKC * kTile; e += 256) {
      const int k = e / kTile, r = e % kTile;
      const int i = k0 + k;
      const int a = a0 + r, c = c0 + r;
      double va = 0.0, vb = 0.0;
      if (i < nrows) {
        if (a < mA) va = Ab[static_cast<size_t>(i) * lda + (ca ? ca[a] : a)];
        if (SYM) {
          if (c < mB) vb = Ab[static_cast<size_t>(i) * lda + (ca ? ca[c] : c)];
        } else if (c < mB) {
          vb = static_cast<double>(Bb[static_cast<size_t>(i) * ldb + c]);
        }
      }
      sAt[k * kTile + r] = va;
      sBt[k * kTile + r] = vb;
    }
    __syncthreads();
    tile_mma(sAt, sBt, acc, wave, lane);
  }
  double* Cb = C + b * sC;
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = a0 + tile_row(wave, lane, ra, i), c = c0 + tile_col(wave, lane, rb);
        if (r < mA && c < mB) {
          Cb[static_cast<size_t>(r) * ldc + c] = acc[ra][rb][i];
          if (SYM && tx != ty) Cb[static_cast<size_t>(c) * ldc + r] = acc[ra][rb][i];
        }
      }
}

// Column sums of P_S: colsum[b][a] = sum_i P_S[b][i][a].  grid (ceil(t/256), B).
__global__ void k_colsum(const double* __restrict__ PS, double* __restrict__ out, int n, int t) {
  const int b = blockIdx.y, a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= t) return;
  const double* p = PS + static_cast<size_t>(b) * n * t + a;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += p[static_cast<size_t>(i) * t];
  out[static_cast<size_t>(b) * t + a] = s;
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

// Pivoting state per head: [0] done, [1] best infeasible count N, [2] backup
// budget p, [3] rounds run.
// H = M + lam_w I (M in H, full), c = colsum + lam_w, lam_w = ridge*tr(M)/t.
// grid (B), block 1024.
__global__ __launch_bounds__(1024) void k_bias_prep(double* __restrict__ H,
                                                    double* __restrict__ cvec,
                                                    double* __restrict__ lam,
                                                    int32_t* __restrict__ mask,
                                                    int32_t* __restrict__ state,
                                                    double* __restrict__ wv, int t,
                                                    double ridge) {
  __shared__ double sh[16];
  const int b = blockIdx.x;
  double* Hb = H + static_cast<size_t>(b) * t * t;
  double tr = 0.0;
  for (int a = threadIdx.x; a < t; a += blockDim.x) tr += Hb[static_cast<size_t>(a) * t + a];
  tr = block_sum(tr, sh);
  const double lw = ridge * tr / t;
  for (int a = threadIdx.x; a < t; a += blockDim.x) {
    Hb[static_cast<size_t>(a) * t + a] += lw;
    cvec[static_cast<size_t>(b) * t + a] += lw;
    mask[static_cast<size_t>(b) * t + a] = 1;
    wv[static_cast<size_t>(b) * t + a] = 0.0;
  }
  if (threadIdx.x == 0) {
    lam[2 * b] = lw;
    state[4 * b + 0] = 0;
    state[4 * b + 1] = t + 1;
    state[4 * b + 2] = 3;
    state[4 * b + 3] = 0;
  }
}

// Passive index list and its size; rhs = c[F].  grid (B), block 1024.
__global__ __launch_bounds__(1024) void k_bpp_index(const int32_t* __restrict__ mask,
                                                    const double* __restrict__ cvec,
                                                    const int32_t* __restrict__ state,
                                                    int32_t* __restrict__ Fidx,
                                                    int32_t* __restrict__ inv,
                                                    int32_t* __restrict__ msz,
                                                    double* __restrict__ rhs, int t) {
  __shared__ int scr[64];
  const int b = blockIdx.x;
  if (state && state[4 * b]) {
    if (threadIdx.x == 0) msz[b] = 0;  // nothing to factor this round
    return;
  }
  const int32_t* mk = mask + static_cast<size_t>(b) * t;
  const int chunk = (t + blockDim.x - 1) / blockDim.x;
  const int c0 = min(t, static_cast<int>(threadIdx.x) * chunk), c1 = min(t, c0 + chunk);
  int cnt = 0;
  for (int j = c0; j < c1; ++j) cnt += mk[j] != 0;
  // exclusive scan over the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scr[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scr[w];
  int pos = base + x - cnt;
  for (int j = c0; j < c1; ++j) {
    if (mk[j]) {
      Fidx[static_cast<size_t>(b) * t + pos] = j;
      inv[static_cast<size_t>(b) * t + j] = pos;
      if (rhs) rhs[static_cast<size_t>(b) * t + pos] = cvec[static_cast<size_t>(b) * t + j];
      ++pos;
    } else {
      inv[static_cast<size_t>(b) * t + j] = -1;
    }
  }
  if (threadIdx.x == blockDim.x - 1) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += scr[w];
    msz[b] = tot;
  }
}

// W[a][a'] = H[F[a]][F[a']] for a' <= a < m.  grid (ceil(t*t/256), B).
__global__ void k_gather_sub(const double* __restrict__ H, const int32_t* __restrict__ Fidx,
                             const int32_t* __restrict__ msz, double* __restrict__ W, int t) {
  const int b = blockIdx.y, m = msz[b];
  const size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int a = static_cast<int>(e / t), a2 = static_cast<int>(e % t);
  if (a >= m || a2 > a) return;
  const int32_t* F = Fidx + static_cast<size_t>(b) * t;
  W[(static_cast<size_t>(b) * t + a) * t + a2] =
      H[(static_cast<size_t>(b) * t + F[a]) * t + F[a2]];
}

// ---------------------------------------------------------------------------
// Blocked right-looking Cholesky, panel width 64, lower triangle in place.
// Per panel k: k_trsm_panel solves the rows below the (already factored)
// diagonal block, then k_syrk_update subtracts the panel's outer product from
// the trailing lower tiles; the workgroup that owns trailing tile (0,0) -- the
// next diagonal block -- also factors it, so every diagonal block is factored
// by exactly one workgroup after its last update.  A non-positive pivot sets
// status bit 1 and is replaced by 1 (the head is flagged, never NaN).
// ---------------------------------------------------------------------------
typedef double DiagBlock[kNB][kNB + 1];

// Factor sD[0:kb][0:kb] (lower) in place; thread r owns row r.  All threads of
// the block must call it.
__device__ void factor_diag(DiagBlock& sD, int kb, int32_t* status, int b) {
  const int r = threadIdx.x;
  for (int c = 0; c < kb; ++c) {
    if (r == c) {
      double dv = sD[c][c];
      if (!(dv > 0.0)) {
        if (status) status[b] |= 1;
        dv = 1.0;
      }
      sD[c][c] = sqrt(dv);
    }
    __syncthreads();
    if (r > c && r < kb) sD[r][c] /= sD[c][c];
    __syncthreads();
    if (r > c && r < kb) {
      const double lrc = sD[r][c];
      for (int j = c + 1; j <= r; ++j) sD[r][j] -= lrc * sD[j][c];
    }
    __syncthreads();
  }
}

// Factor the first diagonal block of each head.  grid (B), block 256.
__global__ __launch_bounds__(256) void k_potrf_first(double* __restrict__ W, int ld,
                                                     const int32_t* __restrict__ msz,
                                                     int32_t* __restrict__ status) {
  __shared__ DiagBlock sD;
  const int b = blockIdx.x, m = msz[b];
  if (m <= 0) return;
  const int kb = min(kNB, m);
  double* Wb = W + static_cast<size_t>(b) * ld * ld;
  for (int e = threadIdx.x; e < kNB * kNB; e += blockDim.x) {
    const int r = e / kNB, c = e % kNB;
    sD[r][c] = (r < kb && c <= r) ? Wb[static_cast<size_t>(r) * ld + c] : 0.0;
  }
  __syncthreads();
  factor_diag(sD, kb, status, b);
  for (int e = threadIdx.x; e < kb * kb; e += blockDim.x) {
    const int r = e / kb, c = e % kb;
    if (c <= r) Wb[static_cast<size_t>(r) * ld + c] = sD[r][c];
  }
}

// L[i, k:k+64] = A[i, k:k+64] L_kk^{-T} for rows i >= k+64.  grid (nchunks, B).
__global__ __launch_bounds__(256) void k_trsm_panel(double* __restrict__ W, int ld,
                                                    const int32_t* __restrict__ msz, int k) {
  __shared__ DiagBlock sD;
  const int b = blockIdx.y, m = msz[b];
  if (k + kNB >= m) return;
  double* Wb = W + static_cast<size_t>(b) * ld * ld;
  for (int e = threadIdx.x; e < kNB * kNB; e += blockDim.x) {
    const int r = e / kNB, c = e % kNB;
    sD[r][c] = c <= r ? Wb[static_cast<size_t>(k + r) * ld + k + c] : 0.0;
  }
  __syncthreads();
  const int i = k + kNB + blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  double* row = Wb + static_cast<size_t>(i) * ld + k;
  double x[kNB];
#pragma unroll
  for (int c = 0; c < kNB; ++c) {
    double v = row[c];
    for (int e = 0; e < c; ++e) v -= x[e] * sD[c][e];
    x[c] = v / sD[c][c];
  }
#pragma unroll
  for (int c = 0; c < kNB; ++c) row[c] = x[c];
}

// Trailing update A[i][j] -= sum_c L[i][k+c] L[j][k+c] over the lower tiles
// of the trailing block; tile (0,0) then factors the next diagonal block.
// grid (tiles, B), block 256.
__global__ __launch_bounds__(256) void k_syrk_update(double* __restrict__ W, int ld,
                                                     const int32_t* __restrict__ msz, int k,
                                                     int32_t* __restrict__ status) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  __shared__ DiagBlock sD;
  const int b = blockIdx.y, m = msz[b];
  const int s0 = k + kNB;  // first trailing row
  if (s0 >= m) return;
  int ty, tx;
  tri_decode(blockIdx.x, ty, tx);
  const int r0 = s0 + ty * kTile, c0 = s0 + tx * kTile;
  if (r0 >= m) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double* Wb = W + static_cast<size_t>(b) * ld * ld;
  f64x4 acc[2][2] = {};
  for (int kk = 0; kk < kNB; kk += kKC) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKC * kTile; e += 256) {
      const int r = e / kKC, c = e % kKC;
      const int i = r0 + r, j = c0 + r;
      sAt[c * kTile + r] = i < m ? Wb[static_cast<size_t>(i) * ld + k + kk + c] : 0.0;
      sBt[c * kTile + r] = j < m ? Wb[static_cast<size_t>(j) * ld + k + kk + c] : 0.0;
    }
    __syncthreads();
    tile_mma(sAt, sBt, acc, wave, lane);
  }
  const bool diag = ty == 0 && tx == 0;
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = tile_row(wave, lane, ra, i), cc = tile_col(wave, lane, rb);
        const int r = r0 + rr, c = c0 + cc;
        if (r < m && c <= r) {
          const double v = Wb[static_cast<size_t>(r) * ld + c] - acc[ra][rb][i];
          if (diag) sD[rr][cc] = v;
          else Wb[static_cast<size_t>(r) * ld + c] = v;
        } else if (diag) {
          sD[rr][cc] = 0.0;
        }
      }
  if (!diag) return;
  __syncthreads();
  const int kb = min(kNB, m - s0);
  factor_diag(sD, kb, status, b);
  for (int e = threadIdx.x; e < kb * kb; e += blockDim.x) {
    const int r = e / kb, c = e % kb;
    if (c <= r) Wb[static_cast<size_t>(s0 + r) * ld + s0 + c] = sD[r][c];
  }
}

// Solve L L^T x = y in place for nrhs columns of Y [ld_y rows][nrhs] (row a of
// the system at Y[a*nrhs + col]).  One wave per column; grid (ceil(nrhs/4), B),
// block 64*min(4,nrhs).
__global__ __launch_bounds__(256) void k_chol_solve(const double* __restrict__ W, int ld,
                                                    const int32_t* __restrict__ msz,
                                                    double* __restrict__ Y, int nrhs) {
  const int b = blockIdx.y, m = msz[b];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = blockIdx.x * (blockDim.x >> 6) + wave;
  if (col >= nrhs || m == 0) return;
  const double* L = W + static_cast<size_t>(b) * ld * ld;
  double* y = Y + static_cast<size_t>(b) * ld * nrhs + col;
  // forward: L z = y
  for (int kb = 0; kb < m; kb += 64) {
    const int r = kb + lane;
    double v = r < m ? y[static_cast<size_t>(r) * nrhs] : 0.0;
    const int nb = min(64, m - kb);
    for (int e = 0; e < nb; ++e) {
      if (lane == e) v /= L[static_cast<size_t>(r) * ld + r];
      const double ze = __shfl(v, e);
      if (lane > e && r < m) v -= L[static_cast<size_t>(r) * ld + kb + e] * ze;
    }
    if (r < m) y[static_cast<size_t>(r) * nrhs] = v;
    for (int r2 = kb + 64 + lane; r2 - lane < m; r2 += 64) {
      double acc = 0.0;
      for (int e = 0; e < nb; ++e) {
        const double ze = __shfl(v, e);
        if (r2 < m) acc += L[static_cast<size_t>(r2) * ld + kb + e] * ze;
      }
      if (r2 < m) y[static_cast<size_t>(r2) * nrhs] -= acc;
    }
  }
  // backward: L^T x = z
  const int nblk = (m + 63) / 64;
  for (int bi = nblk - 1; bi >= 0; --bi) {
    const int kb = bi * 64, r = kb + lane, nb = min(64, m - kb);
    double v = r < m ? y[static_cast<size_t>(r) * nrhs] : 0.0;
    for (int e = nb - 1; e >= 0; --e) {
      if (lane == e) v /= L[static_cast<size_t>(r) * ld + r];
      const double xe = __shfl(v, e);
      if (lane < e) v -= L[static_cast<size_t>(kb + e) * ld + r] * xe;
    }
    if (r < m) y[static_cast<size_t>(r) * nrhs] = v;
    for (int r2 = lane; r2 < kb; r2 += 64) {
      double acc = 0.0;
      for (int e = 0; e < nb; ++e) {
        const double xe = __shfl(v, e);
        acc += L[static_cast<size_t>(kb + e) * ld + r2] * xe;
      }
      y[static_cast<size_t>(r2) * nrhs] -= acc;
    }
  }
}

// One pivoting round's bookkeeping.  x (passive solution) in xs[b][0..m);
// full-length w; gradient y_j = (H w - c)_j for j off F; exchange rule.
// grid (B), block 1024.
__global__ __launch_bounds__(1024) void k_bpp_update(const double* __restrict__ H,
                                                     const double* __restrict__ cvec,
                                                     const double* __restrict__ xs,
                                                     const int32_t* __restrict__ Fidx,
                                                     const int32_t* __restrict__ msz,
                                                     int32_t* __restrict__ mask,
                                                     int32_t* __restrict__ state,
                                                     double* __restrict__ wv,
                                                     int32_t* __restrict__ status, int t,
                                                     int max_iters) {
  __shared__ double shd[16];
  __shared__ int shi[16];
  __shared__ int s_vmax;
  const int b = blockIdx.x;
  int32_t* st = state + 4 * b;
  if (st[0]) return;
  const int m = msz[b];
  const double* Hb = H + static_cast<size_t>(b) * t * t;
  const double* cb = cvec + static_cast<size_t>(b) * t;
  const int32_t* F = Fidx + static_cast<size_t>(b) * t;
  int32_t* mk = mask + static_cast<size_t>(b) * t;
  double* w = wv + static_cast<size_t>(b) * t;
  const double* x = xs + static_cast<size_t>(b) * t;
  for (int j = threadIdx.x; j < t; j += blockDim.x) w[j] = 0.0;
  __syncthreads();
  for (int a = threadIdx.x; a < m; a += blockDim.x) w[F[a]] = x[a];
  __syncthreads();
  double cmax = 0.0, hmax = 0.0, xmax = 0.0;
  for (int j = threadIdx.x; j < t; j += blockDim.x) {
    cmax = fmax(cmax, fabs(cb[j]));
    hmax = fmax(hmax, Hb[static_cast<size_t>(j) * t + j]);
    xmax = fmax(xmax, fabs(w[j]));
  }
  cmax = block_max(cmax, shd);
  hmax = block_max(hmax, shd);
  xmax = block_max(xmax, shd);
  const double tol = 1e-13 * fmax(cmax, hmax) * fmax(1.0, xmax);
  if (threadIdx.x == 0) s_vmax = -1;
  __syncthreads();
  int nv = 0, vmax = -1;
  for (int j = threadIdx.x; j < t; j += blockDim.x) {
    bool infeasible;
    if (mk[j]) {
      infeasible = w[j] < 0.0;
    } else {
      const double* hr = Hb + static_cast<size_t>(j) * t;
      double y = -cb[j];
      for (int a = 0; a < m; ++a) y += hr[F[a]] * x[a];
      infeasible = y < -tol;
    }
    if (infeasible) {
      ++nv;
      vmax = max(vmax, j);
    }
  }
  nv = block_count(nv, shi);
  atomicMax(&s_vmax, vmax);
  __syncthreads();
  vmax = s_vmax;
  const int it = st[3] + 1;
  int mode;  // 0 done, 1 exchange all, 2 exchange the largest index only
  if (nv == 0) {
    mode = 0;
  } else if (nv < st[1]) {
    mode = 1;
  } else if (st[2] >= 1) {
    mode = 1;
  } else {
    mode = 2;
  }
  __syncthreads();
  if (mode == 1) {
    // recompute the infeasible set and flip it (reads mask before writes: the
    // decision for j depends only on j's own entry and on x, H, c)
    for (int j = threadIdx.x; j < t; j += blockDim.x) {
      bool infeasible;
      if (mk[j]) {
        infeasible = w[j] < 0.0;
      } else {
        const double* hr = Hb + static_cast<size_t>(j) * t;
        double y = -cb[j];
        for (int a = 0; a < m; ++a) y += hr[F[a]] * x[a];
        infeasible = y < -tol;
      }
      if (infeasible) mk[j] = !mk[j];
    }
  } else if (mode == 2 && threadIdx.x == 0) {
    mk[vmax] = !mk[vmax];
  }
  if (threadIdx.x == 0) {
    if (mode == 0) st[0] = 1;
    else if (nv < st[1]) {
      st[1] = nv;
      st[2] = 3;
    } else if (st[2] >= 1) {
      st[2] -= 1;
    }
    st[3] = it;
    if (mode != 0 && it >= max_iters) {
      st[0] = 2;
      if (status) status[b] |= 2;
    }
  }
  if (mode != 0 && it >= max_iters) {
    __syncthreads();
    for (int j = threadIdx.x; j < t; j += blockDim.x) w[j] = fmax(w[j], 0.0);
  }
}

// r_i = sum_a P_S[i][a] w'_a, X = P_S diag(w') / r (in place), w' = max(w, 1e-30).
// grid (n, B), block 256.
__global__ __launch_bounds__(256) void k_value_prep(double* __restrict__ PS,
                                                    const double* __restrict__ wv, int n,
                                                    int t) {
  __shared__ double sh[16];
  const int b = blockIdx.y, i = blockIdx.x;
  double* row = PS + (static_cast<size_t>(b) * n + i) * t;
  const double* w = wv + static_cast<size_t>(b) * t;
  double s = 0.0;
  for (int a = threadIdx.x; a < t; a += blockDim.x) s += row[a] * fmax(w[a], 1e-30);
  s = block_sum(s, sh);
  const double inv = 1.0 / s;
  for (int a = threadIdx.x; a < t; a += blockDim.x) row[a] = row[a] * fmax(w[a], 1e-30) * inv;
}

// lam_v = ridge * trace(G) / t; G += lam_v I (G = W, size msz).  grid (B), block 256.
__global__ void k_ridge_v(double* __restrict__ W, const int32_t* __restrict__ msz,
                          double* __restrict__ lam, int t, double ridge) {
  __shared__ double sh[16];
  const int b = blockIdx.x, m = msz[b];
  double* Wb = W + static_cast<size_t>(b) * t * t;
  double tr = 0.0;
  for (int a = threadIdx.x; a < m; a += blockDim.x) tr += Wb[static_cast<size_t>(a) * t + a];
  tr = block_sum(tr, sh);
  const double lv = ridge * tr / t;
  for (int a = threadIdx.x; a < m; a += blockDim.x) Wb[static_cast<size_t>(a) * t + a] += lv;
  if (threadIdx.x == 0) lam[2 * b + 1] = lv;
}

// R[a][c] += lam_v * V[idx[F[a]]][c].  grid (ceil(t*D/256), B).
template <class In>
__global__ void k_rhs_ridge(double* __restrict__ R, const In* __restrict__ V,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ Fidx,
                            const int32_t* __restrict__ msz, const double* __restrict__ lam,
                            int T, int t, int D) {
  const int b = blockIdx.y, m = msz[b];
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= m) return;
  const int j = idx[static_cast<size_t>(b) * t + Fidx[static_cast<size_t>(b) * t + a]];
  R[(static_cast<size_t>(b) * t + a) * D + c] +=
      lam[2 * b + 1] * to_f64<In>(V[(static_cast<size_t>(b) * T + j) * D + c]);
}

// out_V[b][a][c] = fitted value for passive keys, V row (the prior) for keys
// whose multiplier is zero; out_bias = log(max(w, 1e-30)).  grid (ceil(t*D/256), B).
template <class In>
__global__ void k_write_out(const double* __restrict__ R, const In* __restrict__ V,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ inv,
                            const double* __restrict__ wv, float* __restrict__ out_V,
                            float* __restrict__ out_bias, int T, int t, int D) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D;
  if (a >= t) return;
  const int p = inv[static_cast<size_t>(b) * t + a];
  float v;
  if (p >= 0) {
    v = static_cast<float>(R[(static_cast<size_t>(b) * t + p) * D + c]);
  } else {
    const int j = idx[static_cast<size_t>(b) * t + a];
    v = to_f32<In>(V[(static_cast<size_t>(b) * T + j) * D + c]);
  }
  out_V[(static_cast<size_t>(b) * t + a) * D + c] = v;
  if (c == 0)
    out_bias[static_cast<size_t>(b) * t + a] =
        static_cast<float>(log(fmax(wv[static_cast<size_t>(b) * t + a], 1e-30)));
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------

static hipError_t launch_cholesky(double* W, int ld, const int32_t* msz, int B, int tmax,
                                  int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_potrf_first, dim3(B), dim3(256), 0, st, W, ld, msz, status);
  for (int k = 0; k + kNB < tmax; k += kNB) {
    const int below = tmax - k - kNB;
    hipLaunchKernelGGL(k_trsm_panel, dim3((below + 255) / 256, B), dim3(256), 0, st, W, ld, msz,
                       k);
    const int nt = (below + kTile - 1) / kTile;
    hipLaunchKernelGGL(k_syrk_update, dim3(nt * (nt + 1) / 2, B), dim3(256), 0, st, W, ld, msz,
                       k, status);
  }
  return hipGetLastError();
}

template <class In, int D>
hipError_t launch_fit(const void* Qv, const void* Kv, const void* Vv, const float* lse,
                      const float* O, const int32_t* idx, FitBufs fb, float* out_bias,
                      float* out_V, int32_t* status, int B, int n, int T, int t, double ridge,
                      int max_iters, hipStream_t st) {
  const In* Q = static_cast<const In*>(Qv);
  const In* K = static_cast<const In*>(Kv);
  const In* V = static_cast<const In*>(Vv);
  const int tt = (t + kTile - 1) / kTile, tn = (n + kTile - 1) / kTile;
  // P_S, M = P_S^T P_S (into H), colsum (into cvec)
  prof_mark(3, false, st);
  hipLaunchKernelGGL((k_ps<In, D>), dim3(tn * tt, B), dim3(256), 0, st, Q, K, idx, lse, fb.PS, n,
                     T, t, tt);
  prof_mark(3, true, st);
  prof_mark(4, false, st);
  hipLaunchKernelGGL((k_atb<double, true>), dim3(tt * (tt + 1) / 2, B), dim3(256), 0, st, fb.PS,
                     static_cast<size_t>(n) * t, t, nullptr, size_t(0), fb.PS,
                     static_cast<size_t>(n) * t, t, fb.H, static_cast<size_t>(t) * t, t, n,
                     nullptr, t, t, tt);
  prof_mark(4, true, st);
  hipLaunchKernelGGL(k_colsum, dim3((t + 255) / 256, B), dim3(256), 0, st, fb.PS, fb.cvec, n, t);
  hipLaunchKernelGGL(k_bias_prep, dim3(B), dim3(1024), 0, st, fb.H, fb.cvec, fb.lam, fb.mask,
                     fb.state, fb.wv, t, ridge);
  // block principal pivoting rounds
  const size_t tsq = static_cast<size_t>(t) * t;
  prof_mark(5, false, st);
  for (int it = 0; it < max_iters; ++it) {
    hipLaunchKernelGGL(k_bpp_index, dim3(B), dim3(1024), 0, st, fb.mask, fb.cvec, fb.state,
                       fb.Fidx, fb.inv, fb.msz, fb.xs, t);
    hipLaunchKernelGGL(k_gather_sub, dim3((tsq + 255) / 256, B), dim3(256), 0, st, fb.H, fb.Fidx,
                       fb.msz, fb.W, t);
    (void)launch_cholesky(fb.W, t, fb.msz, B, t, status, st);
    hipLaunchKernelGGL(k_chol_solve, dim3(1, B), dim3(64), 0, st, fb.W, t, fb.msz, fb.xs, 1);
    hipLaunchKernelGGL(k_bpp_update, dim3(B), dim3(1024), 0, st, fb.H, fb.cvec, fb.xs, fb.Fidx,
                       fb.msz, fb.mask, fb.state, fb.wv, status, t, max_iters);
  }
  prof_mark(5, true, st);
  // final passive set (done heads keep their mask) -> index lists
  prof_mark(6, false, st);
  hipLaunchKernelGGL(k_bpp_index, dim3(B), dim3(1024), 0, st, fb.mask, fb.cvec,
                     static_cast<const int32_t*>(nullptr), fb.Fidx, fb.inv, fb.msz,
                     static_cast<double*>(nullptr), t);
  // value fit on the passive set
  hipLaunchKernelGGL(k_value_prep, dim3(n, B), dim3(256), 0, st, fb.PS, fb.wv, n, t);
  hipLaunchKernelGGL((k_atb<double, true>), dim3(tt * (tt + 1) / 2, B), dim3(256), 0, st, fb.PS,
                     static_cast<size_t>(n) * t, t, fb.Fidx, static_cast<size_t>(t), fb.PS,
                     static_cast<size_t>(n) * t, t, fb.W, tsq, t, n, fb.msz, t, t, tt);
  hipLaunchKernelGGL(k_ridge_v, dim3(B), dim3(256), 0, st, fb.W, fb.msz, fb.lam, t, ridge);
  const int td = D / kTile;
  hipLaunchKernelGGL((k_atb<float, false>), dim3(tt * td, B), dim3(256), 0, st, fb.PS,
                     static_cast<size_t>(n) * t, t, fb.Fidx, static_cast<size_t>(t), O,
                     static_cast<size_t>(n) * D, D, fb.R, static_cast<size_t>(t) * D, D, n,
                     fb.msz, t, D, td);
  hipLaunchKernelGGL((k_rhs_ridge<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, fb.R, V,
                     idx, fb.Fidx, fb.msz, fb.lam, T, t, D);
  (void)launch_cholesky(fb.W, t, fb.msz, B, t, status, st);
  hipLaunchKernelGGL(k_chol_solve, dim3(D / 4, B), dim3(256), 0, st, fb.W, t, fb.msz, fb.R, D);
  hipLaunchKernelGGL((k_write_out<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, fb.R, V,
                     idx, fb.inv, fb.wv, out_V, out_bias, T, t, D);
  prof_mark(6, true, st);
  return hipGetLastError();
}

#define KVC_INST_FIT(In, D)                                                                   \
  template hipError_t launch_fit<In, D>(const void*, const void*, const void*, const float*,  \
                                        const float*, const int32_t*, FitBufs, float*, float*, \
                                        int32_t*, int, int, int, int, double, int, hipStream_t);
KVC_INST_FIT(bf16_t, 128)
KVC_INST_FIT(bf16_t, 64)
KVC_INST_FIT(float, 128)
KVC_INST_FIT(float, 64)

}  // namespace kvc
