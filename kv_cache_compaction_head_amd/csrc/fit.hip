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
                                            const double* __restrict__ lse,
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
              exp(acc[ra][rb][i] - lse[static_cast<size_t>(b) * n + r]);
      }
}

// ---------------------------------------------------------------------------
// C[b][a][c] = sum_i A[b][i][ca(a)] * Bm[b][i][c]  for a < mA_b, c < mB_b.
// ca: optional per-head column map of A.  SYM: B = A, lower tiles only,
// mirrored.  grid (tiles, ksplit, B): with ksplit > 1 each workgroup sums a
// slice of the rows into part[b][split][tile][64*64] and k_atb_reduce adds
// the slices in order.  The next 16-row chunk is fetched into registers while
// the MFMAs consume the current one.
// ---------------------------------------------------------------------------
template <class TB, bool SYM>
__global__ __launch_bounds__(256) void k_atb(const double* __restrict__ A, size_t sA, int lda,
                                             const int32_t* __restrict__ colA, size_t sColA,
                                             const TB* __restrict__ Bm, size_t sB, int ldb,
                                             double* __restrict__ C, size_t sC, int ldc,
                                             int nrows, const int32_t* __restrict__ msz,
                                             int mA_const, int mB_const, int tiles_x,
                                             double* __restrict__ part, int ntiles) {
  __shared__ double sAt[kKC * kTile], sBt[kKC * kTile];
  const int b = blockIdx.z, split = blockIdx.y, ksplit = gridDim.y;
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
  // this slice's rows, whole 16-row chunks
  const int nchunk = (nrows + kKC - 1) / kKC;
  const int per = (nchunk + ksplit - 1) / ksplit;
  const int k0 = split * per * kKC, k1 = min(nrows, (split + 1) * per * kKC);
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
  f64x4 acc[2][2] = {};
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
  if (ksplit == 1) {
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
  } else {
    double* P = part + ((static_cast<size_t>(b) * ksplit + split) * ntiles + blockIdx.x) * (kTile * kTile);
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          P[tile_row(wave, lane, ra, i) * kTile + tile_col(wave, lane, rb)] = acc[ra][rb][i];
  }
}

// Sum the ksplit row slices of each tile in order and store (mirrored for
// symmetric products).  grid (tiles, B), block 256.
template <bool SYM>
__global__ __launch_bounds__(256) void k_atb_reduce(const double* __restrict__ part,
                                                    double* __restrict__ C, size_t sC, int ldc,
                                                    const int32_t* __restrict__ msz, int mA_const,
                                                    int mB_const, int tiles_x, int ntiles,
                                                    int ksplit) {
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
  double* Cb = C + b * sC;
  const double* P = part + (static_cast<size_t>(b) * ksplit * ntiles + blockIdx.x) * (kTile * kTile);
  for (int e = threadIdx.x; e < kTile * kTile; e += 256) {
    const int r = a0 + e / kTile, c = c0 + e % kTile;
    double v = 0.0;
    for (int sp = 0; sp < ksplit; ++sp) v += P[static_cast<size_t>(sp) * ntiles * kTile * kTile + e];
    if (r < mA && c < mB) {
      Cb[static_cast<size_t>(r) * ldc + c] = v;
      if (SYM && tx != ty) Cb[static_cast<size_t>(c) * ldc + r] = v;
    }
  }
}

// Column sums of P_S in two fixed-order stages: partial sums over 256-row
// slabs, then over slabs.  grid (ceil(t/64), ceil(n/256), B), block (64, 4).
__global__ void k_colsum_part(const double* __restrict__ PS, double* __restrict__ part, int n,
                              int t) {
  __shared__ double sh[4][64];
  const int b = blockIdx.z, a = blockIdx.x * 64 + threadIdx.x;
  const int i0 = blockIdx.y * 256, i1 = min(n, i0 + 256);
  double s = 0.0;
  if (a < t)
    for (int i = i0 + threadIdx.y; i < i1; i += 4) s += PS[(static_cast<size_t>(b) * n + i) * t + a];
  sh[threadIdx.y][threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.y == 0 && a < t)
    part[(static_cast<size_t>(b) * gridDim.y + blockIdx.y) * t + a] =
        ((sh[0][threadIdx.x] + sh[1][threadIdx.x]) + sh[2][threadIdx.x]) + sh[3][threadIdx.x];
}

__global__ void k_colsum_final(const double* __restrict__ part, double* __restrict__ out, int nslab,
                               int t) {
  const int b = blockIdx.y, a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= t) return;
  double s = 0.0;
  for (int k = 0; k < nslab; ++k) s += part[(static_cast<size_t>(b) * nslab + k) * t + a];
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

// ---------------------------------------------------------------------------
// Teams.  The iterative parts of the fits (the pivoting rounds of the NNLS and
// the value system's factorization and solve) run in one cooperative launch:
// each head gets a team of g co-resident workgroups synchronised by
// team_sync, a barrier through a counter in global memory.
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
  unsigned* ctr;
  unsigned gen;
  int* err;
  bool fast;
};

__device__ __forceinline__ int hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xf;  // HW_REG_XCC_ID[3:0]
}

__device__ void team_sync(Team& tm) {
  if (tm.size == 1) {
    __syncthreads();
    return;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!tm.fast) __threadfence();
    atomicAdd(tm.ctr, 1u);
    const unsigned target = (tm.gen + 1) * static_cast<unsigned>(tm.size);
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(tm.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(tm.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
      if (wall_clock64() - t0 > kSpinTicks) {
        atomicOr(tm.err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (tm.fast) asm volatile("buffer_inv sc1" ::: "memory");
    else __threadfence();
  }
  tm.gen++;
  __syncthreads();
}

// Team of this workgroup from the XCD-aligned mapping, then one agent-fenced
// barrier to compare the members' XCC ids (fast barrier if they all match).
__device__ void team_setup(Team& tm, int& team, int& nteams, unsigned* bar, int* err, int* xcc,
                           int tx) {
  nteams = kXcds * tx;
  team = static_cast<int>(blockIdx.x % nteams);
  tm.rank = static_cast<int>(blockIdx.x / nteams);
  tm.size = static_cast<int>(gridDim.x / nteams);
  tm.ctr = bar + team;
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

constexpr int kMaxTeamT = 4096;  // largest t the team kernels stage in LDS
// Team kernels run 256 threads per workgroup; staging loops are unrolled on
// that so every thread issues its loads back to back.
constexpr int kTeamThreads = 256;

struct __align__(16) TeamSmem {
  double sx[kMaxTeamT];
  int sF[kMaxTeamT];
  double sD[kNB][kNB + 1];
  double sA[kKC * kTile];
  double sB[kKC * kTile];
  double col[2][kNB];
  double vec[4][kNB];
  double dpiv[kNB];
  double rdiag[kNB];
  double red[16];
  int ired[16];
  int scan[64];
};
// The team kernels' LDS, at file scope so that the (non-inlined) helpers
// address it as LDS rather than through generic pointers.
__shared__ TeamSmem g_team_smem;


// Factor sD[0:kb][0:kb] (lower) in place, 256 threads.  The block is padded
// to 64 x 64 with the identity, so everything below is fixed-size and
// branch-free: four 16-column micro-panels, each factored by wave 0 alone
// (lane = row, the micro-panel's 16 values in registers, pivot and column
// values broadcast with readlane, so the 16 column steps need no workgroup
// barrier), followed by the rank-16 update of the trailing block on fp64
// MFMA.  Upper-triangle entries are computed but never stored.  sm.rdiag
// receives 1/L[c][c].  A pivot <= 0 is replaced by 1 and flags status bit 1.
__device__ __forceinline__ double bcast(double v, int lane) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// 1/sqrt(x) for x > 0 to full double precision: hardware estimate, two
// Newton steps y <- y (3 - x y^2) / 2.
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x * y, y, 1.5);
  y = y * fma(-0.5 * x * y, y, 1.5);
  return y;
}

__device__ __noinline__ void factor_diag(int kb, int32_t* status, int b) {
  TeamSmem& sm = g_team_smem;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (kb < kNB) {
    for (int e = tid; e < kNB * kNB; e += kTeamThreads) {
      const int r = e >> 6, c = e & 63;
      if (r >= kb || c >= kb) sm.sD[r][c] = r == c ? 1.0 : 0.0;
    }
    __syncthreads();
  }
  constexpr int MP = 16;
#pragma unroll
  for (int p = 0; p < kNB / MP; ++p) {
    const int p0 = p * MP;
    if (wave == 0) {
      double a[MP];
#pragma unroll
      for (int j = 0; j < MP; ++j) a[j] = sm.sD[lane][p0 + j];
      bool bad = false;
#pragma unroll
      for (int c = 0; c < MP; ++c) {
        double piv = bcast(a[c], p0 + c);
        bad |= !(piv > 0.0);
        piv = piv > 0.0 ? piv : 1.0;
        const double y = rsqrt_f64(piv);
        a[c] = lane > p0 + c ? a[c] * y : (lane == p0 + c ? piv * y : a[c]);
        if (lane == 0) sm.rdiag[p0 + c] = y;
#pragma unroll
        for (int j = c + 1; j < MP; ++j) a[j] = fma(-a[c], bcast(a[c], p0 + j), a[j]);
      }
      if (bad && lane == 0 && status) atomicOr(&status[b], 1);
#pragma unroll
      for (int j = 0; j < MP; ++j)
        if (p0 + j <= lane) sm.sD[lane][p0 + j] = a[j];
    }
    __syncthreads();
    if (p + 1 < kNB / MP) {
      // trailing rows/cols [p0+16, 64): C -= P P^T, P = columns p0..p0+15
      const int t0 = p0 + MP, nt = (kNB - t0) / 16;
      for (int tau = wave; tau < nt * nt; tau += 4) {
        const int R = t0 + 16 * (tau / nt), Cc = t0 + 16 * (tau % nt);
        f64x4 acc = {};
#pragma unroll
        for (int ks = 0; ks < MP / 4; ++ks) {
          const int k = p0 + 4 * ks + (lane >> 4);
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(sm.sD[R + (lane & 15)][k],
                                                     sm.sD[Cc + (lane & 15)][k], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.sD[R + (lane >> 4) + 4 * i][Cc + (lane & 15)] -= acc[i];
      }
      __syncthreads();
    }
  }
}

__device__ void load_diag(const double* W, int ld, int k, int kb) {
  TeamSmem& sm = g_team_smem;
  double v[kNB * kNB / kTeamThreads];
#pragma unroll
  for (int i = 0; i < kNB * kNB / kTeamThreads; ++i) {
    const int e = threadIdx.x + i * kTeamThreads, r = e >> 6, c = e & 63;
    v[i] = (r < kb && c <= r) ? ldc(&W[static_cast<size_t>(k + r) * ld + k + c]) : 0.0;
  }
#pragma unroll
  for (int i = 0; i < kNB * kNB / kTeamThreads; ++i) {
    const int e = threadIdx.x + i * kTeamThreads;
    sm.sD[e >> 6][e & 63] = v[i];
  }
  __syncthreads();
  if (threadIdx.x < kNB) sm.rdiag[threadIdx.x] = threadIdx.x < kb ? 1.0 / sm.sD[threadIdx.x][threadIdx.x] : 0.0;
  __syncthreads();
}

__device__ void store_diag(double* W, int ld, int k, int kb) {
  const TeamSmem& sm = g_team_smem;
  for (int e = threadIdx.x; e < kNB * kNB; e += blockDim.x) {
    const int r = e >> 6, c = e & 63;
    if (r < kb && c <= r) stc(&W[static_cast<size_t>(k + r) * ld + k + c], sm.sD[r][c]);
  }
  __syncthreads();
}

// Rows [r0, r1) of the panel at column k: L[i, k:k+64] = A[i, k:k+64] L_kk^{-T}
// with L_kk in sm.sD.  One thread per row; each half row (32 values) is loaded
// in one batch before the substitution uses it.
__device__ __noinline__ void trsm_rows(double* W, int ld, int k, int r0, int r1) {
  const TeamSmem& sm = g_team_smem;
  const int i = r0 + threadIdx.x;
  if (i >= r1) return;
  double* row = W + static_cast<size_t>(i) * ld + k;
  constexpr int H = kNB / 2;
  double x[H], y[H];
#pragma unroll
  for (int c = 0; c < H; ++c) x[c] = ldc(&row[c]);
#pragma unroll
  for (int c = 0; c < H; ++c) y[c] = ldc(&row[H + c]);
// independent partial sums shorten the dependent chains 4x
#pragma unroll
  for (int c = 0; c < H; ++c) {
    double v0 = x[c], v1 = 0.0, v2 = 0.0, v3 = 0.0;
#pragma unroll
    for (int e = 0; e + 3 < c; e += 4) {
      v0 -= x[e] * sm.sD[c][e];
      v1 -= x[e + 1] * sm.sD[c][e + 1];
      v2 -= x[e + 2] * sm.sD[c][e + 2];
      v3 -= x[e + 3] * sm.sD[c][e + 3];
    }
#pragma unroll
    for (int e = c & ~3; e < c; ++e) v0 -= x[e] * sm.sD[c][e];
    x[c] = ((v0 + v1) + (v2 + v3)) * sm.rdiag[c];
  }
#pragma unroll
  for (int c = 0; c < H; ++c) {
    double v0 = y[c], v1 = 0.0, v2 = 0.0, v3 = 0.0;
#pragma unroll
    for (int e = 0; e < H; e += 4) {
      v0 -= x[e] * sm.sD[H + c][e];
      v1 -= x[e + 1] * sm.sD[H + c][e + 1];
      v2 -= x[e + 2] * sm.sD[H + c][e + 2];
      v3 -= x[e + 3] * sm.sD[H + c][e + 3];
    }
#pragma unroll
    for (int e = 0; e + 3 < c; e += 4) {
      v0 -= y[e] * sm.sD[H + c][H + e];
      v1 -= y[e + 1] * sm.sD[H + c][H + e + 1];
      v2 -= y[e + 2] * sm.sD[H + c][H + e + 2];
      v3 -= y[e + 3] * sm.sD[H + c][H + e + 3];
    }
#pragma unroll
    for (int e = c & ~3; e < c; ++e) v0 -= y[e] * sm.sD[H + c][H + e];
    y[c] = ((v0 + v1) + (v2 + v3)) * sm.rdiag[H + c];
  }
#pragma unroll
  for (int c = 0; c < H; ++c) stc(&row[c], x[c]);
#pragma unroll
  for (int c = 0; c < H; ++c) stc(&row[H + c], y[c]);
}

// One lower tile of the trailing update after panel k; tile 0 (the next
// diagonal block) is then factored in place.
__device__ __noinline__ void syrk_tile(double* W, int ld, int m, int k, int tau, int32_t* status,
                                       int b) {
  TeamSmem& sm = g_team_smem;
  const int s0 = k + kNB;
  int ty, tx;
  tri_decode(tau, ty, tx);
  const int r0 = s0 + ty * kTile, c0 = s0 + tx * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f64x4 acc[2][2] = {};
  constexpr int NE = kKC * kTile / kTeamThreads;
  constexpr int NCH = kNB / kKC;
  double va[NCH][NE], vb[NCH][NE];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int e = threadIdx.x + q * kTeamThreads, r = e / kKC, c = e % kKC;
      const int i = r0 + r, j = c0 + r;
      va[ch][q] = i < m ? ldc(&W[static_cast<size_t>(i) * ld + k + ch * kKC + c]) : 0.0;
      vb[ch][q] = j < m ? ldc(&W[static_cast<size_t>(j) * ld + k + ch * kKC + c]) : 0.0;
    }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int e = threadIdx.x + q * kTeamThreads, r = e / kKC, c = e % kKC;
      sm.sA[c * kTile + r] = va[ch][q];
      sm.sB[c * kTile + r] = vb[ch][q];
    }
    __syncthreads();
    tile_mma(sm.sA, sm.sB, acc, wave, lane);
  }
  const bool diag = tau == 0;
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = tile_row(wave, lane, ra, i), cc = tile_col(wave, lane, rb);
        const int r = r0 + rr, c = c0 + cc;
        if (r < m && c <= r) {
          double* p = &W[static_cast<size_t>(r) * ld + c];
          const double v = ldc(p) - acc[ra][rb][i];
          if (diag) sm.sD[rr][cc] = v;
          else stc(p, v);
        } else if (diag) {
          sm.sD[rr][cc] = 0.0;
        }
      }
  __syncthreads();
  if (!diag) return;
  const int kb = min(kNB, m - s0);
  factor_diag(kb, status, b);
  store_diag(W, ld, s0, kb);
}

// Blocked right-looking Cholesky of the m x m lower triangle of W by a team:
// panel rows split over members by 256-row chunks, trailing tiles round-robin.
__device__ __noinline__ void chol_team(double* W, int ld, int m, Team& tm, int32_t* status,
                                       int b) {
  if (m > 0 && tm.rank == 0) {
    const int kb = min(kNB, m);
    load_diag(W, ld, 0, kb);
    factor_diag(kb, status, b);
    store_diag(W, ld, 0, kb);
  }
  team_sync(tm);
  for (int k = 0; k + kNB < m; k += kNB) {
    const int below = m - k - kNB;
    const int nchunk = (below + 255) / 256;
    if (tm.rank < nchunk) {
      load_diag(W, ld, k, kNB);
      for (int ch = tm.rank; ch < nchunk; ch += tm.size)
        trsm_rows(W, ld, k, k + kNB + ch * 256, m);
    }
    team_sync(tm);
    const int nt = (below + kTile - 1) / kTile;
    const int ntiles = nt * (nt + 1) / 2;
    for (int tau = tm.rank; tau < ntiles; tau += tm.size) syrk_tile(W, ld, m, k, tau, status, b);
    team_sync(tm);
  }
}

// Solve L L^T Y = Y in place for columns [c0, c0+4) of Y [m][ncol] (row stride
// ncol), one wave per column (ncol = 1 for a vector).  The waves walk the
// diagonal blocks together: block staged in LDS, triangle with lane = row,
// then the off-diagonal rows.  All accesses coherent (ldc/stc).
__device__ __noinline__ void chol_solve_cols(const double* L, int ld, int m, double* Y, int ncol,
                                             int c0) {
  TeamSmem& sm = g_team_smem;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = c0 + wave;
  const bool on = col < ncol;
  for (int kb = 0; kb < m; kb += kNB) {
    const int nb = min(kNB, m - kb);
    __syncthreads();
    load_diag(L, ld, kb, nb);
    if (on) {
      double v = lane < nb ? ldc(&Y[static_cast<size_t>(kb + lane) * ncol + col]) : 0.0;
      for (int e = 0; e < nb; ++e) {
        if (lane == e) v *= sm.rdiag[e];
        const double ve = bcast(v, e);
        if (lane > e && lane < nb) v -= sm.sD[lane][e] * ve;
      }
      if (lane < nb) stc(&Y[static_cast<size_t>(kb + lane) * ncol + col], v);
      sm.vec[wave][lane] = lane < nb ? v : 0.0;
      for (int r2 = kb + nb + lane; r2 < m; r2 += 64) {
        const double* row = L + static_cast<size_t>(r2) * ld + kb;
        double* py = &Y[static_cast<size_t>(r2) * ncol + col];
        const double yv = ldc(py);
        double acc = 0.0;
#pragma unroll 1
        for (int e0 = 0; e0 < kNB; e0 += 16) {
          double lv[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) lv[e] = e0 + e < nb ? ldc(&row[e0 + e]) : 0.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc += lv[e] * sm.vec[wave][e0 + e];
        }
        stc(py, yv - acc);
      }
    }
  }
  const int nblk = (m + kNB - 1) / kNB;
  for (int bi = nblk - 1; bi >= 0; --bi) {
    const int kb = bi * kNB, nb = min(kNB, m - kb);
    __syncthreads();
    load_diag(L, ld, kb, nb);
    if (on) {
      double v = lane < nb ? ldc(&Y[static_cast<size_t>(kb + lane) * ncol + col]) : 0.0;
      for (int e = nb - 1; e >= 0; --e) {
        if (lane == e) v *= sm.rdiag[e];
        const double ve = bcast(v, e);
        if (lane < e) v -= sm.sD[e][lane] * ve;
      }
      if (lane < nb) stc(&Y[static_cast<size_t>(kb + lane) * ncol + col], v);
      sm.vec[wave][lane] = lane < nb ? v : 0.0;
      for (int r2 = lane; r2 < kb; r2 += 64) {
        double* py = &Y[static_cast<size_t>(r2) * ncol + col];
        const double yv = ldc(py);
        double acc = 0.0;
#pragma unroll 1
        for (int e0 = 0; e0 < kNB; e0 += 16) {
          double lv[16];
#pragma unroll
          for (int e = 0; e < 16; ++e)
            lv[e] = e0 + e < nb ? ldc(&L[static_cast<size_t>(kb + e0 + e) * ld + r2]) : 0.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc += lv[e] * sm.vec[wave][e0 + e];
        }
        stc(py, yv - acc);
      }
    }
  }
  __syncthreads();
}

// Solve L L^T y = y for one vector with a whole workgroup: diagonal blocks
// staged in LDS and solved by wave 0 (lane = row), the off-diagonal updates
// spread over all 256 threads, four threads per row each loading 16 values in
// one batch and combining with shuffles.
__device__ __noinline__ void chol_solve_vec(const double* L, int ld, int m, double* y) {
  TeamSmem& sm = g_team_smem;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int quad = tid & 3, rsub = tid >> 2;  // 64 rows per pass, 4 threads each
  for (int kb = 0; kb < m; kb += kNB) {
    const int nb = min(kNB, m - kb);
    __syncthreads();
    load_diag(L, ld, kb, nb);
    if (wave == 0) {
      double v = lane < nb ? y[kb + lane] : 0.0;
      for (int e = 0; e < nb; ++e) {
        if (lane == e) v *= sm.rdiag[e];
        const double ve = bcast(v, e);
        if (lane > e && lane < nb) v -= sm.sD[lane][e] * ve;
      }
      if (lane < nb) y[kb + lane] = v;
      sm.vec[0][lane] = lane < nb ? v : 0.0;
    }
    __syncthreads();
    for (int r0 = kb + nb; r0 < m; r0 += 64) {
      const int r2 = r0 + rsub;
      const double* row = L + static_cast<size_t>(r2 < m ? r2 : kb) * ld + kb + quad * 16;
      double lv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) lv[e] = (r2 < m && quad * 16 + e < nb) ? row[e] : 0.0;
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc += lv[e] * sm.vec[0][quad * 16 + e];
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (quad == 0 && r2 < m) y[r2] -= acc;
    }
  }
  const int nblk = (m + kNB - 1) / kNB;
  for (int bi = nblk - 1; bi >= 0; --bi) {
    const int kb = bi * kNB, nb = min(kNB, m - kb);
    __syncthreads();
    load_diag(L, ld, kb, nb);
    if (wave == 0) {
      double v = lane < nb ? y[kb + lane] : 0.0;
      for (int e = nb - 1; e >= 0; --e) {
        if (lane == e) v *= sm.rdiag[e];
        const double ve = bcast(v, e);
        if (lane < e) v -= sm.sD[e][lane] * ve;
      }
      if (lane < nb) y[kb + lane] = v;
      sm.vec[0][lane] = lane < nb ? v : 0.0;
    }
    __syncthreads();
    // y[r2] -= sum_e L[kb+e][r2] x_e for r2 < kb: thread per r2, 16-value batches
    for (int r2 = tid; r2 < kb; r2 += kTeamThreads) {
      double acc = 0.0;
#pragma unroll 1
      for (int e0 = 0; e0 < kNB; e0 += 16) {
        double lv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
          lv[e] = e0 + e < nb ? L[static_cast<size_t>(kb + e0 + e) * ld + r2] : 0.0;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += lv[e] * sm.vec[0][e0 + e];
      }
      y[r2] -= acc;
    }
  }
  __syncthreads();
}

// Passive index list F (ascending), inverse map, |F|, rhs = c[F]; one workgroup.
__device__ __noinline__ void build_index(const int32_t* mk, const double* cb, int32_t* F,
                                         int32_t* inv, int32_t* msz, double* rhs, int t) {
  TeamSmem& sm = g_team_smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int chunk = (t + blockDim.x - 1) / blockDim.x;
  const int c0 = min(t, tid * chunk), c1 = min(t, c0 + chunk);
  int cnt = 0;
  for (int j = c0; j < c1; ++j) cnt += ldc(&mk[j]) != 0;
  int x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sm.scan[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sm.scan[w];
  int pos = base + x - cnt;
  for (int j = c0; j < c1; ++j) {
    if (ldc(&mk[j])) {
      stc(&F[pos], j);
      stc(&inv[j], pos);
      if (rhs) stc(&rhs[pos], cb[j]);
      ++pos;
    } else {
      stc(&inv[j], -1);
    }
  }
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += sm.scan[w];
    sta(msz, tot);
  }
  __syncthreads();
}

__device__ double wg_max(double v) {
  TeamSmem& sm = g_team_smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sm.red[wave] = v;
  __syncthreads();
  double s = -INFINITY;
  for (int w = 0; w < nw; ++w) s = fmax(s, sm.red[w]);
  __syncthreads();
  return s;
}

__device__ int wg_isum(int v) {
  TeamSmem& sm = g_team_smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) sm.ired[wave] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < nw; ++w) s += sm.ired[w];
  __syncthreads();
  return s;
}

__device__ int wg_imax(int v) {
  TeamSmem& sm = g_team_smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sm.ired[wave] = v;
  __syncthreads();
  int s = -1;
  for (int w = 0; w < nw; ++w) s = max(s, sm.ired[w]);
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------------------
// NNLS by block principal pivoting, one team per head (cooperative launch).
// Round: passive list -> gather H_FF -> Cholesky -> solve -> infeasibility of
// every variable -> exchange rule.  The loop stops as soon as the head's
// point is feasible and optimal (KKT), or at max_iters (status bit 2).
// State per head: [0] done (1 ok, 2 capped), [1] best infeasible count,
// [2] backup budget, [3] rounds; tolv[b] the round's gradient tolerance.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_nnls_team(
    const double* __restrict__ H, const double* __restrict__ cvec, double* __restrict__ W,
    double* __restrict__ xs, int32_t* __restrict__ mask, int32_t* __restrict__ Fidx,
    int32_t* __restrict__ inv, int32_t* __restrict__ msz, int32_t* __restrict__ state,
    double* __restrict__ tolv, double* __restrict__ wv, int32_t* __restrict__ viol,
    int32_t* __restrict__ status, unsigned* __restrict__ bar, int* __restrict__ err,
    int* __restrict__ xcc, double* __restrict__ flops, int B, int t, int max_iters, int tx) {
  TeamSmem& sm = g_team_smem;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx);
  const int g = tm.size;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int b = team; b < B; b += nteams) {
    const size_t tt = static_cast<size_t>(t) * t;
    if (tm.rank == 0 && tid == 0) flops[2 * b] = 0.0;
    const double* Hb = H + b * tt;
    const double* cb = cvec + static_cast<size_t>(b) * t;
    double* Wb = W + b * tt;
    double* xb = xs + static_cast<size_t>(b) * t;
    int32_t* mk = mask + static_cast<size_t>(b) * t;
    int32_t* Fb = Fidx + static_cast<size_t>(b) * t;
    int32_t* ib = inv + static_cast<size_t>(b) * t;
    int32_t* vb = viol + static_cast<size_t>(b) * t;
    int32_t* st = state + 4 * b;
    double* w = wv + static_cast<size_t>(b) * t;
    for (int it = 0; it < max_iters; ++it) {
      if (tm.rank == 0) build_index(mk, cb, Fb, ib, &msz[b], xb, t);
      team_sync(tm);
      const int m = lda(&msz[b]);
      for (int a = tid; a < m; a += kTeamThreads) sm.sF[a] = ldc(&Fb[a]);
      __syncthreads();
      for (int a = tm.rank; a < m; a += g) {
        const double* hr = Hb + static_cast<size_t>(sm.sF[a]) * t;
        for (int a2 = tid; a2 <= a; a2 += kTeamThreads)
          stc(&Wb[static_cast<size_t>(a) * t + a2], hr[sm.sF[a2]]);
      }
      team_sync(tm);
      chol_team(Wb, t, m, tm, status, b);
      if (tm.rank == 0) {
        chol_solve_vec(Wb, t, m, xb);
        double cmax = 0.0, hmax = 0.0, xmax = 0.0;
        for (int j = tid; j < t; j += blockDim.x) {
          cmax = fmax(cmax, fabs(cb[j]));
          hmax = fmax(hmax, Hb[static_cast<size_t>(j) * t + j]);
        }
        for (int a = tid; a < m; a += blockDim.x) xmax = fmax(xmax, fabs(ldc(&xb[a])));
        cmax = wg_max(cmax);
        hmax = wg_max(hmax);
        xmax = wg_max(xmax);
        if (tid == 0) {
          sta(&tolv[b], 1e-13 * fmax(cmax, hmax) * fmax(1.0, xmax));
          // fp64 work of this round: factorization and the two triangular solves
          const double md = m;
          flops[2 * b] += md * md * md / 3.0 + 2.0 * md * md;
        }
      }
      team_sync(tm);
      const double tol = lda(&tolv[b]);
      // full-length solution (zero off F) in LDS, then infeasibility: a wave
      // per variable, gradient y_j = H[j,:] x - c_j over the whole row
      for (int j = tid; j < t; j += kTeamThreads) sm.sx[j] = 0.0;
      __syncthreads();
      for (int a = tid; a < m; a += kTeamThreads) sm.sx[sm.sF[a]] = ldc(&xb[a]);
      __syncthreads();
      for (int j = tm.rank * 4 + wave; j < t; j += g * 4) {
        int v = 0;
        if (ldc(&mk[j])) {
          v = sm.sx[j] < 0.0;
        } else {
          const double* hr = Hb + static_cast<size_t>(j) * t;
          double acc = 0.0;
          for (int k2 = lane; k2 < t; k2 += 64) acc += hr[k2] * sm.sx[k2];
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
          v = acc - cb[j] < -tol;
        }
        if (lane == 0) stc(&vb[j], v);
      }
      team_sync(tm);
      if (tm.rank == 0) {
        int nv = 0, vmax = -1;
        for (int j = tid; j < t; j += blockDim.x) {
          w[j] = sm.sx[j];
          if (ldc(&vb[j])) {
            ++nv;
            vmax = max(vmax, j);
          }
        }
        nv = wg_isum(nv);
        vmax = wg_imax(vmax);
        const int N = lda(&st[1]), pbud = lda(&st[2]);
        const int mode = nv == 0 ? 0 : (nv < N || pbud >= 1) ? 1 : 2;
        if (mode == 1) {
          for (int j = tid; j < t; j += blockDim.x)
            if (ldc(&vb[j])) stc(&mk[j], !ldc(&mk[j]));
        } else if (mode == 2 && tid == 0) {
          stc(&mk[vmax], !ldc(&mk[vmax]));
        }
        const bool capped = mode != 0 && it + 1 >= max_iters;
        if (capped)
          for (int j = tid; j < t; j += blockDim.x) w[j] = fmax(w[j], 0.0);
        __syncthreads();
        if (tid == 0) {
          if (mode == 0) sta(&st[0], 1);
          else if (nv < N) {
            sta(&st[1], nv);
            sta(&st[2], 3);
          } else if (pbud >= 1) {
            sta(&st[2], pbud - 1);
          }
          sta(&st[3], it + 1);
          if (capped) {
            sta(&st[0], 2);
            if (status) atomicOr(&status[b], 2);
          }
        }
      }
      team_sync(tm);
      if (lda(&st[0]) != 0) break;
    }
    // final passive list for the value fit (the support of w)
    if (tm.rank == 0) build_index(mk, cb, Fb, ib, &msz[b], nullptr, t);
    team_sync(tm);
  }
  if (tm.rank == 0 && tid == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    for (int b = team; b < B; b += nteams) atomicOr(&status[b], 8);
}

// Value system: Cholesky of G_FF + lam_v I (in W) and solve for the D
// right-hand sides in R, one team per head; members split the columns.
__global__ __launch_bounds__(256) void k_value_team(double* __restrict__ W, double* __restrict__ R,
                                                    const int32_t* __restrict__ msz,
                                                    int32_t* __restrict__ status,
                                                    unsigned* __restrict__ bar,
                                                    int* __restrict__ err, int* __restrict__ xcc,
                                                    double* __restrict__ flops, int B, int t,
                                                    int D, int tx) {
  TeamSmem& sm = g_team_smem;
  Team tm;
  int team, nteams;
  team_setup(tm, team, nteams, bar, err, xcc, tx);
  const int g = tm.size;
  for (int b = team; b < B; b += nteams) {
    const size_t tt = static_cast<size_t>(t) * t;
    double* Wb = W + b * tt;
    double* Rb = R + static_cast<size_t>(b) * t * D;
    const int m = msz[b];
    if (tm.rank == 0 && threadIdx.x == 0) {
      const double md = m;
      flops[2 * b + 1] = md * md * md / 3.0 + 2.0 * md * md * D;
    }
    chol_team(Wb, t, m, tm, status, b);
    for (int c0 = tm.rank * 4; c0 < D; c0 += g * 4) chol_solve_cols(Wb, t, m, Rb, D, c0);
    team_sync(tm);
  }
  if (tm.rank == 0 && threadIdx.x == 0 &&
      __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    for (int b = team; b < B; b += nteams) atomicOr(&status[b], 8);
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

// Co-resident workgroups of a team kernel on the current device (cached).
static int coop_capacity(const void* func) {
  static int cache[2][64] = {};
  const int which = func == reinterpret_cast<const void*>(&k_nnls_team) ? 0 : 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[which][dev] == 0) {
    int nb = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, func, 256, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[which][dev] = nb * cus < kMaxTeamGrid ? nb * cus : kMaxTeamGrid;
  }
  return cache[which][dev];
}

// Team shape: nteams = 8*tx teams (a multiple of the XCD count, so each team
// stays on one XCD), g members each: enough for the first trailing update (up
// to 64), no more than the device holds.  Returns the grid size.
static int team_shape(int B, int t, int cap, int& tx) {
  const int nt = (t + kNB - 1) / kNB;
  int tiles = nt * (nt - 1) / 2;
  tiles = tiles < 1 ? 1 : (tiles > 64 ? 64 : tiles);
  tx = (B + kXcds - 1) / kXcds;
  if (kXcds * tx > cap) tx = cap / kXcds > 0 ? cap / kXcds : 1;
  const int nteams = kXcds * tx;
  int g = cap / nteams < tiles ? cap / nteams : tiles;
  if (g < 1) g = 1;
  return g * nteams;
}

// A^T B over heads with split-K chosen so the grid has ~2048 workgroups.
template <class TB, bool SYM>
static void launch_atb(const double* A, size_t sA, int lda, const int32_t* colA, size_t sColA,
                       const TB* Bm, size_t sB, int ldb, double* C, size_t sC, int ldc, int nrows,
                       const int32_t* msz, int mA, int mB, double* part, size_t part_cap, int B,
                       hipStream_t st) {
  const int ta = (mA + kTile - 1) / kTile, tb = (mB + kTile - 1) / kTile;
  const int ntiles = SYM ? ta * (ta + 1) / 2 : ta * tb;
  const int nchunk = (nrows + kKC - 1) / kKC;
  int ksplit = 2048 / (ntiles * B);
  if (ksplit > 16) ksplit = 16;
  if (ksplit > nchunk / 4) ksplit = nchunk / 4;
  while (ksplit > 1 &&
         static_cast<size_t>(B) * ksplit * ntiles * kTile * kTile > part_cap)
    --ksplit;
  if (ksplit < 1) ksplit = 1;
  hipLaunchKernelGGL((k_atb<TB, SYM>), dim3(ntiles, ksplit, B), dim3(256), 0, st, A, sA, lda,
                     colA, sColA, Bm, sB, ldb, C, sC, ldc, nrows, msz, mA, mB, tb, part, ntiles);
  if (ksplit > 1)
    hipLaunchKernelGGL((k_atb_reduce<SYM>), dim3(ntiles, B), dim3(256), 0, st, part, C, sC, ldc,
                       msz, mA, mB, tb, ntiles, ksplit);
}

template <class In, int D>
hipError_t launch_fit(const void* Qv, const void* Kv, const void* Vv, const double* lse,
                      const float* O, const int32_t* idx, FitBufs fb, float* out_bias,
                      float* out_V, int32_t* status, int B, int n, int T, int t, double ridge,
                      int max_iters, hipStream_t st) {
  const In* Q = static_cast<const In*>(Qv);
  const In* K = static_cast<const In*>(Kv);
  const In* V = static_cast<const In*>(Vv);
  const int tt = (t + kTile - 1) / kTile, tn = (n + kTile - 1) / kTile;
  const size_t tsq = static_cast<size_t>(t) * t;
  // P_S, M = P_S^T P_S (into H), column sums (into cvec)
  prof_mark(3, false, st);
  hipLaunchKernelGGL((k_ps<In, D>), dim3(tn * tt, B), dim3(256), 0, st, Q, K, idx, lse, fb.PS, n,
                     T, t, tt);
  prof_mark(3, true, st);
  prof_mark(4, false, st);
  launch_atb<double, true>(fb.PS, static_cast<size_t>(n) * t, t, nullptr, 0, fb.PS,
                           static_cast<size_t>(n) * t, t, fb.H, tsq, t, n, nullptr, t, t, fb.part,
                           fb.part_cap, B, st);
  prof_mark(4, true, st);
  const int nslab = (n + 255) / 256;
  hipLaunchKernelGGL(k_colsum_part, dim3(tt, nslab, B), dim3(64, 4), 0, st, fb.PS, fb.colpart, n,
                     t);
  hipLaunchKernelGGL(k_colsum_final, dim3((t + 255) / 256, B), dim3(256), 0, st, fb.colpart,
                     fb.cvec, nslab, t);
  hipLaunchKernelGGL(k_bias_prep, dim3(B), dim3(1024), 0, st, fb.H, fb.cvec, fb.lam, fb.mask,
                     fb.state, fb.wv, t, ridge);
  // pivoting rounds: one cooperative launch, a team per head
  prof_mark(5, false, st);
  int cap = coop_capacity(reinterpret_cast<const void*>(&k_nnls_team));
  if (cap <= 0) return hipErrorLaunchFailure;
  int tx;
  int grid = team_shape(B, t, cap, tx);
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(fb.bar), 0, kBarWords, st);
  if (e != hipSuccess) return e;
  {
    const double* H = fb.H;
    const double* cv = fb.cvec;
    int* err = reinterpret_cast<int*>(fb.bar + kBarWords - 1);
    int* xcc = fb.xcc;
    void* args[] = {&H,        &cv,        &fb.W,    &fb.xs,   &fb.mask, &fb.Fidx, &fb.inv,
                    &fb.msz,   &fb.state,  &fb.tolv, &fb.wv,   &fb.viol, &status,  &fb.bar,
                    &err,      &xcc,       &fb.flops, &B,      &t,       &max_iters, &tx};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_nnls_team), dim3(grid),
                                   dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
  }
  prof_mark(5, true, st);
  // value fit on the passive set
  prof_mark(6, false, st);
  hipLaunchKernelGGL(k_value_prep, dim3(n, B), dim3(256), 0, st, fb.PS, fb.wv, n, t);
  launch_atb<double, true>(fb.PS, static_cast<size_t>(n) * t, t, fb.Fidx, t, fb.PS,
                           static_cast<size_t>(n) * t, t, fb.W, tsq, t, n, fb.msz, t, t, fb.part,
                           fb.part_cap, B, st);
  hipLaunchKernelGGL(k_ridge_v, dim3(B), dim3(256), 0, st, fb.W, fb.msz, fb.lam, t, ridge);
  launch_atb<float, false>(fb.PS, static_cast<size_t>(n) * t, t, fb.Fidx, t, O,
                           static_cast<size_t>(n) * D, D, fb.R, static_cast<size_t>(t) * D, D, n,
                           fb.msz, t, D, fb.part, fb.part_cap, B, st);
  hipLaunchKernelGGL((k_rhs_ridge<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, fb.R, V,
                     idx, fb.Fidx, fb.msz, fb.lam, T, t, D);
  cap = coop_capacity(reinterpret_cast<const void*>(&k_value_team));
  if (cap <= 0) return hipErrorLaunchFailure;
  grid = team_shape(B, t, cap, tx);
  e = launch_fill_i32(reinterpret_cast<int32_t*>(fb.bar), 0, kBarWords, st);
  if (e != hipSuccess) return e;
  {
    int* err = reinterpret_cast<int*>(fb.bar + kBarWords - 1);
    const int32_t* ms = fb.msz;
    int Dv = D;
    int* xcc = fb.xcc;
    void* args[] = {&fb.W, &fb.R, &ms, &status, &fb.bar, &err, &xcc, &fb.flops, &B, &t, &Dv, &tx};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_value_team), dim3(grid),
                                   dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_write_out<In>), dim3((t * D + 255) / 256, B), dim3(256), 0, st, fb.R, V,
                     idx, fb.inv, fb.wv, out_V, out_bias, T, t, D);
  prof_mark(6, true, st);
  return hipGetLastError();
}

#define KVC_INST_FIT(In, D)                                                                   \
  template hipError_t launch_fit<In, D>(const void*, const void*, const void*, const double*, \
                                        const float*, const int32_t*, FitBufs, float*, float*, \
                                        int32_t*, int, int, int, int, double, int, hipStream_t);
KVC_INST_FIT(bf16_t, 128)
KVC_INST_FIT(bf16_t, 64)
KVC_INST_FIT(float, 128)
KVC_INST_FIT(float, 64)

}  // namespace kvc
