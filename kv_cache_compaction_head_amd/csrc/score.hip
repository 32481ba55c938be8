// Score path: reference queries against the full cache.
//
// "Fast KV Compaction via Attention Matching", section 2 (main objective and
// key selection): both matching equations are built from exp(q K^T); the
// softmax denominator is the attention mass, and keys are ranked by the RMS
// over the reference queries of their softmax weight.
//
//   k_score_lse   s = K Q^T tile by tile on MFMA (bf16 in, fp32 accumulate;
//                 fp32 MFMA for fp32 input), an online (max, sum exp) per
//                 query over one key split -> partial (m, l).
//   k_lse_merge   fixed-order merge of the splits -> lse.
//   k_expweight   recomputes s, p = exp(s - lse); per-key column sums of p^2
//                 (or p) over the workgroup's queries -> importance partials;
//                 O^T += V^T P^T on MFMA, with P split into bf16 hi + lo so the
//                 product keeps ~16 mantissa bits -> partial O per key split.
//   k_o_reduce, k_imp_reduce   fixed-order sums of the partials.
//
// Every reduction runs in a fixed order (no float atomics): results are
// bitwise reproducible run to run.
//
// Tiling: a workgroup is 4 waves; each wave owns 32 reference queries whose
// MFMA B-operands stay in registers.  The scores are produced transposed
// (keys as MFMA rows, queries as columns) so that each lane owns one query and
// 16 keys: the per-query max/sum stays inside the lane, and the P fragment is
// already the B operand of the O^T = V^T P^T product.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "sel.h"

namespace kvc {

template <class In> struct Frag;
template <> struct Frag<bf16_t> {
  static constexpr int KS = 16;  // contraction depth of one MFMA
  using T = bf16x8;
  __device__ static T load(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static T zero() { return T{}; }
  __device__ static f32x16 mma(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<float> {
  static constexpr int KS = 2;
  using T = float;
  __device__ static T load(const float* p) { return *p; }
  __device__ static T zero() { return 0.f; }
  __device__ static f32x16 mma(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // reference queries per workgroup
constexpr int kXcd = 8;           // workgroups are dispatched round-robin over 8 XCDs

// Score-kernel grid: one workgroup per (query block, key split, head), laid
// out so that all query blocks of one (split, head) pair run on the same XCD
// in consecutive slots: the K/V tiles they all read are then shared through
// that XCD's L2 instead of being fetched once per query block.  Pair p goes
// to XCD p mod 8; the grid has roundup(pairs, 8) * nqb workgroups.
__device__ __forceinline__ bool score_grid(int nqb, int nsplit, int B, int& qb, int& split,
                                           int& b) {
  const int w = blockIdx.x, xcd = w % kXcd, slot = w / kXcd;
  qb = slot % nqb;
  const int p = (slot / nqb) * kXcd + xcd;
  if (p >= nsplit * B) return false;
  split = p % nsplit;
  b = p / nsplit;
  return true;
}
static int score_grid_size(int nqb, int nsplit, int B) {
  const int pairs = nsplit * B;
  return (pairs + kXcd - 1) / kXcd * kXcd * nqb;
}

// Copy a [rows x D] tile of a row-major [*, D] matrix into LDS (row stride LD),
// zero-filling rows at or past `valid`.
template <class In, int D, int LD>
__device__ __forceinline__ void load_tile(In* s, const In* g, int rows, int valid) {
  constexpr int VEC = 16 / sizeof(In);
  constexpr int CPR = D / VEC;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < rows * CPR; c += blockDim.x) {
    const int r = c / CPR, col = (c % CPR) * VEC;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < valid) v = *reinterpret_cast<const uint4*>(g + static_cast<size_t>(r) * D + col);
    *reinterpret_cast<uint4*>(s + r * LD + col) = v;
  }
}

template <class In, int D>
__device__ __forceinline__ void load_q_frags(typename Frag<In>::T* bq, const In* Qb, int q, int n,
                                             int g) {
  constexpr int KS = Frag<In>::KS;
#pragma unroll
  for (int ks = 0; ks < D / KS; ++ks)
    bq[ks] = q < n ? Frag<In>::load(Qb + static_cast<size_t>(q) * D + ks * KS + g * (KS / 2))
                   : Frag<In>::zero();
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at dst + 16 l (dst the same for the whole wave).
__device__ __forceinline__ void lds_copy16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// XOR swizzle of the 16-byte chunks of a key row in an unpadded LDS tile
// with CPR chunks per row.  Two reads have to be conflict-free:
//  - an MFMA operand read (16 bytes a lane): lane l takes row l mod 32, one
//    chunk, so 16 consecutive rows must land in 16 distinct 16-byte bank
//    groups;
//  - the value tile's transpose read (8 bytes a lane): 32 lanes take 4
//    consecutive rows (4-aligned) x 4 consecutive chunks (4-aligned), which
//    must also land in 16 distinct groups.
// At 16 chunks a row (d = 128) the swizzle is linear over GF(2) in the row's
// low four bits, bit b contributing 4, 10, 1, 2 for b = 0..3: rows 0..15 map
// to a permutation of 0..15, and the four rows of a 4-aligned quad map to
// four different 4-aligned chunk groups, which serves both reads.  (The plain
// r mod 16 served the first and put the second four rows to a group.)
template <int CPR>
__host__ __device__ constexpr int k_swz(int r) {
  static_assert(CPR == 8 || CPR == 16, "16-byte chunks per row");
  if constexpr (CPR == 16) {
    return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
  } else {
    return (r / 2) & 7;
  }
}

// Bit r set when accumulator row r of this lane holds a live key: tile key
// st*32 + mfma32_row(r, lane) below `valid` and not excluded (bit set in excl).
__device__ __forceinline__ unsigned live_rows(int st, int valid, uint64_t excl, int lane) {
  const uint64_t vm = valid >= 64 ? ~0ull : ((1ull << (valid > 0 ? valid : 0)) - 1ull);
  const unsigned h = static_cast<unsigned>((vm & ~excl) >> (32 * st));
  const int gs = 4 * (lane >> 5);
  unsigned k = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) k |= ((h >> (8 * j + gs)) & 0xFu) << (4 * j);
  return k;
}

// ---------------------------------------------------------------------------
// K1: partial log-sum-exp per (query, key split).
// grid (ceil(n/128), nsplit, B), block 256.  ml[b][split][q] = (m, l) with
// sum_{j in split} exp(s_qj) = l * exp(m).
// ---------------------------------------------------------------------------
template <class In, int D, bool MASK>
__global__ __launch_bounds__(256) void k_score_lse(const In* __restrict__ Q,
                                                   const In* __restrict__ K,
                                                   const uint8_t* __restrict__ mask,
                                                   double2* __restrict__ ml, int n, int T,
                                                   int keys_per_split, int nqb, int nsplit, int B,
                                                   int qg) {
  // bf16 K tiles go global -> LDS directly into swizzled unpadded rows (as
  // in K2); fp32 tiles are staged through registers into padded rows
  constexpr bool DMA = sizeof(In) == 2;
  constexpr int KS = Frag<In>::KS, NK = D / KS, BN = 64, LD = DMA ? D : D + 16 / sizeof(In);
  constexpr int VEC = 16 / sizeof(In), CPR = D / VEC, NCH = BN * CPR / 256;
  __shared__ __align__(16) In sK[2][BN * LD];
  __shared__ uint64_t sMb[2];  // excluded keys of the tile, one bit per key
  int qb, split, b;
  if (!score_grid(nqb, nsplit, B, qb, split, b)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
  const int q = qb * kBM + wave * 32 + (lane & 31);
  const In* Qb = Q + static_cast<size_t>(b / qg) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;
  const uint8_t* Mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;

  typename Frag<In>::T bq[NK];
  load_q_frags<In, D>(bq, Qb, q, n, g);

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  const int ntile = (j1 - j0 + BN - 1) / BN;
  // next tile's K rows in flight while the current tile is computed; rows
  // past the split end read row j1-1 (one batch of loads) and their scores
  // are masked
  uint4 pk[DMA ? 1 : NCH];
  uint64_t pm = 0;
  auto fetch = [&](int jt, int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * 256, r = idx / CPR;
      const bool ok = jt + r < j1;
      if constexpr (DMA) {
        const int lc = (idx % CPR) ^ k_swz<CPR>(r);
        lds_copy16(Kb + static_cast<size_t>(ok ? jt + r : j1 - 1) * D + lc * VEC,
                   &sK[buf][(c * 256 + (threadIdx.x & ~63)) * VEC]);
      } else {
        const int col = (idx % CPR) * VEC;
        const uint4 kv = *reinterpret_cast<const uint4*>(
            Kb + static_cast<size_t>(ok ? jt + r : j1 - 1) * D + col);
        pk[c] = ok ? kv : make_uint4(0, 0, 0, 0);
      }
    }
    if (MASK && wave == 0) pm = __ballot(Mb[min(jt + lane, j1 - 1)] != 0);
  };
  auto stash = [&](int buf) {
    if constexpr (!DMA) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int idx = threadIdx.x + c * 256, r = idx / CPR, col = (idx % CPR) * VEC;
        *reinterpret_cast<uint4*>(&sK[buf][r * LD + col]) = pk[c];
      }
    }
    if (MASK && threadIdx.x == 0) sMb[buf] = pm;
  };
  // running max m (a score, exact in fp32) and sum l = sum exp(s - m) in fp64:
  // each 16-term tile sum is formed in fp32, then accumulated in double, and
  // the rare rescale on a new maximum uses a double exp.  The exponent is
  // s*log2e - m2 with m*log2e = m2 + m2lo (m2 the fp32 rounding); the factor
  // 2^-m2lo is applied once per sum, in double (cm).
  float m = -INFINITY, m2 = 0.f;
  double l = 0.0, cm = 1.0;
  if (ntile > 0) {
    fetch(j0, 0);
    stash(0);
  }
  if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1, jt = j0 + it * BN;
    if (it + 1 < ntile) fetch(jt + BN, cur ^ 1);
    auto scores = [&](int st, f32x16& acc) {
      acc = f32x16{};
      const int row = st * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        int col = ks * KS + g * (KS / 2);
        if constexpr (DMA) col = (col / VEC ^ k_swz<CPR>(row)) * VEC;
        acc = Frag<In>::mma(Frag<In>::load(&sK[cur][row * LD + col]), bq[ks], acc);
      }
    };
    // bf16: both halves' scores are issued first, so the second half's
    // MFMAs run under the first half's exponentials
    f32x16 accS[DMA ? 2 : 1];
    if constexpr (DMA) {
      scores(0, accS[0]);
      scores(1, accS[1]);
    }
#pragma unroll
    for (int st = 0; st < BN / 32; ++st) {
      f32x16& acc = accS[DMA ? st : 0];
      if constexpr (!DMA) scores(st, acc);
      float tmax = -INFINITY;
      const uint64_t mb = MASK ? sMb[cur] : 0;
      if (mb == 0 && jt + BN <= j1) {  // a whole tile, nothing excluded
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
      } else if constexpr (MASK) {
        const unsigned live = live_rows(st, j1 - jt, mb, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = ((live >> r) & 1u) ? acc[r] : -INFINITY;
          acc[r] = s;
          tmax = fmaxf(tmax, s);
        }
      } else {  // the split's last, partial tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = jt + st * 32 + mfma32_row(r, lane) < j1 ? acc[r] : -INFINITY;
          acc[r] = s;
          tmax = fmaxf(tmax, s);
        }
      }
      if (tmax > m) {
        if (m != -INFINITY) l *= exp(static_cast<double>(m) - static_cast<double>(tmax));
        m = tmax;
        m2 = m * KVC_LOG2E;
        const float m2lo = fmaf(m, KVC_LOG2E, -m2);  // m*log2e = m2 + m2lo exactly
        cm = exp2(-static_cast<double>(m2lo));
      }
      if (m != -INFINITY) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -m2));
        l = fma(static_cast<double>(sum), cm, l);
      }
    }
    if (it + 1 < ntile) stash(cur ^ 1);
    if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  // lanes l and l+32 hold the same query over different keys: merge them
  const float mo = __shfl_xor(m, 32);
  const double lo = __shfl_xor(l, 32);
  if (g == 0 && q < n) {
    const float mm = fmaxf(m, mo);
    double ll = 0.0;
    if (mm != -INFINITY) {
      if (m != -INFINITY) ll += l * exp(static_cast<double>(m) - mm);
      if (mo != -INFINITY) ll += lo * exp(static_cast<double>(mo) - mm);
    }
    ml[(static_cast<size_t>(b) * nsplit + split) * n + q] = make_double2(mm, ll);
  }
}

// ---------------------------------------------------------------------------
// K1 for bfloat16 input: the same partial (m, l) per (query, key split).
//   * A wave owns 64 reference queries (two MFMA B-operand sets in
//     registers), so every K fragment read from LDS feeds two MFMAs: one
//     1 KB read per 64 MFMA cycles.
//   * K tiles of 128 keys go global -> LDS by DMA, double-buffered one tile
//     ahead; each thread's chunk offsets inside a tile are fixed, so a fetch
//     is a scalar base plus precomputed 32-bit offsets.
//   * Each query's running sum is kept against an integer reference k in
//     the log2 domain: l = sum 2^(s log2e - k), with k = ceil(max s log2e)
//     so every exponent is <= 0 (as accurate as against the exact maximum).
//     A new maximum that moves k rescales l by an exact power of two
//     (ldexp), so the fold of 16 scores into (k, l) has no branch and no exp
//     or exp2 of its own.
//   * Software pipeline over halves of 32 keys: the MFMAs
//     of half h are issued interleaved with the fold of half h-1 (whose
//     scores are complete), and the LDS reads of half h+2 follow the MFMAs
//     that free their registers, so one wave keeps the matrix pipe and the
//     VALU busy at once.  A tile with an excluded key or past the split end
//     takes a plain path: pending fold, then its halves one by one with the
//     exclusions applied.
// grid: score_grid over 256-query blocks, block 256.
// ---------------------------------------------------------------------------
constexpr int kBM1 = 256;  // reference queries per K1 workgroup (64 per wave)

// The terms are exp2(fp32(s L - k)) with L = fp32(log2 e); the true ones
// carry an extra factor 2^(s (log2 e - L)).  Taking that factor at the
// reference score k ln2 for every term leaves a residual of relative size
// |s - k ln2| * 1.3e-8 per term (negligible for the terms near the maximum
// that carry the sum), and folds the rest into the stored reference:
// m = k ln2 (1 + (log2 e - L) ln2).
constexpr double kLn2Scaled =
    0.6931471805599453 * (1.0 + (1.4426950408889634 - static_cast<double>(KVC_LOG2E)) *
                                    0.6931471805599453);

// running state of one query's partial log-sum-exp over its keys so far:
// sum exp(s) = l 2^k, k an integer (float-valued; -inf before the first
// live key), l in fp64 from fp32 sums of 16 terms.
struct LseState {
  float k = -INFINITY;
  double l = 0.0;
};

// fold 16 scores of one query (one MFMA half tile; -inf for excluded keys)
// into its state, without branches: k' = max(k, ceil(max s log2e)),
// l' = l 2^(k - k') + sum 2^(s log2e - k').  A state with k = -inf has
// l = 0 and rescales to 0; k' = -inf means every score is -inf, whose terms
// vanish against the stand-in reference 0.
__device__ __forceinline__ void lse_fold(LseState& s, const f32x16& acc) {
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
  const float kn = fmaxf(s.k, ceilf(tmax * KVC_LOG2E));
  const float d = fmaxf(s.k - kn, -1024.f);  // (-inf) - (-inf) is NaN: max gives -1024
  const float kref = kn == -INFINITY ? 0.f : kn;
  float sum = __builtin_amdgcn_exp2f(fmaf(acc[0], KVC_LOG2E, -kref));
#pragma unroll
  for (int r = 1; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -kref));
  s.l = ldexp(s.l, static_cast<int>(d)) + static_cast<double>(sum);
  s.k = kn;
}

// scores whose bit in `live` is clear become -inf
__device__ __forceinline__ void mask_scores(f32x16& acc, unsigned live) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = ((live >> r) & 1u) ? acc[r] : -INFINITY;
}

template <int D, bool MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_score_lse_bf16(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const uint8_t* __restrict__ mask,
    double2* __restrict__ ml, int n, int T, int keys_per_split, int nqb, int nsplit, int B,
    int qg) {
  constexpr int NK = D / 16, BN = 128, NH = BN / 32, VEC = 8, CPR = D / VEC;
  constexpr int NCH = BN * CPR / 256;
  constexpr int TILE = BN * D;  // bf16 elements per LDS buffer
  __shared__ __align__(16) bf16_t sK[2 * TILE];
  __shared__ uint64_t sMb[2][2];  // excluded keys of the tile, one bit per key
  int qb, split, b;
  if (!score_grid(nqb, nsplit, B, qb, split, b)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 5;
  const int q0 = qb * kBM1 + wave * 64 + (lane & 31), q1 = q0 + 32;
  const bf16_t* Qb = Q + static_cast<size_t>(b / qg) * n * D;
  const bf16_t* Kb = K + static_cast<size_t>(b) * T * D;
  const uint8_t* Mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;

  bf16x8 bq0[NK], bq1[NK];
  load_q_frags<bf16_t, D>(bq0, Qb, q0, n, g);
  load_q_frags<bf16_t, D>(bq1, Qb, q1, n, g);

  // this thread's chunks of a tile: chunk c is slot threadIdx.x + 256 c of
  // the tile, i.e. row r0 + c (256 / CPR) (r0 = threadIdx.x / CPR), holding
  // source chunk (threadIdx.x % CPR) ^ swz(r0): the swizzle is the same for
  // every c, so chunk c sits 256 * 16 bytes after chunk 0
  static_assert(k_swz<CPR>(0) == 0 && 256 % CPR == 0, "chunk rows");
  const int r0 = threadIdx.x / CPR;
  const uint32_t goff = static_cast<uint32_t>(
      (r0 * D + ((threadIdx.x % CPR) ^ k_swz<CPR>(r0)) * VEC) * 2);
  // LDS element offset of this lane's MFMA A-operand chunk ks in half 0 of
  // buffer 0 (row lane%32; half h adds 32 h rows, buffer 1 adds TILE)
  uint32_t roff[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int row = lane & 31;
    roff[ks] = static_cast<uint32_t>(row * D + ((2 * ks + g) ^ k_swz<CPR>(row)) * VEC);
  }

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  const int ntile = (j1 - j0 + BN - 1) / BN;
  // tile at key jt with `valid` keys before the split end into buffer buf;
  // rows at or past `valid` copy row valid-1 (their scores are masked).
  // The mask bytes are loaded before the copies and turned into the tile's
  // bit sets at the end of the current tile.
  uint8_t mbyte[2] = {0, 0};
  auto fetch = [&](int jt, int valid, int buf) {
    if (MASK && wave == 0) {
      mbyte[0] = Mb[min(jt + lane, j1 - 1)];
      mbyte[1] = Mb[min(jt + 64 + lane, j1 - 1)];
    }
    const char* base = reinterpret_cast<const char*>(Kb + static_cast<size_t>(jt) * D);
    if (valid >= BN) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        lds_copy16(base + goff + c * 4096, &sK[buf * TILE + (c * 256 + wave * 64) * VEC]);
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int r = r0 + c * (256 / CPR);
        const uint32_t o = goff + c * 4096 - static_cast<uint32_t>((r - min(r, valid - 1)) * D * 2);
        lds_copy16(base + o, &sK[buf * TILE + (c * 256 + wave * 64) * VEC]);
      }
    }
  };
  auto publish_mask = [&](int buf) {
    if (MASK && wave == 0) {
      const uint64_t m0 = __ballot(mbyte[0] != 0), m1 = __ballot(mbyte[1] != 0);
      if (lane == 0) {
        sMb[buf][0] = m0;
        sMb[buf][1] = m1;
      }
    }
  };
  LseState s0, s1;
  // K fragments of the next half (read while the current half's MFMAs
  // release them), scores of the half whose fold is pending (-inf: none)
  bf16x8 F[NK];
  f32x16 A0[2], A1[2];
  A0[1] = f32x16{} - INFINITY;
  A1[1] = A0[1];
  auto read_half = [&](int buf, int h, bf16x8* f) {
    const bf16_t* sb = sK + buf * TILE + h * 32 * D;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) f[ks] = *reinterpret_cast<const bf16x8*>(sb + roff[ks]);
  };
  // MFMAs of one half from f into (a0, a1), interleaved with the fold of
  // (p0, p1); then, if `next` >= 0, the reads of half `next` into f
  auto step = [&](bf16x8* f, f32x16& a0, f32x16& a1, const f32x16& p0, const f32x16& p1,
                  int buf, int next) {
    a0 = f32x16{};
    a1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks], bq0[ks], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks], bq1[ks], a1, 0, 0, 0);
    }
    lse_fold(s0, p0);
    lse_fold(s1, p1);
    if (next >= 0) read_half(buf, next, f);
    // per fragment: its two MFMAs with fold arithmetic between them, then
    // the LDS read that reuses its registers for half `next`
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
  };
  auto tile = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int jt = j0 + it * BN, valid = j1 - jt;
    if (it + 1 < ntile) fetch(jt + BN, valid - BN, cur ^ 1);
    const uint64_t mb0 = MASK ? sMb[cur][0] : 0, mb1 = MASK ? sMb[cur][1] : 0;
    if ((mb0 | mb1) == 0 && valid >= BN) {
      // halves 0..3: half 0's frags are in flight on entry
      step(F, A0[0], A1[0], A0[1], A1[1], cur, 1);
      step(F, A0[1], A1[1], A0[0], A1[0], cur, 2);
      step(F, A0[0], A1[0], A0[1], A1[1], cur, 3);
      step(F, A0[1], A1[1], A0[0], A1[0], cur, -1);
    } else {
      // the pending fold, then halves one at a time with the exclusions
      // applied; the last half's masked scores become the pending fold
      lse_fold(s0, A0[1]);
      lse_fold(s1, A1[1]);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 f[NK];
        read_half(cur, h, f);
        f32x16 a0{}, a1{};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks], bq0[ks], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks], bq1[ks], a1, 0, 0, 0);
        }
        const unsigned live = live_rows(h & 1, valid - 64 * (h >> 1), h < 2 ? mb0 : mb1, lane);
        mask_scores(a0, live);
        mask_scores(a1, live);
        if (h + 1 < NH) {
          lse_fold(s0, a0);
          lse_fold(s1, a1);
        } else {
          A0[1] = a0;
          A1[1] = a1;
        }
      }
    }
    // the next tile's copies and mask bits, then its first half's frags
    if (it + 1 < ntile) publish_mask(cur ^ 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < ntile) read_half(cur ^ 1, 0, F);
  };
  if (ntile > 0) {
    fetch(j0, j1 - j0, 0);
    publish_mask(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (ntile > 0) read_half(0, 0, F);
  for (int it = 0; it < ntile; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntile) tile(std::integral_constant<int, 1>{}, it + 1);
  }
  lse_fold(s0, A0[1]);
  lse_fold(s1, A1[1]);
  // lanes l and l+32 hold the same query over different keys: merge them
  // (exactly, by powers of two) and store m = k ln2 with l
  auto finish = [&](const LseState& s, int q) {
    const float ko = __shfl_xor(s.k, 32);
    const double lo = __shfl_xor(s.l, 32);
    if (g == 0 && q < n) {
      const float kk = fmaxf(s.k, ko);
      double ll = 0.0, mm = -INFINITY;
      if (kk != -INFINITY) {
        if (s.k != -INFINITY) ll += ldexp(s.l, static_cast<int>(s.k - kk));
        if (ko != -INFINITY) ll += ldexp(lo, static_cast<int>(ko - kk));
        mm = static_cast<double>(kk) * kLn2Scaled;
      }
      ml[(static_cast<size_t>(b) * nsplit + split) * n + q] = make_double2(mm, ll);
    }
  };
  finish(s0, q0);
  finish(s1, q1);
}

// lse[b][q] (float64) from the split partials, merged in split order.
// Four lanes per query, each taking every fourth split: the maximum over
// all splits, then each lane's sum in split order, then the four sums added
// in lane order.  grid (ceil(4 B n / 256)), block 256.
// It also clears every head's first selection histogram (sel, stride
// sstride words), which the importance reduction fills.
__global__ void k_lse_merge(const double2* __restrict__ ml, double* __restrict__ lse, int n,
                            int nsplit, int B, unsigned* __restrict__ sel, size_t sstride) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x, i = g >> 2, part = g & 3;
  for (size_t e = g; e < static_cast<size_t>(B) * kSelH1;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    sel[(e / kSelH1) * sstride + e % kSelH1] = 0;
  const bool ok = i < B * n;
  const int b = ok ? i / n : 0, q = ok ? i % n : 0;
  const double2* p = ml + static_cast<size_t>(b) * nsplit * n + q;
  double m = -INFINITY;
  if (ok)
    for (int s = part; s < nsplit; s += 4) m = fmax(m, p[static_cast<size_t>(s) * n].x);
  m = fmax(m, __shfl_xor(m, 1));
  m = fmax(m, __shfl_xor(m, 2));
  double l = 0.0;
  if (ok)
    for (int s = part; s < nsplit; s += 4) {
      const double2 v = p[static_cast<size_t>(s) * n];
      if (v.x != -INFINITY) l += v.y * exp(v.x - m);
    }
  const double l1 = __shfl_down(l, 1), l2 = __shfl_down(l, 2), l3 = __shfl_down(l, 3);
  if (ok && part == 0) lse[i] = m + log(((l + l1) + l2) + l3);
}

// Position of key kk (0..31 inside a tile) in the transposed V tile: the
// k-slots of lane group g for MFMA half h are the accumulator rows
// 8*(e/4) + 4*g + e%4 + 16*h, e = 0..7; store those 8 keys contiguously.
__device__ __forceinline__ int vt_pos(int kk) {
  const int h = kk >> 4, o = kk & 15;
  const int gg = (o >> 2) & 1, e = ((o >> 3) << 2) | (o & 3);
  return h * 16 + gg * 8 + e;
}

// ---------------------------------------------------------------------------
// K2: p = exp(s - lse); importance partials and partial O.
// grid (ceil(n/128), nsplit, B), block 256.
//   Opart[b][split][dd][q]  partial (P V)^T over the split's keys
//   imp_part[b][qb][j]      sum over the 128 queries of block qb of p^2 (or p)
// Keys go in tiles of 64: the next tile's K and V rows are fetched into
// registers while the current one is computed, then written to the other
// half of a double-buffered LDS tile, so each tile needs one barrier.  Each
// wave reduces its 32 queries' p^2 per key with a butterfly that halves the
// kept key slots at every exchange (16 shuffles for 16 keys); the four waves'
// partials are added after the tile's barrier.
// ---------------------------------------------------------------------------

// Sum of v[0..15] (accumulator rows) over the 32 lanes of this lane's half
// wave; the result for row 8*b4 + 4*b3 + 2*b2 + b1 (b_i = bit i of the lane)
// ends up in both lanes of the pair differing in bit 0.  Each level halves the
// values a lane keeps and adds its partner's copy of the same rows, with
// VALU cross-lane moves only: v_permlane16_swap pairs lane l with l ^ 16 (it
// exchanges odd 16-lane rows of one register with even rows of another, so
// swapping v[i] and v[8+i] leaves each lane its kept half plus the partner's
// matching half), DPP row_ror:8 pairs l with l ^ 8 within a row,
// row_half_mirror pairs l with 7 - l within 8 lanes (the partner has the
// other bit 2), and quad permutations pair bits 1 and 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <bool SQ, class Vec>
__device__ __forceinline__ float half_wave_rowsum(const Vec& v, int lane) {
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float w[8], x[4], y[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // the swap moves the values themselves; squaring after it takes one
    // multiply and one FMA per pair instead of two multiplies and an add
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[8 + i]), false, false);
    const float r0 = __uint_as_float(r[0]), r1 = __uint_as_float(r[1]);
    w[i] = SQ ? fmaf(r0, r0, r1 * r1) : r0 + r1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = b3 ? w[4 + i] : w[i], send = b3 ? w[i] : w[4 + i];
    x[i] = keep + dpp_f32<0x128>(send);  // row_ror:8
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = b2 ? x[2 + i] : x[i], send = b2 ? x[i] : x[2 + i];
    y[i] = keep + dpp_f32<0x141>(send);  // row_half_mirror
  }
  const float z = (b1 ? y[1] : y[0]) + dpp_f32<0x4E>(b1 ? y[0] : y[1]);  // quad_perm 2,3,0,1
  return z + dpp_f32<0xB1>(z);                                           // quad_perm 1,0,3,2
}

template <class In, int D, bool RMS, bool MASK>
__global__ __launch_bounds__(256) void k_expweight(const In* __restrict__ Q,
                                                   const In* __restrict__ K,
                                                   const In* __restrict__ V,
                                                   const double* __restrict__ lse,
                                                   const uint8_t* __restrict__ mask,
                                                   float* __restrict__ Opart,
                                                   float* __restrict__ imp_part, int n, int T,
                                                   int keys_per_split, int nqb, int nsplit,
                                                   int B, int qg) {
  constexpr int KS = Frag<In>::KS, NK = D / KS, BN = 64;
  // bf16 K tiles go global -> LDS directly (no registers), unpadded, with
  // the 16-byte chunks of a row XOR-swizzled; fp32 tiles are staged through
  // registers into padded rows
  constexpr bool DMA = sizeof(In) == 2;
  constexpr bool EARLY = DMA;
  constexpr int LD = DMA ? D : D + 16 / sizeof(In);
  constexpr int LDV = BN + 16 / sizeof(In);
  constexpr int ND = D / 32;
  constexpr int VEC = 16 / sizeof(In), CPR = D / VEC;  // 16-byte chunks per row
  constexpr int NCH = BN * CPR / 256;                   // chunks per thread per tile
  static_assert(BN == 64 && NCH * 4 == CPR, "V fetch: a wave per column chunk of 64 keys");
  __shared__ __align__(16) In sK[2][BN * LD];
  __shared__ __align__(16) In sVt[2][D * LDV];
  __shared__ float sImp[2][kWaves][BN];
  __shared__ uint64_t sMb[2];  // excluded keys of the tile, one bit per key

  int qb, split, b;
  if (!score_grid(nqb, nsplit, B, qb, split, b)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
  const int q = qb * kBM + wave * 32 + (lane & 31);
  const In* Qb = Q + static_cast<size_t>(b / qg) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;
  const In* Vb = V + static_cast<size_t>(b) * T * D;
  const uint8_t* Mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;

  typename Frag<In>::T bq[NK];
  load_q_frags<In, D>(bq, Qb, q, n, g);
  // lse*log2e as an unevaluated fp32 pair, so exp2(s*log2e - hi - lo) keeps
  // the float64 log-sum-exp's accuracy
  // (a query past n gets an infinite lse: its zero scores give p = 0 with no
  // per-element test)
  const double l2 = q < n ? lse[static_cast<size_t>(b) * n + q] * 1.4426950408889634 : 0.0;
  const float ml2 = q < n ? static_cast<float>(l2) : INFINITY;
  const float ml2lo = q < n ? static_cast<float>(l2 - static_cast<double>(ml2)) : 0.f;

  f32x16 accO[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) accO[dt] = f32x16{};

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  const int ntile = (j1 - j0 + BN - 1) / BN;
  uint4 pk[DMA ? 1 : NCH], pv[NCH];
  uint64_t pm = 0;
  // rows past the split end read row j1-1 (always valid) and are zeroed, so
  // the fetch is one unconditional batch of loads
  // K rows go to LDS as they are (consecutive lanes: consecutive 16-byte
  // chunks of a row).  V is transposed on the way in, so a wave takes one
  // 16-byte column chunk of 64 consecutive keys: each of its transposed
  // writes then covers one contiguous 128-byte run of a V^T row, free of
  // bank conflicts.
  auto fetch = [&](int jt, int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * 256, r = idx / CPR;
      const bool ok = jt + r < j1;
      if constexpr (DMA) {
        // one wave's 64 lanes fill 1 KB of the tile (slots idx of the wave,
        // 16 bytes each); slot (r, p) holds chunk p ^ swz(r) of key row r.
        // Rows past the split end copy row j1-1: their p is masked to zero.
        const int lc = (idx % CPR) ^ k_swz<CPR>(r);
        lds_copy16(Kb + static_cast<size_t>(ok ? jt + r : j1 - 1) * D + lc * VEC,
                   &sK[buf][(c * 256 + (threadIdx.x & ~63)) * VEC]);
      } else {
        const int col = (idx % CPR) * VEC;
        const uint4 kv = *reinterpret_cast<const uint4*>(
            Kb + static_cast<size_t>(ok ? jt + r : j1 - 1) * D + col);
        pk[c] = ok ? kv : make_uint4(0, 0, 0, 0);
      }
      const int rv = threadIdx.x & (BN - 1), colv = ((threadIdx.x >> 6) + 4 * c) * VEC;
      const bool okv = jt + rv < j1;
      const uint4 vv = *reinterpret_cast<const uint4*>(
          Vb + static_cast<size_t>(okv ? jt + rv : j1 - 1) * D + colv);
      pv[c] = okv ? vv : make_uint4(0, 0, 0, 0);
    }
    if (MASK && wave == 0) pm = __ballot(Mb[min(jt + lane, j1 - 1)] != 0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (!DMA) {
        const int idx = threadIdx.x + c * 256, r = idx / CPR, col = (idx % CPR) * VEC;
        *reinterpret_cast<uint4*>(&sK[buf][r * LD + col]) = pk[c];
      }
      const int rv = threadIdx.x & (BN - 1), colv = ((threadIdx.x >> 6) + 4 * c) * VEC;
      In v[VEC];
      *reinterpret_cast<uint4*>(v) = pv[c];
      // V^T [dd][key slot]; bf16 slots follow the accumulator rows
      const int pos = sizeof(In) == 2 ? (rv >> 5) * 32 + vt_pos(rv & 31) : rv;
#pragma unroll
      for (int e = 0; e < VEC; ++e) sVt[buf][(colv + e) * LDV + pos] = v[e];
    }
    if (MASK && threadIdx.x == 0) sMb[buf] = pm;
  };
  if (ntile > 0) {
    fetch(j0, 0);
    stash(0);
  }
  if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int cur = it & 1, jt = j0 + it * BN, valid = j1 - jt;
    if (it + 1 < ntile) fetch(jt + BN, cur ^ 1);
    auto scores = [&](int st, f32x16& acc) {
      acc = f32x16{};
      const int row = st * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        int col = ks * KS + g * (KS / 2);
        if constexpr (DMA) col = (col / VEC ^ k_swz<CPR>(row)) * VEC;
        acc = Frag<In>::mma(Frag<In>::load(&sK[cur][row * LD + col]), bq[ks], acc);
      }
    };
    // bf16: both 32-key halves' scores are issued first, so the second
    // half's MFMAs run while the first half's exponentials are computed
    f32x16 accS[EARLY ? 2 : 1];
    if constexpr (EARLY) {
      scores(0, accS[0]);
      scores(1, accS[1]);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16& acc = accS[EARLY ? st : 0];
      if constexpr (!EARLY) scores(st, acc);
      const uint64_t mb = MASK ? sMb[cur] : 0;
      if (mb == 0 && valid >= BN) {  // a whole tile, nothing excluded: no test
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2) - ml2lo);
        }
      } else if constexpr (MASK) {
        const unsigned live = live_rows(st, valid, mb, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2) - ml2lo);
          acc[r] = ((live >> r) & 1u) ? e : 0.f;
        }
      } else {  // the split's last, partial tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2) - ml2lo);
          acc[r] = st * 32 + mfma32_row(r, lane) < valid ? e : 0.f;
        }
      }
      {
        const float tot = half_wave_rowsum<RMS>(acc, lane);
        const int r = ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 +
                      ((lane >> 1) & 1);
        if ((lane & 1) == 0) sImp[cur][wave][st * 32 + mfma32_row(r, lane)] = tot;
      }
      if constexpr (sizeof(In) == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = acc[h * 8 + e];
            const __bf16 ph = static_cast<__bf16>(p);
            hi[e] = ph;
            lo[e] = static_cast<__bf16>(p - static_cast<float>(ph));
          }
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                &sVt[cur][(dt * 32 + (lane & 31)) * LDV + st * 32 + h * 16 + g * 8]);
            accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, accO[dt], 0, 0, 0);
            accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, accO[dt], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = st * 32 + mfma32_row(r, lane);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const float a = static_cast<float>(sVt[cur][(dt * 32 + (lane & 31)) * LDV + kk]);
            accO[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, acc[r], accO[dt], 0, 0, 0);
          }
        }
      }
    }
    if (it + 1 < ntile) stash(cur ^ 1);
    // the next tile's K copies must have landed before the barrier
    if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x < BN && static_cast<int>(threadIdx.x) < valid) {
      const int t = threadIdx.x;
      imp_part[(static_cast<size_t>(b) * nqb + qb) * T + jt + t] =
          ((sImp[cur][0][t] + sImp[cur][1][t]) + sImp[cur][2][t]) + sImp[cur][3][t];
    }
  }
  if (q < n) {
    float* Ob = Opart + (static_cast<size_t>(b) * nsplit + split) * D * n;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Ob[static_cast<size_t>(dt * 32 + mfma32_row(r, lane)) * n + q] = accO[dt][r];
  }
}

// ---------------------------------------------------------------------------
// K2 for bfloat16 input: p = exp(s - lse); importance partials and partial O.
// grid (score_grid over 128-query blocks), block 256; outputs as k_expweight.
//   * K and V tiles both go global -> LDS by DMA, in the same XOR-swizzled
//     row layout, double-buffered, one tile ahead.
//   * The A operand of O^T += V^T P^T (32 value columns x 16 keys) is read
//     straight from the key-major V tile with LDS transpose reads
//     (ds_read_b64_tr_b16): in each 16-lane group, output lane i, element e
//     comes from the 8-byte read of lane 4e + i/4 at position i % 4, so a lane
//     whose group reads 4 consecutive key rows gets 4 consecutive keys of one
//     value column.  Two such reads give the 8 keys of a lane's k-slots, in
//     the order the score accumulator holds them (keys 4g..4g+3 and
//     8+4g..8+4g+3 of each 16-key step, g = lane / 32), so P needs no
//     permutation and V no transposed copy.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// p = hi + lo for eight values: hi = bf16(p), lo = bf16(p - hi), both rounded
// to nearest even, two values per conversion; hi's float value is its bf16
// bits shifted (low half) or masked (high half) into place.
__device__ __forceinline__ void split_hi_lo(const f32x16& p, int base, bf16x8& hi, bf16x8& lo) {
  bf16x2 h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = p[base + 2 * i], p1 = p[base + 2 * i + 1];
    h[i] = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
    const uint32_t u = __builtin_bit_cast(uint32_t, h[i]);
    const float h0 = __uint_as_float(u << 16), h1 = __uint_as_float(u & 0xffff0000u);
    l[i] = __builtin_convertvector((f32x2{p0 - h0, p1 - h1}), bf16x2);
  }
  const bf16x4 h01 = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3);
  const bf16x4 h23 = __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3);
  const bf16x4 l01 = __builtin_shufflevector(l[0], l[1], 0, 1, 2, 3);
  const bf16x4 l23 = __builtin_shufflevector(l[2], l[3], 0, 1, 2, 3);
  hi = __builtin_shufflevector(h01, h23, 0, 1, 2, 3, 4, 5, 6, 7);
  lo = __builtin_shufflevector(l01, l23, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

template <int D, bool RMS, bool MASK>
__global__ __launch_bounds__(256) void k_expweight_bf16(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const double* __restrict__ lse, const uint8_t* __restrict__ mask, float* __restrict__ Opart,
    float* __restrict__ imp_part, int n, int T, int keys_per_split, int nqb, int nsplit, int B,
    int qg) {
  constexpr int NK = D / 16, BN = 64, VEC = 8, CPR = D / VEC, NCH = BN * CPR / 256, ND = D / 32;
  constexpr int TILE = BN * D;  // bf16 elements per LDS buffer
  __shared__ __align__(16) bf16_t sK[2 * TILE];
  __shared__ __align__(16) bf16_t sV[2 * TILE];
  __shared__ float sImp[2][kWaves][BN];
  __shared__ uint64_t sMb[2];  // excluded keys of the tile, one bit per key

  int qb, split, b;
  if (!score_grid(nqb, nsplit, B, qb, split, b)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 5;
  const int q = qb * kBM + wave * 32 + (lane & 31);
  const bf16_t* Qb = Q + static_cast<size_t>(b / qg) * n * D;
  const bf16_t* Kb = K + static_cast<size_t>(b) * T * D;
  const bf16_t* Vb = V + static_cast<size_t>(b) * T * D;
  const uint8_t* Mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;

  bf16x8 bq[NK];
  load_q_frags<bf16_t, D>(bq, Qb, q, n, g);
  // lse*log2e as an unevaluated fp32 pair, so exp2(s*log2e - hi - lo) keeps
  // the float64 log-sum-exp's accuracy (a query past n gets an infinite lse:
  // its zero scores give p = 0 with no per-element test)
  const double l2 = q < n ? lse[static_cast<size_t>(b) * n + q] * 1.4426950408889634 : 0.0;
  const float ml2 = q < n ? static_cast<float>(l2) : INFINITY;
  const float ml2lo = q < n ? static_cast<float>(l2 - static_cast<double>(ml2)) : 0.f;
  // The low part enters as the score accumulators' initial value (divided by
  // log2e), so each p costs one FMA and one exp2: the accumulator holds
  // s - ml2lo/log2e, rounded once like s alone.
  const float c0 = -ml2lo * (1.0f / KVC_LOG2E);
  f32x16 cinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = c0;

  // this thread's chunks of a tile (K and V alike): chunk c is slot
  // threadIdx.x + 256 c, i.e. row r = slot / CPR holding source chunk
  // (slot % CPR) ^ swz(r)
  uint32_t goff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = threadIdx.x + c * 256, r = idx / CPR, lc = (idx % CPR) ^ k_swz<CPR>(r);
    goff[c] = static_cast<uint32_t>((r * D + lc * VEC) * 2);
  }
  // K A-operand chunk ks of half 0 (row lane%32; half 1 adds 32 rows)
  uint32_t roff[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int row = lane & 31;
    roff[ks] = static_cast<uint32_t>(row * D + ((2 * ks + g) ^ k_swz<CPR>(row)) * VEC);
  }
  // V transpose reads for value tile dt, part r2 (keys +0 / +8) of 16-key
  // step 0 (step kk adds 16 rows): this lane reads key row
  // 4 (G/2) + 8 r2 + j/4 at value column 32 dt + 16 (G%2) + 4 (j%4), where
  // G = lane / 16 and j = lane % 16
  uint32_t voff[ND][2];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      const int G = lane >> 4, j = lane & 15;
      const int row = 4 * (G >> 1) + 8 * r2 + (j >> 2);
      const int col = 32 * dt + 16 * (G & 1) + 4 * (j & 3);
      const int pos = (col / VEC) ^ k_swz<CPR>(row);
      voff[dt][r2] = static_cast<uint32_t>(row * D + pos * VEC + col % VEC);
    }

  f32x16 accO[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) accO[dt] = f32x16{};

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  const int ntile = (j1 - j0 + BN - 1) / BN;
  // tile at key jt with `valid` keys before the split end into buffer buf;
  // rows at or past `valid` copy row valid-1 (their p is masked to zero)
  auto fetch = [&](int jt, int valid, int buf, uint8_t& mbyte) {
    if (MASK && wave == 0) mbyte = Mb[min(jt + lane, j1 - 1)];
    const char* kb = reinterpret_cast<const char*>(Kb + static_cast<size_t>(jt) * D);
    const char* vb = reinterpret_cast<const char*>(Vb + static_cast<size_t>(jt) * D);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t o = goff[c];
      if (valid < BN) {
        const int r = (threadIdx.x + c * 256) / CPR;
        o -= static_cast<uint32_t>((r - min(r, valid - 1)) * D * 2);
      }
      const int dst = buf * TILE + (c * 256 + wave * 64) * VEC;
      lds_copy16(kb + o, &sK[dst]);
      lds_copy16(vb + o, &sV[dst]);
    }
  };
  uint8_t mb_next = 0;
  auto tile = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int jt = j0 + it * BN, valid = j1 - jt;
    if (it + 1 < ntile) fetch(jt + BN, valid - BN, cur ^ 1, mb_next);
    const bf16_t* sk = sK + cur * TILE;
    const bf16_t* sv = sV + cur * TILE;
    const uint64_t mb = MASK ? sMb[cur] : 0;
    const bool whole = mb == 0 && valid >= BN;
    // Two halves of 32 keys, software-pipelined inside the tile: the scores
    // of half 1 go to the matrix pipe while half 0's weights are formed, and
    // half 0's P.V products while half 1's weights are formed.
    auto scores = [&](int st, f32x16& acc) {
      bf16x8 ka[NK];
#pragma unroll
      for (int ks = 0; ks < NK; ++ks)
        ka[ks] = *reinterpret_cast<const bf16x8*>(sk + roff[ks] + st * 32 * D);
      acc = cinit;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], bq[ks], acc, 0, 0, 0);
    };
    // p = exp(s - lse) of half st (excluded keys and keys past the split
    // end: 0), its bf16 hi/lo split, then its importance partial (the
    // butterfly overwrites acc)
    auto weights = [&](auto whole_c, int st, f32x16& acc, bf16x8 (&hi)[2], bf16x8 (&lo)[2]) {
      if constexpr (decltype(whole_c)::value) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2));
      } else {
        const unsigned live = live_rows(st, valid, mb, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2));
          acc[r] = ((live >> r) & 1u) ? e : 0.f;
        }
      }
      split_hi_lo(acc, 0, hi[0], lo[0]);
      split_hi_lo(acc, 8, hi[1], lo[1]);
      const float tot = half_wave_rowsum<RMS>(acc, lane);
      const int r = ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 +
                    ((lane >> 1) & 1);
      if ((lane & 1) == 0) sImp[cur][wave][st * 32 + mfma32_row(r, lane)] = tot;
    };
    auto pv = [&](int st, const bf16x8 (&hi)[2], const bf16x8 (&lo)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 2 * st + h;  // 16-key step of the tile
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const bf16x4 v0 = lds_read_tr16(sv + voff[dt][0] + kk * 16 * D);
          const bf16x4 v1 = lds_read_tr16(sv + voff[dt][1] + kk * 16 * D);
          const bf16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi[h], accO[dt], 0, 0, 0);
          accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo[h], accO[dt], 0, 0, 0);
        }
      }
    };
    auto halves = [&](auto whole_c) {
      f32x16 a0, a1;
      bf16x8 h0[2], l0[2], h1[2], l1[2];
      __builtin_amdgcn_sched_barrier(0);
      scores(0, a0);
      __builtin_amdgcn_sched_barrier(0);
      scores(1, a1);
      weights(whole_c, 0, a0, h0, l0);
      // the K reads of half 1, then each of its MFMAs followed by weight work
      __builtin_amdgcn_sched_group_barrier(0x100, NK, 1);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 14, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      pv(0, h0, l0);
      weights(whole_c, 1, a1, h1, l1);
      // half 0's P.V (two value reads, two MFMAs) interleaved with weight work
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
        __builtin_amdgcn_sched_group_barrier(0x002, 14, 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      pv(1, h1, l1);
    };
    if (whole) halves(std::true_type{});
    else halves(std::false_type{});
    // publish the next tile's mask bits; its copies must have landed
    if (MASK && wave == 0 && it + 1 < ntile) {
      const uint64_t pm = __ballot(mb_next != 0);
      if (lane == 0) sMb[cur ^ 1] = pm;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x < BN && static_cast<int>(threadIdx.x) < valid) {
      const int t = threadIdx.x;
      imp_part[(static_cast<size_t>(b) * nqb + qb) * T + jt + t] =
          ((sImp[cur][0][t] + sImp[cur][1][t]) + sImp[cur][2][t]) + sImp[cur][3][t];
    }
  };
  if (ntile > 0) {
    uint8_t mb0 = 0;
    fetch(j0, j1 - j0, 0, mb0);
    if (MASK && wave == 0) {
      const uint64_t pm = __ballot(mb0 != 0);
      if (lane == 0) sMb[0] = pm;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntile; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntile) tile(std::integral_constant<int, 1>{}, it + 1);
  }
  if (q < n) {
    float* Ob = Opart + (static_cast<size_t>(b) * nsplit + split) * D * n;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Ob[static_cast<size_t>(dt * 32 + mfma32_row(r, lane)) * n + q] = accO[dt][r];
  }
}

// O[b][q][dd] = sum over splits (in order) of Opart[b][s][dd][q]; 32x32 tiles
// transposed through LDS.  grid (ceil(n/32), D/32, B), block (32, 8).
__global__ void k_o_reduce(const float* __restrict__ Opart, float* __restrict__ O, int n, int D,
                           int nsplit) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z, q0 = blockIdx.x * 32, d0 = blockIdx.y * 32;
  for (int y = threadIdx.y; y < 32; y += 8) {
    const int dd = d0 + y, q = q0 + threadIdx.x;
    float s = 0.f;
    if (q < n)
      for (int sp = 0; sp < nsplit; ++sp)
        s += Opart[((static_cast<size_t>(b) * nsplit + sp) * D + dd) * n + q];
    tile[y][threadIdx.x] = s;
  }
  __syncthreads();
  for (int y = threadIdx.y; y < 32; y += 8) {
    const int q = q0 + y, dd = d0 + threadIdx.x;
    if (q < n) O[(static_cast<size_t>(b) * n + q) * D + dd] = tile[threadIdx.x][y];
  }
}

// imp[b][j] = sum over query blocks (in order) of imp_part[b][qb][j], and the
// first pass of the top-t selection (select.hip): the histogram of the
// ranking keys' top 11 bits, per workgroup of kImpKeys keys in LDS, added
// into the head's histogram in sel (cleared by k_lse_merge).  The workgroups
// also clear the later passes' histograms.  A non-finite importance sets
// status bit 4.  grid (ceil(T / kImpKeys), B), block 256; key j = workgroup
// start + 256 i + thread (coalesced), four query blocks' loads in flight.
constexpr int kImpKeys = 1024;
__global__ __launch_bounds__(256) void k_imp_reduce(const float* __restrict__ part,
                                                    float* __restrict__ imp,
                                                    unsigned* __restrict__ sel,
                                                    const uint8_t* __restrict__ mask,
                                                    int32_t* __restrict__ status, int T, int nqb,
                                                    size_t sstride) {
  constexpr int PER = kImpKeys / 256;
  __shared__ unsigned hist[kSelH1];
  __shared__ int s_bad;
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const float* p = part + static_cast<size_t>(b) * nqb * T;
  float s[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) s[i] = 0.f;
  int qb = 0;
  for (; qb + 4 <= nqb; qb += 4) {
    float v[4][PER];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = g * kImpKeys + i * 256 + tid;
        v[u][i] = j < T ? p[static_cast<size_t>(qb + u) * T + j] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) s[i] += v[u][i];
  }
  for (; qb < nqb; ++qb)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = g * kImpKeys + i * 256 + tid;
      if (j < T) s[i] += p[static_cast<size_t>(qb) * T + j];
    }
  for (int i = tid; i < kSelH1; i += 256) hist[i] = 0;
  if (tid == 0) s_bad = 0;
  unsigned* st = sel + b * sstride;
  {
    constexpr int later = kSelH2 + kSelH3;
    const int per = (later + gridDim.x - 1) / gridDim.x;
    for (int i = g * per + tid; i < min(later, (g + 1) * per); i += 256) st[kSelH1 + i] = 0;
  }
  __syncthreads();
  const uint8_t* mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = g * kImpKeys + i * 256 + tid;
    if (j < T) {
      imp[static_cast<size_t>(b) * T + j] = s[i];
      bad |= __float_as_uint(s[i]) >= 0x7f800000u;  // inf / nan (non-negative values)
      atomicAdd(&hist[sel_key_of(s[i], mb, j) >> 21], 1u);
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();
  for (int i = tid; i < kSelH1; i += 256)
    if (hist[i]) atomicAdd(&st[i], hist[i]);
  if (tid == 0 && s_bad && status) atomicOr(&status[b], 4);
}

// ---------------------------------------------------------------------------
// Host-side launchers (same library).
// ---------------------------------------------------------------------------
template <class In, int D>
hipError_t launch_score(const void* Q, const void* K, const void* V, double2* ml, double* lse,
                        float* Opart, float* O, float* imp_part, float* imp, uint32_t* sel,
                        int32_t* status, int B, int n, int T, int nsplit1, int kps1, int nsplit2,
                        int kps2, bool rms, int qg, const uint8_t* mask, hipStream_t st) {
  const int nqb = (n + kBM - 1) / kBM;
  const In* q = static_cast<const In*>(Q);
  const In* k = static_cast<const In*>(K);
  const In* v = static_cast<const In*>(V);
  prof_mark(0, false, st);
  const int nqb1 = sizeof(In) == 2 ? (n + kBM1 - 1) / kBM1 : nqb;
  const dim3 g1(score_grid_size(nqb1, nsplit1, B)), g2(score_grid_size(nqb, nsplit2, B));
  if constexpr (sizeof(In) == 2) {
    if (mask)
      hipLaunchKernelGGL((k_score_lse_bf16<D, true>), g1, dim3(256), 0, st, q, k, mask, ml, n, T,
                         kps1, nqb1, nsplit1, B, qg);
    else
      hipLaunchKernelGGL((k_score_lse_bf16<D, false>), g1, dim3(256), 0, st, q, k, mask, ml, n,
                         T, kps1, nqb1, nsplit1, B, qg);
  } else {
    if (mask)
      hipLaunchKernelGGL((k_score_lse<In, D, true>), g1, dim3(256), 0, st, q, k, mask, ml, n, T,
                         kps1, nqb, nsplit1, B, qg);
    else
      hipLaunchKernelGGL((k_score_lse<In, D, false>), g1, dim3(256), 0, st, q, k, mask, ml, n, T,
                         kps1, nqb, nsplit1, B, qg);
  }
  prof_mark(0, true, st);
  const size_t ss = sel_words(T);
  hipLaunchKernelGGL(k_lse_merge, dim3((4 * B * n + 255) / 256), dim3(256), 0, st, ml, lse, n,
                     nsplit1, B, sel, ss);
  prof_mark(1, false, st);
#define KVC_K2(R, M)                                                                          \
  if constexpr (sizeof(In) == 2)                                                              \
    hipLaunchKernelGGL((k_expweight_bf16<D, R, M>), g2, dim3(256), 0, st, q, k, v, lse, mask,  \
                       Opart, imp_part, n, T, kps2, nqb, nsplit2, B, qg);                     \
  else                                                                                        \
    hipLaunchKernelGGL((k_expweight<In, D, R, M>), g2, dim3(256), 0, st, q, k, v, lse, mask,   \
                       Opart, imp_part, n, T, kps2, nqb, nsplit2, B, qg)
  if (rms) {
    if (mask) KVC_K2(true, true);
    else KVC_K2(true, false);
  } else {
    if (mask) KVC_K2(false, true);
    else KVC_K2(false, false);
  }
#undef KVC_K2
  prof_mark(1, true, st);
  hipLaunchKernelGGL(k_o_reduce, dim3((n + 31) / 32, D / 32, B), dim3(32, 8), 0, st, Opart, O, n,
                     D, nsplit2);
  prof_mark(8, false, st);
  hipLaunchKernelGGL(k_imp_reduce, dim3((T + kImpKeys - 1) / kImpKeys, B), dim3(256), 0, st,
                     imp_part, imp, sel, mask, status, T, nqb, ss);
  prof_mark(8, true, st);
  return hipGetLastError();
}

#define KVC_INST_SCORE(In, D)                                                                  \
  template hipError_t launch_score<In, D>(const void*, const void*, const void*, double2*,     \
                                          double*, float*, float*, float*, float*, uint32_t*,  \
                                          int32_t*, int, int, int, int, int, int, int, bool,   \
                                          int, const uint8_t*, hipStream_t);
KVC_INST_SCORE(bf16_t, 128)
KVC_INST_SCORE(bf16_t, 64)
KVC_INST_SCORE(float, 128)
KVC_INST_SCORE(float, 64)
#undef KVC_INST_SCORE

}  // namespace kvc
