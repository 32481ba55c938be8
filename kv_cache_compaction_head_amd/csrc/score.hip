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
#include "common.h"
#include "launch.h"

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
// with CPR chunks per row: the 16 rows an MFMA operand read takes at once
// land in 16 distinct 16-byte bank groups of a 256-byte bank row.
template <int CPR>
__device__ __forceinline__ int k_swz(int r) {
  static_assert(CPR == 8 || CPR == 16, "16-byte chunks per row");
  return (r / (16 / CPR)) & (CPR - 1);
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

// lse[b][q] (float64) from the split partials, merged in split order.
// Four lanes per query, each taking every fourth split: the maximum over
// all splits, then each lane's sum in split order, then the four sums added
// in lane order.  grid (ceil(4 B n / 256)), block 256.
__global__ void k_lse_merge(const double2* __restrict__ ml, double* __restrict__ lse, int n,
                            int nsplit, int B) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x, i = g >> 2, part = g & 3;
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
    const float a = SQ ? v[i] * v[i] : v[i], c = SQ ? v[8 + i] * v[8 + i] : v[8 + i];
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(c),
                                                    false, false);
    w[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// imp[b][j] = sum over query blocks (in order) of imp_part[b][qb][j].
__global__ void k_imp_reduce(const float* __restrict__ part, float* __restrict__ imp, int T,
                             int nqb, int B) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(B) * T) return;
  const size_t b = i / T, j = i % T;
  const float* p = part + b * nqb * T + j;
  float s = 0.f;
  for (int qb = 0; qb < nqb; ++qb) s += p[static_cast<size_t>(qb) * T];
  imp[i] = s;
}

// ---------------------------------------------------------------------------
// Host-side launchers (same library).
// ---------------------------------------------------------------------------
template <class In, int D>
hipError_t launch_score(const void* Q, const void* K, const void* V, double2* ml, double* lse,
                        float* Opart, float* O, float* imp_part, float* imp, int B, int n, int T,
                        int nsplit1, int kps1, int nsplit2, int kps2, bool rms, int qg,
                        const uint8_t* mask, hipStream_t st) {
  const int nqb = (n + kBM - 1) / kBM;
  const In* q = static_cast<const In*>(Q);
  const In* k = static_cast<const In*>(K);
  const In* v = static_cast<const In*>(V);
  prof_mark(0, false, st);
  const dim3 g1(score_grid_size(nqb, nsplit1, B)), g2(score_grid_size(nqb, nsplit2, B));
  if (mask)
    hipLaunchKernelGGL((k_score_lse<In, D, true>), g1, dim3(256), 0, st, q, k, mask, ml, n, T, kps1,
                       nqb, nsplit1, B, qg);
  else
    hipLaunchKernelGGL((k_score_lse<In, D, false>), g1, dim3(256), 0, st, q, k, mask, ml, n, T,
                       kps1, nqb, nsplit1, B, qg);
  prof_mark(0, true, st);
  hipLaunchKernelGGL(k_lse_merge, dim3((4 * B * n + 255) / 256), dim3(256), 0, st, ml, lse, n,
                     nsplit1, B);
  prof_mark(1, false, st);
#define KVC_K2(R, M)                                                                           \
  hipLaunchKernelGGL((k_expweight<In, D, R, M>), g2, dim3(256), 0, st, q, k, v, lse, mask, Opart, \
                     imp_part, n, T, kps2, nqb, nsplit2, B, qg)
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
  const size_t tot = static_cast<size_t>(B) * T;
  hipLaunchKernelGGL(k_imp_reduce, dim3((tot + 255) / 256), dim3(256), 0, st, imp_part, imp, T,
                     nqb, B);
  return hipGetLastError();
}

template hipError_t launch_score<bf16_t, 128>(const void*, const void*, const void*, double2*,
                                              double*, float*, float*, float*, float*, int, int,
                                              int, int, int, int, int, bool, int, const uint8_t*,
                                             hipStream_t);
template hipError_t launch_score<bf16_t, 64>(const void*, const void*, const void*, double2*,
                                             double*, float*, float*, float*, float*, int, int,
                                             int, int, int, int, int, bool, int, const uint8_t*,
                                             hipStream_t);
template hipError_t launch_score<float, 128>(const void*, const void*, const void*, double2*,
                                             double*, float*, float*, float*, float*, int, int,
                                             int, int, int, int, int, bool, int, const uint8_t*,
                                             hipStream_t);
template hipError_t launch_score<float, 64>(const void*, const void*, const void*, double2*,
                                            double*, float*, float*, float*, float*, int, int,
                                            int, int, int, int, int, bool, int, const uint8_t*,
                                             hipStream_t);

}  // namespace kvc
