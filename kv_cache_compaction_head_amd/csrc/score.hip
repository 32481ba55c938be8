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

// ---------------------------------------------------------------------------
// K1: partial log-sum-exp per (query, key split).
// grid (ceil(n/128), nsplit, B), block 256.  ml[b][split][q] = (m, l) with
// sum_{j in split} exp(s_qj) = l * exp(m).
// ---------------------------------------------------------------------------
template <class In, int D>
__global__ __launch_bounds__(256) void k_score_lse(const In* __restrict__ Q,
                                                   const In* __restrict__ K,
                                                   double2* __restrict__ ml, int n, int T,
                                                   int keys_per_split) {
  constexpr int KS = Frag<In>::KS, NK = D / KS, BN = 64, LD = D + 16 / sizeof(In);
  __shared__ __align__(16) In sK[BN * LD];
  const int b = blockIdx.z, split = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
  const int q = blockIdx.x * kBM + wave * 32 + (lane & 31);
  const In* Qb = Q + static_cast<size_t>(b) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;

  typename Frag<In>::T bq[NK];
  load_q_frags<In, D>(bq, Qb, q, n, g);

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  // running max m (a score, exact in fp32) and sum l = sum exp(s - m) in fp64:
  // each 16-term tile sum is formed in fp32, then accumulated in double, and
  // the rare rescale on a new maximum uses a double exp.
  float m = -INFINITY;
  double l = 0.0;
  for (int jt = j0; jt < j1; jt += BN) {
    __syncthreads();
    load_tile<In, D, LD>(sK, Kb + static_cast<size_t>(jt) * D, BN, j1 - jt);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < BN / 32; ++st) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        auto a = Frag<In>::load(&sK[(st * 32 + (lane & 31)) * LD + ks * KS + g * (KS / 2)]);
        acc = Frag<In>::mma(a, bq[ks], acc);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jt + st * 32 + mfma32_row(r, lane);
        const float s = j < j1 ? acc[r] : -INFINITY;
        acc[r] = s;
        tmax = fmaxf(tmax, s);
      }
      if (tmax > m) {
        if (m != -INFINITY) l *= exp(static_cast<double>(m) - static_cast<double>(tmax));
        m = tmax;
      }
      if (m != -INFINITY) {
        const float m2 = m * KVC_LOG2E;
        const float m2lo = fmaf(m, KVC_LOG2E, -m2);  // m*log2e = m2 + m2lo exactly
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sum += __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -m2) - m2lo);
        l += static_cast<double>(sum);
      }
    }
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
    ml[(static_cast<size_t>(b) * gridDim.y + split) * n + q] = make_double2(mm, ll);
  }
}

// lse[b][q] (float64) from the split partials, merged in split order.
__global__ void k_lse_merge(const double2* __restrict__ ml, double* __restrict__ lse, int n,
                            int nsplit, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * n) return;
  const int b = i / n, q = i % n;
  const double2* p = ml + static_cast<size_t>(b) * nsplit * n + q;
  double m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmax(m, p[static_cast<size_t>(s) * n].x);
  double l = 0.0;
  for (int s = 0; s < nsplit; ++s) {
    const double2 v = p[static_cast<size_t>(s) * n];
    if (v.x != -INFINITY) l += v.y * exp(v.x - m);
  }
  lse[i] = m + log(l);
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
// ---------------------------------------------------------------------------
template <class In, int D, bool RMS>
__global__ __launch_bounds__(256) void k_expweight(const In* __restrict__ Q,
                                                   const In* __restrict__ K,
                                                   const In* __restrict__ V,
                                                   const double* __restrict__ lse,
                                                   float* __restrict__ Opart,
                                                   float* __restrict__ imp_part, int n, int T,
                                                   int keys_per_split) {
  constexpr int KS = Frag<In>::KS, NK = D / KS, BN = 32;
  constexpr int LD = D + 16 / sizeof(In);
  constexpr int LDV = BN + 16 / sizeof(In);
  constexpr int ND = D / 32;
  __shared__ __align__(16) In sK[BN * LD];
  __shared__ __align__(16) In sVt[D * LDV];
  __shared__ float sImp[kWaves * 16 * 64];

  const int b = blockIdx.z, split = blockIdx.y, nsplit = gridDim.y, nqb = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
  const int q = blockIdx.x * kBM + wave * 32 + (lane & 31);
  const In* Qb = Q + static_cast<size_t>(b) * n * D;
  const In* Kb = K + static_cast<size_t>(b) * T * D;
  const In* Vb = V + static_cast<size_t>(b) * T * D;

  typename Frag<In>::T bq[NK];
  load_q_frags<In, D>(bq, Qb, q, n, g);
  // lse*log2e as an unevaluated fp32 pair, so exp2(s*log2e - hi - lo) keeps
  // the float64 log-sum-exp's accuracy
  const double l2 = q < n ? lse[static_cast<size_t>(b) * n + q] * 1.4426950408889634 : 0.0;
  const float ml2 = static_cast<float>(l2);
  const float ml2lo = static_cast<float>(l2 - static_cast<double>(ml2));

  f32x16 accO[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) accO[dt] = f32x16{};

  const int j0 = split * keys_per_split;
  const int j1 = min(T, j0 + keys_per_split);
  for (int jt = j0; jt < j1; jt += BN) {
    const int valid = j1 - jt;
    __syncthreads();
    load_tile<In, D, LD>(sK, Kb + static_cast<size_t>(jt) * D, BN, valid);
    {  // V tile, transposed to [dd][key slot]
      constexpr int VEC = 16 / sizeof(In), CPR = D / VEC;
      for (int c = threadIdx.x; c < BN * CPR; c += blockDim.x) {
        const int r = c / CPR, col = (c % CPR) * VEC;
        In v[VEC];
        if (r < valid) {
          *reinterpret_cast<uint4*>(v) =
              *reinterpret_cast<const uint4*>(Vb + static_cast<size_t>(jt + r) * D + col);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = In(0);
        }
        const int pos = sizeof(In) == 2 ? vt_pos(r) : r;
#pragma unroll
        for (int e = 0; e < VEC; ++e) sVt[(col + e) * LDV + pos] = v[e];
      }
    }
    __syncthreads();

    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      auto a = Frag<In>::load(&sK[(lane & 31) * LD + ks * KS + g * (KS / 2)]);
      acc = Frag<In>::mma(a, bq[ks], acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = mfma32_row(r, lane);
      float p = 0.f;
      if (kk < valid && q < n)
        p = __builtin_amdgcn_exp2f(fmaf(acc[r], KVC_LOG2E, -ml2) - ml2lo);
      acc[r] = p;
      sImp[(wave * 16 + r) * 64 + lane] = RMS ? p * p : p;
    }
    __syncthreads();
    {  // column sums over the workgroup's 128 queries, fixed order
      const int kk = threadIdx.x >> 3, part = threadIdx.x & 7;
      const int gk = (kk >> 2) & 1, rk = ((kk >> 3) << 2) | (kk & 3);
      const int w = part >> 1, lb = gk * 32 + (part & 1) * 16;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += sImp[(w * 16 + rk) * 64 + lb + i];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (part == 0 && kk < valid)
        imp_part[(static_cast<size_t>(b) * nqb + blockIdx.x) * T + jt + kk] = s;
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
              &sVt[(dt * 32 + (lane & 31)) * LDV + h * 16 + g * 8]);
          accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, accO[dt], 0, 0, 0);
          accO[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, accO[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = mfma32_row(r, lane);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const float a = static_cast<float>(sVt[(dt * 32 + (lane & 31)) * LDV + kk]);
          accO[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, acc[r], accO[dt], 0, 0, 0);
        }
      }
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
                        int nsplit1, int kps1, int nsplit2, int kps2, bool rms,
                        hipStream_t st) {
  const int nqb = (n + kBM - 1) / kBM;
  const In* q = static_cast<const In*>(Q);
  const In* k = static_cast<const In*>(K);
  const In* v = static_cast<const In*>(V);
  prof_mark(0, false, st);
  hipLaunchKernelGGL((k_score_lse<In, D>), dim3(nqb, nsplit1, B), dim3(256), 0, st, q, k, ml, n,
                     T, kps1);
  prof_mark(0, true, st);
  hipLaunchKernelGGL(k_lse_merge, dim3((B * n + 255) / 256), dim3(256), 0, st, ml, lse, n,
                     nsplit1, B);
  prof_mark(1, false, st);
  if (rms)
    hipLaunchKernelGGL((k_expweight<In, D, true>), dim3(nqb, nsplit2, B), dim3(256), 0, st, q, k,
                       v, lse, Opart, imp_part, n, T, kps2);
  else
    hipLaunchKernelGGL((k_expweight<In, D, false>), dim3(nqb, nsplit2, B), dim3(256), 0, st, q,
                       k, v, lse, Opart, imp_part, n, T, kps2);
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
                                              int, int, int, int, int, bool, hipStream_t);
template hipError_t launch_score<bf16_t, 64>(const void*, const void*, const void*, double2*,
                                             double*, float*, float*, float*, float*, int, int,
                                             int, int, int, int, int, bool, hipStream_t);
template hipError_t launch_score<float, 128>(const void*, const void*, const void*, double2*,
                                             double*, float*, float*, float*, float*, int, int,
                                             int, int, int, int, int, bool, hipStream_t);
template hipError_t launch_score<float, 64>(const void*, const void*, const void*, double2*,
                                            double*, float*, float*, float*, float*, int, int,
                                            int, int, int, int, int, bool, hipStream_t);

}  // namespace kvc
