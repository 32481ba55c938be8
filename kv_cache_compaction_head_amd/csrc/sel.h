// Device helpers of the top-t selection's radix passes (select.hip), shared
// with the importance reduction in score.hip, which runs the first pass.
#pragma once
#include "common.h"
#include "launch.h"

namespace kvc {

constexpr int kSelBlock = 256;                    // threads of a selection workgroup
constexpr int kSelPer = kSelChunk / kSelBlock;    // keys per thread
static_assert(kSelPer == 16, "chunk of 4096 keys over 256 threads");

// Ranking key of a key: its importance's bit pattern (order-preserving for
// non-negative floats), plus one, or 0 where the mask excludes the key.
__device__ __forceinline__ unsigned sel_key_of(float v, const uint8_t* mask_b, int j) {
  const unsigned raw = __float_as_uint(v);
  return mask_b ? (mask_b[j] ? 0u : raw + 1u) : raw;
}

// Exclusive prefix sum over a 256-thread block; the total in *total.
__device__ __forceinline__ int scan256(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = x - v;
  for (int w = 0; w < wave; ++w) before += sh[w];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return before;
}

// The digit of the need-th largest key among those a head's histogram
// counts (NB bins, bin NB-1 the largest digit): *dig, and how many keys with
// that digit are still needed (need minus the count of the larger digits).
// Every thread of the block returns the same.
template <int NB>
__device__ void sel_digit(const unsigned* __restrict__ h, int need, int* sh, int* dig,
                          int* rest) {
  constexpr int PER = NB / kSelBlock;
  const int tid = threadIdx.x;
  // thread i sums bins [NB - PER (i+1), NB - PER i), the largest digits first
  const int hi = NB - PER * tid;
  unsigned c[PER];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    c[k] = h[hi - 1 - k];
    sum += static_cast<int>(c[k]);
  }
  int tot;
  const int above = scan256(sum, sh, &tot);
  if (above < need && above + sum >= need) {
    int acc = above;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (acc < need && acc + static_cast<int>(c[k]) >= need) {
        sh[8] = hi - 1 - k;
        sh[9] = need - acc;
      }
      acc += static_cast<int>(c[k]);
    }
  }
  __syncthreads();
  *dig = sh[8];
  *rest = sh[9];
  __syncthreads();
}

// Key prefix after the first P-1 digits of tau (P = 2, 3: the prefix bits;
// P = 4: tau itself) and how many keys with it are still needed.
template <int P>
__device__ void sel_prefix(const unsigned* __restrict__ st, int need, int* sh, unsigned* pre,
                           int* rest) {
  int d1, r1;
  sel_digit<kSelH1>(st, need, sh, &d1, &r1);
  *pre = static_cast<unsigned>(d1) << 21;
  *rest = r1;
  if (P == 2) return;
  int d2, r2;
  sel_digit<kSelH2>(st + kSelH1, r1, sh, &d2, &r2);
  *pre |= static_cast<unsigned>(d2) << 10;
  *rest = r2;
  if (P == 3) return;
  int d3, r3;
  sel_digit<kSelH3>(st + kSelH1 + kSelH2, r2, sh, &d3, &r3);
  *pre |= static_cast<unsigned>(d3);
  *rest = r3;
}

}  // namespace kvc
