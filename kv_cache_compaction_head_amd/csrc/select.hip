// Key selection and gather.
//
// "Fast KV Compaction via Attention Matching", section 2, algorithmic
// pipeline: keep the original keys with the highest aggregated attention.
// The ranking key is the per-key sum over reference queries of p^2 (RMS
// aggregation) or p (mean); the page's sqrt(./n) and ./n are monotone and do
// not change the order.  Equal values go to the lower index, and the kept
// indices are emitted in ascending order so the compacted cache keeps the
// positional order of the original (a contiguous re-indexing of the survivors).
//
//   k_sel_*    MSB-first radix select over the uint32 bit patterns of the
//              (non-negative) importances, several workgroups per head, finds
//              the t-th largest value tau exactly; an order-preserving
//              compaction then keeps every value > tau and the lowest-index
//              values == tau.
//   k_gather   C_k = K[idx] (exact copies, input dtype).
#include "common.h"
#include "launch.h"
#include "sel.h"

namespace kvc {

constexpr int kSelThreads = 1024;

// Exclusive prefix sum over the block (kSelThreads threads), returns the
// total in *total.  Deterministic (integer).
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kSelThreads / 64 ? scratch[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < kSelThreads / 64) scratch[32 + lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int before = (wave ? scratch[32 + wave - 1] : 0) + x - v;
  *total = scratch[32 + kSelThreads / 64 - 1];
  __syncthreads();
  return before;
}

// ---------------------------------------------------------------------------
// Top-t selection, several workgroups per head.  The ranking key of key j is
// the uint32 bit pattern of its importance (order-preserving for the
// non-negative floats), plus one, or 0 when the mask excludes it.  The exact
// t-th largest key tau is found MSB first in three digits (bits 31-21, 20-10,
// 9-0): each pass histograms, per chunk of kSelChunk keys, the next digit of
// the keys that match the digits found so far, and adds the chunk's
// histogram into the head's (integer atomics: the counts do not depend on
// the order).  Pass 1 runs inside the importance reduction (score.hip); each
// later kernel reads the digits found so far from the head's histograms.
// Then every chunk counts its keys above and equal to tau, and a compaction
// keeps every key above tau and the lowest-index keys equal to it, in
// ascending order, from the chunks' counts in chunk order.
// ---------------------------------------------------------------------------

// The chunk's 16 keys of this thread: key chunk start + 256 i + thread.
__device__ __forceinline__ void sel_load_strided(const float* ib, const uint8_t* mb, int T, int g,
                                                 unsigned (&kv)[kSelPer]) {
  float v[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = g * kSelChunk + i * kSelBlock + threadIdx.x;
    v[i] = j < T ? ib[j] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = g * kSelChunk + i * kSelBlock + threadIdx.x;
    kv[i] = j < T ? sel_key_of(v[i], mb, j) : 0u;
  }
}

// Passes 2 and 3: histogram of digit P of the chunk's keys that match tau's
// first P-1 digits.  grid (chunks, B), block 256.
template <int P>
__global__ __launch_bounds__(kSelBlock) void k_sel_refine(const float* __restrict__ imp,
                                                          unsigned* __restrict__ sel,
                                                          const int32_t* __restrict__ tv,
                                                          const uint8_t* __restrict__ mask,
                                                          int T, int t, size_t sstride) {
  constexpr int NB = P == 2 ? kSelH2 : kSelH3;
  constexpr int SH = P == 2 ? 10 : 0;
  constexpr unsigned PM = P == 2 ? 0xFFE00000u : 0xFFFFFC00u;
  __shared__ unsigned hist[NB];
  __shared__ int sh[16];
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  unsigned* st = sel + b * sstride;
  const float* ib = imp + static_cast<size_t>(b) * T;
  const uint8_t* mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;
  unsigned kv[kSelPer];
  sel_load_strided(ib, mb, T, g, kv);  // in flight while the prefix is found
  for (int i = tid; i < NB; i += kSelBlock) hist[i] = 0;
  unsigned pre;
  int rest;
  sel_prefix<P>(st, tv ? tv[b] : t, sh, &pre, &rest);
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = g * kSelChunk + i * kSelBlock + tid;
    if (j < T && (kv[i] & PM) == pre) atomicAdd(&hist[(kv[i] >> SH) & (NB - 1)], 1u);
  }
  __syncthreads();
  unsigned* gh = st + (P == 2 ? kSelH1 : kSelH1 + kSelH2);
  for (int i = tid; i < NB; i += kSelBlock)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// tau and the number of keys equal to it that are kept (chunk 0 records
// them), and the chunk's counts above and equal to tau.  grid (chunks, B).
__global__ __launch_bounds__(kSelBlock) void k_sel_count(const float* __restrict__ imp,
                                                         unsigned* __restrict__ sel,
                                                         const int32_t* __restrict__ tv,
                                                         const uint8_t* __restrict__ mask, int T,
                                                         int t, size_t sstride) {
  __shared__ int sh[16];
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  unsigned* st = sel + b * sstride;
  const float* ib = imp + static_cast<size_t>(b) * T;
  const uint8_t* mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;
  unsigned kv[kSelPer];
  sel_load_strided(ib, mb, T, g, kv);
  unsigned tau;
  int need_eq;
  sel_prefix<4>(st, tv ? tv[b] : t, sh, &tau, &need_eq);
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = g * kSelChunk + i * kSelBlock + tid;
    if (j < T) {
      gt += kv[i] > tau;
      eq += kv[i] == tau;
    }
  }
  int tgt, teq;
  scan256(gt, sh, &tgt);
  scan256(eq, sh, &teq);
  if (tid == 0) {
    st[kSelCnt + 2 * g] = static_cast<unsigned>(tgt);
    st[kSelCnt + 2 * g + 1] = static_cast<unsigned>(teq);
    if (g == 0) {
      st[kSelTau] = tau;
      st[kSelTau + 1] = static_cast<unsigned>(need_eq);
    }
  }
}

// Order-preserving compaction: chunk g starts after the keys kept by the
// chunks before it (all above tau, plus the equal ones while need_eq lasts);
// inside the chunk each thread takes 16 contiguous keys, in thread order.
// idx [B][t]: the tb = tv[b] (or t) kept indices ascending, -1 in the
// remaining slots.  grid (chunks, B).
__global__ __launch_bounds__(kSelBlock) void k_sel_compact(const float* __restrict__ imp,
                                                           const unsigned* __restrict__ sel,
                                                           int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ tv,
                                                           const uint8_t* __restrict__ mask,
                                                           int T, int t, size_t sstride) {
  __shared__ int sh[16];
  __shared__ int s_base[2];
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const unsigned* st = sel + b * sstride;
  const float* ib = imp + static_cast<size_t>(b) * T;
  const uint8_t* mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;
  const int j0 = g * kSelChunk + tid * kSelPer;
  float v[kSelPer];
  if (j0 + kSelPer <= T && (T & 3) == 0) {
    // whole and 16-byte aligned: four 16-byte loads
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
      const float4 w4 = *reinterpret_cast<const float4*>(ib + j0 + 4 * q);
      v[4 * q] = w4.x;
      v[4 * q + 1] = w4.y;
      v[4 * q + 2] = w4.z;
      v[4 * q + 3] = w4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) v[i] = j0 + i < T ? ib[j0 + i] : 0.f;
  }
  const unsigned tau = st[kSelTau];
  const int need_eq = static_cast<int>(st[kSelTau + 1]);
  if (tid == 0) {
    int kept = 0, eqb = 0;
    for (int c = 0; c < g; ++c) {
      const int gt = static_cast<int>(st[kSelCnt + 2 * c]);
      const int eq = static_cast<int>(st[kSelCnt + 2 * c + 1]);
      kept += gt + max(0, min(eq, need_eq - eqb));
      eqb += eq;
    }
    s_base[0] = kept;
    s_base[1] = eqb;
  }
  unsigned kv[kSelPer];
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    kv[i] = j0 + i < T ? sel_key_of(v[i], mb, j0 + i) : 0u;
    if (j0 + i < T) {
      gt += kv[i] > tau;
      eq += kv[i] == tau;
    }
  }
  __syncthreads();
  int tot;
  const int eq_before = s_base[1] + scan256(eq, sh, &tot);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  int pos = s_base[0] + scan256(gt + take_eq, sh, &tot);
  int32_t* out = idx + static_cast<size_t>(b) * t;
  int taken = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = j0 + i;
    if (j < T) {
      bool keep = kv[i] > tau;
      if (kv[i] == tau && taken < take_eq) {
        keep = true;
        ++taken;
      }
      if (keep) out[pos++] = j;
    }
  }
  if (g == 0) {
    const int tb = tv ? tv[b] : t;
    for (int a = tb + tid; a < t; a += kSelBlock) out[a] = -1;
  }
}

// out_K[b][a][:] = K[b][idx[b][a]][:], zeros where idx is -1 (unused slots
// of a smaller per-head budget).  grid (ceil(t*D*es/16/256), B).
__global__ void k_gather_rows(const uint4* __restrict__ K, const int32_t* __restrict__ idx,
                              uint4* __restrict__ out, int T, int t, int row_vecs) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= t * row_vecs) return;
  const int a = i / row_vecs, c = i % row_vecs;
  const int j = idx[static_cast<size_t>(b) * t + a];
  out[(static_cast<size_t>(b) * t + a) * row_vecs + c] =
      j >= 0 ? K[(static_cast<size_t>(b) * T + j) * row_vecs + c] : make_uint4(0, 0, 0, 0);
}

// Per-head budgets: tv[b] = tin[b] clamped to [1, t]; status |= 16 where it
// had to be clamped.  grid (ceil(B/256)).
__global__ void k_budgets(const int32_t* __restrict__ tin, int32_t* __restrict__ tv,
                          int32_t* __restrict__ status, int B, int t) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int v = tin[b];
  const int c = v < 1 ? 1 : (v > t ? t : v);
  tv[b] = c;
  if (c != v && status) status[b] |= 16;
}

hipError_t launch_budgets(const int32_t* tin, int32_t* tv, int32_t* status, int B, int t,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_budgets, dim3((B + 255) / 256), dim3(256), 0, st, tin, tv, status, B, t);
  return hipGetLastError();
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int32_t v, size_t count) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t count, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_i32, dim3((count + 255) / 256), dim3(256), 0, st, p, v, count);
  return hipGetLastError();
}

hipError_t launch_select(const float* imp, uint32_t* sel, int32_t* idx, const int32_t* tv,
                         const uint8_t* mask, int B, int T, int t, hipStream_t st) {
  const dim3 grid(sel_chunks(T), B);
  const size_t ss = sel_words(T);
  hipLaunchKernelGGL(k_sel_refine<2>, grid, dim3(kSelBlock), 0, st, imp, sel, tv, mask, T, t, ss);
  hipLaunchKernelGGL(k_sel_refine<3>, grid, dim3(kSelBlock), 0, st, imp, sel, tv, mask, T, t, ss);
  hipLaunchKernelGGL(k_sel_count, grid, dim3(kSelBlock), 0, st, imp, sel, tv, mask, T, t, ss);
  hipLaunchKernelGGL(k_sel_compact, grid, dim3(kSelBlock), 0, st, imp, sel, idx, tv, mask, T, t,
                     ss);
  return hipGetLastError();
}

hipError_t launch_gather(const void* K, const int32_t* idx, void* outK, int B, int T, int t,
                         int row_bytes, hipStream_t st) {
  const int row_vecs = row_bytes / 16;
  const int tot = t * row_vecs;
  hipLaunchKernelGGL(k_gather_rows, dim3((tot + 255) / 256, B), dim3(256), 0, st,
                     static_cast<const uint4*>(K), idx, static_cast<uint4*>(outK), T, t,
                     row_vecs);
  return hipGetLastError();
}

// Chunked compaction: batch entry b' = head * C + chunk holds the chunk's
// kept indices relative to the chunk; make them positions in the head's cache.
__global__ void k_idx_offset(int32_t* __restrict__ idx, int Bc, int t, int C, int Tc) {
  const size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<size_t>(Bc) * t) return;
  const int bc = static_cast<int>(e / t);
  if (idx[e] >= 0) idx[e] += (bc % C) * Tc;
}

hipError_t launch_idx_offset(int32_t* idx, int Bc, int t, int C, int Tc, hipStream_t st) {
  const size_t tot = static_cast<size_t>(Bc) * t;
  hipLaunchKernelGGL(k_idx_offset, dim3((tot + 255) / 256), dim3(256), 0, st, idx, Bc, t, C, Tc);
  return hipGetLastError();
}

// Protected keys ("Thought-Aware KV Cache Compaction ...", section 2C: pivot
// tokens kept exactly, with zero bias, and the rest of the budget spread over
// the others).  One workgroup per head scans the caller's mask in order: the
// first pp = min(count, t - 1) marked keys are listed in plist and marked in
// emask, so the fitted part always keeps at least one key; marks beyond them
// are dropped (status |= 32).  tv[b] = t - pp.  grid (B), block kSelThreads.
__global__ __launch_bounds__(kSelThreads) void k_protect_prep(const uint8_t* __restrict__ mask,
                                                              uint8_t* __restrict__ emask,
                                                              int32_t* __restrict__ plist,
                                                              int32_t* __restrict__ tv,
                                                              int32_t* __restrict__ status, int T,
                                                              int t) {
  __shared__ int scratch[64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* mb = mask + static_cast<size_t>(b) * T;
  uint8_t* eb = emask + static_cast<size_t>(b) * T;
  int32_t* pl = plist + static_cast<size_t>(b) * t;
  const int chunk = (T + kSelThreads - 1) / kSelThreads;
  const int c0 = min(T, tid * chunk), c1 = min(T, c0 + chunk);
  int cnt = 0;
  for (int j = c0; j < c1; ++j) cnt += mb[j] != 0;
  int total;
  int pos = block_exclusive_scan(cnt, scratch, &total);
  const int cap = t - 1;
  for (int j = c0; j < c1; ++j) {
    const bool m = mb[j] != 0 && pos < cap;
    if (m) pl[pos] = j;
    pos += mb[j] != 0;
    eb[j] = m;
  }
  if (tid == 0) {
    const int pp = min(total, cap);
    tv[b] = t - pp;
    if (total > cap && status) status[b] |= 32;
  }
}

hipError_t launch_protect_prep(const uint8_t* mask, uint8_t* emask, int32_t* plist, int32_t* tv,
                               int32_t* status, int B, int T, int t, hipStream_t st) {
  hipLaunchKernelGGL(k_protect_prep, dim3(B), dim3(kSelThreads), 0, st, mask, emask, plist, tv,
                     status, T, t);
  return hipGetLastError();
}

// Slots a in [tv[b], t) of head b hold protected key plist[b][a - tv[b]]:
// out_K = K row (bytes), out_V = V row as OutT (float, or bfloat16 of the
// float value), bias 0, idx = position.  grid (ceil(t*D/256), B).
template <class In, class OutT>
__global__ void k_fill_protected(const int32_t* __restrict__ plist, const int32_t* __restrict__ tv,
                                 const In* __restrict__ K, const In* __restrict__ V,
                                 In* __restrict__ out_K, OutT* __restrict__ out_V,
                                 float* __restrict__ out_bias, int32_t* __restrict__ out_idx,
                                 int T, int t, int D) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = e / D, c = e % D, a0 = tv[b];
  if (a >= t || a < a0) return;
  const int j = plist[static_cast<size_t>(b) * t + (a - a0)];
  const size_t src = (static_cast<size_t>(b) * T + j) * D + c;
  const size_t dst = (static_cast<size_t>(b) * t + a) * D + c;
  out_K[dst] = K[src];
  out_V[dst] = from_f32<OutT>(to_f32<In>(V[src]));
  if (c == 0) {
    out_bias[static_cast<size_t>(b) * t + a] = 0.f;
    if (out_idx) out_idx[static_cast<size_t>(b) * t + a] = j;
  }
}

template <class In, class OutT>
static void fill_protected(const int32_t* plist, const int32_t* tv, const void* K, const void* V,
                           void* out_K, void* out_V, float* out_bias, int32_t* out_idx, int B,
                           int T, int t, int D, hipStream_t st) {
  const dim3 grid((static_cast<size_t>(t) * D + 255) / 256, B);
  hipLaunchKernelGGL((k_fill_protected<In, OutT>), grid, dim3(256), 0, st, plist, tv,
                     static_cast<const In*>(K), static_cast<const In*>(V), static_cast<In*>(out_K),
                     static_cast<OutT*>(out_V), out_bias, out_idx, T, t, D);
}

hipError_t launch_fill_protected(const int32_t* plist, const int32_t* tv, const void* K,
                                 const void* V, void* out_K, void* out_V, float* out_bias,
                                 int32_t* out_idx, int B, int T, int t, int D, bool bf16,
                                 bool v_bf16, hipStream_t st) {
  if (bf16) {
    if (v_bf16) fill_protected<bf16_t, bf16_t>(plist, tv, K, V, out_K, out_V, out_bias, out_idx, B, T, t, D, st);
    else fill_protected<bf16_t, float>(plist, tv, K, V, out_K, out_V, out_bias, out_idx, B, T, t, D, st);
  } else {
    if (v_bf16) fill_protected<float, bf16_t>(plist, tv, K, V, out_K, out_V, out_bias, out_idx, B, T, t, D, st);
    else fill_protected<float, float>(plist, tv, K, V, out_K, out_V, out_bias, out_idx, B, T, t, D, st);
  }
  return hipGetLastError();
}

}  // namespace kvc
