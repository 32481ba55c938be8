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
//   k_select   one workgroup per head: MSB-first radix select over the
//              uint32 bit patterns of the (non-negative) importances finds the
//              t-th largest value tau exactly; an order-preserving block scan
//              then keeps every value > tau and the lowest-index values == tau.
//   k_gather   C_k = K[idx] (exact copies, input dtype).
#include "common.h"
#include "launch.h"

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

// grid (B), block kSelThreads.  imp [B][T] (non-negative floats), idx [B][t]:
// the tb = tv[b] (or t) kept indices ascending, then -1 in the remaining slots.
// Keys marked in mask (if given) are never kept: the ranking key is the bit
// pattern plus one, and 0 for a marked key, which keeps the order of the
// others (patterns of finite non-negative floats stay below 0x7f800000).
// status[b] |= 4 if an importance is not finite (NaN/Inf input upstream).
// PER > 0: every thread holds its contiguous chunk of ceil(T / kSelThreads)
// <= PER keys in registers, read once, for all passes and the compaction;
// PER == 0 streams the keys from memory in every pass (any T).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ imp,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ status,
                                                        const int32_t* __restrict__ tv,
                                                        const uint8_t* __restrict__ mask, int T,
                                                        int t) {
  // one 256-bin histogram per wave: no contention between waves on the few
  // top-byte bins most keys share; the digit is then found by a parallel scan
  // of the combined bins
  __shared__ unsigned int hist[kSelThreads / 64][256];
  __shared__ int scratch[64];
  __shared__ unsigned int s_prefix, s_mask;
  __shared__ int s_need, s_bad;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const unsigned int* u = reinterpret_cast<const unsigned int*>(imp) + static_cast<size_t>(b) * T;
  const uint8_t* mb = mask ? mask + static_cast<size_t>(b) * T : nullptr;
  auto key = [&](int j) -> unsigned int {
    const unsigned int v = u[j];
    return mb ? (mb[j] ? 0u : v + 1u) : v;
  };

  const int tb = tv ? tv[b] : t;
  if (tid == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_need = tb;
    s_bad = 0;
  }
  // the thread's contiguous chunk (also the compaction's)
  const int chunk = (T + kSelThreads - 1) / kSelThreads;
  const int c0 = min(T, tid * chunk), c1 = min(T, c0 + chunk);
  constexpr int NR = PER > 0 ? PER : 1;
  unsigned int kv[NR];
  if (PER > 0) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = c0 + i;
      const unsigned int raw = j < c1 ? u[j] : 0u;
      bad |= raw >= 0x7f800000u;  // inf / nan (non-negative inputs)
      kv[i] = j < c1 ? (mb ? (mb[j] ? 0u : raw + 1u) : raw) : 0u;
    }
    __syncthreads();
    if (bad) s_bad = 1;
  }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < (kSelThreads / 64) * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const unsigned int prefix = s_prefix, mask = s_mask;
    unsigned int* hw = hist[wave];
    if (PER > 0) {
#pragma unroll
      for (int i = 0; i < NR; ++i)
        if (c0 + i < c1 && (kv[i] & mask) == prefix) atomicAdd(&hw[(kv[i] >> shift) & 255u], 1u);
    } else {
      for (int j0 = 0; j0 < T; j0 += kSelThreads) {
        const int j = j0 + tid;
        bool in = false;
        unsigned int dig = 0;
        if (j < T) {
          if (shift == 24 && u[j] >= 0x7f800000u) s_bad = 1;  // inf / nan (non-negative inputs)
          const unsigned int v = key(j);
          in = (v & mask) == prefix;
          dig = (v >> shift) & 255u;
        }
        if (in) atomicAdd(&hw[dig], 1u);
      }
    }
    __syncthreads();
    // digit of the need-th largest: scan the bins from the top (bin 255 first)
    unsigned int h = 0;
    if (tid < 256)
      for (int w = 0; w < kSelThreads / 64; ++w) h += hist[w][255 - tid];
    int tot;
    const int above = block_exclusive_scan(static_cast<int>(h), scratch, &tot);
    const int need = s_need;
    __syncthreads();
    if (tid < 256 && above < need && above + static_cast<int>(h) >= need) {
      s_need = need - above;
      s_prefix = prefix | (static_cast<unsigned int>(255 - tid) << shift);
      s_mask = mask | (255u << shift);
    }
    __syncthreads();
  }
  const unsigned int tau = s_prefix;
  const int need_eq = s_need;  // how many values equal to tau are kept

  // order-preserving compaction over the contiguous chunks
  int n_gt = 0, n_eq = 0;
  if (PER > 0) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (c0 + i < c1) {
        n_gt += kv[i] > tau;
        n_eq += kv[i] == tau;
      }
  } else {
    for (int j = c0; j < c1; ++j) {
      const unsigned int v = key(j);
      n_gt += v > tau;
      n_eq += v == tau;
    }
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, scratch, &tot);
  const int take_eq = max(0, min(n_eq, need_eq - eq_before));
  const int pos0 = block_exclusive_scan(n_gt + take_eq, scratch, &tot);
  int32_t* out = idx + static_cast<size_t>(b) * t;
  int pos = pos0, eq_taken = 0;
  if (PER > 0) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (c0 + i < c1) {
        bool keep = kv[i] > tau;
        if (kv[i] == tau && eq_taken < take_eq) {
          keep = true;
          ++eq_taken;
        }
        if (keep) out[pos++] = c0 + i;
      }
  } else {
    for (int j = c0; j < c1; ++j) {
      const unsigned int v = key(j);
      bool keep = v > tau;
      if (v == tau && eq_taken < take_eq) {
        keep = true;
        ++eq_taken;
      }
      if (keep) out[pos++] = j;
    }
  }
  for (int a = tb + tid; a < t; a += kSelThreads) out[a] = -1;
  if (tid == 0 && status && s_bad) status[b] |= 4;
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

hipError_t launch_select(const float* imp, int32_t* idx, int32_t* status, const int32_t* tv,
                         const uint8_t* mask, int B, int T, int t, hipStream_t st) {
  // keys in registers up to 32 per thread (T <= 32768), streamed beyond
  if (T <= 32 * kSelThreads)
    hipLaunchKernelGGL(k_select<32>, dim3(B), dim3(kSelThreads), 0, st, imp, idx, status, tv, mask,
                       T, t);
  else
    hipLaunchKernelGGL(k_select<0>, dim3(B), dim3(kSelThreads), 0, st, imp, idx, status, tv, mask,
                       T, t);
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
