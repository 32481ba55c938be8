// Greedy key selection by orthogonal matching pursuit.
//
// "Fast KV Compaction via Attention Matching", section 2, algorithmic
// pipeline, key selection: pick keys greedily so that they best satisfy the
// attention-mass matching objective, then fit their weights by NNLS.  Here
// the dictionary is the whole-cache softmax weights P [n][T] (column j = key
// j's weight on every reference query) and the target is the relative mass
// y = 1 (each query's kept mass, re-weighted, equals its full mass).  Step k:
//
//   c_j = p_j . r / ||p_j||  over keys not yet chosen (r: current residual),
//   j* = argmax c_j (equal values: the lower index),
//   r  = y minus its orthogonal projection on span{p_j : j chosen}.
//
// The projection is kept as an orthonormal basis Q of the chosen columns,
// extended each step by classical Gram-Schmidt applied twice (the second pass
// restores orthogonality lost to nearly dependent columns), so
// r <- r - q (q . r).  After t steps the chosen set, sorted, goes to the same
// NNLS bias fit and least-squares value fit as the highest-attention keys.
//
// P is stored in float32 (the fp64 weights rounded to nearest); correlations,
// norms, the basis and the residual are float64.  Each step is a handful of
// launches on the caller's stream: the correlation pass reads P once (it
// dominates: n*T*4 bytes per head per step), the rest touches O(n*k).
#include "common.h"
#include "launch.h"

namespace kvc {

constexpr int kCorrCols = 1024;  // keys per workgroup of the correlation pass

// nrm[b][j] = sqrt(sum_i P[b][i][j]^2) in fp64.  grid (ceil(T/256), B).
__global__ void k_omp_norms(const float* __restrict__ P, double* __restrict__ nrm, int n, int T) {
  const int b = blockIdx.y, j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  const float* Pb = P + static_cast<size_t>(b) * n * T + j;
  double s = 0.0;
  for (int i = 0; i < n; ++i) {
    const double v = Pb[static_cast<size_t>(i) * T];
    s = fma(v, v, s);
  }
  nrm[static_cast<size_t>(b) * T + j] = sqrt(s);
}

// r = 1, chosen flags cleared.  grid (ceil(max(n,T)/256), B).
__global__ void k_omp_init(double* __restrict__ r, uint8_t* __restrict__ chosen, int n, int T) {
  const int b = blockIdx.y, e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) r[static_cast<size_t>(b) * n + e] = 1.0;
  if (e < T) chosen[static_cast<size_t>(b) * T + e] = 0;
}

__device__ __forceinline__ bool better(double v, int j, double bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

// Correlation pass: each workgroup scores kCorrCols keys (4 consecutive per
// thread, rows in order) and writes its best (value, key) to part[b][blk].
// grid (ceil(T/kCorrCols), B), block 256.
__global__ __launch_bounds__(256) void k_omp_corr(const float* __restrict__ P,
                                                  const double* __restrict__ r,
                                                  const double* __restrict__ nrm,
                                                  const uint8_t* __restrict__ chosen,
                                                  double2* __restrict__ part, int n, int T) {
  __shared__ double sr[1024];
  __shared__ double bv[4];
  __shared__ int bj[4];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int j0 = blockIdx.x * kCorrCols + tid * 4;
  const float* Pb = P + static_cast<size_t>(b) * n * T;
  const double* rb = r + static_cast<size_t>(b) * n;
  double c[4] = {0.0, 0.0, 0.0, 0.0};
  const bool full = j0 + 3 < T && (T & 3) == 0;
  for (int i0 = 0; i0 < n; i0 += 1024) {
    const int ni = min(1024, n - i0);
    __syncthreads();
    for (int i = tid; i < ni; i += 256) sr[i] = rb[i0 + i];
    __syncthreads();
    if (full) {
      const float* col = Pb + static_cast<size_t>(i0) * T + j0;
      int i = 0;
      for (; i + 4 <= ni; i += 4) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = *reinterpret_cast<const float4*>(col + static_cast<size_t>(i + u) * T);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const double ri = sr[i + u];
          c[0] = fma(static_cast<double>(v[u].x), ri, c[0]);
          c[1] = fma(static_cast<double>(v[u].y), ri, c[1]);
          c[2] = fma(static_cast<double>(v[u].z), ri, c[2]);
          c[3] = fma(static_cast<double>(v[u].w), ri, c[3]);
        }
      }
      for (; i < ni; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(col + static_cast<size_t>(i) * T);
        const double ri = sr[i];
        c[0] = fma(static_cast<double>(v.x), ri, c[0]);
        c[1] = fma(static_cast<double>(v.y), ri, c[1]);
        c[2] = fma(static_cast<double>(v.z), ri, c[2]);
        c[3] = fma(static_cast<double>(v.w), ri, c[3]);
      }
    } else {
      for (int i = 0; i < ni; ++i) {
        const double ri = sr[i];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + u < T)
            c[u] = fma(static_cast<double>(Pb[static_cast<size_t>(i0 + i) * T + j0 + u]), ri, c[u]);
      }
    }
  }
  double best = -INFINITY;
  int bestj = 0x7fffffff;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = j0 + u;
    if (j >= T) continue;
    const double nj = nrm[static_cast<size_t>(b) * T + j];
    if (chosen[static_cast<size_t>(b) * T + j] || !(nj > 0.0)) continue;
    const double v = c[u] / nj;
    if (better(v, j, best, bestj)) {
      best = v;
      bestj = j;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(best, off);
    const int oj = __shfl_xor(bestj, off);
    if (better(ov, oj, best, bestj)) {
      best = ov;
      bestj = oj;
    }
  }
  if ((tid & 63) == 0) {
    bv[tid >> 6] = best;
    bj[tid >> 6] = bestj;
  }
  __syncthreads();
  if (tid == 0) {
    double bb = bv[0];
    int jj = bj[0];
    for (int w = 1; w < 4; ++w)
      if (better(bv[w], bj[w], bb, jj)) {
        bb = bv[w];
        jj = bj[w];
      }
    part[static_cast<size_t>(b) * gridDim.x + blockIdx.x] = make_double2(bb, static_cast<double>(jj));
  }
}

// Reduce the workgroup bests in order, record the pick, gather its column
// a = P[:, j*] (fp64).  grid (B), block 256.
__global__ __launch_bounds__(256) void k_omp_pick(const float* __restrict__ P,
                                                  const double2* __restrict__ part, int nblk,
                                                  uint8_t* __restrict__ chosen,
                                                  int32_t* __restrict__ order,
                                                  double* __restrict__ a, int n, int T, int t,
                                                  int k) {
  __shared__ int sj;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    double best = -INFINITY;
    int bj = 0x7fffffff;
    for (int q = 0; q < nblk; ++q) {
      const double2 v = part[static_cast<size_t>(b) * nblk + q];
      const int j = static_cast<int>(v.y);
      if (better(v.x, j, best, bj)) {
        best = v.x;
        bj = j;
      }
    }
    if (!(best > -INFINITY)) {  // no scorable key left (zero columns): the lowest unchosen
      bj = 0;
      while (bj < T - 1 && chosen[static_cast<size_t>(b) * T + bj]) ++bj;
    }
    sj = bj;
    chosen[static_cast<size_t>(b) * T + bj] = 1;
    order[static_cast<size_t>(b) * t + k] = bj;
  }
  __syncthreads();
  const int j = sj;
  const float* Pb = P + static_cast<size_t>(b) * n * T + j;
  for (int i = tid; i < n; i += 256)
    a[static_cast<size_t>(b) * n + i] = static_cast<double>(Pb[static_cast<size_t>(i) * T]);
}

// h[b][m] = Qb[m] . v for m < k (one wave per m).  grid (ceil(k/4), B), block 256.
__global__ __launch_bounds__(256) void k_omp_proj(const double* __restrict__ Qb,
                                                  const double* __restrict__ v,
                                                  double* __restrict__ h, int n, int t, int k) {
  const int b = blockIdx.y, m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= k) return;
  const double* q = Qb + (static_cast<size_t>(b) * t + m) * n;
  const double* vb = v + static_cast<size_t>(b) * n;
  double s = 0.0;
  for (int i = lane; i < n; i += 64) s = fma(q[i], vb[i], s);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) h[static_cast<size_t>(b) * t + m] = s;
}

// out_i = v_i - sum_{m<k} h_m Qb[m][i]; with PART, also per-workgroup sums of
// out_i^2 and out_i r_i into part2[b][blk].  grid (ceil(n/256), B), block 256.
template <bool PART>
__global__ __launch_bounds__(256) void k_omp_orth(const double* __restrict__ Qb,
                                                  const double* __restrict__ h,
                                                  const double* __restrict__ v,
                                                  double* __restrict__ out,
                                                  const double* __restrict__ r,
                                                  double2* __restrict__ part2, int n, int t,
                                                  int k) {
  __shared__ double sh[4096];
  __shared__ double2 red[4];
  const int b = blockIdx.y, tid = threadIdx.x, i = blockIdx.x * 256 + tid;
  for (int m = tid; m < k; m += 256) sh[m] = h[static_cast<size_t>(b) * t + m];
  __syncthreads();
  double x = 0.0;
  if (i < n) {
    x = v[static_cast<size_t>(b) * n + i];
    const double* q = Qb + static_cast<size_t>(b) * t * n + i;
    for (int m = 0; m < k; ++m) x = fma(-sh[m], q[static_cast<size_t>(m) * n], x);
    out[static_cast<size_t>(b) * n + i] = x;
  }
  if (PART) {
    double s2 = x * x, sr = i < n ? x * r[static_cast<size_t>(b) * n + i] : 0.0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      s2 += __shfl_xor(s2, off);
      sr += __shfl_xor(sr, off);
    }
    if ((tid & 63) == 0) red[tid >> 6] = make_double2(s2, sr);
    __syncthreads();
    if (tid == 0)
      part2[static_cast<size_t>(b) * gridDim.x + blockIdx.x] =
          make_double2(((red[0].x + red[1].x) + red[2].x) + red[3].x,
                       ((red[0].y + red[1].y) + red[2].y) + red[3].y);
  }
}

// Append q / ||q|| to the basis as row k and take it out of the residual:
// r -= q (q . r) / ||q||^2.  grid (ceil(n/256), B), block 256.
__global__ __launch_bounds__(256) void k_omp_update(const double* __restrict__ qv,
                                                    const double2* __restrict__ part2, int nblk,
                                                    double* __restrict__ Qb,
                                                    double* __restrict__ r, int n, int t, int k) {
  const int b = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  double s2 = 0.0, sr = 0.0;
  for (int q = 0; q < nblk; ++q) {
    const double2 v = part2[static_cast<size_t>(b) * nblk + q];
    s2 += v.x;
    sr += v.y;
  }
  if (i >= n) return;
  const double x = qv[static_cast<size_t>(b) * n + i];
  const double inv = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
  Qb[(static_cast<size_t>(b) * t + k) * n + i] = x * inv;
  if (s2 > 0.0) r[static_cast<size_t>(b) * n + i] -= x * (sr / s2);
}

// Chosen flags -> ascending index list (one workgroup per head; the flags
// hold exactly t ones).  grid (B), block 1024.
__global__ __launch_bounds__(1024) void k_omp_list(const uint8_t* __restrict__ chosen,
                                                   int32_t* __restrict__ idx, int T, int t) {
  __shared__ int cnt[1024];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* cb = chosen + static_cast<size_t>(b) * T;
  const int chunk = (T + 1023) / 1024, c0 = min(T, tid * chunk), c1 = min(T, c0 + chunk);
  int c = 0;
  for (int j = c0; j < c1; ++j) c += cb[j] != 0;
  cnt[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int y = tid >= off ? cnt[tid - off] : 0;
    __syncthreads();
    cnt[tid] += y;
    __syncthreads();
  }
  int pos = cnt[tid] - c;
  for (int j = c0; j < c1; ++j)
    if (cb[j] && pos < t) idx[static_cast<size_t>(b) * t + pos++] = j;
}

hipError_t launch_omp(const float* P, OmpBufs ob, int32_t* idx, int B, int n, int T, int t,
                      hipStream_t st) {
  const dim3 blk(256);
  hipLaunchKernelGGL(k_omp_norms, dim3((T + 255) / 256, B), blk, 0, st, P, ob.nrm, n, T);
  const int ne = n > T ? n : T;
  hipLaunchKernelGGL(k_omp_init, dim3((ne + 255) / 256, B), blk, 0, st, ob.r, ob.chosen, n, T);
  const int ncb = (T + kCorrCols - 1) / kCorrCols, nib = (n + 255) / 256;
  for (int k = 0; k < t; ++k) {
    hipLaunchKernelGGL(k_omp_corr, dim3(ncb, B), blk, 0, st, P, ob.r, ob.nrm, ob.chosen, ob.part,
                       n, T);
    hipLaunchKernelGGL(k_omp_pick, dim3(B), blk, 0, st, P, ob.part, ncb, ob.chosen, ob.order,
                       ob.a, n, T, t, k);
    if (k > 0) {
      // q = a - Q^T (Q a), twice
      hipLaunchKernelGGL(k_omp_proj, dim3((k + 3) / 4, B), blk, 0, st, ob.Q, ob.a, ob.h, n, t, k);
      hipLaunchKernelGGL(k_omp_orth<false>, dim3(nib, B), blk, 0, st, ob.Q, ob.h, ob.a, ob.q,
                         ob.r, ob.part2, n, t, k);
      hipLaunchKernelGGL(k_omp_proj, dim3((k + 3) / 4, B), blk, 0, st, ob.Q, ob.q, ob.h, n, t, k);
      hipLaunchKernelGGL(k_omp_orth<true>, dim3(nib, B), blk, 0, st, ob.Q, ob.h, ob.q, ob.q,
                         ob.r, ob.part2, n, t, k);
    } else {
      hipLaunchKernelGGL(k_omp_orth<true>, dim3(nib, B), blk, 0, st, ob.Q, ob.h, ob.a, ob.q,
                         ob.r, ob.part2, n, t, 0);
    }
    hipLaunchKernelGGL(k_omp_update, dim3(nib, B), blk, 0, st, ob.q, ob.part2, nib, ob.Q, ob.r,
                       n, t, k);
  }
  hipLaunchKernelGGL(k_omp_list, dim3(B), dim3(1024), 0, st, ob.chosen, idx, T, t);
  return hipGetLastError();
}

}  // namespace kvc
