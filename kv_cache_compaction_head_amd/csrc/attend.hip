// Attention over a (compacted) cache followed by an appended fixed block.
//
// "Fast KV Compaction via Attention Matching", section 2, main objective: the
// compact cache (C_k, beta, C_v) must keep the attention output for any query
// and any fixed or future block (K_fixed, V_fixed) appended after it, which
// holds when the compact block reproduces the original block's output and
// attention mass (attention over concatenated blocks is the mass-weighted mix
// of the blocks' outputs).  This kernel evaluates the consumer's side of that
// statement on the GPU:
//
//   out_i = sum_j softmax_j(s_ij) v_j,  s_ij = q_i . k_j + bias_j  over the
//   keys of block 1 (K1, V1, bias, e.g. a compact cache) then block 2 (K2, V2,
//   no bias, e.g. the appended block),  lse_i = log sum_j exp(s_ij).
//
// The keys are cut into splits of whole 64-key tiles so the grid has ~2048
// workgroups; a split's partial (max, sum, output) goes to the workspace and
// k_attend_merge combines the splits in order (one split: written directly).
// One workgroup of 256 threads takes 64 queries of one head; four lanes share
// a query, each holding a quarter of its d coordinates (dot-product quarters
// are summed with two xor shuffles, so all four lanes see every score).  Keys
// and values of 64-key tiles are staged in LDS as float32, in rows split into
// quarters padded by 4 floats so the four lanes' 16-byte reads fall in
// different banks.  Softmax is online in float32 with max subtraction; the
// output is accumulated in float32.
#include "common.h"
#include "launch.h"

namespace kvc {

template <class In>
__device__ __forceinline__ float ld_f32(const In* p, size_t i) {
  return to_f32<In>(p[i]);
}

// V1 is float32 (fitted values) when V1F32, else the input type.
template <class In, int D, bool V1F32>
__global__ __launch_bounds__(256) void k_attend(const In* __restrict__ Q, const In* __restrict__ K1,
                                                const float* __restrict__ bias,
                                                const void* __restrict__ V1v,
                                                const In* __restrict__ K2,
                                                const In* __restrict__ V2,
                                                float* __restrict__ out,
                                                double* __restrict__ out_lse,
                                                float2* __restrict__ pml,
                                                float* __restrict__ po, int m, int t1, int t2,
                                                int kps) {
  constexpr int BN = 64, DQ = D / 4, SEG = DQ + 4, ROW = 4 * SEG;
  __shared__ __align__(16) float sK[BN * ROW];
  __shared__ __align__(16) float sV[BN * ROW];
  __shared__ float sB[BN];
  const int b = blockIdx.z, split = blockIdx.y, nsplit = gridDim.y, tid = threadIdx.x;
  const int qi = blockIdx.x * 64 + (tid >> 2), part = tid & 3;
  const bool qok = qi < m;
  const In* Qb = Q + static_cast<size_t>(b) * m * D;
  float qv[DQ], o[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    qv[c] = qok ? ld_f32(Qb, static_cast<size_t>(qi) * D + part * DQ + c) : 0.f;
    o[c] = 0.f;
  }
  float mx = -INFINITY, l = 0.f;
  const int tot = min(t1 + t2, (split + 1) * kps);
  for (int j0 = split * kps; j0 < tot; j0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += 256) {
      const int r = e / D, c = e % D, j = j0 + r;
      float kv = 0.f, vv = 0.f;
      if (j < t1) {
        const size_t at = (static_cast<size_t>(b) * t1 + j) * D + c;
        kv = ld_f32(K1, at);
        vv = V1F32 ? static_cast<const float*>(V1v)[at] : ld_f32(static_cast<const In*>(V1v), at);
      } else if (j < tot) {
        const size_t at = (static_cast<size_t>(b) * t2 + (j - t1)) * D + c;
        kv = ld_f32(K2, at);
        vv = ld_f32(V2, at);
      }
      const int pos = r * ROW + (c / DQ) * SEG + c % DQ;
      sK[pos] = kv;
      sV[pos] = vv;
    }
    for (int r = tid; r < BN; r += 256) {
      const int j = j0 + r;
      sB[r] = j < t1 ? (bias ? bias[static_cast<size_t>(b) * t1 + j] : 0.f) : 0.f;
    }
    __syncthreads();
    const int nk = min(BN, tot - j0);
    for (int r = 0; r < nk; ++r) {
      const float* kr = &sK[r * ROW + part * SEG];
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; c += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(kr + c);
        s = fmaf(qv[c], k4.x, s);
        s = fmaf(qv[c + 1], k4.y, s);
        s = fmaf(qv[c + 2], k4.z, s);
        s = fmaf(qv[c + 3], k4.w, s);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += sB[r];
      if (s == -INFINITY) continue;  // a key with bias -inf has weight zero
      if (s > mx) {
        const float sc = mx == -INFINITY ? 0.f : __expf(mx - s);
        l *= sc;
#pragma unroll
        for (int c = 0; c < DQ; ++c) o[c] *= sc;
        mx = s;
      }
      const float p = __expf(s - mx);
      l += p;
      const float* vr = &sV[r * ROW + part * SEG];
#pragma unroll
      for (int c = 0; c < DQ; c += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(vr + c);
        o[c] = fmaf(p, v4.x, o[c]);
        o[c + 1] = fmaf(p, v4.y, o[c + 1]);
        o[c + 2] = fmaf(p, v4.z, o[c + 2]);
        o[c + 3] = fmaf(p, v4.w, o[c + 3]);
      }
    }
  }
  if (nsplit > 1) {
    if (qok) {
      const size_t row = (static_cast<size_t>(b) * nsplit + split) * m + qi;
      float* ob = po + row * D + part * DQ;
#pragma unroll
      for (int c = 0; c < DQ; ++c) ob[c] = o[c];
      if (part == 0) pml[row] = make_float2(mx, l);
    }
    return;
  }
  if (qok) {
    const float inv = 1.f / l;
    float* ob = out + (static_cast<size_t>(b) * m + qi) * D + part * DQ;
#pragma unroll
    for (int c = 0; c < DQ; ++c) ob[c] = o[c] * inv;
    if (out_lse && part == 0)
      out_lse[static_cast<size_t>(b) * m + qi] = static_cast<double>(mx) + log(static_cast<double>(l));
  }
}

// Combine the key splits of each query in split order: M = max of the split
// maxima, L = sum l_s exp(m_s - M), out = sum o_s exp(m_s - M) / L,
// lse = M + log L.  grid (ceil(m*D/256), B), block 256.
template <int D>
__global__ void k_attend_merge(const float2* __restrict__ pml, const float* __restrict__ po,
                               float* __restrict__ out, double* __restrict__ out_lse, int m,
                               int nsplit) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m * D) return;
  const int qi = e / D, c = e % D;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    M = fmaxf(M, pml[(static_cast<size_t>(b) * nsplit + s) * m + qi].x);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const size_t row = (static_cast<size_t>(b) * nsplit + s) * m + qi;
    const float2 v = pml[row];
    if (v.x == -INFINITY) continue;
    const float w = __expf(v.x - M);
    L = fmaf(v.y, w, L);
    o = fmaf(po[row * D + c], w, o);
  }
  out[(static_cast<size_t>(b) * m + qi) * D + c] = o / L;
  if (out_lse && c == 0)
    out_lse[static_cast<size_t>(b) * m + qi] = static_cast<double>(M) + log(static_cast<double>(L));
}

// Splits for (m, keys, B): whole 64-key tiles, ~2048 workgroups.
void attend_plan(int B, int m, int keys, int& nsplit, int& kps) {
  const int mb = (m + 63) / 64, tiles = (keys + 63) / 64;
  int want = (2048 + mb * B - 1) / (mb * B);
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  kps = (tiles + want - 1) / want * 64;
  nsplit = (keys + kps - 1) / kps;
}

size_t attend_ws_bytes(int B, int m, int keys, int D) {
  int nsplit, kps;
  attend_plan(B, m, keys, nsplit, kps);
  if (nsplit <= 1) return 0;
  const size_t rows = static_cast<size_t>(B) * nsplit * m;
  return (rows * 8 + 255) / 256 * 256 + rows * D * 4;
}

template <class In, int D>
hipError_t launch_attend(const void* Q, const void* K1, const float* bias, const void* V1,
                         bool v1_f32, const void* K2, const void* V2, float* out,
                         double* out_lse, void* ws, int B, int m, int t1, int t2,
                         hipStream_t st) {
  int nsplit, kps;
  attend_plan(B, m, t1 + t2, nsplit, kps);
  const size_t rows = static_cast<size_t>(B) * nsplit * m;
  float2* pml = static_cast<float2*>(ws);
  float* po = reinterpret_cast<float*>(static_cast<char*>(ws) + (rows * 8 + 255) / 256 * 256);
  const dim3 grid((m + 63) / 64, nsplit, B);
  const In* q = static_cast<const In*>(Q);
  const In* k1 = static_cast<const In*>(K1);
  const In* k2 = static_cast<const In*>(K2);
  const In* v2 = static_cast<const In*>(V2);
  if (v1_f32)
    hipLaunchKernelGGL((k_attend<In, D, true>), grid, dim3(256), 0, st, q, k1, bias, V1, k2, v2,
                       out, out_lse, pml, po, m, t1, t2, kps);
  else
    hipLaunchKernelGGL((k_attend<In, D, false>), grid, dim3(256), 0, st, q, k1, bias, V1, k2, v2,
                       out, out_lse, pml, po, m, t1, t2, kps);
  if (nsplit > 1)
    hipLaunchKernelGGL((k_attend_merge<D>), dim3((m * D + 255) / 256, B), dim3(256), 0, st, pml,
                       po, out, out_lse, m, nsplit);
  return hipGetLastError();
}

#define KVC_INST_ATTEND(In, D)                                                              \
  template hipError_t launch_attend<In, D>(const void*, const void*, const float*,          \
                                           const void*, bool, const void*, const void*,     \
                                           float*, double*, void*, int, int, int, int,      \
                                           hipStream_t);
KVC_INST_ATTEND(bf16_t, 128)
KVC_INST_ATTEND(bf16_t, 64)
KVC_INST_ATTEND(float, 128)
KVC_INST_ATTEND(float, 64)

}  // namespace kvc
