// Host side of the C ABI declared in include/kvc.h: argument checks,
// workspace layout and the launch sequence on the caller's stream.
//
// Pipeline ("Fast KV Compaction via Attention Matching", section 2): scores
// and log-sum-exp over the full cache, full-cache output and per-key
// importance, top-t selection of original keys, NNLS bias fit on the relative
// attention mass, least-squares value fit.  Nothing here allocates device
// memory or synchronises with the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/kvc.h"

#include "launch.h"

namespace {

struct ProfState {
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev[KVC_NUM_STAGES];  // start, stop, start, stop, ...
  size_t used[KVC_NUM_STAGES] = {};
};
ProfState g_prof;

// bound on each wait of a fit team (100 MHz ticks); kvc_set_wait_limit
constexpr uint64_t kDefaultWaitTicks = 2000000000ull;
uint64_t g_wait_ticks = kDefaultWaitTicks;

}  // namespace

namespace kvc {
void prof_mark(int stage, bool end, hipStream_t st) {
  if (!(g_prof.mask & (1u << stage))) return;
  auto& v = g_prof.ev[stage];
  size_t& u = g_prof.used[stage];
  if (!end && (u & 1)) return;  // unmatched start: ignore
  if (end && !(u & 1)) return;
  if (u == v.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    v.push_back(e);
  }
  if (hipEventRecord(v[u], st) == hipSuccess) ++u;
}
}  // namespace kvc

namespace {

constexpr int64_t kMaxT = 1 << 30;
constexpr int64_t kMaxT_keep = 4096;  // the fit kernels stage t values in LDS
constexpr int64_t kMaxB = 65535;
constexpr int kMaxRefine = 4;  // value-fit refinement steps
constexpr int kBM = 128;  // reference queries per score workgroup

struct Plan {
  int nqb, nsplit1, kps1, nsplit2, kps2;
};

// Split the key range so the score grid has about `target` workgroups;
// splits are a multiple of 64 keys (a whole number of tiles).
void split_keys(int64_t T, int64_t work_per_split, int64_t target, int& nsplit, int& kps) {
  int64_t want = (target + work_per_split - 1) / work_per_split;
  int64_t maxs = T / 512 > 0 ? T / 512 : 1;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  int64_t per = (T + want - 1) / want;
  per = (per + 63) / 64 * 64;
  kps = static_cast<int>(per);
  nsplit = static_cast<int>((T + per - 1) / per);
}

Plan make_plan(const kvc_params_t* p) {
  Plan pl;
  pl.nqb = static_cast<int>((p->n + kBM - 1) / kBM);
  // K1's partials are one (max, sum) pair per query and split, so it takes
  // ~4 rounds of its 3-workgroups-per-CU residency (a short tail); K2's carry
  // a d x n output slice per split, so it keeps ~1024 workgroups (two full
  // rounds at 2 per CU)
  split_keys(p->T, static_cast<int64_t>(pl.nqb) * p->B, 3072, pl.nsplit1, pl.kps1);
  split_keys(p->T, static_cast<int64_t>(pl.nqb) * p->B, 1024, pl.nsplit2, pl.kps2);
  return pl;
}

struct Layout {
  size_t ml, lse, Opart, O, imp_part, imp, sel, idx, status, tv, emask, plist, PS, S, U, V, stage, cvec, wv, lam,
      colpart, Fidx, inv, msz, bar, xcc, flops, part, E, Rp, Cn, total;
  size_t part_cap;
  // greedy selection only (zero otherwise)
  size_t P32, o_nrm, o_r, o_chosen, o_part, o_order, o_a, o_Q, o_h, o_q, o_part2;
};

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

Layout make_layout(const kvc_params_t* p, bool omp = false) {
  const Plan pl = make_plan(p);
  const size_t B = p->B, T = p->T, n = p->n, d = p->d, t = p->t;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.ml = take(B * pl.nsplit1 * n * 16);
  L.lse = take(B * n * 8);
  L.Opart = take(B * pl.nsplit2 * d * n * 4);
  L.O = take(B * n * d * 4);
  L.imp_part = take(B * pl.nqb * T * 4);
  L.imp = take(B * T * 4);
  L.sel = take(B * kvc::sel_words(static_cast<int>(T)) * 4);
  L.idx = take(B * t * 4);
  L.status = take(B * 4);
  L.tv = take(B * 4);
  L.emask = take(B * T);
  L.plist = take(B * t * 4);
  L.PS = take(B * n * t * 8);
  {
    const size_t ld = static_cast<size_t>(kvc::sweep_ld(static_cast<int>(t), static_cast<int>(d)));
    L.S = take(B * ld * ld * 8);
    L.U = take(B * ld * 64 * 8);
    L.V = take(B * ld * 64 * 8);
  }
  L.stage = take(B * static_cast<size_t>(kvc::kSweepStage) * 8);
  L.cvec = take(B * t * 8);
  L.wv = take(B * t * 8);
  L.lam = take(B * 2 * 8);
  L.colpart = take(B * ((n + 63) / 64) * t * 8);
  L.Fidx = take(B * t * 4);
  L.inv = take(B * t * 4);
  L.msz = take(B * 4);
  L.bar = take(static_cast<size_t>(kvc::kBarWords) * 4);
  L.xcc = take(static_cast<size_t>(kvc::kMaxTeamGrid) * 4);
  L.flops = take(B * 2 * 8);
  // split-K partials: up to 2048 * 4 tile slices of 64 x 64 doubles, never
  // more than the (already needed) t x t matrix per head times 4
  {
    size_t cap = static_cast<size_t>(8192) * 64 * 64;
    const size_t lim = 4 * B * t * t + 64 * 64;
    L.part_cap = cap < lim ? cap : lim;
    L.part = take(L.part_cap * 8);
  }
  // value-fit refinement: the residual, X_F^T of it and the refined solution
  if (p->refine_steps > 0) {
    L.E = take(B * n * d * 8);
    L.Rp = take(B * t * d * 8);
    L.Cn = take(B * t * d * 8);
  }
  if (omp) {
    L.P32 = take(B * n * T * 4);
    L.o_nrm = take(B * T * 8);
    L.o_r = take(B * n * 8);
    L.o_chosen = take(B * T);
    L.o_part = take(B * ((T + 1023) / 1024) * 16);
    L.o_order = take(B * t * 4);
    L.o_a = take(B * n * 8);
    L.o_Q = take(B * t * n * 8);
    L.o_h = take(B * t * 8);
    L.o_q = take(B * n * 8);
    L.o_part2 = take(B * ((n + 255) / 256) * 16);
  }
  L.total = off;
  return L;
}

bool params_ok(const kvc_params_t* p) {
  if (!p) return false;
  if (p->B < 1 || p->B > kMaxB) return false;
  if (p->T < 1 || p->T > kMaxT) return false;
  if (p->n < 1 || p->n > kMaxT) return false;
  if (p->d != 64 && p->d != 128) return false;
  if (p->t < 1 || p->t > p->T || p->t > kMaxT_keep) return false;
  if (p->in_dtype != KVC_F32 && p->in_dtype != KVC_BF16) return false;
  if (p->agg != KVC_AGG_RMS && p->agg != KVC_AGG_MEAN) return false;
  if (!(p->ridge_rel >= 0.0) || !std::isfinite(p->ridge_rel)) return false;
  if (p->max_nnls_iters < 1 || p->max_nnls_iters > 1000) return false;
  if (p->out_v_dtype != KVC_F32 && p->out_v_dtype != KVC_BF16) return false;
  if (p->refine_steps < 0 || p->refine_steps > kMaxRefine) return false;
  if (p->reserved != 0) return false;
  return true;
}

bool aligned(const void* ptr) { return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

kvc::FitBufs fit_bufs(void* ws, const Layout& L) {
  kvc::FitBufs fb;
  fb.PS = at<double>(ws, L.PS);
  fb.S = at<double>(ws, L.S);
  fb.U = at<double>(ws, L.U);
  fb.V = at<double>(ws, L.V);
  fb.stage = at<double>(ws, L.stage);
  fb.cvec = at<double>(ws, L.cvec);
  fb.wv = at<double>(ws, L.wv);
  fb.lam = at<double>(ws, L.lam);
  fb.colpart = at<double>(ws, L.colpart);
  fb.bar = at<unsigned>(ws, L.bar);
  fb.xcc = at<int32_t>(ws, L.xcc);
  fb.flops = at<double>(ws, L.flops);
  fb.part = at<double>(ws, L.part);
  fb.part_cap = L.part_cap;
  fb.Fidx = at<int32_t>(ws, L.Fidx);
  fb.inv = at<int32_t>(ws, L.inv);
  fb.msz = at<int32_t>(ws, L.msz);
  fb.tv = nullptr;
  fb.refine = 0;
  fb.E = fb.Rp = fb.Cn = nullptr;
  if (L.E) {
    fb.E = at<double>(ws, L.E);
    fb.Rp = at<double>(ws, L.Rp);
    fb.Cn = at<double>(ws, L.Cn);
  }
  return fb;
}

// qg: batch entries per reference-query set.  Entry b reads Q_ref[b / qg]
// (chunked compaction runs every chunk of a head against that head's queries).
template <class In, int D>
hipError_t run_score(const kvc_params_t* p, const void* Q, const void* K, const void* V,
                     void* ws, const Layout& L, int qg, const uint8_t* mask, int32_t* status,
                     hipStream_t st) {
  const Plan pl = make_plan(p);
  return kvc::launch_score<In, D>(Q, K, V, at<double2>(ws, L.ml), at<double>(ws, L.lse),
                                  at<float>(ws, L.Opart), at<float>(ws, L.O),
                                  at<float>(ws, L.imp_part), at<float>(ws, L.imp),
                                  at<uint32_t>(ws, L.sel), status,
                                  static_cast<int>(p->B), static_cast<int>(p->n),
                                  static_cast<int>(p->T), pl.nsplit1, pl.kps1, pl.nsplit2,
                                  pl.kps2, p->agg == KVC_AGG_RMS, qg, mask, st);
}

template <class In, int D>
hipError_t run_fit(const kvc_params_t* p, const void* Q, const void* K, const void* V,
                   const int32_t* idx, float* out_bias, void* out_V, int32_t* status, void* ws,
                   const Layout& L, int qg, const int32_t* tv, hipStream_t st) {
  kvc::FitBufs fb = fit_bufs(ws, L);
  fb.tv = tv;
  fb.wait_ticks = g_wait_ticks;
  fb.refine = p->refine_steps;
  return kvc::launch_fit<In, D>(Q, K, V, at<double>(ws, L.lse), at<float>(ws, L.O), idx,
                                fb, out_bias, out_V, p->out_v_dtype == KVC_BF16, status,
                                static_cast<int>(p->B), static_cast<int>(p->n),
                                static_cast<int>(p->T), static_cast<int>(p->t), p->ridge_rel,
                                p->max_nnls_iters, qg, st);
}

// Dispatch on (dtype, head dim).
template <template <class, int> class F, class... A>
hipError_t dispatch(const kvc_params_t* p, A... args) {
  if (p->in_dtype == KVC_BF16) {
    if (p->d == 128) return F<kvc::bf16_t, 128>::run(p, args...);
    return F<kvc::bf16_t, 64>::run(p, args...);
  }
  if (p->d == 128) return F<float, 128>::run(p, args...);
  return F<float, 64>::run(p, args...);
}

template <class In, int D>
struct ScoreOp {
  static hipError_t run(const kvc_params_t* p, const void* Q, const void* K, const void* V,
                        void* ws, const Layout* L, int qg, const uint8_t* mask,
                        int32_t* status, hipStream_t st) {
    return run_score<In, D>(p, Q, K, V, ws, *L, qg, mask, status, st);
  }
};
template <class In, int D>
struct FitOp {
  static hipError_t run(const kvc_params_t* p, const void* Q, const void* K, const void* V,
                        const int32_t* idx, float* ob, void* ov, int32_t* status, void* ws,
                        const Layout* L, int qg, const int32_t* tv, hipStream_t st) {
    return run_fit<In, D>(p, Q, K, V, idx, ob, ov, status, ws, *L, qg, tv, st);
  }
};

template <class In, int D>
struct ProbsOp {
  static hipError_t run(const kvc_params_t* p, const void* Q, const void* K, const double* lse,
                        float* P, hipStream_t st) {
    return kvc::launch_probs_all<In, D>(Q, K, lse, P, static_cast<int>(p->B),
                                        static_cast<int>(p->n), static_cast<int>(p->T), 1, st);
  }
};

kvc::OmpBufs omp_bufs(void* ws, const Layout& L) {
  kvc::OmpBufs ob;
  ob.nrm = at<double>(ws, L.o_nrm);
  ob.r = at<double>(ws, L.o_r);
  ob.chosen = at<uint8_t>(ws, L.o_chosen);
  ob.part = at<double2>(ws, L.o_part);
  ob.order = at<int32_t>(ws, L.o_order);
  ob.a = at<double>(ws, L.o_a);
  ob.Q = at<double>(ws, L.o_Q);
  ob.h = at<double>(ws, L.o_h);
  ob.q = at<double>(ws, L.o_q);
  ob.part2 = at<double2>(ws, L.o_part2);
  return ob;
}

int common_checks(const kvc_params_t* p, const void* Q, const void* K, const void* V,
                  const void* out_bias, const void* out_V, void* ws, size_t ws_bytes) {
  if (!params_ok(p)) return KVC_EINVAL;
  if (!aligned(Q) || !aligned(K) || !aligned(V) || !aligned(out_bias) || !aligned(out_V) ||
      !aligned(ws))
    return KVC_EINVAL;
  if (ws_bytes < make_layout(p).total) return KVC_EWORKSPACE;
  return KVC_OK;
}

// Chunked compaction as a batch: entry b' = head * C + chunk is the chunk's
// T / C contiguous keys (a view of the head's K and V, no copy) with the same
// per-entry budget t.  False when the split is not representable.
bool chunk_params(const kvc_params_t* p, int64_t C, kvc_params_t* out) {
  if (!p || C < 1 || C > kMaxB) return false;
  if (p->T < 1 || p->T % C != 0) return false;
  *out = *p;
  out->B = p->B * C;
  out->T = p->T / C;
  return params_ok(out) && p->B >= 1;
}

// Select, gather and fit for every batch entry of p; qg as in run_score;
// t_in: per-entry budgets (device) or null for p->t everywhere; protect: the
// caller's protected-key mask [B][T] (device) or null.
int compact_impl(const kvc_params_t* p, int qg, const int32_t* t_in, const uint8_t* protect,
                 const void* Q_ref, const void* K, const void* V, void* out_K, float* out_bias,
                 void* out_V, int32_t* out_idx, int32_t* out_status, void* workspace,
                 hipStream_t stream, bool omp = false) {
  const Layout L = make_layout(p, omp);
  int32_t* idx = out_idx ? out_idx : at<int32_t>(workspace, L.idx);
  int32_t* status = out_status ? out_status : at<int32_t>(workspace, L.status);
  const int B = static_cast<int>(p->B), T = static_cast<int>(p->T), t = static_cast<int>(p->t);
  const int es = p->in_dtype == KVC_BF16 ? 2 : 4;
  kvc::prof_mark(KVC_STAGE_TOTAL, false, stream);
  hipError_t e = kvc::launch_fill_i32(status, 0, p->B, stream);
  int32_t* tv = nullptr;
  const uint8_t* emask = nullptr;
  int32_t* plist = at<int32_t>(workspace, L.plist);
  if (t_in) {
    tv = at<int32_t>(workspace, L.tv);
    if (e == hipSuccess) e = kvc::launch_budgets(t_in, tv, status, B, t, stream);
  } else if (protect) {
    tv = at<int32_t>(workspace, L.tv);
    uint8_t* em = at<uint8_t>(workspace, L.emask);
    emask = em;
    if (e == hipSuccess) e = kvc::launch_protect_prep(protect, em, plist, tv, status, B, T, t, stream);
  }
  if (e == hipSuccess)
    e = dispatch<ScoreOp>(p, Q_ref, K, V, workspace, &L, qg, emask, status, stream);
  kvc::prof_mark(KVC_STAGE_SELECT, false, stream);
  if (e == hipSuccess && omp) {
    float* P32 = at<float>(workspace, L.P32);
    e = dispatch<ProbsOp>(p, Q_ref, K, static_cast<const double*>(at<double>(workspace, L.lse)),
                          P32, stream);
    if (e == hipSuccess)
      e = kvc::launch_omp(P32, omp_bufs(workspace, L), idx, B, static_cast<int>(p->n), T, t,
                          stream);
  } else if (e == hipSuccess) {
    kvc::prof_mark(KVC_STAGE_TOPT, false, stream);
    e = kvc::launch_select(at<float>(workspace, L.imp), at<uint32_t>(workspace, L.sel), idx, tv,
                           emask, B, T, t, stream);
    kvc::prof_mark(KVC_STAGE_TOPT, true, stream);
  }
  kvc::prof_mark(KVC_STAGE_GATHER, false, stream);
  if (e == hipSuccess)
    e = kvc::launch_gather(K, idx, out_K, B, T, t, static_cast<int>(p->d) * es, stream);
  kvc::prof_mark(KVC_STAGE_GATHER, true, stream);
  kvc::prof_mark(KVC_STAGE_SELECT, true, stream);
  if (e == hipSuccess)
    e = dispatch<FitOp>(p, Q_ref, K, V, static_cast<const int32_t*>(idx), out_bias, out_V,
                        status, workspace, &L, qg, tv, stream);
  if (e == hipSuccess && protect)
    e = kvc::launch_fill_protected(plist, tv, K, V, out_K, out_V, out_bias, idx, B, T, t,
                                   static_cast<int>(p->d), p->in_dtype == KVC_BF16,
                                   p->out_v_dtype == KVC_BF16, stream);
  if (e == hipSuccess && qg > 1 && out_idx)
    e = kvc::launch_idx_offset(out_idx, B, t, qg, T, stream);
  kvc::prof_mark(KVC_STAGE_TOTAL, true, stream);
  return e == hipSuccess ? KVC_OK : KVC_EHIP;
}

}  // namespace

extern "C" {

void kvc_params_default(kvc_params_t* p) {
  if (!p) return;
  std::memset(p, 0, sizeof(*p));
  p->in_dtype = KVC_BF16;
  p->agg = KVC_AGG_RMS;
  p->ridge_rel = 1e-6;
  p->max_nnls_iters = 32;
  p->out_v_dtype = KVC_F32;
  p->refine_steps = 0;
  p->reserved = 0;
}

size_t kvc_workspace_bytes(const kvc_params_t* p) {
  if (!params_ok(p)) return 0;
  return make_layout(p).total;
}

int kvc_workspace_layout(const kvc_params_t* p, kvc_ws_layout_t* out) {
  if (!params_ok(p) || !out) return KVC_EINVAL;
  const Layout L = make_layout(p);
  out->lse = L.lse;
  out->O = L.O;
  out->imp = L.imp;
  out->w = L.wv;
  out->fit_flops = L.flops;
  out->omp_order = make_layout(p, true).o_order;
  {
    const size_t ld = static_cast<size_t>(kvc::sweep_ld(static_cast<int>(p->t), static_cast<int>(p->d)));
    const size_t rv = (static_cast<size_t>(p->d) + 63) / 64 * 64;  // right-hand-side rows
    out->value_C = L.S + rv * ld * 8;
    out->value_ld = ld;
  }
  return KVC_OK;
}

int kvc_compact(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
                void* out_K, float* out_bias, void* out_V, int32_t* out_idx,
                int32_t* out_status, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  int rc = common_checks(p, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (!aligned(out_K) || (out_idx && !aligned(out_idx)) || (out_status && !aligned(out_status)))
    return KVC_EINVAL;
  return compact_impl(p, 1, nullptr, nullptr, Q_ref, K, V, out_K, out_bias, out_V, out_idx,
                      out_status, workspace, stream);
}

size_t kvc_workspace_bytes_omp(const kvc_params_t* p) {
  if (!params_ok(p)) return 0;
  return make_layout(p, true).total;
}

int kvc_compact_omp(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
                    void* out_K, float* out_bias, void* out_V, int32_t* out_idx,
                    int32_t* out_status, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  int rc = common_checks(p, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (workspace_bytes < make_layout(p, true).total) return KVC_EWORKSPACE;
  if (!aligned(out_K) || (out_idx && !aligned(out_idx)) || (out_status && !aligned(out_status)))
    return KVC_EINVAL;
  return compact_impl(p, 1, nullptr, nullptr, Q_ref, K, V, out_K, out_bias, out_V, out_idx,
                      out_status, workspace, stream, true);
}

int kvc_compact_protected(const kvc_params_t* p, const uint8_t* protect_mask, const void* Q_ref,
                          const void* K, const void* V, void* out_K, float* out_bias,
                          void* out_V, int32_t* out_idx, int32_t* out_status, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int rc = common_checks(p, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (!protect_mask || !aligned(out_K) || (out_idx && !aligned(out_idx)) ||
      (out_status && !aligned(out_status)))
    return KVC_EINVAL;
  return compact_impl(p, 1, nullptr, protect_mask, Q_ref, K, V, out_K, out_bias, out_V, out_idx,
                      out_status, workspace, stream);
}

int kvc_compact_ragged(const kvc_params_t* p, const int32_t* t_heads, const void* Q_ref,
                       const void* K, const void* V, void* out_K, float* out_bias, void* out_V,
                       int32_t* out_idx, int32_t* out_status, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int rc = common_checks(p, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (!t_heads || (reinterpret_cast<uintptr_t>(t_heads) & 3u) || !aligned(out_K) ||
      (out_idx && !aligned(out_idx)) || (out_status && !aligned(out_status)))
    return KVC_EINVAL;
  return compact_impl(p, 1, t_heads, nullptr, Q_ref, K, V, out_K, out_bias, out_V, out_idx,
                      out_status, workspace, stream);
}

size_t kvc_workspace_bytes_chunked(const kvc_params_t* p, int64_t n_chunks) {
  kvc_params_t pc;
  if (!chunk_params(p, n_chunks, &pc)) return 0;
  return make_layout(&pc).total;
}

int kvc_compact_chunked(const kvc_params_t* p, int64_t n_chunks, const void* Q_ref,
                        const void* K, const void* V, void* out_K, float* out_bias, void* out_V,
                        int32_t* out_idx, int32_t* out_status, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  kvc_params_t pc;
  if (!chunk_params(p, n_chunks, &pc)) return KVC_EINVAL;
  int rc = common_checks(&pc, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (!aligned(out_K) || (out_idx && !aligned(out_idx)) || (out_status && !aligned(out_status)))
    return KVC_EINVAL;
  return compact_impl(&pc, static_cast<int>(n_chunks), nullptr, nullptr, Q_ref, K, V, out_K,
                      out_bias, out_V, out_idx, out_status, workspace, stream);
}

int kvc_fit(const kvc_params_t* p, const void* Q_ref, const void* K, const void* V,
            const int32_t* idx, float* out_bias, void* out_V, int32_t* out_status,
            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = common_checks(p, Q_ref, K, V, out_bias, out_V, workspace, workspace_bytes);
  if (rc) return rc;
  if (!aligned(idx) || (out_status && !aligned(out_status))) return KVC_EINVAL;
  const Layout L = make_layout(p);
  int32_t* status = out_status ? out_status : at<int32_t>(workspace, L.status);
  kvc::prof_mark(KVC_STAGE_TOTAL, false, stream);
  hipError_t e = kvc::launch_fill_i32(status, 0, p->B, stream);
  if (e == hipSuccess)
    e = dispatch<ScoreOp>(p, Q_ref, K, V, workspace, &L, 1, static_cast<const uint8_t*>(nullptr),
                          status, stream);
  if (e == hipSuccess)
    e = dispatch<FitOp>(p, Q_ref, K, V, idx, out_bias, out_V, status, workspace, &L, 1,
                        static_cast<const int32_t*>(nullptr), stream);
  kvc::prof_mark(KVC_STAGE_TOTAL, true, stream);
  return e == hipSuccess ? KVC_OK : KVC_EHIP;
}

static bool attend_ok(const kvc_attend_params_t* p) {
  if (!p || p->B < 1 || p->B > kMaxB || p->m < 1 || p->m > kMaxT || (p->d != 64 && p->d != 128))
    return false;
  if (p->t1 < 0 || p->t2 < 0 || p->t1 + p->t2 < 1 || p->t1 + p->t2 > kMaxT) return false;
  if (p->in_dtype != KVC_F32 && p->in_dtype != KVC_BF16) return false;
  if ((p->v1_f32 != 0 && p->v1_f32 != 1) || p->reserved != 0 || p->reserved2 != 0) return false;
  return true;
}

size_t kvc_attend_workspace_bytes(const kvc_attend_params_t* p) {
  if (!attend_ok(p)) return 0;
  return kvc::attend_ws_bytes(static_cast<int>(p->B), static_cast<int>(p->m),
                              static_cast<int>(p->t1 + p->t2), static_cast<int>(p->d));
}

int kvc_attend(const kvc_attend_params_t* p, const void* Q, const void* K1, const float* bias1,
               const void* V1, const void* K2, const void* V2, float* out, double* out_lse,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!attend_ok(p)) return KVC_EINVAL;
  const size_t need = kvc_attend_workspace_bytes(p);
  if (need > 0 && (!workspace || !aligned(workspace))) return KVC_EINVAL;
  if (workspace_bytes < need) return KVC_EWORKSPACE;
  if (!aligned(Q) || !aligned(out) || (out_lse && !aligned(out_lse))) return KVC_EINVAL;
  if (p->t1 > 0 && (!aligned(K1) || !aligned(V1) || (bias1 && !aligned(bias1)))) return KVC_EINVAL;
  if (p->t2 > 0 && (!aligned(K2) || !aligned(V2))) return KVC_EINVAL;
  const int B = static_cast<int>(p->B), m = static_cast<int>(p->m);
  const int t1 = static_cast<int>(p->t1), t2 = static_cast<int>(p->t2);
  const bool v1f = p->v1_f32 != 0;
  hipError_t e;
  if (p->in_dtype == KVC_BF16)
    e = p->d == 128 ? kvc::launch_attend<kvc::bf16_t, 128>(Q, K1, bias1, V1, v1f, K2, V2, out,
                                                           out_lse, workspace, B, m, t1, t2,
                                                           stream)
                    : kvc::launch_attend<kvc::bf16_t, 64>(Q, K1, bias1, V1, v1f, K2, V2, out,
                                                          out_lse, workspace, B, m, t1, t2,
                                                          stream);
  else
    e = p->d == 128 ? kvc::launch_attend<float, 128>(Q, K1, bias1, V1, v1f, K2, V2, out, out_lse,
                                                     workspace, B, m, t1, t2, stream)
                    : kvc::launch_attend<float, 64>(Q, K1, bias1, V1, v1f, K2, V2, out, out_lse,
                                                    workspace, B, m, t1, t2, stream);
  return e == hipSuccess ? KVC_OK : KVC_EHIP;
}

int kvc_set_wait_limit(uint64_t ticks) {
  g_wait_ticks = ticks == 0 ? kDefaultWaitTicks : ticks;
  return KVC_OK;
}

int kvc_profile_enable(uint32_t stage_mask) {
  g_prof.mask = stage_mask & ((1u << KVC_NUM_STAGES) - 1);
  for (int s = 0; s < KVC_NUM_STAGES; ++s) {
    g_prof.used[s] = 0;
    if (g_prof.mask == 0) {  // off: release the events (none outlive their use)
      for (hipEvent_t e : g_prof.ev[s]) (void)hipEventDestroy(e);
      g_prof.ev[s].clear();
    }
  }
  return KVC_OK;
}

int kvc_profile_read(int stage, double* total_ms, int64_t* launches) {
  if (stage < 0 || stage >= KVC_NUM_STAGES || !total_ms || !launches) return KVC_EINVAL;
  const auto& v = g_prof.ev[stage];
  const size_t pairs = g_prof.used[stage] / 2;
  double sum = 0.0;
  for (size_t i = 0; i < pairs; ++i) {
    if (hipEventSynchronize(v[2 * i + 1]) != hipSuccess) return KVC_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, v[2 * i], v[2 * i + 1]) != hipSuccess) return KVC_EHIP;
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(pairs);
  return KVC_OK;
}

const char* kvc_strerror(int code) {
  switch (code) {
    case KVC_OK: return "ok";
    case KVC_EINVAL: return "invalid argument (null/misaligned pointer, bad size or enum)";
    case KVC_EWORKSPACE: return "workspace smaller than kvc_workspace_bytes()";
    case KVC_EHIP: return "HIP launch failed";
    case KVC_EUNSUPPORTED: return "unsupported configuration";
    default: return "unknown error code";
  }
}

}  // extern "C"
