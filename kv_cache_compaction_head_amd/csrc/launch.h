// Host-callable launchers of the kernels (each enqueues on the given stream
// and returns hipGetLastError()).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {
using bf16_t = uint16_t;

// Selection state of a head, sel_words(T) uint32 words in the workspace: the
// histograms of the radix select's three digits (bits 31-21, 20-10, 9-0 of
// the ranking key), the threshold key tau and how many keys equal to it are
// kept, then per chunk of kSelChunk keys its counts above and equal to tau.
constexpr int kSelChunk = 4096;
constexpr int kSelH1 = 2048, kSelH2 = 2048, kSelH3 = 1024;
constexpr int kSelTau = kSelH1 + kSelH2 + kSelH3;  // tau, then need_eq
constexpr int kSelCnt = kSelTau + 2;               // [chunk][2]: above, equal
inline int sel_chunks(int T) { return (T + kSelChunk - 1) / kSelChunk; }
inline size_t sel_words(int T) {
  return (kSelCnt + 2 * static_cast<size_t>(sel_chunks(T)) + 63) / 64 * 64;
}

// The score path; its importance reduction also runs the selection's first
// pass into sel (which the lse merge clears first) from the ranking keys
// (mask: keys never selected, or null; status |= 4 for a non-finite
// importance).
template <class In, int D>
hipError_t launch_score(const void* Q, const void* K, const void* V, double2* ml, double* lse,
                        float* Opart, float* O, float* imp_part, float* imp, uint32_t* sel,
                        int32_t* status, int B, int n, int T, int nsplit1, int kps1,
                        int nsplit2, int kps2, bool rms, int qg, const uint8_t* mask,
                        hipStream_t st);
// The rest of the top-t selection, after launch_score.  tv: per-head budgets
// (device, each in [1, t]) or null for t everywhere; mask: [B][T] keys never
// selected (nonzero), or null (the one given to launch_score).
hipError_t launch_select(const float* imp, uint32_t* sel, int32_t* idx, const int32_t* tv,
                         const uint8_t* mask, int B, int T, int t, hipStream_t st);
// Protected keys: from the caller's mask [B][T], per head the first (by
// position) pp_b = min(count, t - 1) protected keys are listed in plist [B][t]
// and marked in emask [B][T] (the rest of the mask is dropped, status |= 32);
// tv[b] = t - pp_b is the budget left for the fitted keys.
hipError_t launch_protect_prep(const uint8_t* mask, uint8_t* emask, int32_t* plist, int32_t* tv,
                               int32_t* status, int B, int T, int t, hipStream_t st);
// Slots [tv[b], t) of head b: the protected keys, exact (K, V converted to
// float32, or to bfloat16 when v_bf16; bias 0).
hipError_t launch_fill_protected(const int32_t* plist, const int32_t* tv, const void* K,
                                 const void* V, void* out_K, void* out_V, float* out_bias,
                                 int32_t* out_idx, int B, int T, int t, int D, bool bf16,
                                 bool v_bf16, hipStream_t st);
// tv[b] = tin[b] clamped to [1, t]; status[b] |= 16 where clamped
hipError_t launch_budgets(const int32_t* tin, int32_t* tv, int32_t* status, int B, int t,
                          hipStream_t st);
hipError_t launch_gather(const void* K, const int32_t* idx, void* outK, int B, int T, int t,
                         int row_bytes, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t count, hipStream_t st);

// Float64 work buffers of the fits (device pointers into the workspace).
struct FitBufs {
  double *PS, *cvec, *wv, *lam, *colpart;
  double* S;  // [B][ld][ld] sweep matrices (lower triangle), ld = sweep_ld(t, d)
  double* U;  // [B][ld][64] staged pivot columns of a sweep step
  double* V;  // [B][ld][64] the same times the inverse pivot block
  double* stage;  // [B][kSweepStage] inverse of the next pivot block (lookahead)
  int32_t *Fidx, *inv, *msz;
  const int32_t* tv;  // [B] per-head budgets (<= t), or null: t for every head
  unsigned* bar;  // kBarWords words: team barrier flags (kFlagStride words per team workgroup), tile-task
                  // counters and lookahead ready counts (kFlagStride words per team, from
                  // kTicketOffset and kReadyOffset), the last word the timeout flag
  int32_t* xcc;   // kMaxTeamGrid words: each team workgroup's XCC id
  double* flops;    // [B][2] fp64 work of the NNLS sweeps and of the value sweeps
  double* part;     // split-K partial tiles of the fit GEMMs
  size_t part_cap;  // its capacity in doubles
  uint64_t wait_ticks;  // bound on each team wait (100 MHz constant clock)
  int refine;           // refinement steps of the value fit (0: none)
  double* E;            // [B][n][d] residual O - X_F C (refinement only)
  double* Rp;           // [B][t][d] X_F^T E (refinement only)
  double* Cn;           // [B][t][d] the refined solution (refinement only)
};
// Order of a head's sweep matrix: right-hand-side rows (d rounded up to 64)
// plus the variables (t rounded up to 64).
int sweep_ld(int t, int d);
constexpr int kSweepStage = 2 * 64 * 64 + 64;
constexpr int kMaxTeamGrid = 8192;
constexpr int kFlagStride = 16;  // one 64-byte slot per team workgroup's barrier flag
constexpr int kTicketOffset = kMaxTeamGrid * kFlagStride;
constexpr int kReadyOffset = 2 * kMaxTeamGrid * kFlagStride;
constexpr int kBarWords = 3 * kMaxTeamGrid * kFlagStride + 1;
template <class In, int D>
// out_V: float32, or bfloat16 (the float32 value rounded to nearest-even)
// when v_bf16
hipError_t launch_fit(const void* Qv, const void* Kv, const void* Vv, const double* lse,
                      const float* O, const int32_t* idx, FitBufs fb, float* out_bias,
                      void* out_V, bool v_bf16, int32_t* status, int B, int n, int T, int t,
                      double ridge, int max_iters, int qg, hipStream_t st);
// kept indices of (head, chunk) b' made global: idx[b'][a] += (b' mod C) * Tc
hipError_t launch_idx_offset(int32_t* idx, int Bc, int t, int C, int Tc, hipStream_t st);
// Attention over block 1 (K1, V1 with a per-key bias) then block 2 (K2, V2);
// ws holds attend_ws_bytes() of split partials.
size_t attend_ws_bytes(int B, int m, int keys, int D);
template <class In, int D>
hipError_t launch_attend(const void* Q, const void* K1, const float* bias, const void* V1,
                         bool v1_f32, const void* K2, const void* V2, float* out,
                         double* out_lse, void* ws, int B, int m, int t1, int t2,
                         hipStream_t st);
// P [B][n][T] float32 of every key: exp(q_i . k_j - lse_i).
template <class In, int D>
hipError_t launch_probs_all(const void* Q, const void* K, const double* lse, float* P, int B,
                            int n, int T, int qg, hipStream_t st);
// Work buffers of the greedy (matching pursuit) selection.
struct OmpBufs {
  double* nrm;     // [B][T] column norms of P
  double* r;       // [B][n] residual
  uint8_t* chosen; // [B][T] flags
  double2* part;   // [B][ceil(T/1024)] workgroup bests (value, key)
  int32_t* order;  // [B][t] keys in the order chosen
  double* a;       // [B][n] the chosen column
  double* Q;       // [B][t][n] orthonormal basis of the chosen columns
  double* h;       // [B][t] projections
  double* q;       // [B][n] new basis vector before normalisation
  double2* part2;  // [B][ceil(n/256)] partial sums (q.q, q.r)
};
// t greedy steps over P; writes the chosen keys ascending to idx [B][t].
hipError_t launch_omp(const float* P, OmpBufs ob, int32_t* idx, int B, int n, int T, int t,
                      hipStream_t st);
// Event-pair instrumentation (defined with the C ABI): no-op unless enabled.
void prof_mark(int stage, bool end, hipStream_t st);
}  // namespace kvc
