"""Float64 CPU oracle for attention-matching KV-cache compaction.

TEST INFRASTRUCTURE.  This package is the independent checker of the GPU path:
only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import it.  It shares no code with the HIP library and never calls it.

Source: "Fast KV Compaction via Attention Matching" (Zweiger, Fu, Guo, Kim),
technical summary, section 2 ("Methodology: Attention Matching"): the
"main objective" paragraph (output- and mass-matching equations, the per-key
scalar bias) and the "algorithmic pipeline" paragraph (highest-attention key
selection aggregated by RMS, bias by non-negative least squares, values by
ordinary least squares given the keys and the fitted bias).

Notation, per (layer, KV head):
    Q  [n, d]  reference queries (already carrying the softmax scale)
    K, V [T, d] the full cache
    s_ij = q_i . k_j,   lse_i = log sum_j exp(s_ij),   p_ij = exp(s_ij - lse_i)
    O = P V            full-cache attention output on the reference queries
    S                  the kept index set, |S| = t, ascending
    C_k = K[S]         kept original keys
    w_j = exp(beta_j)  per-kept-key mass multiplier, beta the logit bias
    C_v                fitted values

Readings taken where the page is silent (each one is a documented choice):
  * no softmax scale inside the method: exp(q K^T) as written; Q carries it;
  * the aggregated "attention scores" are the full-cache softmax weights p,
    aggregated over the reference queries by RMS (or mean, a switch);
  * ties at the top-t cutoff go to the lower index; S is returned ascending;
  * mass matching is relative: each query's equation is divided by its own
    full-cache mass, i.e. sum_{j in S} p_ij w_j ~= 1;
  * both fits carry a vanishing ridge toward the prior (w -> 1, C_v -> V[S])
    of weight ridge_rel * trace(Gram) / t, which keeps each fit unique;
  * beta_j = log(max(w_j, 1e-30)), so a key whose multiplier is pinned at 0
    keeps a finite bias;
  * the bias is fitted first, then the values with the compacted softmax
    weights that use the fitted bias.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import cho_factor, cho_solve
from scipy.special import logsumexp

W_FLOOR = 1e-30           # smallest multiplier; beta >= log(1e-30) ~= -69.08
DEFAULT_RIDGE_REL = 1e-6
BLOCK = 16384             # cache rows per block (memory only)


# ---------------------------------------------------------------------------
# Scores over the full cache (section 2, main objective: both equations use
# exp(q K^T); the denominator of the softmax is the attention mass).
# ---------------------------------------------------------------------------
def row_lse(Q: np.ndarray, K: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """lse_i = log sum_j exp(q_i . k_j), float64.

    The cache is taken in contiguous blocks only to bound memory; the
    log-mass of a concatenation is the log-sum of the blocks' masses, which
    is the block decomposition the page builds its objective on."""
    acc = np.full(Q.shape[0], -np.inf)
    for j0 in range(0, K.shape[0], block):
        s = Q @ K[j0:j0 + block].T
        acc = np.logaddexp(acc, logsumexp(s, axis=1))
    return acc


def attention_stats(Q, K, V, lse, agg: str = "rms", block: int = BLOCK):
    """Full-cache attention output O = P V and per-key importance.

    importance_j = sqrt(mean_i p_ij^2) for RMS aggregation (the page's key
    selection), or mean_i p_ij for the mean aggregator."""
    n, T = Q.shape[0], K.shape[0]
    O = np.zeros((n, V.shape[1]))
    acc = np.zeros(T)
    for j0 in range(0, T, block):
        p = np.exp(Q @ K[j0:j0 + block].T - lse[:, None])
        O += p @ V[j0:j0 + block]
        acc[j0:j0 + block] = (p * p).sum(axis=0) if agg == "rms" else p.sum(axis=0)
    imp = np.sqrt(acc / n) if agg == "rms" else acc / n
    return O, imp


# ---------------------------------------------------------------------------
# Key selection (section 2, pipeline, "highest-attention keys").
# ---------------------------------------------------------------------------
def select_topt(imp: np.ndarray, t: int) -> np.ndarray:
    """The t largest importances; equal values go to the lower index.
    Returned in ascending index order (the cache keeps positional order)."""
    order = np.argsort(-imp, kind="stable")
    return np.sort(order[:t]).astype(np.int64)


def compact_probs(Q, Ck, lse) -> np.ndarray:
    """P_S [n, t]: the full-cache softmax weights of the kept keys."""
    return np.exp(Q @ Ck.T - lse[:, None])


# ---------------------------------------------------------------------------
# Non-negative least squares (section 2, pipeline, bias fit).
# ---------------------------------------------------------------------------
def nnls_normal(H: np.ndarray, c: np.ndarray, w0: np.ndarray | None = None,
                max_outer: int | None = None):
    """argmin_{w >= 0} 1/2 w^T H w - c^T w for symmetric positive definite H.

    This is the active-set method of Lawson and Hanson (Solving Least Squares
    Problems, 1974, chapter 23), written on the normal equations: an inner
    loop that solves the unconstrained problem on the passive set and steps
    back to the feasible region when a passive variable would go negative
    (dropping the variables that reach zero), and an outer loop that frees the
    active variable whose dual (c - H w)_j is largest positive.  It may start
    from any feasible point; the caller passes the ridge prior.

    Returns (w, passive mask, outer iterations)."""
    t = c.shape[0]
    w = np.zeros(t) if w0 is None else np.maximum(np.asarray(w0, float), 0.0)
    P = w > 0
    scale = max(np.abs(c).max(), np.abs(H).max(), 1e-300)
    tol = 1e-13 * scale * max(1.0, np.abs(w).max())
    max_outer = 3 * t + 10 if max_outer is None else max_outer
    it = 0
    while True:
        # inner loop: solve on P, back-track while a passive variable is <= 0
        while True:
            z = np.zeros(t)
            if P.any():
                idx = np.flatnonzero(P)
                z[idx] = cho_solve(cho_factor(H[np.ix_(idx, idx)]), c[idx])
            bad = P & (z <= 0)
            if not bad.any():
                w = z
                break
            bi = np.flatnonzero(bad)
            ratio = w[bi] / (w[bi] - z[bi])
            alpha = ratio.min()
            w = w + alpha * (z - w)
            # the blocking variable(s) reach zero and leave the passive set
            w[bi[ratio <= alpha]] = 0.0
            P &= w > 0
            w[~P] = 0.0
        g = c - H @ w
        cand = ~P & (g > tol)
        if not cand.any() or it >= max_outer:
            return w, P, it
        j = int(np.argmax(np.where(cand, g, -np.inf)))
        P[j] = True
        it += 1


def fit_bias(PS: np.ndarray, ridge_rel: float = DEFAULT_RIDGE_REL):
    """Per-kept-key multipliers w >= 0 and bias beta = log max(w, 1e-30).

    Solves min_{w >= 0} ||P_S w - 1||^2 + lam_w ||w - 1||^2 with
    lam_w = ridge_rel * trace(P_S^T P_S) / t: each reference query's mass over
    the kept keys, re-weighted by w, should equal its full-cache mass."""
    n, t = PS.shape
    lam = ridge_rel * float((PS * PS).sum()) / t
    H = PS.T @ PS + lam * np.eye(t)
    c = PS.T @ np.ones(n) + lam * np.ones(t)
    w, P, iters = nnls_normal(H, c, w0=np.ones(t))
    # final passive-set solve by orthogonal factorisation of the augmented
    # system (the normal equations only located the passive set)
    idx = np.flatnonzero(P)
    if idx.size:
        A = np.vstack([PS[:, idx], np.sqrt(lam) * np.eye(idx.size)])
        rhs = np.concatenate([np.ones(n), np.sqrt(lam) * np.ones(idx.size)])
        wp = np.linalg.lstsq(A, rhs, rcond=None)[0]
        if (wp > 0).all():
            w = np.zeros(t)
            w[idx] = wp
    beta = np.log(np.maximum(w, W_FLOOR))
    return w, beta, {"lam_w": lam, "outer_iters": iters, "n_zero": int(t - idx.size)}


# ---------------------------------------------------------------------------
# Value fit (section 2, pipeline, ordinary least squares on the outputs).
# ---------------------------------------------------------------------------
def compacted_weights(PS: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """x_ij = exp(s_ij + beta_j) / sum_{k in S} exp(s_ik + beta_k), the
    softmax of the compacted cache (right side of the output equation).
    exp(s_ij) differs from p_ij only by the row factor exp(lse_i), which
    cancels in the ratio."""
    e = PS * np.exp(beta)[None, :]
    return e / e.sum(axis=1, keepdims=True)


def fit_values(X: np.ndarray, O: np.ndarray, VS: np.ndarray,
               ridge_rel: float = DEFAULT_RIDGE_REL):
    """C_v = argmin ||X C - O||_F^2 + lam_v ||C - V_S||_F^2,
    lam_v = ridge_rel * trace(X^T X) / t, by orthogonal factorisation of the
    augmented system (never the normal equations)."""
    n, t = X.shape
    lam = ridge_rel * float((X * X).sum()) / t
    A = np.vstack([X, np.sqrt(lam) * np.eye(t)])
    R = np.vstack([O, np.sqrt(lam) * VS])
    C = np.linalg.lstsq(A, R, rcond=None)[0]
    return C, {"lam_v": lam}


# ---------------------------------------------------------------------------
# Whole pipeline for one head, and the consumer's view of the result.
# ---------------------------------------------------------------------------
def fit(Q, K, V, idx, lse=None, O=None, ridge_rel: float = DEFAULT_RIDGE_REL):
    """Bias and value fit for a given kept set (no selection)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    if lse is None:
        lse = row_lse(Q, K)
    if O is None:
        O, _ = attention_stats(Q, K, V, lse)
    idx = np.asarray(idx, dtype=np.int64)
    PS = compact_probs(Q, K[idx], lse)
    w, beta, info_b = fit_bias(PS, ridge_rel)
    X = compacted_weights(PS, beta)
    Cv, info_v = fit_values(X, O, V[idx], ridge_rel)
    info = {**info_b, **info_v, "PS": PS, "X": X}
    return w, beta, Cv, info


def compact(Q, K, V, t: int, agg: str = "rms", ridge_rel: float = DEFAULT_RIDGE_REL):
    """One head: (C_k, beta, C_v, idx) plus intermediates, all float64."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T = K.shape[0]
    if not 1 <= t <= T:
        raise ValueError("t must lie in [1, T]")
    lse = row_lse(Q, K)
    O, imp = attention_stats(Q, K, V, lse, agg)
    idx = select_topt(imp, t)
    w, beta, Cv, info = fit(Q, K, V, idx, lse=lse, O=O, ridge_rel=ridge_rel)
    return {"idx": idx, "Ck": K[idx], "beta": beta, "w": w, "Cv": Cv,
            "lse": lse, "O": O, "imp": imp, **info}


def omp_dictionary(Q, K, lse):
    """The dictionary of the greedy selection: the whole-cache softmax weights
    P [n, T] in float64 (column j = key j's weight on every reference query;
    each row sums to one over the T keys)."""
    return np.exp(np.asarray(Q, float) @ np.asarray(K, float).T - np.asarray(lse, float)[:, None])


def omp_select(P: np.ndarray, t: int):
    """Orthogonal matching pursuit on the attention mass (section 2, key
    selection, the greedy alternative to the highest-attention keys): target
    y = 1 over the reference queries (relative mass), dictionary columns p_j.
    Each step picks the unchosen key with the largest p_j . r / ||p_j|| (ties
    to the lower index; all-zero columns only when nothing else is left) and
    sets r to y minus its least-squares projection on the chosen columns.
    Returns (chosen keys ascending, keys in the order chosen, residual norms)."""
    n, T = P.shape
    if not 1 <= t <= T:
        raise ValueError("t must lie in [1, T]")
    y = np.ones(n)
    nrm = np.sqrt((P * P).sum(axis=0))
    r = y.copy()
    order, norms = [], []
    taken = np.zeros(T, bool)
    for _ in range(t):
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.where(nrm > 0, (P.T @ r) / nrm, -np.inf)
        c[taken] = -np.inf
        j = int(np.argmax(c)) if np.isfinite(c.max()) else int(np.flatnonzero(~taken)[0])
        order.append(j)
        taken[j] = True
        A = P[:, order]
        w = np.linalg.lstsq(A, y, rcond=None)[0]
        r = y - A @ w
        norms.append(float(np.linalg.norm(r)))
    return np.sort(np.array(order)), np.array(order), np.array(norms)


def compact_omp(Q, K, V, t: int, ridge_rel: float = DEFAULT_RIDGE_REL):
    """One head with the greedy selection: keys by omp_select on the float64
    dictionary, then the same bias (NNLS) and value fits as compact()."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    lse = row_lse(Q, K)
    O, _ = attention_stats(Q, K, V, lse)
    idx, order, norms = omp_select(omp_dictionary(Q, K, lse), t)
    w, beta, Cv, info = fit(Q, K, V, idx, lse=lse, O=O, ridge_rel=ridge_rel)
    return {"idx": idx, "order": order, "res_norms": norms, "Ck": K[idx], "beta": beta, "w": w,
            "Cv": Cv, "lse": lse, "O": O, **info}


def compact_chunked(Q, K, V, t: int, n_chunks: int, agg: str = "rms",
                    ridge_rel: float = DEFAULT_RIDGE_REL):
    """Chunked compaction ("Compaction par blocs" paragraph of the same summary):
    the KV states of one head are cut into n_chunks contiguous chunks of equal
    length, each chunk is compacted on its own against all reference queries
    (its own lse, output, importance and fits), and the compact chunks are
    concatenated in order.  Kept indices are returned as positions in the
    whole cache.  The merge needs no re-fit: attention over concatenated blocks
    is the mass-weighted mix of the per-block attentions (main objective,
    block-concatenation decomposition)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T = K.shape[0]
    if n_chunks < 1 or T % n_chunks:
        raise ValueError("T must be a positive multiple of n_chunks")
    Tc = T // n_chunks
    parts = []
    for c in range(n_chunks):
        lo = c * Tc
        r = compact(Q, K[lo:lo + Tc], V[lo:lo + Tc], t, agg, ridge_rel)
        r["idx"] = r["idx"] + lo
        parts.append(r)
    out = {k: np.concatenate([r[k] for r in parts]) for k in ("idx", "Ck", "beta", "w", "Cv")}
    out["chunks"] = parts
    return out


def compact_ragged(Qs, Ks, Vs, budgets, agg: str = "rms",
                   ridge_rel: float = DEFAULT_RIDGE_REL):
    """Per-head budgets (the per-head retention ratios of the non-uniform
    schedule in section 2 of the same summary): head b is compacted on its own
    with t = budgets[b].  Results are padded to max(budgets): a padded slot
    holds index -1, zero key and value rows and bias -inf, whose softmax weight
    is exactly zero, so attention over the padded cache equals attention over
    the head's own compact cache."""
    budgets = [int(x) for x in budgets]
    tm = max(budgets)
    B = len(budgets)
    d, dv = np.asarray(Ks[0]).shape[1], np.asarray(Vs[0]).shape[1]
    out = {"idx": np.full((B, tm), -1, np.int64), "Ck": np.zeros((B, tm, d)),
           "beta": np.full((B, tm), -np.inf), "w": np.zeros((B, tm)),
           "Cv": np.zeros((B, tm, dv)), "heads": []}
    for h, tb in enumerate(budgets):
        r = compact(Qs[h], Ks[h], Vs[h], tb, agg, ridge_rel)
        for k in ("idx", "Ck", "beta", "w", "Cv"):
            out[k][h, :tb] = r[k]
        out["heads"].append(r)
    return out


def compact_protected(Q, K, V, t: int, protect, agg: str = "rms",
                      ridge_rel: float = DEFAULT_RIDGE_REL):
    """Protected (pivot) keys, "Thought-Aware KV Cache Compaction ...",
    section 2C: the marked keys are kept exactly with zero bias and the rest of
    the budget goes to the other keys.  At most t - 1 keys are protected (the
    first by position), so at least one slot is fitted.  The unprotected keys
    R form their own block: they are compacted to t - |P| slots against their
    own log-sum-exp and output (the protected block is exact, so by the block
    decomposition of the main objective the fitted part has to match R alone).
    Slots: the fitted part first (ascending), then the protected keys
    (ascending)."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T = K.shape[0]
    if not 1 <= t <= T:
        raise ValueError("t must lie in [1, T]")
    marked = np.flatnonzero(np.asarray(protect, dtype=bool))
    P = marked[:t - 1]
    R = np.setdiff1d(np.arange(T), P)
    r = compact(Q, K[R], V[R], t - P.size, agg, ridge_rel)
    idx = np.concatenate([R[r["idx"]], P])
    return {"idx": idx, "Ck": K[idx], "beta": np.concatenate([r["beta"], np.zeros(P.size)]),
            "w": np.concatenate([r["w"], np.ones(P.size)]),
            "Cv": np.concatenate([r["Cv"], V[P]]), "n_protected": int(P.size),
            "dropped": int(marked.size - P.size), "rest": r}


def attend(Q, K, V, bias=None):
    """softmax(Q K^T + bias) V in float64 (the consumer's attention)."""
    s = np.asarray(Q, float) @ np.asarray(K, float).T
    if bias is not None:
        s = s + np.asarray(bias, float)[None, :]
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ np.asarray(V, float)


def attend_appended(Q, K1, V1, bias1, K2, V2):
    """Attention over a cache (K1, V1, per-key bias1) followed by an appended
    block (K2, V2) with no bias: the setting of the main objective, where a
    compact cache must keep the output for any fixed or future block appended
    after it.  Returns (output, lse)."""
    K = np.vstack([np.asarray(K1, float), np.asarray(K2, float)])
    V = np.vstack([np.asarray(V1, float), np.asarray(V2, float)])
    b1 = np.zeros(len(K1)) if bias1 is None else np.asarray(bias1, float)
    bias = np.concatenate([b1, np.zeros(len(K2))])
    s = np.asarray(Q, float) @ K.T + bias[None, :]
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ V, (mx + np.log(z))[:, 0]


def rel_l2(a, b) -> float:
    a = np.asarray(a, float)
    b = np.asarray(b, float)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
