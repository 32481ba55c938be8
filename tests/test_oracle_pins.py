"""Pins for the float64 oracle: closed forms, invariants, brute force.

Each test ties an oracle function to something fixed outside the oracle's own
code (the mathematics, a worked example on the page, an exhaustive search),
chosen so that a dropped term, a wrong sign or a transposed operand fails.
Source of the method: "Fast KV Compaction via Attention Matching", technical
summary section 2 (main objective; algorithmic pipeline)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import nnls as scipy_nnls

import oracle as orc
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------- P1
def test_lse_and_output_match_elementwise_fsum():
    """lse, O and the RMS importance against scalar loops with math.fsum."""
    Q, K, V = _rand(1, 5, 3, scale=0.7), _rand(2, 11, 3), _rand(3, 11, 2)
    lse = orc.row_lse(Q, K, block=4)
    O, imp = orc.attention_stats(Q, K, V, lse, block=3)
    for i in range(5):
        s = [math.fsum(Q[i, c] * K[j, c] for c in range(3)) for j in range(11)]
        z = math.fsum(math.exp(x) for x in s)
        assert abs(lse[i] - math.log(z)) < 1e-13
        for c in range(2):
            o = math.fsum(math.exp(s[j]) * V[j, c] for j in range(11)) / z
            assert abs(O[i, c] - o) < 1e-13
    for j in range(11):
        p2 = [math.exp(2 * (math.fsum(Q[i, c] * K[j, c] for c in range(3))))
              / math.exp(2 * lse[i]) for i in range(5)]
        assert abs(imp[j] - math.sqrt(math.fsum(p2) / 5)) < 1e-13
    _, imp_mean = orc.attention_stats(Q, K, V, lse, agg="mean")
    p = np.exp(Q @ K.T - lse[:, None])
    assert np.allclose(imp_mean, p.mean(axis=0), rtol=1e-13, atol=0)


def test_lse_blocking_invariance_and_large_logits():
    """Any block size gives the same lse (concatenation identity), and logits
    of size 700 neither overflow nor lose precision."""
    Q, K = _rand(4, 7, 16, scale=0.3), _rand(5, 1000, 16)
    ref = orc.row_lse(Q, K, block=1000)
    for b in (1, 7, 64, 333):
        assert np.allclose(orc.row_lse(Q, K, block=b), ref, rtol=0, atol=1e-12)
    K2 = np.zeros((3, 1))
    K2[:, 0] = [700.0, 699.0, -5.0]
    got = orc.row_lse(np.ones((1, 1)), K2)[0]
    assert abs(got - (700.0 + math.log(1 + math.exp(-1) + math.exp(-705)))) < 1e-12


def test_zero_query_uniform_attention():
    """q = 0 -> every p_ij = 1/T, lse = log T, O = column mean of V,
    importance 1/T for both aggregators."""
    T = 37
    Q, K, V = np.zeros((4, 5)), _rand(6, T, 5), _rand(7, T, 3)
    lse = orc.row_lse(Q, K)
    assert np.allclose(lse, math.log(T), atol=1e-14)
    O, imp = orc.attention_stats(Q, K, V, lse)
    assert np.allclose(O, V.mean(axis=0)[None, :], atol=1e-14)
    assert np.allclose(imp, 1.0 / T, rtol=1e-13)


# --------------------------------------------------------------------- P7
def test_block_decomposition_identity():
    """Attention over [A; B] = mass-weighted mix of the two blocks' outputs."""
    Q = _rand(8, 6, 4, scale=0.5)
    KA, VA, KB, VB = _rand(9, 13, 4), _rand(10, 13, 3), _rand(11, 9, 4), _rand(12, 9, 3)
    full = orc.attend(Q, np.vstack([KA, KB]), np.vstack([VA, VB]))
    la, lb = orc.row_lse(Q, KA), orc.row_lse(Q, KB)
    oa, ob = orc.attend(Q, KA, VA), orc.attend(Q, KB, VB)
    za, zb = np.exp(la)[:, None], np.exp(lb)[:, None]
    assert np.allclose(full, (za * oa + zb * ob) / (za + zb), atol=1e-13)


def test_bias_acts_as_key_multiplicity():
    """A logit bias of log m on one key equals m copies of that key, for the
    attention output and the mass (the role of beta on the page)."""
    Q, K, V = _rand(13, 5, 4, scale=0.5), _rand(14, 6, 4), _rand(15, 6, 2)
    bias = np.zeros(6)
    bias[2] = math.log(3.0)
    Kr, Vr = np.vstack([K, K[2], K[2]]), np.vstack([V, V[2], V[2]])
    assert np.allclose(orc.attend(Q, K, V, bias), orc.attend(Q, Kr, Vr), atol=1e-13)


# --------------------------------------------------------------------- P9
@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_exhaustive_subset_search(seed):
    """top-t with the lower-index tie rule = the lexicographically smallest
    subset that maximises the summed importance (exhaustive over C(T, t))."""
    rng = np.random.default_rng(100 + seed)
    T, t = 12 + seed % 3, 2 + seed % 5
    imp = rng.integers(0, 5, size=T).astype(float)      # many exact ties
    best, best_set = -1.0, None
    for S in itertools.combinations(range(T), t):          # lexicographic order
        v = imp[list(S)].sum()
        if v > best:
            best, best_set = v, S
    assert list(orc.select_topt(imp, t)) == list(best_set)


def test_selection_ties_from_duplicate_keys_go_low():
    """Bitwise-identical keys tie exactly; the lower index is kept."""
    K = _rand(16, 10, 4)
    K[7] = K[2]
    Q = _rand(17, 8, 4, scale=0.4)
    lse = orc.row_lse(Q, K)
    _, imp = orc.attention_stats(Q, K, np.zeros((10, 1)), lse)
    assert imp[7] == imp[2]
    order = np.argsort(-imp, kind="stable")
    r = list(order).index(2)
    idx = orc.select_topt(imp, r + 1)
    assert 2 in idx and 7 not in idx


# -------------------------------------------------------------------- P10
def _kkt(H, c, w, tol):
    g = H @ w - c
    assert (w >= 0).all()
    assert np.all(np.abs(g[w > 0]) <= tol)
    assert np.all(g[w == 0] >= -tol)


@pytest.mark.parametrize("seed", range(8))
def test_nnls_brute_force_over_passive_sets(seed):
    """For t <= 10 exactly one passive set satisfies the KKT conditions; its
    solution is the oracle's."""
    rng = np.random.default_rng(200 + seed)
    n, t = 14, 6 + seed % 5
    A = np.abs(rng.standard_normal((n, t))) * rng.uniform(0.1, 1, t)
    A[:, 1] = A[:, 0] * 0.9 + 0.1 * A[:, 2]                 # near-collinear pair
    b = rng.uniform(0.5, 1.5, n)
    H, c = A.T @ A + 1e-3 * np.eye(t), A.T @ b + 1e-3 * rng.standard_normal(t)
    found = []
    for mask in itertools.product([False, True], repeat=t):
        F = np.array(mask)
        x = np.zeros(t)
        if F.any():
            x[F] = np.linalg.solve(H[np.ix_(F, F)], c[F])
        g = H @ x - c
        if (x[F] > 0).all() and (g[~F] >= 0).all():
            found.append(x)
    assert len(found) == 1
    w, _, _ = orc.nnls_normal(H, c, w0=np.ones(t))
    assert np.allclose(w, found[0], atol=1e-11)
    w0, _, _ = orc.nnls_normal(H, c)                      # start at zero
    assert np.allclose(w0, found[0], atol=1e-11)


@pytest.mark.parametrize("cfg", [1, 2])
def test_bias_fit_kkt_and_independent_nnls(cfg):
    """On real compaction problems: KKT holds, and scipy's independent
    Lawson-Hanson code on the augmented system agrees."""
    w = synth.CONFIGS[cfg]
    if cfg == 2:
        w = synth.custom(3, 1, 2048, 256, 128, 205, "bf16", "channel_lognormal")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r = orc.compact(Q, K, V, w.t)
    PS, lam, t = r["PS"], r["lam_w"], w.t
    H = PS.T @ PS + lam * np.eye(t)
    c = PS.sum(axis=0) + lam
    _kkt(H, c, r["w"], 1e-9 * np.abs(c).max())
    A = np.vstack([PS, math.sqrt(lam) * np.eye(t)])
    rhs = np.concatenate([np.ones(PS.shape[0]), math.sqrt(lam) * np.ones(t)])
    ws = scipy_nnls(A, rhs, maxiter=50 * t)[0]
    assert orc.rel_l2(r["w"], ws) < 1e-7
    assert r["n_zero"] > 0      # the constraint is active on these problems


# --------------------------------------------------------------------- P2
@pytest.mark.parametrize("n,ridge", [(40, 1e-6), (8, 1e-6), (40, 1e-3)])
def test_keep_everything_is_exact(n, ridge):
    """t = T: all indices kept, w = 1 (beta = 0), C_v = V, output unchanged,
    for any number of reference queries (the ridge prior makes the zero-loss
    point unique)."""
    T, d = 24, 8
    Q, K, V = _rand(20, n, d, scale=0.4), _rand(21, T, d), _rand(22, T, 5)
    r = orc.compact(Q, K, V, T, ridge_rel=ridge)
    assert list(r["idx"]) == list(range(T))
    assert np.allclose(r["w"], 1.0, atol=1e-10)
    assert np.allclose(r["beta"], 0.0, atol=1e-10)
    assert np.allclose(r["Cv"], V, atol=1e-9)
    Qn = _rand(23, 9, d, scale=0.4)
    assert np.allclose(orc.attend(Qn, r["Ck"], r["Cv"], r["beta"]), orc.attend(Qn, K, V),
                       atol=1e-9)


# --------------------------------------------------------------------- P4
def test_zero_queries_golden_bias():
    """Page example (q = 0: full mass T versus t kept keys), stored under
    tests/golden with its citation: beta -> log(T/t)."""
    with open(os.path.join(GOLDEN, "q0_mass_example.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        T, t, n, d = case["T"], case["t"], case["n"], case["d"]
        Q, K, V = np.zeros((n, d)), _rand(T, T, d), _rand(T + 1, T, 3)
        r = orc.compact(Q, K, V, t, ridge_rel=1e-12)
        assert list(r["idx"]) == list(range(t))          # all tie -> lowest indices
        assert np.allclose(r["beta"], case["beta"], atol=1e-9)


@pytest.mark.parametrize("rho", [1e-6, 1e-2, 0.5])
def test_zero_queries_closed_form_with_ridge(rho):
    """q = 0 at finite ridge: w = (T + rho)/(t + rho) and
    C_v,j = V_j + (mean(V) - mean(V_S)) / (1 + rho/t)."""
    T, t, n = 30, 7, 5
    V = _rand(31, T, 4)
    r = orc.compact(np.zeros((n, 6)), _rand(30, T, 6), V, t, ridge_rel=rho)
    assert np.allclose(r["w"], (T + rho) / (t + rho), rtol=1e-9)
    VS = V[:t]
    expect = VS + (V.mean(axis=0) - VS.mean(axis=0)) / (1 + rho / t)
    assert np.allclose(r["Cv"], expect, atol=1e-7)


# --------------------------------------------------------------------- P5
@pytest.mark.parametrize("rho", [1e-6, 1e-3, 0.3])
def test_single_query_closed_form(rho):
    """n = 1: w = 1 + p (1 - sum p) / (|p|^2 + lam_w) (inactive constraint),
    C_v = V_S + x (o - x V_S) / (|x|^2 + lam_v)   (Sherman-Morrison)."""
    T, t, d = 40, 9, 6
    q, K, V = _rand(40, 1, d, scale=0.6), _rand(41, T, d), _rand(42, T, 3)
    r = orc.compact(q, K, V, t, ridge_rel=rho)
    s = (q @ K.T)[0]
    p_all = np.exp(s - s.max())
    p_all /= p_all.sum()
    S = np.sort(np.argsort(-p_all, kind="stable")[:t])
    assert list(r["idx"]) == list(S)
    p = p_all[S]
    lam_w = rho * (p @ p) / t
    w = 1 + p * (1 - p.sum()) / (p @ p + lam_w)
    assert np.allclose(r["w"], w, rtol=1e-9)
    x = p * w / (p @ w)
    o = p_all @ V
    lam_v = rho * (x @ x) / t
    Cv = V[S] + np.outer(x, o - x @ V[S]) / (x @ x + lam_v)
    assert np.allclose(r["Cv"], Cv, atol=1e-8)


# --------------------------------------------------------------------- P6
def test_duplicated_keys_recovered_exactly_for_all_queries():
    """t distinct keys, key j repeated m_j times, fit on the first copies:
    w_j = m_j, C_v,j = mean of V over the copies, exact for fresh queries."""
    rng = np.random.default_rng(50)
    t, d = 5, 6
    base = rng.standard_normal((t, d))
    mult = np.array([1, 3, 2, 4, 1])
    rows = np.repeat(np.arange(t), mult)
    perm = rng.permutation(rows.size)
    K = base[rows[perm]]
    V = rng.standard_normal((rows.size, 3))
    first = np.array([np.flatnonzero(rows[perm] == j)[0] for j in range(t)])
    order = np.argsort(first)
    idx = first[order]
    Q = rng.standard_normal((12, d)) * 0.5
    w, beta, Cv, _ = orc.fit(Q, K, V, idx, ridge_rel=1e-12)
    assert np.allclose(w, mult[order], rtol=1e-8)
    means = np.array([V[rows[perm] == j].mean(axis=0) for j in range(t)])[order]
    assert np.allclose(Cv, means, atol=1e-7)
    Qn = rng.standard_normal((20, d)) * 0.5
    assert np.allclose(orc.attend(Qn, K[idx], Cv, beta), orc.attend(Qn, K, V), atol=1e-7)


# --------------------------------------------------------------------- P3
@pytest.mark.parametrize("ridge", [1e-6, 1e-2])
def test_value_fit_gradient_vanishes_and_normal_equations_agree(ridge):
    w = synth.custom(7, 1, 700, 96, 32, 70, "f32", "normal")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r = orc.compact(Q, K, V, w.t, ridge_rel=ridge)
    X, O, VS, C = r["X"], r["O"], V[r["idx"]], r["Cv"]
    lam = r["lam_v"]
    grad = X.T @ (X @ C - O) + lam * (C - VS)
    scale = np.linalg.norm(X.T @ O) + lam * np.linalg.norm(VS)
    assert np.linalg.norm(grad) <= 1e-10 * scale
    Cne = np.linalg.solve(X.T @ X + lam * np.eye(w.t), X.T @ O + lam * VS)
    assert orc.rel_l2(C, Cne) < 1e-6
    # the compacted weights are a softmax over the kept keys with the bias
    s = Q @ K[r["idx"]].T + r["beta"][None, :]
    e = np.exp(s - s.max(axis=1, keepdims=True))
    assert np.allclose(X, e / e.sum(axis=1, keepdims=True), atol=1e-14)


def test_bias_mass_equation_and_relative_weighting():
    """The fitted multipliers minimise the relative mass residual: perturbing
    any positive w_j along +-eps does not lower the objective."""
    w = synth.custom(8, 1, 600, 80, 32, 40, "f32", "normal")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r = orc.compact(Q, K, V, w.t)
    PS, lam, wv = r["PS"], r["lam_w"], r["w"]

    def obj(x):
        return np.sum((PS @ x - 1) ** 2) + lam * np.sum((x - 1) ** 2)

    f0 = obj(wv)
    rng = np.random.default_rng(0)
    for _ in range(20):
        dx = rng.standard_normal(wv.size) * 1e-4
        x = np.maximum(wv + dx, 0)
        assert obj(x) >= f0 - 1e-15
    # relative mass: with the full mass on the left, p sums to one per query
    full = np.exp(Q @ K.T - r["lse"][:, None]).sum(axis=1)
    assert np.allclose(full, 1.0, atol=1e-13)


# --------------------------------------------------------------------- P8
@pytest.mark.parametrize("cfg_seed", range(3))
def test_eviction_error_bound(cfg_seed):
    """Eviction only (beta = 0, values kept): |o - o'| <= 2 Vmax delta per
    query, delta the dropped attention mass (error-bound page, section 2B)."""
    w = synth.custom(20 + cfg_seed, 1, 300, 40, 16, 30, "f32", "normal")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r = orc.compact(Q, K, V, w.t)
    idx = r["idx"]
    o = orc.attend(Q, K, V)
    o2 = orc.attend(Q, K[idx], V[idx])
    delta = 1 - r["PS"].sum(axis=1)
    vmax = np.linalg.norm(V, axis=1).max()
    assert np.all(np.linalg.norm(o - o2, axis=1) <= 2 * vmax * delta + 1e-12)


def test_am_fit_beats_eviction_on_reference_queries():
    """Eviction (w = 1, C_v = V_S) is a feasible point of both fits, so the
    fitted cache cannot be worse on the reference queries' objective."""
    w = synth.custom(30, 1, 1024, 128, 32, 64, "bf16", "clusters")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r = orc.compact(Q, K, V, w.t)
    am = orc.attend(Q, r["Ck"], r["Cv"], r["beta"])
    ev = orc.attend(Q, r["Ck"], V[r["idx"]])
    assert orc.rel_l2(am, r["O"]) < orc.rel_l2(ev, r["O"])


def test_argument_checks():
    with pytest.raises(ValueError):
        orc.compact(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros((4, 3)), 5)
    with pytest.raises(ValueError):
        orc.compact(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros((4, 3)), 0)


# ----------------------------------------------------------------- synth
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.3e38,
                  1e-40], dtype=np.float64)
    b = synth.round_bf16_bits(x)
    back = synth.bf16_bits_to_f64(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                    # tie -> even mantissa
    assert back[2] == 1.0 + 4 * 2 ** -8      # tie -> even (up)
    assert back[3] == 1.0
    assert back[4] == -2.5
    for v, r in zip(x[:5], back[:5]):
        assert abs(v - r) <= abs(v) * 2 ** -8


def test_workload_shapes_and_determinism():
    w = synth.CONFIGS[3]
    small = synth.Workload(3, "c3_small", 2, 512, 32, 128, 10, "bf16", "clusters", 8)
    a, b = synth.batch(small), synth.batch(small)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["K"].shape == (2, 512, 128) and a["K"].dtype == np.uint16
    assert w.T // w.t == 50
    assert synth.CONFIGS[4].B == 256 and synth.CONFIGS[5].T == 131072


# ------------------------------------------------------------ chunked (f1)
def test_chunked_one_chunk_is_compact():
    w = synth.custom(9, 1, 256, 24, 16, 20, "f32", "normal")
    a = synth.head(w, 0)
    Q, K, V = (synth.to_f64(a[k]) for k in ("Q", "K", "V"))
    r1, rc = orc.compact(Q, K, V, 20), orc.compact_chunked(Q, K, V, 20, 1)
    for k in ("idx", "beta", "w", "Cv"):
        assert np.array_equal(r1[k], rc[k])


def test_chunked_chunks_partition_the_cache():
    """The chunks' own log-sum-exps combine to the whole cache's (the chunks
    are disjoint and cover every key), and every kept index lies in its own
    chunk's range, ascending overall."""
    Q, K, V = _rand(60, 7, 8, scale=0.5), _rand(61, 96, 8), _rand(62, 96, 4)
    r = orc.compact_chunked(Q, K, V, 5, 4)
    lses = np.stack([c["lse"] for c in r["chunks"]])
    assert np.allclose(np.logaddexp.reduce(lses, axis=0), orc.row_lse(Q, K), atol=1e-13)
    idx = r["idx"]
    assert idx.shape == (20,) and np.all(np.diff(idx) > 0)
    assert np.array_equal(idx // 24, np.repeat(np.arange(4), 5))
    assert np.array_equal(r["Ck"], K[idx])


@pytest.mark.parametrize("C", [2, 3, 6])
def test_chunked_keep_everything_reproduces_full_attention(C):
    """t = T / C keeps every key of every chunk with w = 1 and C_v = V, so the
    merged cache is the original one and attention on fresh queries is
    unchanged (no re-fit after the merge)."""
    T, d = 36, 6
    Q, K, V = _rand(63, 30, d, scale=0.4), _rand(64, T, d), _rand(65, T, 3)
    r = orc.compact_chunked(Q, K, V, T // C, C)
    assert list(r["idx"]) == list(range(T))
    assert np.allclose(r["beta"], 0.0, atol=1e-9)
    assert np.allclose(r["Cv"], V, atol=1e-8)
    Qn = _rand(66, 11, d, scale=0.4)
    assert np.allclose(orc.attend(Qn, r["Ck"], r["Cv"], r["beta"]), orc.attend(Qn, K, V),
                       atol=1e-8)


def test_chunked_merge_is_mass_weighted_mix_of_chunks():
    """Attention over the merged compact cache = the per-chunk compact
    attentions mixed by their compact masses (block decomposition applied to
    the compacted blocks), and each chunk's bias brings its compact mass on the
    reference queries closer to that chunk's own mass than plain eviction
    (w = 1 is feasible for the chunk's NNLS)."""
    Q, K, V = _rand(67, 40, 8, scale=0.5), _rand(68, 120, 8), _rand(69, 120, 3)
    r = orc.compact_chunked(Q, K, V, 10, 3)
    Qn = _rand(70, 9, 8, scale=0.5)
    num, den = 0.0, 0.0
    for c in r["chunks"]:
        s = Qn @ c["Ck"].T + c["beta"][None, :]
        z = np.exp(s).sum(axis=1)[:, None]
        num = num + z * orc.attend(Qn, c["Ck"], c["Cv"], c["beta"])
        den = den + z
    assert np.allclose(orc.attend(Qn, r["Ck"], r["Cv"], r["beta"]), num / den, atol=1e-13)
    for j, c in enumerate(r["chunks"]):
        Kc = K[j * 40:(j + 1) * 40]
        m_true = np.exp(orc.row_lse(Q, Kc))
        m_comp = np.exp(Q @ c["Ck"].T + c["beta"][None, :]).sum(axis=1)
        m_evict = np.exp(Q @ c["Ck"].T).sum(axis=1)
        e_am = np.sum((m_comp / m_true - 1) ** 2)
        assert e_am < 0.5 * np.sum((m_evict / m_true - 1) ** 2)


def test_chunked_argument_checks():
    with pytest.raises(ValueError):
        orc.compact_chunked(np.zeros((2, 3)), np.zeros((10, 3)), np.zeros((10, 3)), 2, 3)
    with pytest.raises(ValueError):
        orc.compact_chunked(np.zeros((2, 3)), np.zeros((10, 3)), np.zeros((10, 3)), 6, 2)


# ------------------------------------------------------ ragged budgets (f2)
def test_ragged_heads_are_independent_compactions_and_padding_is_inert():
    """Each head's slots equal compact() at its own budget; the padding
    (index -1, zero rows, bias -inf) gives attention over the padded cache
    exactly the value over the head's own compact cache, for fresh queries."""
    rng = np.random.default_rng(71)
    budgets = [7, 19, 1, 12]
    Qs = [rng.standard_normal((16, 8)) * 0.4 for _ in budgets]
    Ks = [rng.standard_normal((60, 8)) for _ in budgets]
    Vs = [rng.standard_normal((60, 3)) for _ in budgets]
    r = orc.compact_ragged(Qs, Ks, Vs, budgets)
    assert r["idx"].shape == (4, 19)
    for h, tb in enumerate(budgets):
        own = orc.compact(Qs[h], Ks[h], Vs[h], tb)
        assert np.array_equal(r["idx"][h, :tb], own["idx"])
        assert np.all(r["idx"][h, tb:] == -1) and np.all(np.isneginf(r["beta"][h, tb:]))
        Qn = rng.standard_normal((5, 8)) * 0.4
        padded = orc.attend(Qn, r["Ck"][h], r["Cv"][h], r["beta"][h])
        trimmed = orc.attend(Qn, own["Ck"], own["Cv"], own["beta"])
        assert np.allclose(padded, trimmed, atol=1e-14, rtol=0)


# --------------------------------------------------- protected keys (f4)
def test_protected_none_is_compact_and_keep_rest_is_exact():
    Q, K, V = _rand(80, 20, 8, scale=0.5), _rand(81, 50, 8), _rand(82, 50, 3)
    r0 = orc.compact(Q, K, V, 12)
    rp = orc.compact_protected(Q, K, V, 12, np.zeros(50, bool))
    for k in ("idx", "beta", "Cv"):
        assert np.array_equal(r0[k], rp[k])
    # protect 8 keys and keep all 42 others: the compact cache is the cache
    prot = np.zeros(50, bool)
    prot[[1, 5, 9, 20, 33, 34, 40, 49]] = True
    r = orc.compact_protected(Q, K, V, 50, prot)
    assert sorted(r["idx"]) == list(range(50))
    assert np.allclose(r["beta"], 0.0, atol=1e-9)
    Qn = _rand(83, 7, 8, scale=0.5)
    assert np.allclose(orc.attend(Qn, r["Ck"], r["Cv"], r["beta"]), orc.attend(Qn, K, V),
                       atol=1e-8)


def test_protected_keys_exact_and_rest_fitted_on_its_own_block():
    """Protected slots: the key and value rows as they are with bias 0 (w = 1);
    the fitted part equals compact() of the unprotected keys alone; the rest's
    log-sum-exp and the protected block's combine to the whole cache's; and
    attention over the result is the two blocks' attentions mixed by mass."""
    Q, K, V = _rand(84, 30, 8, scale=0.5), _rand(85, 90, 8), _rand(86, 90, 3)
    prot = np.zeros(90, bool)
    prot[[3, 17, 18, 60, 88]] = True
    t = 20
    r = orc.compact_protected(Q, K, V, t, prot)
    P = np.flatnonzero(prot)
    R = np.flatnonzero(~prot)
    assert r["n_protected"] == 5 and r["dropped"] == 0
    assert np.array_equal(r["idx"][15:], P)
    assert np.array_equal(r["Cv"][15:], V[P]) and np.all(r["beta"][15:] == 0)
    own = orc.compact(Q, K[R], V[R], 15)
    assert np.array_equal(r["idx"][:15], R[own["idx"]])
    assert np.allclose(r["Cv"][:15], own["Cv"], atol=1e-12)
    assert np.allclose(np.logaddexp(r["rest"]["lse"], orc.row_lse(Q, K[P])), orc.row_lse(Q, K),
                       atol=1e-13)
    Qn = _rand(87, 6, 8, scale=0.5)
    za = np.exp(Qn @ own["Ck"].T + own["beta"]).sum(axis=1)[:, None]
    zb = np.exp(Qn @ K[P].T).sum(axis=1)[:, None]
    mix = (za * orc.attend(Qn, own["Ck"], own["Cv"], own["beta"]) +
           zb * orc.attend(Qn, K[P], V[P])) / (za + zb)
    assert np.allclose(orc.attend(Qn, r["Ck"], r["Cv"], r["beta"]), mix, atol=1e-13)


def test_protected_overflow_keeps_first_t_minus_one():
    Q, K, V = _rand(88, 10, 4, scale=0.5), _rand(89, 30, 4), _rand(90, 30, 2)
    prot = np.zeros(30, bool)
    prot[[2, 4, 6, 8, 10, 12]] = True
    r = orc.compact_protected(Q, K, V, 4, prot)
    assert r["n_protected"] == 3 and r["dropped"] == 3
    assert list(r["idx"][1:]) == [2, 4, 6]
    assert r["idx"][0] not in (2, 4, 6)


# ------------------------------------------ appended fixed block (f4, P7)
def test_exact_compaction_survives_any_appended_block():
    """Duplicated keys fitted exactly (w = multiplicity, C_v = mean over the
    copies) match output and mass for every query; by the block decomposition
    the attention then stays exact with any block appended after the cache."""
    rng = np.random.default_rng(91)
    t, d = 6, 5
    base = rng.standard_normal((t, d))
    mult = np.array([2, 1, 4, 3, 1, 2])
    rows = rng.permutation(np.repeat(np.arange(t), mult))
    K, V = base[rows], rng.standard_normal((rows.size, 3))
    first = np.sort([np.flatnonzero(rows == j)[0] for j in range(t)])
    Q = rng.standard_normal((20, d)) * 0.5
    w, beta, Cv, _ = orc.fit(Q, K, V, first, ridge_rel=1e-12)
    Kf, Vf = rng.standard_normal((7, d)), rng.standard_normal((7, 3))
    Qn = rng.standard_normal((9, d)) * 0.5
    o_c, l_c = orc.attend_appended(Qn, K[first], Cv, beta, Kf, Vf)
    o_f, l_f = orc.attend_appended(Qn, K, V, None, Kf, Vf)
    assert np.allclose(o_c, o_f, atol=1e-7) and np.allclose(l_c, l_f, atol=1e-7)
    # and the lse is the whole concatenation's (block identity)
    assert np.allclose(l_f, np.logaddexp(orc.row_lse(Qn, K), orc.row_lse(Qn, Kf)), atol=1e-13)


def test_attend_appended_matches_scalar_loops():
    rng = np.random.default_rng(92)
    Q, K1, V1 = rng.standard_normal((3, 4)), rng.standard_normal((5, 4)), rng.standard_normal((5, 2))
    K2, V2 = rng.standard_normal((2, 4)), rng.standard_normal((2, 2))
    b1 = np.array([0.5, -np.inf, 0.0, 1.5, -2.0])
    o, lse = orc.attend_appended(Q, K1, V1, b1, K2, V2)
    for i in range(3):
        s = [math.fsum(Q[i, c] * K1[j, c] for c in range(4)) + b1[j] for j in range(5)]
        s += [math.fsum(Q[i, c] * K2[j, c] for c in range(4)) for j in range(2)]
        vs = list(V1) + list(V2)
        z = math.fsum(math.exp(x) for x in s)
        assert abs(lse[i] - math.log(z)) < 1e-13
        for c in range(2):
            assert abs(o[i, c] - math.fsum(math.exp(x) * v[c] for x, v in zip(s, vs)) / z) < 1e-13


# ------------------------------------------------ greedy selection (f3)
@pytest.mark.parametrize("seed", range(4))
def test_omp_first_pick_is_best_single_key_fit(seed):
    """Step 1 of the pursuit = the key whose column alone fits y = 1 best in
    least squares (brute force over keys: ||y||^2 - (p.y)^2 / ||p||^2)."""
    rng = np.random.default_rng(100 + seed)
    P = rng.random((15, 40)) ** 3
    _, order, norms = orc.omp_select(P, 1)
    res = [np.linalg.norm(np.ones(15) - P[:, [j]] @ np.linalg.lstsq(P[:, [j]], np.ones(15),
                                                                       rcond=None)[0])
           for j in range(40)]
    assert order[0] == int(np.argmin(res))
    assert abs(norms[0] - min(res)) < 1e-12


def test_omp_orthogonal_dictionary_recovers_exact_support():
    """Columns with disjoint supports are orthogonal: if y = 1 is a positive
    combination of k of them, the pursuit picks exactly those k (textbook
    exact recovery) and the residual vanishes; distractors overlap no more
    than half a block."""
    n = 24
    blocks = [range(0, 6), range(6, 10), range(10, 18), range(18, 24)]
    P = np.zeros((n, 9))
    for c, blk in zip((1, 4, 6, 8), blocks):
        P[list(blk), c] = 0.5
    P[[0, 1, 2], 0] = 0.9       # distractors: part of one block each
    P[[6, 7], 2] = 0.4
    P[[10, 11, 12], 3] = 0.3
    P[[18, 19, 20], 5] = 0.7
    P[[12], 7] = 1.0
    idx, order, norms = orc.omp_select(P, 4)
    assert list(idx) == [1, 4, 6, 8]
    assert norms[-1] < 1e-12
    assert np.all(np.diff(norms) <= 1e-15)


def test_omp_residual_orthogonal_and_duplicates_skipped():
    """After each step the residual is orthogonal to every chosen column (the
    'orthogonal' of the pursuit), so an exact duplicate of a chosen column
    scores zero and is not picked while another column correlates."""
    rng = np.random.default_rng(7)
    P = rng.random((30, 12))
    P[:, 5] = P[:, 2]
    for t in range(1, 8):
        _, order, _ = orc.omp_select(P, t)
        A = P[:, order]
        r = np.ones(30) - A @ np.linalg.lstsq(A, np.ones(30), rcond=None)[0]
        assert np.max(np.abs(A.T @ r)) < 1e-10
        assert not (2 in order and 5 in order)


def test_omp_keep_everything_is_exact_and_zero_columns_last():
    Q, K, V = _rand(110, 20, 6, scale=0.4), _rand(111, 16, 6), _rand(112, 16, 3)
    r = orc.compact_omp(Q, K, V, 16)
    assert list(r["idx"]) == list(range(16))
    assert np.allclose(r["Cv"], V, atol=1e-8)
    P = np.abs(_rand(113, 10, 6))
    P[:, [1, 4]] = 0.0
    _, order, _ = orc.omp_select(P, 6)
    assert list(order[-2:]) == [1, 4]


def _softmax_weights_by_loops(Q, K):
    """p_ij = exp(q_i . k_j) / sum_k exp(q_i . k_k), scalar math.fsum loops."""
    n, T, d = Q.shape[0], K.shape[0], Q.shape[1]
    P = np.zeros((n, T))
    for i in range(n):
        s = [math.fsum(Q[i, c] * K[j, c] for c in range(d)) for j in range(T)]
        z = math.fsum(math.exp(x) for x in s)
        for j in range(T):
            P[i, j] = math.exp(s[j]) / z
    return P


def test_omp_dictionary_is_the_full_cache_softmax():
    """The greedy selection's dictionary is the whole-cache softmax weights in
    float64: scalar loops agree to 1e-15, every row sums to one over the T keys
    (a dropped log-sum-exp breaks this), zero queries give 1/T everywhere, and
    its column RMS and column mean are the two aggregators' importances."""
    Q, K, V = _rand(120, 6, 4, scale=0.8), _rand(121, 13, 4), _rand(122, 13, 2)
    lse = orc.row_lse(Q, K)
    P = orc.omp_dictionary(Q, K, lse)
    assert P.dtype == np.float64 and P.shape == (6, 13)
    assert np.max(np.abs(P - _softmax_weights_by_loops(Q, K))) < 1e-15
    assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    _, imp_rms = orc.attention_stats(Q, K, V, lse, agg="rms")
    _, imp_mean = orc.attention_stats(Q, K, V, lse, agg="mean")
    assert np.allclose(np.sqrt((P * P).mean(axis=0)), imp_rms, rtol=1e-13, atol=0)
    assert np.allclose(P.mean(axis=0), imp_mean, rtol=1e-13, atol=0)
    Z = np.zeros((3, 4))
    assert np.allclose(orc.omp_dictionary(Z, K, orc.row_lse(Z, K)), 1.0 / 13, rtol=1e-14, atol=0)
    # not rounded to a storage precision: weights that differ below float32's
    # resolution stay distinct
    K2 = np.zeros((3, 1))
    K2[:, 0] = [0.0, 1e-9, 2e-9]
    Q2 = np.ones((1, 1))
    P2 = orc.omp_dictionary(Q2, K2, orc.row_lse(Q2, K2))
    assert P2[0, 0] < P2[0, 1] < P2[0, 2]


def _greedy_by_brute_force(Q, K, t):
    """Matching pursuit written out by hand: softmax weights by scalar loops;
    at each step every unchosen key's column is scored by
    sum_i p_ij r_i / sqrt(sum_i p_ij^2) with math.fsum (the reduction of
    ||r||^2 a non-negative single-column fit would give, signed), the first
    best key (lowest index on equal scores) is taken, and the residual is
    y = 1 minus its least-squares fit on the chosen columns, solved through
    the normal equations (a different route from the oracle's lstsq)."""
    P = _softmax_weights_by_loops(Q, K)
    n, T = P.shape
    y = np.ones(n)
    r = y.copy()
    order = []
    for _ in range(t):
        best, bj = -math.inf, -1
        for j in range(T):
            if j in order:
                continue
            nrm = math.sqrt(math.fsum(P[i, j] ** 2 for i in range(n)))
            c = math.fsum(P[i, j] * r[i] for i in range(n)) / nrm
            if c > best:
                best, bj = c, j
        order.append(bj)
        A = P[:, order]
        w = np.linalg.solve(A.T @ A, A.T @ y)
        r = y - A @ w
    return order


@pytest.mark.parametrize("seed", range(4))
def test_compact_omp_matches_brute_force_greedy(seed):
    """compact_omp at t < T picks, in order, the keys the hand-written pursuit
    picks (softmax by loops, scores by fsum, residual by normal equations)."""
    rng = np.random.default_rng(130 + seed)
    T, t = 11, 4
    Q = rng.standard_normal((16, 5)) * 0.9
    K = rng.standard_normal((T, 5))
    V = rng.standard_normal((T, 3))
    ref = _greedy_by_brute_force(Q, K, t)
    r = orc.compact_omp(Q, K, V, t)
    assert list(r["order"]) == ref
    assert list(r["idx"]) == sorted(ref)
