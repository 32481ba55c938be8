"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.  Bars: kept indices identical up to near-ties below
1e-6 relative importance gap; multipliers w, fitted values and the compacted
attention output within 2e-3 relative L2 for bf16 inputs, 1e-4 for float32."""
import dataclasses

import numpy as np
import pytest

import oracle as orc
import synth
from parity import TOL_BF16, TOL_F32, compare_head, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _tol(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


SMALL = [
    synth.CONFIGS[1],
    synth.custom(1, 3, 1000, 200, 128, 77, "bf16", "clusters"),          # ragged T, n, t
    synth.custom(2, 2, 4096, 256, 64, 100, "bf16", "channel_lognormal"),  # d = 64
    synth.custom(3, 2, 777, 130, 128, 64, "f32", "sinks"),               # fp32, d = 128
    synth.custom(4, 1, 2500, 384, 128, 250, "bf16", "student_t3"),
    synth.custom(5, 4, 640, 64, 128, 1, "bf16", "normal"),               # t = 1
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_cases_match_oracle(w):
    data = synth.batch(w)
    gpu = run_gpu(w, data)
    for h in range(w.B):
        err = compare_head(gpu, h, data, w.t, _tol(w))
        print(w.name, h, {k: (round(v, 9) if isinstance(v, float) else v) for k, v in err.items()},
              flush=True)


def test_mean_aggregator():
    w = synth.custom(6, 2, 1500, 128, 128, 120, "bf16", "clusters")
    data = synth.batch(w)
    gpu = run_gpu(w, data, agg="mean")
    for h in range(w.B):
        compare_head(gpu, h, data, w.t, TOL_BF16, agg="mean")


@pytest.mark.parametrize("n", [40, 130])
def test_keep_everything_is_exact(n):
    """t = T: every index kept, w = 1, C_v = V (the ridge prior makes this the
    unique zero-loss point for any n).  The GPU's P_S rows carry the float32
    log-sum-exp's rounding (~1e-7 relative); with n > T that perturbs the
    least-squares point by about cond(P) * 1e-7, hence the 1e-4 bound."""
    w = synth.custom(7, 2, 96, n, 128, 96, "bf16", "normal")
    data = synth.batch(w)
    gpu = run_gpu(w, data)
    for h in range(w.B):
        assert list(gpu["idx"][h]) == list(range(96))
        assert np.allclose(gpu["w"][h], 1.0, atol=1e-4)
        V = synth.to_f64(data["V"][h])
        assert orc.rel_l2(gpu["values"][h], V) < 1e-4


def test_zero_queries_tie_rule_and_closed_form():
    """q = 0: all importances tie -> indices 0..t-1; w = (T + rho)/(t + rho)."""
    w = synth.custom(8, 2, 700, 64, 128, 50, "bf16", "normal")
    data = synth.batch(w)
    data["Q"][:] = 0
    gpu = run_gpu(w, data, ridge_rel=1e-2)
    for h in range(w.B):
        assert list(gpu["idx"][h]) == list(range(50))
        assert np.allclose(gpu["w"][h], (700 + 1e-2) / (50 + 1e-2), rtol=1e-6)


def test_duplicated_keys_fit_recovers_multiplicities():
    """kvc_fit on the first copies of t distinct keys repeated m_j times:
    w_j = m_j and C_v,j = mean of V over the copies (ridge -> 0)."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    rng = np.random.default_rng(9)
    t, d = 6, 128
    mult = np.array([1, 3, 2, 5, 1, 4])
    rows = rng.permutation(np.repeat(np.arange(t), mult))
    base = rng.standard_normal((t, d)) * 0.7
    K = synth.round_bf16_bits(base[rows])
    V = synth.round_bf16_bits(rng.standard_normal((rows.size, d)))
    Q = synth.round_bf16_bits(rng.standard_normal((64, d)) / np.sqrt(d))
    first = np.sort([np.flatnonzero(rows == j)[0] for j in range(t)])
    res = kvc.fit(to_device(Q[None]), to_device(K[None]), to_device(V[None]),
                  torch.from_numpy(first.astype(np.int32)[None]).cuda(), ridge_rel=1e-12)
    torch.cuda.synchronize()
    wgpu = kvc.intermediates(res)["w"].cpu().numpy()[0]
    assert np.allclose(wgpu, mult[rows[first]], rtol=1e-6)
    Vf = synth.to_f64(V)
    means = np.array([Vf[rows == rows[j]].mean(axis=0) for j in first])
    assert orc.rel_l2(res.values.cpu().numpy()[0], means) < 1e-5


def test_bitwise_deterministic():
    w = synth.custom(10, 2, 3000, 300, 128, 90, "bf16", "clusters")
    data = synth.batch(w)
    a, b = run_gpu(w, data), run_gpu(w, data)
    for k in ("idx", "bias", "values", "lse", "O", "imp", "w"):
        assert np.array_equal(a[k], b[k]), k


def test_nonfinite_input_is_flagged():
    w = synth.custom(11, 2, 512, 64, 128, 16, "bf16", "normal")
    data = synth.batch(w)
    data["K"][1, 3, 5] = 0x7FC0  # NaN in head 1
    gpu = run_gpu(w, data)
    assert gpu["status"][0] == 0
    assert gpu["status"][1] & 4


@pytest.mark.parametrize("cfg,heads", [(2, list(range(8))), (3, list(range(8))),
                                       (4, [0, 131, 255]), (5, [3])])
def test_full_configs(cfg, heads):
    """The full-size workloads, launched exactly as the benchmark times them
    (the score kernels' full-size split counts): every head of the 8-head
    layers, a sample of the 256-head stack and of the 128k-token layer, each
    compared with the oracle in full, lse, O and importance included (lse
    within 1e-4 absolute, O and importance within 1e-4 relative)."""
    w = synth.CONFIGS[cfg]
    data = synth.batch(w)
    gpu = run_gpu(w, data)
    assert (gpu["status"] == 0).all(), gpu["status"]
    for h in heads:
        err = compare_head(gpu, h, data, w.t, _tol(w))
        print(f"C{cfg} head {h}:", {k: (float(f"{v:.3g}") if isinstance(v, float) else v)
                                    for k, v in err.items()}, flush=True)


@pytest.mark.parametrize("seed,T,n,d,t,keys", [(60, 2048, 512, 128, 600, "clusters"),
                                                (61, 2048, 512, 64, 333, "student_t3")])
def test_value_elimination_on_one_workgroup_teams(seed, T, n, d, t, keys):
    """256 heads give each head a team of one workgroup, whose value system is
    solved by forward elimination and back substitution (the sweep's swept
    bands left alone): the fitted values of sampled heads against the
    oracle's least squares, with ragged last bands (m not a multiple of 64)
    and one or two right-hand-side bands."""
    w = synth.custom(seed, 256, T, n, d, t, "bf16", keys)
    data = synth.batch(w)
    gpu = run_gpu(w, data)
    assert (gpu["status"] == 0).all(), gpu["status"]
    for h in (0, 77, 255):
        err = compare_head(gpu, h, data, w.t, _tol(w))
        print(f"elim head {h}:", {k: (float(f"{v:.3g}") if isinstance(v, float) else v)
                                  for k, v in err.items()}, flush=True)


@pytest.mark.parametrize("seed,T,n,t,keys", [(62, 4096, 1024, 680, "clusters"),
                                              (63, 3000, 900, 650, "sinks")])
def test_bias_sweep_rhs_column_outside_the_tiles(seed, T, n, t, keys):
    """Eleven variable bands (t in 641..704) on teams of 32 workgroups (two
    heads): the bias sweep updates its one right-hand-side column after the
    tile tasks and takes each diagonal tile as one task, so every task has a
    wave of its own.  Every head against the oracle."""
    w = synth.custom(seed, 2, T, n, 128, t, "bf16", keys)
    data = synth.batch(w)
    gpu = run_gpu(w, data)
    assert (gpu["status"] == 0).all(), gpu["status"]
    for h in range(w.B):
        err = compare_head(gpu, h, data, w.t, _tol(w))
        print(f"rhs-column head {h}:", {k: (float(f"{v:.3g}") if isinstance(v, float) else v)
                                        for k, v in err.items()}, flush=True)


def _chunk_view(w, data, gpu_res, C):
    """Recast a chunked result as B*C independent heads (entry h*C + c is chunk c
    of head h, with chunk-local indices) so each entry compares against the
    oracle's compaction of that chunk alone."""
    import kv_cache_compaction_head_amd as kvc
    B, T, t = w.B, w.T, w.t
    Tc = T // C
    cd = {"Q": np.repeat(data["Q"], C, axis=0),
          "K": data["K"].reshape(B * C, Tc, -1), "V": data["V"].reshape(B * C, Tc, -1)}
    idx = gpu_res.idx.cpu().numpy().astype(np.int64).reshape(B, C, t)
    off = (np.arange(C) * Tc)[None, :, None]
    assert np.all((idx >= off) & (idx < off + Tc)), "kept index outside its chunk"
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(gpu_res).items()}
    g = {"keys": gpu_res.keys.cpu().reshape(B * C, t, -1),
         "bias": gpu_res.bias.cpu().numpy().astype(np.float64).reshape(B * C, t),
         "values": gpu_res.values.cpu().numpy().astype(np.float64).reshape(B * C, t, -1),
         "idx": (idx - off).reshape(B * C, t),
         "status": gpu_res.status.cpu().numpy().reshape(B * C), **inter}
    return cd, g


@pytest.mark.parametrize("w,C", [
    (synth.custom(12, 2, 3000, 200, 128, 77, "bf16", "clusters"), 3),
    (synth.custom(13, 1, 2048, 96, 64, 40, "f32", "sinks"), 4),
], ids=["bf16_C3", "f32_d64_C4"])
def test_chunked_matches_oracle_per_chunk(w, C):
    import torch
    import kv_cache_compaction_head_amd as kvc
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_chunked(Q, K, V, w.t, C)
    torch.cuda.synchronize()
    assert res.idx.shape == (w.B, C * w.t) and res.status.shape == (w.B, C)
    cd, g = _chunk_view(w, data, res, C)
    for e in range(w.B * C):
        err = compare_head(g, e, cd, w.t, _tol(w))
        print(w.name, "head", e // C, "chunk", e % C,
              {k: (float(f"{v:.3g}") if isinstance(v, float) else v) for k, v in err.items()},
              flush=True)
    # the merged cache, read as one head, against the oracle's merged cache
    for h in range(w.B):
        Qh, Kh, Vh = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
        ref = orc.compact_chunked(Qh, Kh, Vh, w.t, C)
        o_gpu = orc.attend(Qh, res.keys[h].float().cpu().numpy().astype(np.float64),
                           res.values[h].cpu().numpy().astype(np.float64),
                           res.bias[h].cpu().numpy().astype(np.float64))
        o_ref = orc.attend(Qh, ref["Ck"], ref["Cv"], ref["beta"])
        assert orc.rel_l2(o_gpu, o_ref) <= _tol(w)


def test_chunked_one_chunk_is_bitwise_compact():
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(14, 2, 1200, 128, 128, 60, "bf16", "clusters")
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    a = kvc.compact(Q, K, V, w.t)
    b = kvc.compact_chunked(Q, K, V, w.t, 1)
    torch.cuda.synchronize()
    for k in ("keys", "bias", "values", "idx"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    assert torch.equal(a.status, b.status.view(-1))
    with pytest.raises(ValueError):
        kvc.compact_chunked(Q, K, V, w.t, 7)      # 1200 % 7 != 0
    with pytest.raises(ValueError):
        kvc.compact_chunked(Q, K, V, 601, 2)      # t > T / C


def test_chunked_long_context_sampled():
    """131072 keys per head in 4 chunks of 32768 (each kept at 50x), the
    long-context shape the chunking is for; a sample of (head, chunk) entries
    against the oracle."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w0 = synth.CONFIGS[5]
    C = 4
    w = dataclasses.replace(w0, t=w0.t // C)
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_chunked(Q, K, V, w.t, C)
    torch.cuda.synchronize()
    assert (res.status.cpu().numpy() == 0).all()
    cd, g = _chunk_view(w, data, res, C)
    for e in (3 * C + 0, 3 * C + 3, 6 * C + 1):
        err = compare_head(g, e, cd, w.t, _tol(w), tight=False)
        print("C5/4 entry", e, {k: (float(f"{v:.3g}") if isinstance(v, float) else v)
                                for k, v in err.items()}, flush=True)


@pytest.mark.parametrize("w,budgets", [
    (synth.custom(15, 4, 2000, 160, 128, 0, "bf16", "clusters"), [40, 131, 1, 64]),
    (synth.custom(16, 3, 900, 96, 64, 0, "f32", "normal"), [200, 65, 128]),
    # one head with eleven variable bands (its right-hand-side column updated
    # outside the tile tasks), one with ten (the usual split)
    (synth.custom(17, 2, 3000, 1024, 128, 0, "bf16", "clusters"), [690, 600]),
], ids=["bf16", "f32_d64", "bf16_11_10_bands"])
def test_ragged_budgets_match_oracle_per_head(w, budgets):
    """kvc_compact_ragged: head b against the oracle's compaction at its own
    budget; the padded slots are inert (index -1, zero rows, bias -inf)."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_ragged(Q, K, V, budgets)
    torch.cuda.synchronize()
    tm = max(budgets)
    assert res.idx.shape == (w.B, tm)
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    idx = res.idx.cpu().numpy().astype(np.int64)
    bias = res.bias.cpu().numpy().astype(np.float64)
    vals = res.values.cpu().numpy().astype(np.float64)
    keys = res.keys.float().cpu().numpy()
    st = res.status.cpu().numpy()
    for h, tb in enumerate(budgets):
        assert np.all(idx[h, tb:] == -1) and np.all(np.isneginf(bias[h, tb:]))
        assert not keys[h, tb:].any() and not vals[h, tb:].any()
        g = {"keys": res.keys[h:h + 1, :tb].cpu(), "bias": bias[h:h + 1, :tb],
             "values": vals[h:h + 1, :tb], "idx": idx[h:h + 1, :tb], "status": st[h:h + 1],
             "lse": inter["lse"][h:h + 1], "O": inter["O"][h:h + 1],
             "imp": inter["imp"][h:h + 1], "w": inter["w"][h:h + 1, :tb]}
        hd = {k: data[k][h:h + 1] for k in ("Q", "K", "V")}
        err = compare_head(g, 0, hd, tb, _tol(w))
        print(w.name, "head", h, "t", tb, {k: (float(f"{v:.3g}") if isinstance(v, float) else v)
                                            for k, v in err.items()}, flush=True)
        Qh = synth.to_f64(data["Q"][h])
        o_pad = orc.attend(Qh, keys[h].astype(np.float64), vals[h], bias[h])
        o_own = orc.attend(Qh, keys[h, :tb].astype(np.float64), vals[h, :tb], bias[h, :tb])
        assert orc.rel_l2(o_pad, o_own) < 1e-12


def test_ragged_equal_budgets_is_bitwise_compact_and_clamps():
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(17, 3, 1100, 128, 128, 70, "bf16", "sinks")
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    a = kvc.compact(Q, K, V, w.t)
    b = kvc.compact_ragged(Q, K, V, [w.t] * w.B)
    torch.cuda.synchronize()
    for k in ("keys", "bias", "values", "idx", "status"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    # a budget of 0 is clamped to 1 and flagged (status bit 16)
    c = kvc.compact_ragged(Q, K, V, [0, 5, 70])
    torch.cuda.synchronize()
    st = c.status.cpu().numpy()
    assert st[0] == 16 and st[1] == 0 and st[2] == 0
    assert (c.idx[0, 1:] == -1).all() and c.idx[0, 0] >= 0


@pytest.mark.parametrize("w,frac", [
    (synth.custom(18, 3, 2400, 192, 128, 90, "bf16", "clusters"), 0.01),
    (synth.custom(19, 2, 1000, 64, 64, 48, "f32", "sinks"), 0.02),
    (synth.custom(24, 2, 1500, 96, 64, 60, "bf16", "normal"), 0.03),   # ragged T, d = 64
], ids=["bf16", "f32_d64", "bf16_d64"])
def test_protected_keys_match_oracle(w, frac):
    """kvc_compact_protected against the oracle: protected slots exact (bias 0),
    the fitted part against the oracle's compaction of the unprotected keys
    (their own lse, output and importance; protected keys carry importance 0)."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    data = synth.batch(w)
    rng = np.random.default_rng(w.cfg)
    prot = rng.random((w.B, w.T)) < frac
    prot[:, 0] = True                      # a sink-like first token
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_protected(Q, K, V, w.t, torch.from_numpy(prot))
    torch.cuda.synchronize()
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    idx = res.idx.cpu().numpy().astype(np.int64)
    bias = res.bias.cpu().numpy().astype(np.float64)
    vals = res.values.cpu().numpy().astype(np.float64)
    st = res.status.cpu().numpy()
    for h in range(w.B):
        P = np.flatnonzero(prot[h])
        assert P.size <= w.t - 1
        R = np.flatnonzero(~prot[h])
        tb = w.t - P.size
        Kf, Vf = synth.to_f64(data["K"][h]), synth.to_f64(data["V"][h])
        assert np.array_equal(idx[h, tb:], P)
        assert np.all(bias[h, tb:] == 0.0)
        assert np.array_equal(vals[h, tb:], Vf[P])
        assert np.array_equal(res.keys[h, tb:].float().cpu().numpy().astype(np.float64), Kf[P])
        assert np.all(inter["imp"][h][P] == 0.0)
        loc = np.searchsorted(R, idx[h, :tb])
        assert np.array_equal(R[loc], idx[h, :tb])
        g = {"keys": res.keys[h:h + 1, :tb].cpu(), "bias": bias[h:h + 1, :tb],
             "values": vals[h:h + 1, :tb], "idx": loc[None], "status": st[h:h + 1],
             "lse": inter["lse"][h:h + 1], "O": inter["O"][h:h + 1],
             "imp": inter["imp"][h:h + 1][:, R], "w": inter["w"][h:h + 1, :tb]}
        hd = {"Q": data["Q"][h:h + 1], "K": data["K"][h:h + 1][:, R],
              "V": data["V"][h:h + 1][:, R]}
        err = compare_head(g, 0, hd, tb, _tol(w))
        print(w.name, "head", h, "protected", P.size,
              {k: (float(f"{v:.3g}") if isinstance(v, float) else v) for k, v in err.items()},
              flush=True)
        Qh = synth.to_f64(data["Q"][h])
        ref = orc.compact_protected(Qh, Kf, Vf, w.t, prot[h])
        o_gpu = orc.attend(Qh, res.keys[h].float().cpu().numpy().astype(np.float64), vals[h],
                           bias[h])
        o_ref = orc.attend(Qh, ref["Ck"], ref["Cv"], ref["beta"])
        assert orc.rel_l2(o_gpu, o_ref) <= _tol(w)


def test_protected_none_is_bitwise_compact_and_overflow_flags():
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(20, 2, 800, 96, 128, 40, "bf16", "normal")
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    a = kvc.compact(Q, K, V, w.t)
    none = torch.zeros((w.B, w.T), dtype=torch.uint8)
    b = kvc.compact_protected(Q, K, V, w.t, none)
    torch.cuda.synchronize()
    for k in ("keys", "bias", "values", "idx", "status"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    many = torch.zeros((w.B, w.T), dtype=torch.uint8)
    many[1, ::10] = 1                        # 80 marks > t - 1 = 39
    c = kvc.compact_protected(Q, K, V, w.t, many)
    torch.cuda.synchronize()
    st = c.status.cpu().numpy()
    assert st[0] == 0 and st[1] == 32
    assert c.idx[1, 1:].cpu().tolist() == list(range(0, 390, 10))


@pytest.mark.parametrize("dtype,d,t1,t2,m", [("bf16", 128, 700, 37, 130), ("f32", 64, 65, 0, 64),
                                             ("bf16", 64, 0, 200, 1), ("f32", 128, 1, 1, 300)])
def test_attend_matches_oracle(dtype, d, t1, t2, m):
    """kvc_attend: the float32 online-softmax kernel against the float64
    definition, with a bias that includes -inf (a zero-weight key)."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    rng = np.random.default_rng(t1 * 7 + t2)
    B = 2

    def arr(*shape, scale=1.0):
        x = rng.standard_normal(shape) * scale
        return synth.round_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    Q, K1, K2, V2 = arr(B, m, d, scale=d ** -0.5), arr(B, t1, d), arr(B, t2, d), arr(B, t2, d)
    V1 = rng.standard_normal((B, t1, d)).astype(np.float32)
    b1 = (rng.standard_normal((B, t1)) * 2).astype(np.float32)
    if t1 > 3:
        b1[:, 3] = -np.inf
    out, lse = kvc.attend(to_device(Q), to_device(K1), torch.from_numpy(V1).cuda(),
                          torch.from_numpy(b1).cuda(),
                          to_device(K2) if t2 else None, to_device(V2) if t2 else None)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy()
    f = synth.to_f64 if dtype == "bf16" else (lambda x: x.astype(np.float64))
    for h in range(B):
        o_ref, l_ref = orc.attend_appended(f(Q[h]), f(K1[h]), V1[h].astype(np.float64),
                                           b1[h].astype(np.float64), f(K2[h]), f(V2[h]))
        assert orc.rel_l2(out[h], o_ref) < 2e-6
        assert np.max(np.abs(lse[h] - l_ref)) < 1e-4


def test_compacted_cache_with_appended_block_on_gpu():
    """The evaluation path end to end: compact on the GPU, then attend over
    [compact cache; appended block] and [full cache; appended block] with
    kvc_attend.  Each equals the float64 value of the same cache within float32
    rounding, and the compaction error with the block appended stays within
    the oracle's own error for the same setting (x1.05)."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(21, 2, 3000, 256, 128, 150, "bf16", "clusters", n_hold=96)
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact(Q, K, V, w.t)
    rng = np.random.default_rng(5)
    Kf = synth.round_bf16_bits(rng.standard_normal((w.B, 64, w.d)))
    Vf = synth.round_bf16_bits(rng.standard_normal((w.B, 64, w.d)))
    Qh = to_device(data["Qhold"])
    oc, _ = kvc.attend(Qh, res.keys, res.values, res.bias, to_device(Kf), to_device(Vf))
    of, _ = kvc.attend(Qh, K, V, None, to_device(Kf), to_device(Vf))
    torch.cuda.synchronize()
    oc, of = oc.cpu().numpy().astype(np.float64), of.cpu().numpy().astype(np.float64)
    for h in range(w.B):
        Qn = synth.to_f64(data["Qhold"][h])
        Kh, Vh = synth.to_f64(data["K"][h]), synth.to_f64(data["V"][h])
        full_ref, _ = orc.attend_appended(Qn, Kh, Vh, None, synth.to_f64(Kf[h]),
                                          synth.to_f64(Vf[h]))
        assert orc.rel_l2(of[h], full_ref) < 2e-6
        ck = res.keys[h].float().cpu().numpy().astype(np.float64)
        comp_ref, _ = orc.attend_appended(Qn, ck, res.values[h].cpu().numpy().astype(np.float64),
                                          res.bias[h].cpu().numpy().astype(np.float64),
                                          synth.to_f64(Kf[h]), synth.to_f64(Vf[h]))
        assert orc.rel_l2(oc[h], comp_ref) < 2e-6
        ref = orc.compact(synth.to_f64(data["Q"][h]), Kh, Vh, w.t)
        oracle_err = orc.rel_l2(orc.attend_appended(Qn, ref["Ck"], ref["Cv"], ref["beta"],
                                                    synth.to_f64(Kf[h]), synth.to_f64(Vf[h]))[0],
                                full_ref)
        gpu_err = orc.rel_l2(oc[h], of[h])
        print(f"head {h}: appended-block compaction error gpu {gpu_err:.4g} oracle {oracle_err:.4g}",
              flush=True)
        assert gpu_err <= oracle_err * 1.05 + 1e-5


OMP_PICK_TOL = 1e-6   # GPU pick vs float64 best, relative to the residual norm


def _omp_replay(P, order, steps, tol=OMP_PICK_TOL):
    """Check that each sampled step k of a pursuit run picked a best key given
    the run's own earlier picks.  P is the float64 dictionary; the scores
    p_j . r / ||p_j|| are bounded by ||r|| (Cauchy-Schwarz), and the GPU stores
    P in float32, which moves a score by at most 2 * 2^-24 * ||r|| plus what
    the rounded columns change in the residual; a pick is valid when its
    float64 score is within tol * ||r|| of the float64 best.  Returns the steps
    where the GPU's pick was not the float64 argmax (near-ties)."""
    n, T = P.shape
    y = np.ones(n)
    nrm = np.sqrt((P * P).sum(axis=0))
    near = []
    for k in steps:
        pre = list(order[:k])
        if pre:
            A = P[:, pre]
            r = y - A @ np.linalg.lstsq(A, y, rcond=None)[0]
        else:
            r = y
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.where(nrm > 0, (P.T @ r) / nrm, -np.inf)
        c[pre] = -np.inf
        best = c.max()
        got = c[order[k]]
        assert got >= best - tol * np.linalg.norm(r), (k, order[k], got, best)
        if order[k] != int(np.argmax(c)):
            near.append(k)
    return near


@pytest.mark.parametrize("w", [
    synth.custom(22, 2, 1000, 128, 128, 40, "bf16", "clusters"),
    synth.custom(23, 2, 777, 96, 64, 33, "f32", "normal"),
], ids=["bf16", "f32_d64"])
def test_omp_matches_oracle(w):
    """kvc_compact_omp against the float64 oracle's pursuit: every GPU pick is
    a best key (within the float32 dictionary's rounding bound) given the
    GPU's own earlier picks, the order matches the oracle's up to such
    near-ties, and the fits on the GPU's set are within the usual bar."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_omp(Q, K, V, w.t)
    torch.cuda.synchronize()
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    idx = res.idx.cpu().numpy().astype(np.int64)
    assert (res.status.cpu().numpy() == 0).all()
    for h in range(w.B):
        Qh, Kh, Vh = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
        ref = orc.compact_omp(Qh, Kh, Vh, w.t)
        order = inter["omp_order"][h].astype(np.int64)
        assert np.array_equal(np.sort(order), idx[h]) and np.all(np.diff(idx[h]) > 0)
        P = orc.omp_dictionary(Qh, Kh, ref["lse"])
        near = _omp_replay(P, order, range(w.t))
        same = np.array_equal(order, ref["order"])
        if not same:  # the first divergence is a near-tie of the float64 scores
            k = int(np.flatnonzero(order != ref["order"])[0])
            assert k in near, (k, near)
        wv, beta, Cv, _ = orc.fit(Qh, Kh, Vh, idx[h])
        err_w = orc.rel_l2(inter["w"][h], wv)
        err_c = orc.rel_l2(res.values[h].cpu().numpy().astype(np.float64), Cv)
        o_gpu = orc.attend(Qh, Kh[idx[h]], res.values[h].cpu().numpy().astype(np.float64),
                           res.bias[h].cpu().numpy().astype(np.float64))
        err_o = orc.rel_l2(o_gpu, orc.attend(Qh, Kh[idx[h]], Cv, beta))
        print(w.name, "head", h, "same order", same, "near-ties", near, "w", err_w, "Cv", err_c,
              "Ohat", err_o, flush=True)
        assert max(err_w, err_c, err_o) <= _tol(w)


def test_omp_full_size_sampled_steps():
    """32768 keys, 2048 queries, 655 picks per head (the 32k/50x workload):
    sampled steps of the GPU's pursuit replayed against the oracle given the
    GPU's own earlier picks; the fits of one head against the oracle."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = dataclasses.replace(synth.CONFIGS[3], B=2)
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_omp(Q, K, V, w.t)
    torch.cuda.synchronize()
    assert (res.status.cpu().numpy() == 0).all()
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    h = 1
    Qh, Kh, Vh = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
    lse = orc.row_lse(Qh, Kh)
    assert np.max(np.abs(inter["lse"][h] - lse)) < 1e-4
    P = orc.omp_dictionary(Qh, Kh, lse)
    order = inter["omp_order"][h].astype(np.int64)
    assert len(set(order.tolist())) == w.t
    _omp_replay(P, order, [0, 1, 2, 50, 300, w.t - 1])
    idx = res.idx[h].cpu().numpy().astype(np.int64)
    wv, beta, Cv, _ = orc.fit(Qh, Kh, Vh, idx)
    o_gpu = orc.attend(Qh, Kh[idx], res.values[h].cpu().numpy().astype(np.float64),
                       res.bias[h].cpu().numpy().astype(np.float64))
    err = orc.rel_l2(o_gpu, orc.attend(Qh, Kh[idx], Cv, beta))
    print("omp C3 head 1: Ohat vs oracle fits", err, flush=True)
    assert orc.rel_l2(inter["w"][h], wv) <= TOL_BF16 and err <= TOL_BF16


@pytest.mark.slow
def test_omp_full_size_chosen_set():
    """One head of the 32k/50x workload: the GPU's whole pursuit against the
    float64 oracle's.  Either the pick orders agree, or at the first step where
    they part the GPU's pick is a near-tie of the float64 scores given the same
    earlier picks (the two runs then continue from different residuals, so
    later picks are not comparable one by one); the chosen sets are reported."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = dataclasses.replace(synth.CONFIGS[3], B=1)
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact_omp(Q, K, V, w.t)
    torch.cuda.synchronize()
    assert (res.status.cpu().numpy() == 0).all()
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    order = inter["omp_order"][0].astype(np.int64)
    Qh, Kh, Vh = (synth.to_f64(data[k][0]) for k in ("Q", "K", "V"))
    ref = orc.compact_omp(Qh, Kh, Vh, w.t)
    common = len(set(order.tolist()) & set(ref["order"].tolist()))
    same = np.array_equal(order, ref["order"])
    print(f"omp C3 head 0: same order {same}, chosen sets share {common} of {w.t}", flush=True)
    if not same:
        k = int(np.flatnonzero(order != ref["order"])[0])
        P = orc.omp_dictionary(Qh, Kh, ref["lse"])
        near = _omp_replay(P, order, [k])
        print(f"first divergence at step {k}: near-tie {k in near}", flush=True)
        assert k in near, (k, near)


def _value_gradient(Q, K, V, idx, lse, w, O, CF, ridge_rel, t):
    """Relative size of the value fit's optimality gradient (oracle pin P3)
    for the GPU's kept set, multipliers and float64 solution CF (passive
    slots in order):
    g = X_F^T (X_F C_F - O) + lam_v (C_F - V_F), over ||X_F^T O|| + lam_v ||V_F||,
    with X_F = P_S[:, F] diag(w_F) / r and lam_v = ridge_rel tr(X_F^T X_F) / t."""
    F = np.flatnonzero(w > 0)
    P = np.exp(Q @ K[idx[F]].T - lse[:, None])
    Xw = P * w[F][None, :]
    X = Xw / Xw.sum(axis=1, keepdims=True)
    lam = ridge_rel * float((X * X).sum()) / t
    VF = V[idx[F]]
    C = CF[:F.size]
    g = X.T @ (X @ C - O) + lam * (C - VF)
    return float(np.linalg.norm(g) / (np.linalg.norm(X.T @ O) + lam * np.linalg.norm(VF)))


def test_value_refinement_reduces_the_normal_equation_error():
    """refine_steps > 0 takes corrected semi-normal-equation steps on the value
    fit.  The swept normal equations leave a gradient of about cond(G) times
    the unit roundoff in the float64 solution; a step against O itself
    removes most of it, and further steps keep it there.  The fitted values
    move by far less than the parity bar, and the other outputs do not move."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(8, 2, 4096, 512, 128, 300, "bf16", "clusters")
    data = synth.batch(w)
    Qd, Kd, Vd = (to_device(data[k]) for k in ("Q", "K", "V"))
    rr = 1e-9
    out = {}
    for steps in (0, 1, 2):
        res = kvc.compact(Qd, Kd, Vd, w.t, ridge_rel=rr, refine_steps=steps)
        torch.cuda.synchronize()
        inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
        out[steps] = {"values": res.values.cpu().numpy().astype(np.float64),
                      "bias": res.bias.cpu().numpy(), "idx": res.idx.cpu().numpy(),
                      "status": res.status.cpu().numpy(), **inter}
        assert not out[steps]["status"].any(), out[steps]["status"]
    for h in range(w.B):
        Q, K, V = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
        g = {}
        for steps in (0, 1, 2):
            o = out[steps]
            assert np.array_equal(o["idx"][h], out[0]["idx"][h])
            assert np.array_equal(o["bias"][h], out[0]["bias"][h])
            g[steps] = _value_gradient(Q, K, V, o["idx"][h], o["lse"][h], o["w"][h],
                                       o["O"][h].astype(np.float64), o["value_C"][h], rr, w.t)
            assert orc.rel_l2(o["values"][h], out[0]["values"][h]) < 1e-5
        print("head", h, "gradient", g, flush=True)
        assert g[1] < 1e-11 and g[2] < 1e-11, g
        assert g[0] > 1e-15 and g[1] < g[0] / 10, g
