"""Benchmark: KV tokens compacted per second on one MI355X.

Workload: one Llama-3-8B-shaped layer, 8 KV heads x d = 128, T = 32768 cached
tokens per head, 2048 reference queries per head, keep t = 655 (50x), keys from
a 64-cluster mixture, bf16 (synthetic, seeded).  One step = one kvc_compact
call over all 8 heads: scores + log-sum-exp, full-cache output and importance,
top-t select and gather, NNLS bias fit and least-squares value fit.

Prints one JSON line.  `value` = B*T / (seconds per step), inputs resident in
HBM before the timed region.  Also reported: the dominant kernel against its
roofline (algorithmic work / measured duration, HIP events on the library's
stream), the float64 CPU oracle on a bounded sample, and the compacted
attention's relative L2 error on held-out queries.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 MFMA (and packed-fp32 vector)
PEAK_F32_VALU_TFLOPS = 78.6  # fp32 vector FMA without packed ops: 256 CU x 64 lanes x 2 x 2.4 GHz
PEAK_F64_TFLOPS = 78.6       # MI355X fp64 (vector and matrix)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_nnls_sweep_T32k_50x_hbm_traffic.md")
FIT_SRC = os.path.join(ROOT, "kv_cache_compaction_head_amd", "csrc", "fit.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="synthetic workload (1-5)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of CPU oracle work: heads are timed in order until this is "
                         "spent (at least one, at most all)")
    ap.add_argument("--prof-steps", type=int, default=3,
                    help="calls of the separate instrumented pass (per-kernel times)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--variant", default="compact",
                    choices=["compact", "omp", "chunked", "ragged", "protected", "attend"],
                    help="omp: keys chosen by orthogonal matching pursuit; chunked: the cache cut into --chunks equal chunks, t/chunks kept per "
                         "chunk; ragged: per-head budgets from 0.5t to 1.5t (mean t); "
                         "protected: 1%% of the keys (and the first) kept exactly; "
                         "attend: the evaluation kernel over the whole cache plus an appended "
                         "block of 1024 tokens, for the held-out queries")
    ap.add_argument("--chunks", type=int, default=4)
    return ap.parse_args()


def cpu_baseline(w, data, budget_s, one_head=None):
    """The oracle as it stands, head after head of the same workload until
    budget_s seconds are spent (at least one head, at most all of them).
    one_head(orc, h, Q, K, V) runs the oracle's form of the benchmarked call on
    head h (default: compact at budget t)."""
    import oracle as orc
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    heads = 0
    while heads < w.B and (heads == 0 or time.perf_counter() - t0 < budget_s):
        Q, K, V = (synth.to_f64(data[k][heads]) for k in ("Q", "K", "V"))
        if one_head is None:
            orc.compact(Q, K, V, w.t)
        else:
            one_head(orc, heads, Q, K, V)
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": heads * w.T / dt, "unit": "KV tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads} of {w.B} heads of {w.name} through the float64 oracle, in order "
                      f"until {budget_s:.0f} s were spent ({dt:.1f} s; BLAS threads={cores}, "
                      f"numpy exp single-threaded)"}


def copy_probe(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy of nbytes (read nbytes + write nbytes), timed with
    events on torch's stream: the measured HBM rate beside the spec peak, and
    the known-size kernel the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def traffic_record():
    """HBM bytes per launch of the NNLS kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^traffic_json: (\{.*\})$", text, re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    sha = hashlib.sha256(open(FIT_SRC, "rb").read()).hexdigest()
    return rec if rec.get("fit_hip_sha256") == sha else None


def bench_attend(args, torch, kvc, w, data, dev):
    """kvc_attend over [K; K_fixed] for the held-out queries: float32 vector
    arithmetic, 4 m (T + f) d flops per head (scores and the weighted sum)."""
    rng = np.random.default_rng(7)
    f = 1024
    import synth
    Kf = dev(synth.round_bf16_bits(rng.standard_normal((w.B, f, w.d))))
    Vf = dev(synth.round_bf16_bits(rng.standard_normal((w.B, f, w.d))))
    Qh, K, V = dev(data["Qhold"]), dev(data["K"]), dev(data["V"])
    for _ in range(args.warmup):
        kvc.attend(Qh, K, V, None, Kf, Vf)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        kvc.attend(Qh, K, V, None, Kf, Vf)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / args.steps
    m = w.n_hold
    flops = 4.0 * m * (w.T + f) * w.d * w.B
    ach = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "attention evaluation over cache + appended block: query-key pairs/s",
        "value": m * (w.T + f) * w.B / (ms * 1e-3), "unit": "query-key pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": "attend", "B": w.B, "m": m, "T": w.T,
                   "appended": f, "d": w.d},
        "roofline": {"bound": "alu", "kernel": "k_attend", "achieved": round(ach, 3),
                     "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_F32_VALU_TFLOPS, 5), "traffic": None,
                     "peak_note": "fp32 vector FMA, packed fp32 ops off in this build"}}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); heads are "
              "independent, so more GPUs would shard B with no communication.", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_compaction_head_amd as kvc
    from kv_cache_compaction_head_amd import _lib
    import synth

    w = synth.CONFIGS[args.config]
    data = synth.batch(w)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    if args.variant == "attend":
        bench_attend(args, torch, kvc, w, data, dev)
        return
    Q, K, V = dev(data["Q"]), dev(data["K"]), dev(data["V"])
    p = kvc.make_params(w.B, w.T, w.n, w.d, w.t, w.dtype)
    variant = {"workload": w.name}
    oracle_head = None
    if args.variant == "chunked":
        tc = w.t // args.chunks
        need = kvc.workspace_bytes_chunked(kvc.make_params(w.B, w.T, w.n, w.d, tc, w.dtype),
                                           args.chunks)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        variant.update(variant="chunked", chunks=args.chunks, t_per_chunk=tc)

        def oracle_head(orc, h, Qh, Kh, Vh):
            orc.compact_chunked(Qh, Kh, Vh, tc, args.chunks)

        def call():
            return kvc.compact_chunked(Q, K, V, tc, args.chunks, workspace=ws)
    elif args.variant == "ragged":
        budgets = [max(1, int(round(w.t * (0.5 + h / max(1, w.B - 1))))) for h in range(w.B)]
        pr = kvc.make_params(w.B, w.T, w.n, w.d, max(budgets), w.dtype)
        ws = torch.empty(kvc.workspace_bytes(pr), dtype=torch.uint8, device="cuda")
        tv = torch.tensor(budgets, dtype=torch.int32, device="cuda")
        variant.update(variant="ragged", budgets=budgets)

        def oracle_head(orc, h, Qh, Kh, Vh):
            orc.compact(Qh, Kh, Vh, budgets[h])

        def call():
            return kvc.compact_ragged(Q, K, V, tv, workspace=ws)
    elif args.variant == "omp":
        ws = torch.empty(kvc.workspace_bytes_omp(p), dtype=torch.uint8, device="cuda")
        variant.update(variant="omp")

        def oracle_head(orc, h, Qh, Kh, Vh):
            orc.compact_omp(Qh, Kh, Vh, w.t)

        def call():
            return kvc.compact_omp(Q, K, V, w.t, workspace=ws)
    elif args.variant == "protected":
        g = torch.Generator().manual_seed(w.cfg)
        prot = (torch.rand((w.B, w.T), generator=g) < 0.01)
        prot[:, 0] = True
        prot = prot.to(torch.uint8).cuda()
        ws = torch.empty(kvc.workspace_bytes(p), dtype=torch.uint8, device="cuda")
        variant.update(variant="protected", protected_frac=0.01)
        prot_host = prot.cpu().numpy()

        def oracle_head(orc, h, Qh, Kh, Vh):
            orc.compact_protected(Qh, Kh, Vh, w.t, prot_host[h])

        def call():
            return kvc.compact_protected(Q, K, V, w.t, prot, workspace=ws)
    else:
        ws = torch.empty(kvc.workspace_bytes(p), dtype=torch.uint8, device="cuda")

        def call():
            return kvc.compact(Q, K, V, w.t, workspace=ws)
    for _ in range(args.warmup):
        res = call()
    torch.cuda.synchronize()

    # timed region: the calls alone (no instrumentation)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps

    # a separate instrumented pass: HIP event pairs on the library's stream
    # around each kernel stage
    stages = list(_lib.STAGES)
    prof = {}
    if not args.no_profile and args.prof_steps > 0:
        _lib.profile_enable(stages)
        for _ in range(args.prof_steps):
            res = call()
        torch.cuda.synchronize()
        for s in stages:
            ms, cnt = _lib.profile_read(s)
            if cnt:
                prof[s] = ms / cnt
        _lib.profile_enable([])

    copy_gbs = copy_probe(torch)
    status = res.status.cpu().numpy()
    B, T, n, d = w.B, w.T, w.n, w.d
    es = 2 if w.dtype == "bf16" else 4
    # per-entry shapes of the batched call (a chunked call runs B*C entries of
    # T/C keys, t/C kept each)
    Be, Te, te = B, T, w.t
    if args.variant == "chunked":
        Be, Te, te = B * args.chunks, T // args.chunks, w.t // args.chunks
    elif args.variant == "ragged":
        te = max(variant["budgets"])
    # fitted keys per entry (the order of its bias system): the budget, a
    # ragged head's own budget, or what the protected keys leave
    t_fit = np.full(Be, te, dtype=np.float64)
    if args.variant == "ragged":
        t_fit = np.array(variant["budgets"], dtype=np.float64)
    elif args.variant == "protected":
        t_fit = w.t - np.minimum(prot_host.sum(axis=1), w.t - 1).astype(np.float64)
    nqb = -(-n // 128)
    mm_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    inter = kvc.intermediates(res)
    fit_flops = inter["fit_flops"].cpu().numpy().sum(axis=0)  # [nnls, value] over entries
    wv = inter["w"].cpu().numpy()
    m_pass = (wv > 0).sum(axis=1)                           # value-system order per entry
    # algorithmic work per launch of each separately timed kernel (formulas and
    # units in the design notes):
    #   k_score_lse    2 n T d per entry (S = Q K^T once)
    #   k_expweight    4 n T d per entry (S recomputed + P V)
    #   k_imp_reduce   reads the ceil(n/128) partials of every key, writes imp (and
    #                  the selection's first histogram): 4 T (nqb + 1) B
    #   k_sel_*        the rest of the selection (two refining passes, the counts,
    #                  the compaction: four launches), algorithmically one read of
    #                  imp and the idx write: 4 T B + 4 t B
    #   k_gather_rows  reads and writes the kept K rows: 2 t d es B
    #   Grams          n t^2 per entry, t its fitted keys (symmetric half); the value
    #                  system's Gram and right-hand side in one launch: n (m^2 + m d),
    #                  m passive
    #   k_nnls_sweep   the block sweeps of the pivoting rounds (counted on device)
    #   k_value_sweep  the value system's block sweeps (counted on device)
    work = {"score_lse": ("k_score_lse", 2.0 * n * Te * d * Be, mm_peak, "mfma"),
            "expweight": ("k_expweight", 4.0 * n * Te * d * Be, mm_peak, "mfma"),
            "imp_reduce": ("k_imp_reduce", 4.0 * Te * (nqb + 1) * Be, PEAK_HBM_GBS, "hbm"),
            "topt": ("k_sel_* (refine x2, count, compact)", 4.0 * (Te + te) * Be, PEAK_HBM_GBS, "hbm"),
            "gather": ("k_gather_rows", 2.0 * te * d * es * Be, PEAK_HBM_GBS, "hbm"),
            "gram": ("k_atb (mass Gram)", float(n * (t_fit ** 2).sum()), PEAK_F64_TFLOPS, "mfma"),
            "value_gram": ("k_atb2 (value Gram + X_F^T O)",
                           float(n * (m_pass.astype(float) ** 2 + m_pass.astype(float) * d).sum()),
                           PEAK_F64_TFLOPS, "mfma"),
            "nnls": ("k_nnls_sweep", float(fit_flops[0]), PEAK_F64_TFLOPS, "mfma"),
            "value_sweep": ("k_value_sweep", float(fit_flops[1]), PEAK_F64_TFLOPS, "mfma")}
    if args.variant == "omp":
        # the pursuit's t correlation passes read P (n T float32 per head) once
        # each, plus P's write and the norms pass: HBM-bound by design
        work["select"] = ("omp selection (k_ps<float>, k_omp_*)",
                          float((w.t + 2) * n * T * 4 * B), PEAK_HBM_GBS, "hbm")
    kernels = []
    for stage, (kname, amount, peak, bound) in work.items():
        if stage not in prof or amount <= 0:
            continue
        hbm = bound == "hbm"
        ach = amount / (prof[stage] * 1e-3) / (1e9 if hbm else 1e12)
        k = {"kernel": kname, "bound": bound, "ms": round(prof[stage], 4),
             "achieved": round(ach, 3), "peak": peak, "unit": "GB/s" if hbm else "TFLOP/s",
             "frac": round(ach / peak, 5), "work": amount}
        if kname in ("k_nnls_sweep", "k_value_sweep"):
            k["limited_by"] = "latency of the chain of dependent block steps"
        kernels.append(k)
    roof = None
    if kernels:
        dom = max((k for k in kernels if k["kernel"].startswith("k_") and " " not in k["kernel"]
                   or k["bound"] == "hbm"), key=lambda k: k["ms"])
        tr = (traffic_record() if (dom["kernel"] == "k_nnls_sweep" and args.config == 3 and
                                   args.variant == "compact") else None)
        roof = {"bound": dom["bound"], "kernel": dom["kernel"], "achieved": dom["achieved"],
                "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"],
                "traffic": tr["bytes_per_launch"] if tr else None,
                "traffic_detail": tr,
                **({"limited_by": dom["limited_by"]} if "limited_by" in dom else {}),
                "kernels": kernels, "stage_ms": {k: round(v, 4) for k, v in prof.items()},
                "hbm_copy_measured_GBs": round(copy_gbs, 1), "hbm_peak_GBs": PEAK_HBM_GBS}

    quality = diagnostics(w, data, res, inter, args.variant, B, status)
    out = {
        "metric": "KV tokens compacted/sec (1 GPU) at T=32k, 50x; compacted-attn rel. L2 error",
        "value": B * T / dt,
        "unit": "KV tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {**variant, "B": B, "T": T, "n": n, "d": d, "t": w.t,
                   "ratio": T / w.t},
        "quality": quality,
        "roofline": roof,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, data, args.cpu_budget, oracle_head)
    print(json.dumps(out), flush=True)


def diagnostics(w, data, res, inter, variant, B, status, max_heads=8):
    """Quality of the compacted cache on the first max_heads heads (float64 on
    the host): the relative L2 error of the compacted attention output on
    held-out queries (and of keeping the same keys without fitting), and, for
    kvc_compact, on the reference queries themselves, the mass ratio r_i =
    sum_{j kept} p_ij w_j per reference query (1 = exact mass), and the
    condition numbers of the two regularised Grams."""
    import oracle as orc
    import synth
    heads = list(range(min(B, max_heads)))
    held, evict, qref, r_all, cond_m, cond_g = [], [], [], [], [], []
    lse_all = inter["lse"].cpu().numpy() if variant == "compact" else None
    O_all = inter["O"].cpu().numpy() if variant == "compact" else None
    wv_all = inter["w"].cpu().numpy()
    for h in heads:
        Kf = synth.to_f64(data["K"][h])
        Vf = synth.to_f64(data["V"][h])
        Qh = synth.to_f64(data["Qhold"][h])
        ih = res.idx[h].cpu().numpy()
        live = ih >= 0
        vals = res.values[h].float().cpu().numpy().astype(np.float64)[live]
        bias = res.bias[h].cpu().numpy().astype(np.float64)[live]
        Ck = Kf[ih[live]]
        full = orc.attend(Qh, Kf, Vf)
        held.append(orc.rel_l2(orc.attend(Qh, Ck, vals, bias), full))
        evict.append(orc.rel_l2(orc.attend(Qh, Ck, Vf[ih[live]]), full))
        if variant != "compact":
            continue
        Q = synth.to_f64(data["Q"][h])
        qref.append(orc.rel_l2(orc.attend(Q, Ck, vals, bias), O_all[h].astype(np.float64)))
        PS = np.exp(Q @ Ck.T - lse_all[h][:, None])
        wh = wv_all[h]
        r = PS @ wh
        r_all.append(r)
        M = PS.T @ PS
        t = M.shape[0]
        ev = np.linalg.eigvalsh(M + 1e-6 * np.trace(M) / t * np.eye(t))
        cond_m.append(float(ev[-1] / ev[0]))
        F = wh > 0
        X = PS[:, F] * wh[F][None, :] / r[:, None]
        G = X.T @ X
        ev = np.linalg.eigvalsh(G + 1e-6 * np.trace(G) / t * np.eye(G.shape[0]))
        cond_g.append(float(ev[-1] / ev[0]))
    q = {"heads": len(heads), "of_heads": B,
         "heldout_rel_l2": float(np.mean(held)), "heldout_rel_l2_max": float(np.max(held)),
         "heldout_rel_l2_head0": held[0],
         "eviction_only_rel_l2": float(np.mean(evict)),
         "status_nonzero_heads": int((status != 0).sum())}
    if qref:
        r = np.concatenate(r_all)
        pct = lambda x: [float(np.percentile(x, p)) for p in (0, 50, 90, 100)]
        q.update({"qref_rel_l2": float(np.mean(qref)), "qref_rel_l2_max": float(np.max(qref)),
                  "mass_ratio": {"min": float(r.min()), "mean": float(r.mean()),
                                 "max": float(r.max())},
                  "cond_mass_gram_p0_50_90_100": pct(cond_m),
                  "cond_value_gram_p0_50_90_100": pct(cond_g)})
    return q


if __name__ == "__main__":
    main()
