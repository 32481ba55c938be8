"""Helpers shared by the GPU parity tests: upload seeded workloads, run the
HIP path through the C ABI, run the oracle on the same bits, compare."""
from __future__ import annotations

import numpy as np

import oracle as orc
import synth

TOL_BF16 = 2e-3   # relative L2 on w, C_v and the compacted output (bf16 inputs)
TOL_F32 = 1e-4    # the same for float32 inputs
TIE_REL = 1e-6    # selected-index swaps allowed only below this importance gap


def to_device(arr: np.ndarray):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def run_gpu(w: synth.Workload, data: dict, agg: str = "rms", ridge_rel: float = 1e-6):
    import torch
    import kv_cache_compaction_head_amd as kvc
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    res = kvc.compact(Q, K, V, w.t, agg=agg, ridge_rel=ridge_rel)
    torch.cuda.synchronize()
    inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(res).items()}
    out = {"keys": res.keys.cpu(), "bias": res.bias.cpu().numpy().astype(np.float64),
           "values": res.values.cpu().numpy().astype(np.float64),
           "idx": res.idx.cpu().numpy().astype(np.int64),
           "status": res.status.cpu().numpy(), **inter}
    return out


def oracle_head(data: dict, h: int, t: int, agg: str = "rms", ridge_rel: float = 1e-6):
    Q, K, V = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
    return orc.compact(Q, K, V, t, agg=agg, ridge_rel=ridge_rel), (Q, K, V)


def check_selection(gpu_idx, ref_idx, ref_imp, t):
    """Identical, or every disagreement is a near-tie (relative gap <= 1e-6
    judged on the oracle's importances).  Returns True if identical."""
    a, b = set(gpu_idx.tolist()), set(ref_idx.tolist())
    assert np.all(np.diff(gpu_idx) > 0), "indices must ascend"
    if a == b:
        return True
    cutoff = np.sort(ref_imp)[::-1][t - 1]
    only_gpu, only_ref = sorted(a - b), sorted(b - a)
    assert len(only_gpu) == len(only_ref)
    for j in only_gpu + only_ref:
        assert abs(ref_imp[j] - cutoff) <= TIE_REL * cutoff, (j, ref_imp[j], cutoff)
    return False


def rel(a, b):
    return orc.rel_l2(a, b)


def compare_head(gpu: dict, h: int, data: dict, t: int, tol: float, agg: str = "rms",
                 ridge_rel: float = 1e-6, tight: bool = True):
    """Full comparison of one head; returns a dict of measured errors."""
    ref, (Q, K, V) = oracle_head(data, h, t, agg, ridge_rel)
    n = Q.shape[0]
    err = {}
    # score path intermediates
    err["lse_abs"] = float(np.abs(gpu["lse"][h] - ref["lse"]).max())
    err["O"] = rel(gpu["O"][h], ref["O"])
    acc_ref = ref["imp"] ** 2 * n if agg == "rms" else ref["imp"] * n
    err["imp"] = rel(gpu["imp"][h], acc_ref)
    same = check_selection(gpu["idx"][h], ref["idx"], ref["imp"], t)
    if not same:  # compare the fits on the GPU's own kept set
        wv, beta, Cv, info = orc.fit(Q, K, V, gpu["idx"][h], ridge_rel=ridge_rel)
        ref = {**ref, "idx": gpu["idx"][h], "Ck": K[gpu["idx"][h]], "w": wv, "beta": beta,
               "Cv": Cv}
    err["same_idx"] = same
    keys = gpu["keys"][h]
    keys = keys.float().numpy().astype(np.float64)
    assert np.array_equal(keys, K[gpu["idx"][h]]), "kept keys must be exact copies"
    err["w"] = rel(gpu["w"][h], ref["w"])
    err["w_from_bias"] = rel(np.maximum(np.exp(gpu["bias"][h]), 0), np.maximum(ref["w"], 1e-30))
    err["Cv"] = rel(gpu["values"][h], ref["Cv"])
    o_gpu = orc.attend(Q, keys, gpu["values"][h], gpu["bias"][h])
    o_ref = orc.attend(Q, ref["Ck"], ref["Cv"], ref["beta"])
    err["Ohat"] = rel(o_gpu, o_ref)
    err["status"] = int(gpu["status"][h])
    assert err["status"] == 0, err
    for k in ("w", "w_from_bias", "Cv", "Ohat"):
        assert err[k] <= tol, (k, err)
    if tight:
        assert err["lse_abs"] <= 1e-4, err
        assert err["O"] <= 1e-4, err
        assert err["imp"] <= 1e-4, err
    return err
