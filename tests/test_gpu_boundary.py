"""GPU tests of the boundary's options: ridge_rel = 0 (the literal NNLS and
least squares of "Fast KV Compaction via Attention Matching", section 2,
algorithmic pipeline), fitted values stored as bfloat16, and the bounded team
wait forced to run out from the host (the time-out path ends normally and is
reported)."""
import numpy as np
import pytest

import oracle as orc
import synth
from parity import TOL_BF16, check_selection, run_gpu, to_device

pytestmark = pytest.mark.gpu


def test_ridge_zero_keep_everything_reproduces_values():
    """t = T with n >= T and no ridge: idx = all keys, w = 1 and C_v = V (the
    full cache is the unique zero-loss point when P has full column rank)."""
    w = synth.custom(30, 2, 96, 130, 128, 96, "bf16", "normal")
    data = synth.batch(w)
    gpu = run_gpu(w, data, ridge_rel=0.0)
    assert (gpu["status"] == 0).all(), gpu["status"]
    for h in range(w.B):
        assert list(gpu["idx"][h]) == list(range(96))
        assert np.allclose(gpu["w"][h], 1.0, atol=1e-4)
        assert orc.rel_l2(gpu["values"][h], synth.to_f64(data["V"][h])) < 1e-4


def test_ridge_zero_matches_oracle():
    """No ridge on a well-conditioned case (n >> t): w, the fitted values of
    the keys with a positive multiplier, and the compacted attention against
    the oracle at ridge 0.  A key whose multiplier is zero has no weight in
    the compacted softmax, so its fitted value is not unique: the GPU keeps
    the original value, the oracle's least squares a minimum-norm one; those
    rows are not compared."""
    w = synth.custom(31, 2, 1500, 512, 128, 40, "bf16", "normal")
    data = synth.batch(w)
    gpu = run_gpu(w, data, ridge_rel=0.0)
    assert (gpu["status"] == 0).all(), gpu["status"]
    for h in range(w.B):
        Q, K, V = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
        ref = orc.compact(Q, K, V, w.t, ridge_rel=0.0)
        check_selection(gpu["idx"][h], ref["idx"], ref["imp"], w.t)
        if not np.array_equal(gpu["idx"][h], ref["idx"]):
            wv, beta, Cv, _ = orc.fit(Q, K, V, gpu["idx"][h], ridge_rel=0.0)
            ref = {**ref, "w": wv, "beta": beta, "Cv": Cv, "Ck": K[gpu["idx"][h]]}
        live = ref["w"] > 0
        err_w = orc.rel_l2(gpu["w"][h], ref["w"])
        err_c = orc.rel_l2(gpu["values"][h][live], ref["Cv"][live])
        o_gpu = orc.attend(Q, K[gpu["idx"][h]], gpu["values"][h], gpu["bias"][h])
        o_ref = orc.attend(Q, ref["Ck"], ref["Cv"], ref["beta"])
        err_o = orc.rel_l2(o_gpu, o_ref)
        print(f"head {h}: passive {live.sum()} of {w.t}, w {err_w:.3g}, Cv {err_c:.3g}, "
              f"Ohat {err_o:.3g}", flush=True)
        assert max(err_w, err_c, err_o) <= TOL_BF16


def test_bf16_values_are_the_rounded_f32_values():
    """out_v_dtype = bfloat16 stores exactly the float32 result rounded to
    nearest-even, for fitted slots and for protected (copied) slots."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(32, 3, 1200, 160, 128, 70, "bf16", "clusters")
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    a = kvc.compact(Q, K, V, w.t)
    b = kvc.compact(Q, K, V, w.t, out_v_dtype=torch.bfloat16)
    prot = torch.zeros((w.B, w.T), dtype=torch.uint8)
    prot[:, ::97] = 1
    c = kvc.compact_protected(Q, K, V, w.t, prot)
    d = kvc.compact_protected(Q, K, V, w.t, prot, out_v_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for f32, bf in ((a, b), (c, d)):
        assert bf.values.dtype == torch.bfloat16
        ref_bits = synth.round_bf16_bits(f32.values.cpu().numpy())
        got_bits = bf.values.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got_bits, ref_bits)
        for k in ("keys", "bias", "idx", "status"):
            assert torch.equal(getattr(f32, k), getattr(bf, k)), k


def test_wait_time_out_is_reported_and_every_kernel_ends():
    """A one-tick bound on the fit teams' waits (set from the host): the first
    wait that finds a member missing gives up and turns the launch's later
    waits into no-ops, every kernel still ends, and every head of the launch
    reports KVC_STATUS_SYNC_TIMEOUT.  With the default bound restored the same
    call is exact again."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    from parity import compare_head
    w = synth.custom(33, 2, 2000, 256, 128, 200, "bf16", "clusters")
    data = synth.batch(w)
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    print("time-out case: B=2 T=2000 n=256 t=200, wait bound 1 tick", flush=True)
    kvc.set_wait_limit(1)
    try:
        res = kvc.compact(Q, K, V, w.t)
        torch.cuda.synchronize()
        st = res.status.cpu().numpy()
    finally:
        kvc.set_wait_limit(0)
    print("status with a 1-tick bound:", st, flush=True)
    assert np.all(st & kvc.STATUS_SYNC_TIMEOUT), st
    gpu = run_gpu(w, data)
    for h in range(w.B):
        compare_head(gpu, h, data, w.t, TOL_BF16)


def test_singular_bias_gram_raises_the_ridge():
    """Two kept keys with identical rows make P_S's columns equal, so at
    ridge 0 the bias Gram is singular and a pivot vanishes once both are
    passive (adjacent slots 5 and 6 enter together in one 16-pivot block,
    where both columns get bit-identical updates and the second pivot
    cancels to rounding size, far under the relative pivot bound).  The NNLS restarts with the ridge raised (status bit 64, the
    count in bits 8-9), ends without KVC_STATUS_NOT_SPD, gives both copies
    the same bias, and its compacted attention matches the oracle's fit at
    the raised relative ridge (1e-9 at the first raise from 0).  At the
    default ridge the same Gram plus lam I is definite: no raise."""
    import torch
    import kv_cache_compaction_head_amd as kvc
    w = synth.custom(34, 2, 700, 256, 128, 48, "bf16", "normal")
    data = synth.batch(w)
    rng = np.random.default_rng(34)
    idx = np.sort(rng.choice(w.T, size=w.t, replace=False)).astype(np.int32)
    idx = np.tile(idx, (w.B, 1))
    for h in range(w.B):  # kept slots 5 and 6 share one key row
        data["K"][h, idx[h, 6]] = data["K"][h, idx[h, 5]]
    Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
    tidx = torch.from_numpy(idx).cuda()
    print("duplicated kept key: B=2 T=700 n=256 t=48, slots 5 and 6, ridge 0", flush=True)
    res = kvc.fit(Q, K, V, tidx, ridge_rel=0.0)
    torch.cuda.synchronize()
    st = res.status.cpu().numpy()
    print("status at ridge 0:", st, [kvc.status_raises(s) for s in st], flush=True)
    bias = res.bias.cpu().numpy().astype(np.float64)
    vals = res.values.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(bias)) and np.all(np.isfinite(vals))
    for h in range(w.B):
        assert st[h] & kvc.STATUS_RIDGE_RAISED, st
        e = kvc.status_raises(st[h])
        assert 1 <= e <= 3 and not st[h] & kvc.STATUS_NOT_SPD, st
        assert abs(bias[h, 5] - bias[h, 6]) < 1e-3, (bias[h, 5], bias[h, 6])
        rel = max(0.0, 1e-9 * 10.0 ** (e - 1))
        Qh, Kh, Vh = (synth.to_f64(data[k][h]) for k in ("Q", "K", "V"))
        _, beta, Cv, _ = orc.fit(Qh, Kh, Vh, idx[h], ridge_rel=rel)
        o_gpu = orc.attend(Qh, Kh[idx[h]], vals[h], bias[h])
        o_ref = orc.attend(Qh, Kh[idx[h]], Cv, beta)
        err = orc.rel_l2(o_gpu, o_ref)
        print(f"head {h}: raises {e}, Ohat vs oracle at ridge {rel:g}: {err:.3g}", flush=True)
        assert err <= TOL_BF16
    res2 = kvc.fit(Q, K, V, tidx)
    torch.cuda.synchronize()
    assert (res2.status.cpu().numpy() == 0).all(), res2.status
