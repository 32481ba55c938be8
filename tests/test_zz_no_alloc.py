"""kvc_compact_noalloc, the entry point that allocates nothing, against
kvc_compact on the same inputs: two calls in a row, the second on a smaller
problem (different dtype and head dim) that reuses the device's scratch array
after the first.  Same kernels, so the outputs must be bitwise equal."""
import numpy as np
import pytest

import synth
from parity import TOL_BF16, TOL_F32, compare_head, to_device

pytestmark = pytest.mark.gpu


def test_noalloc_equals_compact_on_two_calls_in_a_row():
    import torch
    import kv_cache_compaction_head_amd as kvc
    from kv_cache_compaction_head_amd import _lib
    cases = [synth.custom(40, 3, 3000, 256, 128, 120, "bf16", "clusters"),
             synth.custom(41, 2, 700, 64, 64, 33, "f32", "normal")]
    for w in cases:
        p = kvc.make_params(w.B, w.T, w.n, w.d, w.t, w.dtype)
        assert kvc.workspace_bytes(p) <= _lib.NOALLOC_SCRATCH_BYTES
        print(f"noalloc case: B={w.B} T={w.T} n={w.n} d={w.d} t={w.t} {w.dtype}", flush=True)
        data = synth.batch(w)
        Q, K, V = (to_device(data[k]) for k in ("Q", "K", "V"))
        b = kvc.compact_noalloc(Q, K, V, w.t)
        a = kvc.compact(Q, K, V, w.t)
        torch.cuda.synchronize()
        for k in ("keys", "bias", "values", "idx", "status"):
            assert torch.equal(getattr(a, k), getattr(b, k)), k
        # and the shared result against the oracle, at the usual bar
        inter = {k: v.cpu().numpy() for k, v in kvc.intermediates(a).items()}
        g = {"keys": b.keys.cpu(), "bias": b.bias.cpu().numpy().astype(np.float64),
             "values": b.values.cpu().numpy().astype(np.float64),
             "idx": b.idx.cpu().numpy().astype(np.int64), "status": b.status.cpu().numpy(),
             **inter}
        for h in range(w.B):
            compare_head(g, h, data, w.t, TOL_F32 if w.dtype == "f32" else TOL_BF16)
