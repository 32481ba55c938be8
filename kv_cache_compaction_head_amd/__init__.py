"""Attention-matching KV-cache compaction on AMD MI355X (gfx950).

Python front of the C ABI in include/kvc.h.  Torch tensors supply device
memory and the stream; every step of the computation runs in the HIP library
(libkvc.so), which must be built first (`python -m
kv_cache_compaction_head_amd.build`).  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses

from . import _lib
from ._lib import (KVC_AGG_MEAN, KVC_AGG_RMS, KVC_BF16, KVC_F32, STATUS_NNLS_CAP,
                   STATUS_NONFINITE, STATUS_NOT_SPD, STATUS_RIDGE_RAISED, STATUS_SYNC_TIMEOUT,
                   Params, load, status_raises,
                   make_params, set_wait_limit, strerror, workspace_bytes,
                   workspace_bytes_chunked, workspace_bytes_omp, workspace_layout)

__all__ = ["compact", "compact_noalloc", "compact_omp", "compact_chunked", "compact_ragged", "compact_protected", "attend", "fit", "Compacted", "intermediates", "load", "make_params",
           "workspace_bytes", "workspace_bytes_chunked", "workspace_bytes_omp", "workspace_layout", "strerror", "Params",
           "set_wait_limit", "status_raises", "STATUS_RIDGE_RAISED"]


@dataclasses.dataclass
class Compacted:
    """Outputs of one call (device tensors; valid once the stream completes)."""
    keys: "object"       # [B, t, d] input dtype, exact copies of kept K rows
    bias: "object"       # [B, t] float32, additive logit bias per kept key
    values: "object"     # [B, t, d] float32, fitted values
    idx: "object"        # [B, t] int32, kept indices (ascending)
    status: "object"     # [B] int32, KVC_STATUS_* bits per head
    workspace: "object"  # uint8 device buffer holding the intermediates
    params: Params
    omp: bool = False    # keys chosen by the greedy pursuit (intermediates: omp_order)


def _vp(x):
    return ctypes.c_void_p(x.data_ptr())


def _vdt(out_v_dtype):
    """Storage of the fitted values: float32 (default) or bfloat16 (the
    float32 result rounded to nearest-even)."""
    import torch
    if out_v_dtype is None or out_v_dtype == torch.float32:
        return "f32", torch.float32
    if out_v_dtype == torch.bfloat16:
        return "bf16", torch.bfloat16
    raise ValueError("out_v_dtype must be torch.float32 or torch.bfloat16")


def _prep(Q, K, V):
    import torch
    squeeze = Q.dim() == 2
    if squeeze:
        Q, K, V = Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0)
    if Q.dim() != 3 or K.dim() != 3 or V.dim() != 3:
        raise ValueError("expected Q_ref [B,n,d], K [B,T,d], V [B,T,d] (or unbatched)")
    if not (Q.is_cuda and K.is_cuda and V.is_cuda):
        raise ValueError("tensors must be on a HIP device")
    if not (Q.dtype == K.dtype == V.dtype) or Q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("Q_ref, K, V must share one dtype: bfloat16 or float32")
    if K.shape != V.shape or Q.shape[0] != K.shape[0] or Q.shape[2] != K.shape[2]:
        raise ValueError("shape mismatch between Q_ref, K and V")
    return Q.contiguous(), K.contiguous(), V.contiguous(), squeeze


def _stream(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(p, device, workspace, need=None):
    import torch
    need = workspace_bytes(p) if need is None else need
    if need == 0:
        raise ValueError("invalid compaction parameters")
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace


def compact(Q, K, V, t: int, *, agg: str = "rms", ridge_rel: float = 1e-6,
            max_nnls_iters: int = 32, refine_steps: int = 0, out_v_dtype=None, workspace=None,
            stream=None) -> Compacted:
    """Compact each head's cache to t kept keys with fitted bias and values."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, agg, ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    ws = _workspace(p, dev, workspace)
    keys = torch.empty((B, t, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    idx = torch.empty((B, t), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_compact(ctypes.byref(p), _vp(Q), _vp(K), _vp(V), _vp(keys), _vp(bias),
                            _vp(values), _vp(idx), _vp(status), _vp(ws),
                            ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream, dev))
    _lib.check(rc)
    return Compacted(keys, bias, values, idx, status, ws, p)


def compact_noalloc(Q, K, V, t: int, *, agg: str = "rms", ridge_rel: float = 1e-6,
                    max_nnls_iters: int = 32, refine_steps: int = 0, out_v_dtype=None,
                    stream=None) -> Compacted:
    """compact() through kvc_compact_noalloc: the library takes its workspace
    from its own per-device scratch array (at most _lib.NOALLOC_SCRATCH_BYTES)
    instead of a caller buffer.  Only the outputs are allocated here."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, agg, ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    keys = torch.empty((B, t, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    idx = torch.empty((B, t), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_compact_noalloc(ctypes.byref(p), _vp(Q), _vp(K), _vp(V), _vp(keys),
                                    _vp(bias), _vp(values), _vp(idx), _vp(status),
                                    _stream(stream, dev))
    _lib.check(rc)
    return Compacted(keys, bias, values, idx, status, None, p)


def compact_omp(Q, K, V, t: int, *, ridge_rel: float = 1e-6, max_nnls_iters: int = 32,
                refine_steps: int = 0, out_v_dtype=None, workspace=None, stream=None) -> Compacted:
    """Compact each head to t keys chosen by orthogonal matching pursuit on
    the attention mass (t greedy steps), then the same bias and value fits as
    compact()."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, "rms", ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    need = workspace_bytes_omp(p)
    if need == 0:
        raise ValueError("invalid compaction parameters")
    ws = _workspace(p, dev, workspace, need)
    keys = torch.empty((B, t, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    idx = torch.empty((B, t), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_compact_omp(ctypes.byref(p), _vp(Q), _vp(K), _vp(V), _vp(keys), _vp(bias),
                                _vp(values), _vp(idx), _vp(status), _vp(ws),
                                ctypes.c_size_t(ws.numel() * ws.element_size()),
                                _stream(stream, dev))
    _lib.check(rc)
    return Compacted(keys, bias, values, idx, status, ws, p, omp=True)


def compact_ragged(Q, K, V, t_heads, *, agg: str = "rms", ridge_rel: float = 1e-6,
                   max_nnls_iters: int = 32, refine_steps: int = 0,
                   out_v_dtype=None, workspace=None,
            stream=None) -> Compacted:
    """Compact head b to t_heads[b] keys (a per-head budget).  Outputs are
    padded to max(t_heads): head b's slots from t_heads[b] on hold idx -1,
    zero keys and values and bias -inf, which attention ignores."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    tv = torch.as_tensor(t_heads, dtype=torch.int32)
    if tv.shape != (B,):
        raise ValueError(f"t_heads must hold one budget per head ({B})")
    t = int(tv.max())
    tv = tv.to(Q.device).contiguous()
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, agg, ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    ws = _workspace(p, dev, workspace)
    keys = torch.empty((B, t, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    idx = torch.empty((B, t), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_compact_ragged(ctypes.byref(p), _vp(tv), _vp(Q), _vp(K), _vp(V), _vp(keys),
                                   _vp(bias), _vp(values), _vp(idx), _vp(status), _vp(ws),
                                   ctypes.c_size_t(ws.numel() * ws.element_size()),
                                   _stream(stream, dev))
    _lib.check(rc)
    return Compacted(keys, bias, values, idx, status, ws, p)


def compact_protected(Q, K, V, t: int, protect, *, agg: str = "rms", ridge_rel: float = 1e-6,
                      max_nnls_iters: int = 32, refine_steps: int = 0,
                      out_v_dtype=None, workspace=None,
            stream=None) -> Compacted:
    """Keep the marked keys of protect [B, T] (bool/uint8) exactly with bias 0
    (at most t - 1 per head, the first by position) and compact the others
    into the remaining slots.  Head b's slots [0, t - p_b) hold the fitted
    part, slots [t - p_b, t) the protected keys, both ascending."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    if tuple(protect.shape) != (B, T):
        raise ValueError(f"protect must be [B, T] = [{B}, {T}]")
    m = protect.to(device=Q.device, dtype=torch.uint8).contiguous()
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, agg, ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    ws = _workspace(p, dev, workspace)
    keys = torch.empty((B, t, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    idx = torch.empty((B, t), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_compact_protected(ctypes.byref(p), _vp(m), _vp(Q), _vp(K), _vp(V), _vp(keys),
                                      _vp(bias), _vp(values), _vp(idx), _vp(status), _vp(ws),
                                      ctypes.c_size_t(ws.numel() * ws.element_size()),
                                      _stream(stream, dev))
    _lib.check(rc)
    return Compacted(keys, bias, values, idx, status, ws, p)


def compact_chunked(Q, K, V, t: int, n_chunks: int, *, agg: str = "rms",
                    ridge_rel: float = 1e-6, max_nnls_iters: int = 32, refine_steps: int = 0,
                    out_v_dtype=None, workspace=None, stream=None) -> Compacted:
    """Cut each head's cache into n_chunks contiguous chunks, compact every chunk
    to t entries on its own, concatenate.  keys/bias/values/idx are
    [B, n_chunks * t, ...] (idx in whole-cache positions); status is
    [B, n_chunks]."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    B, n, d = Q.shape
    T = K.shape[1]
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, agg, ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    need = workspace_bytes_chunked(p, n_chunks)
    if need == 0:
        raise ValueError("invalid chunked compaction parameters (T % n_chunks, t <= T/n_chunks)")
    ws = _workspace(p, dev, workspace, need)
    m = n_chunks * t
    keys = torch.empty((B, m, d), dtype=Q.dtype, device=dev)
    bias = torch.empty((B, m), dtype=torch.float32, device=dev)
    values = torch.empty((B, m, d), dtype=vt, device=dev)
    idx = torch.empty((B, m), dtype=torch.int32, device=dev)
    status = torch.empty((B, n_chunks), dtype=torch.int32, device=dev)
    rc = load().kvc_compact_chunked(ctypes.byref(p), ctypes.c_int64(n_chunks), _vp(Q), _vp(K),
                                    _vp(V), _vp(keys), _vp(bias), _vp(values), _vp(idx),
                                    _vp(status), _vp(ws),
                                    ctypes.c_size_t(ws.numel() * ws.element_size()),
                                    _stream(stream, dev))
    _lib.check(rc)
    # intermediates() of this result index (head, chunk) entries b * n_chunks + c
    pc = make_params(B * n_chunks, T // n_chunks, n, d, t, dt, agg, ridge_rel, max_nnls_iters,
                     vs, refine_steps)
    return Compacted(keys, bias, values, idx, status, ws, pc)


def fit(Q, K, V, idx, *, ridge_rel: float = 1e-6, max_nnls_iters: int = 32,
        refine_steps: int = 0, out_v_dtype=None, workspace=None, stream=None) -> Compacted:
    """Bias and value fit for a given kept set idx [B, t] (int32, ascending)."""
    import torch
    Q, K, V, _ = _prep(Q, K, V)
    if idx.dim() == 1:
        idx = idx.unsqueeze(0)
    idx = idx.to(torch.int32).contiguous()
    B, n, d = Q.shape
    T, t = K.shape[1], idx.shape[1]
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f32"
    vs, vt = _vdt(out_v_dtype)
    p = make_params(B, T, n, d, t, dt, "rms", ridge_rel, max_nnls_iters, vs, refine_steps)
    dev = Q.device
    ws = _workspace(p, dev, workspace)
    bias = torch.empty((B, t), dtype=torch.float32, device=dev)
    values = torch.empty((B, t, d), dtype=vt, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = load().kvc_fit(ctypes.byref(p), _vp(Q), _vp(K), _vp(V), _vp(idx), _vp(bias),
                        _vp(values), _vp(status), _vp(ws),
                        ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(stream, dev))
    _lib.check(rc)
    keys = None
    return Compacted(keys, bias, values, idx, status, ws, p)


def attend(Q, K1, V1, bias1=None, K2=None, V2=None, *, workspace=None, stream=None):
    """Attention of Q [B,m,d] over block 1 (K1, V1, optional per-key bias1)
    followed by block 2 (K2, V2, no bias): returns (out [B,m,d] float32,
    lse [B,m] float64).  K1, K2, V2 and Q share one dtype (bfloat16 or
    float32); V1 may also be float32 (fitted values)."""
    import torch
    if Q.dim() != 3 or K1.dim() != 3 or V1.dim() != 3:
        raise ValueError("expected Q [B,m,d], K1 and V1 [B,t1,d]")
    B, m, d = Q.shape
    t1 = K1.shape[1]
    if Q.dtype not in (torch.bfloat16, torch.float32) or K1.dtype != Q.dtype:
        raise ValueError("Q and K1 must share one dtype: bfloat16 or float32")
    if V1.shape != K1.shape or V1.dtype not in (Q.dtype, torch.float32):
        raise ValueError("V1 must match K1's shape, in Q's dtype or float32")
    t2 = 0 if K2 is None else K2.shape[1]
    if t2:
        if K2.dtype != Q.dtype or V2 is None or V2.dtype != Q.dtype or V2.shape != K2.shape:
            raise ValueError("K2 and V2 must be [B,t2,d] in Q's dtype")
    if bias1 is not None and (bias1.dtype != torch.float32 or tuple(bias1.shape) != (B, t1)):
        raise ValueError("bias1 must be float32 [B, t1]")
    p = _lib.AttendParams()
    p.B, p.m, p.d, p.t1, p.t2 = B, m, d, t1, t2
    p.in_dtype = KVC_BF16 if Q.dtype == torch.bfloat16 else KVC_F32
    p.v1_f32 = 1 if (V1.dtype == torch.float32 and Q.dtype != torch.float32) else 0
    dev = Q.device
    Q, K1, V1 = Q.contiguous(), K1.contiguous(), V1.contiguous()
    out = torch.empty((B, m, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, m), dtype=torch.float64, device=dev)
    null = ctypes.c_void_p(None)
    need = int(load().kvc_attend_workspace_bytes(ctypes.byref(p)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if need and workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    wsp = _vp(workspace) if need else null
    b1 = _vp(bias1.contiguous()) if bias1 is not None else null
    k2 = _vp(K2.contiguous()) if t2 else null
    v2 = _vp(V2.contiguous()) if t2 else null
    rc = load().kvc_attend(ctypes.byref(p), _vp(Q), _vp(K1), b1, _vp(V1), k2, v2, _vp(out),
                           _vp(lse), wsp, ctypes.c_size_t(need), _stream(stream, dev))
    _lib.check(rc)
    return out, lse


def intermediates(res: Compacted) -> dict:
    """Views into the workspace: lse [B,n] (float64), O [B,n,d], imp [B,T] (sum of p^2 or
    p per key), w [B,t] (float64 NNLS multipliers), fit_flops [B,2] (fp64
    operations of the NNLS rounds and the value solve), value_C [B,t,d] (the
    value fit's float64 solution; row a is the a-th kept slot with w > 0, rows
    past the passive count unused).  Synchronise first."""
    import torch
    p = res.params
    L = workspace_layout(p)
    ws = res.workspace
    B, T, n, d, t = p.B, p.T, p.n, p.d, p.t

    def view(off, count, dtype, shape):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype).view(*shape)

    return {"lse": view(L.lse, B * n, torch.float64, (B, n)),
            "O": view(L.O, B * n * d, torch.float32, (B, n, d)),
            "imp": view(L.imp, B * T, torch.float32, (B, T)),
            "w": view(L.w, B * t, torch.float64, (B, t)),
            "fit_flops": view(L.fit_flops, B * 2, torch.float64, (B, 2)),
            # the value fit's float64 solution, row a = the a-th kept slot with w > 0
            "value_C": torch.as_strided(
                view(L.value_C, (B - 1) * L.value_ld ** 2 + t * L.value_ld, torch.float64,
                     ((B - 1) * L.value_ld ** 2 + t * L.value_ld,)),
                (B, t, d), (L.value_ld ** 2, L.value_ld, 1)),
            **({"omp_order": view(L.omp_order, B * t, torch.int32, (B, t))} if res.omp else {})}
