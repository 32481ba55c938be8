"""ctypes binding of libkvc.so (include/kvc.h).  Argument marshalling only:
every step of the compaction runs in the library's HIP kernels; torch only
supplies device memory and the stream."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

KVC_OK, KVC_EINVAL, KVC_EWORKSPACE, KVC_EHIP, KVC_EUNSUPPORTED = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 64 << 20  # KVC_NOALLOC_SCRATCH_BYTES
KVC_F32, KVC_BF16 = 0, 1
KVC_AGG_RMS, KVC_AGG_MEAN = 0, 1
(STATUS_NOT_SPD, STATUS_NNLS_CAP, STATUS_NONFINITE, STATUS_SYNC_TIMEOUT, STATUS_BUDGET,
 STATUS_PROTECT, STATUS_RIDGE_RAISED) = 1, 2, 4, 8, 16, 32, 64


def status_raises(status: int) -> int:
    """Number of tenfold ridge raises recorded in a status word (bits 8-9)."""
    return (int(status) >> 8) & 3

EXPORTS = ("kvc_params_default", "kvc_workspace_bytes", "kvc_compact", "kvc_compact_noalloc",
           "kvc_fit",
           "kvc_workspace_bytes_chunked", "kvc_compact_chunked", "kvc_compact_ragged",
           "kvc_compact_protected", "kvc_attend", "kvc_attend_workspace_bytes", "kvc_workspace_bytes_omp",
           "kvc_compact_omp",
           "kvc_workspace_layout", "kvc_profile_enable", "kvc_profile_read", "kvc_set_wait_limit",
           "kvc_strerror")
STAGES = {"score_lse": 0, "expweight": 1, "select": 2, "ps": 3, "gram": 4, "nnls": 5,
          "value": 6, "total": 7, "imp_reduce": 8, "topt": 9, "gather": 10, "value_gram": 11,
          "value_sweep": 12}


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("n", ctypes.c_int64),
                ("d", ctypes.c_int64), ("t", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("agg", ctypes.c_int32), ("ridge_rel", ctypes.c_double),
                ("max_nnls_iters", ctypes.c_int32), ("out_v_dtype", ctypes.c_int32),
                ("refine_steps", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AttendParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("m", ctypes.c_int64), ("d", ctypes.c_int64),
                ("t1", ctypes.c_int64), ("t2", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("v1_f32", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("reserved2", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [("lse", ctypes.c_size_t), ("O", ctypes.c_size_t), ("imp", ctypes.c_size_t),
                ("w", ctypes.c_size_t), ("fit_flops", ctypes.c_size_t),
                ("omp_order", ctypes.c_size_t), ("value_C", ctypes.c_size_t),
                ("value_ld", ctypes.c_size_t)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raises if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                           "kv_cache_compaction_head_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.kvc_params_default.argtypes = [P]
    lib.kvc_params_default.restype = None
    lib.kvc_workspace_bytes.argtypes = [P]
    lib.kvc_workspace_bytes.restype = ctypes.c_size_t
    lib.kvc_compact.argtypes = [P, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp, ctypes.c_size_t, vp]
    lib.kvc_compact.restype = ctypes.c_int
    lib.kvc_compact_noalloc.argtypes = [P, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp]
    lib.kvc_compact_noalloc.restype = ctypes.c_int
    lib.kvc_fit.argtypes = [P, vp, vp, vp, i32p, f32p, f32p, i32p, vp, ctypes.c_size_t, vp]
    lib.kvc_fit.restype = ctypes.c_int
    lib.kvc_workspace_bytes_chunked.argtypes = [P, ctypes.c_int64]
    lib.kvc_workspace_bytes_chunked.restype = ctypes.c_size_t
    lib.kvc_compact_chunked.argtypes = [P, ctypes.c_int64, vp, vp, vp, vp, f32p, f32p, i32p, i32p,
                                        vp, ctypes.c_size_t, vp]
    lib.kvc_compact_chunked.restype = ctypes.c_int
    lib.kvc_compact_ragged.argtypes = [P, vp, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp,
                                       ctypes.c_size_t, vp]
    lib.kvc_compact_ragged.restype = ctypes.c_int
    lib.kvc_compact_protected.argtypes = [P, vp, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp,
                                          ctypes.c_size_t, vp]
    lib.kvc_compact_protected.restype = ctypes.c_int
    lib.kvc_workspace_bytes_omp.argtypes = [P]
    lib.kvc_workspace_bytes_omp.restype = ctypes.c_size_t
    lib.kvc_compact_omp.argtypes = [P, vp, vp, vp, vp, f32p, f32p, i32p, i32p, vp, ctypes.c_size_t,
                                    vp]
    lib.kvc_compact_omp.restype = ctypes.c_int
    lib.kvc_attend_workspace_bytes.argtypes = [ctypes.POINTER(AttendParams)]
    lib.kvc_attend_workspace_bytes.restype = ctypes.c_size_t
    lib.kvc_attend.argtypes = [ctypes.POINTER(AttendParams), vp, vp, f32p, vp, vp, vp, f32p, vp,
                               vp, ctypes.c_size_t, vp]
    lib.kvc_attend.restype = ctypes.c_int
    lib.kvc_workspace_layout.argtypes = [P, ctypes.POINTER(WsLayout)]
    lib.kvc_workspace_layout.restype = ctypes.c_int
    lib.kvc_profile_enable.argtypes = [ctypes.c_uint32]
    lib.kvc_profile_enable.restype = ctypes.c_int
    lib.kvc_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.kvc_profile_read.restype = ctypes.c_int
    lib.kvc_set_wait_limit.argtypes = [ctypes.c_uint64]
    lib.kvc_set_wait_limit.restype = ctypes.c_int
    lib.kvc_strerror.argtypes = [ctypes.c_int]
    lib.kvc_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_params(B, T, n, d, t, dtype, agg="rms", ridge_rel=1e-6, max_nnls_iters=32,
                out_v_dtype="f32", refine_steps=0) -> Params:
    p = Params()
    load().kvc_params_default(ctypes.byref(p))
    p.B, p.T, p.n, p.d, p.t = int(B), int(T), int(n), int(d), int(t)
    p.in_dtype = {"bf16": KVC_BF16, "f32": KVC_F32}[dtype]
    p.agg = {"rms": KVC_AGG_RMS, "mean": KVC_AGG_MEAN}[agg]
    p.ridge_rel = float(ridge_rel)
    p.max_nnls_iters = int(max_nnls_iters)
    p.out_v_dtype = {"bf16": KVC_BF16, "f32": KVC_F32}[out_v_dtype]
    p.refine_steps = int(refine_steps)
    return p


def set_wait_limit(ticks: int) -> None:
    """Bound on each fit-team wait, in 100 MHz ticks (0: the 20 s default)."""
    check(load().kvc_set_wait_limit(int(ticks)))


def workspace_bytes(p: Params) -> int:
    return int(load().kvc_workspace_bytes(ctypes.byref(p)))


def workspace_bytes_chunked(p: Params, n_chunks: int) -> int:
    return int(load().kvc_workspace_bytes_chunked(ctypes.byref(p), int(n_chunks)))


def workspace_bytes_omp(p: Params) -> int:
    return int(load().kvc_workspace_bytes_omp(ctypes.byref(p)))


def workspace_layout(p: Params) -> WsLayout:
    out = WsLayout()
    rc = load().kvc_workspace_layout(ctypes.byref(p), ctypes.byref(out))
    if rc:
        raise ValueError(strerror(rc))
    return out


def profile_enable(stages) -> None:
    """Record event pairs around the named stages in subsequent calls."""
    mask = 0
    for s in stages:
        mask |= 1 << STAGES[s]
    check(load().kvc_profile_enable(mask))


def profile_read(stage: str):
    """(total milliseconds, recorded launches) for one stage; waits for it."""
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    check(load().kvc_profile_read(STAGES[stage], ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value


def strerror(code: int) -> str:
    return load().kvc_strerror(int(code)).decode()


def check(rc: int) -> None:
    if rc == KVC_OK:
        return
    msg = f"kvc error {rc}: {strerror(rc)}"
    if rc in (KVC_EINVAL, KVC_EWORKSPACE, KVC_EUNSUPPORTED):
        raise ValueError(msg)
    raise RuntimeError(msg)
