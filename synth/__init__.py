"""Seeded synthetic workloads for attention-matching KV-cache compaction.

This module only draws and rounds numbers; it holds none of the method's
arithmetic.  Both the float64 oracle and the GPU path take their inputs from
here, so that the two see the very same bits.

The workloads stand in for the long-context question-answering suites that
"Fast KV Compaction via Attention Matching" (section 4, results) evaluates on;
no text, model weights or real caches are available, so every tensor is drawn
from a fixed distribution with the shapes of a Llama-3-8B-style cache
(32 layers x 8 KV heads, head dim 128, 4 query heads per KV head).

Every draw comes from ``numpy.random.default_rng([config, head, role])`` with
roles 0 = reference queries, 1 = keys, 2 = values, 3 = held-out queries,
4 = auxiliary draws (channel scales, cluster centres, sink positions).
Values are drawn in float64, then rounded to the storage dtype: float32, or
bfloat16 through float32 with round-to-nearest-even at each step.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROLE_Q, ROLE_K, ROLE_V, ROLE_QHOLD, ROLE_AUX = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and key distribution of one synthetic compaction workload."""

    cfg: int            # seed namespace (the config number for the named ones)
    name: str
    B: int              # independent (layer, KV head) problems
    T: int              # cache length per head
    n: int              # reference queries per head
    d: int              # head dim
    t: int              # kept keys per head
    dtype: str          # "f32" or "bf16"
    keys: str           # key distribution, see ``_keys``
    n_hold: int = 256   # held-out queries per head (quality only)

    @property
    def ratio(self) -> float:
        return self.T / self.t


CONFIGS: dict[int, Workload] = {
    1: Workload(1, "single_head_fp32_T512_8x", 1, 512, 64, 64, 64, "f32", "normal", 64),
    2: Workload(2, "llama3_8b_layer_T8k_10x_channel_outliers", 8, 8192, 1024, 128, 819,
                "bf16", "channel_lognormal"),
    3: Workload(3, "llama3_8b_layer_T32k_50x_clustered", 8, 32768, 2048, 128, 655,
                "bf16", "clusters"),
    4: Workload(4, "llama3_8b_32layer_stack_T16k_20x_sinks", 256, 16384, 1024, 128, 819,
                "bf16", "sinks"),
    5: Workload(5, "long_T128k_50x_student_t", 8, 131072, 4096, 128, 2621,
                "bf16", "student_t3"),
}


def custom(seed: int, B: int, T: int, n: int, d: int, t: int, dtype: str = "bf16",
           keys: str = "normal", n_hold: int = 64) -> Workload:
    """A workload of arbitrary shape (tests).  Seeds live in their own namespace."""
    return Workload(1000 + seed, f"custom{seed}", B, T, n, d, t, dtype, keys, n_hold)


def _rng(cfg: int, head: int, role: int) -> np.random.Generator:
    return np.random.default_rng([cfg, head, role])


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> bfloat16 bit patterns (uint16), via float32, RNE."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16_bits(x)
    raise ValueError(dtype)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Stored array (float32 or bf16 bits) -> exact float64 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def _keys(w: Workload, head: int) -> np.ndarray:
    rk, ra = _rng(w.cfg, head, ROLE_K), _rng(w.cfg, head, ROLE_AUX)
    T, d = w.T, w.d
    if w.keys == "normal":
        return rk.standard_normal((T, d))
    if w.keys == "channel_lognormal":
        # per-(head, channel) scale ~ LogNormal(0, 0.5): channel outliers
        scale = ra.lognormal(0.0, 0.5, size=d)
        return rk.standard_normal((T, d)) * scale
    if w.keys == "clusters":
        # 64 unit-norm centres, isotropic noise of std 0.3 per coordinate
        g = ra.standard_normal((64, d))
        centres = g / np.linalg.norm(g, axis=1, keepdims=True)
        assign = ra.integers(0, 64, size=T)
        return centres[assign] + 0.3 * rk.standard_normal((T, d))
    if w.keys == "sinks":
        # 1% of tokens (without replacement) get their key scaled x4
        k = rk.standard_normal((T, d))
        n_sink = max(1, (T + 50) // 100)
        sinks = ra.choice(T, size=n_sink, replace=False)
        k[sinks] *= 4.0
        return k
    if w.keys == "student_t3":
        # i.i.d. Student-t (nu = 3) elements: heavy-tailed token norms
        return rk.standard_t(3.0, size=(T, d))
    if w.keys == "zeros":
        return np.zeros((T, d))
    raise ValueError(w.keys)


def head(w: Workload, h: int) -> dict[str, np.ndarray]:
    """Stored arrays of one head: Q [n,d], K [T,d], V [T,d], Qhold [n_hold,d]."""
    scale = 1.0 / np.sqrt(w.d)
    q = _rng(w.cfg, h, ROLE_Q).standard_normal((w.n, w.d)) * scale
    v = _rng(w.cfg, h, ROLE_V).standard_normal((w.T, w.d))
    qh = _rng(w.cfg, h, ROLE_QHOLD).standard_normal((w.n_hold, w.d)) * scale
    return {"Q": _store(q, w.dtype), "K": _store(_keys(w, h), w.dtype),
            "V": _store(v, w.dtype), "Qhold": _store(qh, w.dtype)}


def batch(w: Workload, heads=None, threads: int = 8) -> dict[str, np.ndarray]:
    """Stacked stored arrays [Bh, ...] for the given heads (default: all B)."""
    hs = list(range(w.B)) if heads is None else list(heads)
    store_dt = np.float32 if w.dtype == "f32" else np.uint16
    out = {"Q": np.empty((len(hs), w.n, w.d), store_dt),
           "K": np.empty((len(hs), w.T, w.d), store_dt),
           "V": np.empty((len(hs), w.T, w.d), store_dt),
           "Qhold": np.empty((len(hs), w.n_hold, w.d), store_dt)}

    def fill(i_h):
        i, h = i_h
        a = head(w, h)
        for k in out:
            out[k][i] = a[k]

    with ThreadPoolExecutor(max(1, min(threads, len(hs)))) as ex:
        list(ex.map(fill, enumerate(hs)))
    return out
