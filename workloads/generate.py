"""Seeded synthetic inputs for RocketKV's hot path (shared by the oracle tests and the GPU path).

Holds no arithmetic of the method: only random draws, the planting of needle keys, and
round-to-nearest-even narrowing to bfloat16 storage.

Recipe (per layer, per sequence b, per KV head h):
  * Q_win [B,Hq,W,D], K [B,Hkv,L,D], V [B,Hkv,L,D] and every decode query [steps,B,Hq,D] are
    i.i.d. N(0,1) in float32.
  * K is multiplied channel-wise by exp(N(0,1)) factors, one per (layer, b, h, channel).
  * Needles: u_h = unit vector along the sum of the group's window queries
    sum_{g in group(h)} sum_i Q_win[b,g,i]; n_needles distinct positions drawn uniformly from the
    prefix [0, L-W); each needle key is replaced by NEEDLE_GAIN * ||K||_rms * u_h, where ||K||_rms is
    the root-mean-square norm of that head's scaled keys, i.e. a key three times as long as a
    typical key of the head, pointing along the query direction.
  * bf16 workloads round every tensor to bfloat16 (round to nearest even) after planting.
Sub-seeds come from numpy SeedSequence([seed, cfg_id, layer, tensor_id(, step)]).
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

NEEDLE_GAIN = 3.0

_T_QWIN, _T_K, _T_V, _T_SCALE, _T_NEEDLE, _T_QDEC = range(6)


def _rng(w: Workload, layer: int, tensor: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, w.cfg_id, layer, tensor, *extra]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> the workload's storage form (float32, or uint16 bf16 bits)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def prompt_layer(w: Workload, layer: int = 0) -> dict:
    """One layer's prefill inputs: q_win, k, v (storage form), needle positions and directions."""
    B, Hq, Hkv, D, L, W, G = w.B, w.Hq, w.Hkv, w.D, w.L, w.W, w.G
    q_win = _rng(w, layer, _T_QWIN).standard_normal((B, Hq, W, D), dtype=np.float32)
    k = _rng(w, layer, _T_K).standard_normal((B, Hkv, L, D), dtype=np.float32)
    v = _rng(w, layer, _T_V).standard_normal((B, Hkv, L, D), dtype=np.float32)
    chan_scale = np.exp(_rng(w, layer, _T_SCALE).standard_normal((B, Hkv, 1, D))).astype(np.float32)
    k *= chan_scale
    n = min(w.n_needles, max(L - W, 0))
    needle_pos = np.zeros((B, Hkv, n), dtype=np.int64)
    u = np.zeros((B, Hkv, D), dtype=np.float32)
    nrng = _rng(w, layer, _T_NEEDLE)
    for b in range(B):
        for h in range(Hkv):
            s = q_win[b, h * G:(h + 1) * G].astype(np.float64).sum(axis=(0, 1))
            u[b, h] = (s / np.linalg.norm(s)).astype(np.float32)
            rms = np.sqrt(np.mean(np.sum(k[b, h].astype(np.float64) ** 2, axis=1)))
            pos = np.sort(nrng.choice(L - W, size=n, replace=False)) if n else needle_pos[b, h]
            needle_pos[b, h] = pos
            k[b, h, pos] = (NEEDLE_GAIN * rms) * u[b, h]
    return dict(q_win=to_storage(q_win, w.dtype), k=to_storage(k, w.dtype),
                v=to_storage(v, w.dtype), needle_pos=needle_pos, needle_dir=u)


def decode_queries(w: Workload, layer: int = 0, steps: int | None = None) -> np.ndarray:
    """Decode queries [steps, B, Hq, D] in storage form, one independent draw per step."""
    steps = w.steps if steps is None else steps
    out = np.empty((steps, w.B, w.Hq, w.D), dtype=np.float32)
    for s in range(steps):
        out[s] = _rng(w, layer, _T_QDEC, s).standard_normal((w.B, w.Hq, w.D), dtype=np.float32)
    return to_storage(out, w.dtype)


def needle_queries(w: Workload, needle_dir: np.ndarray) -> np.ndarray:
    """Decode queries [B, Hq, D] aimed at the needles: q_g = sqrt(D) * u_h for every g in group h."""
    q = np.repeat(needle_dir, w.G, axis=1) * np.float32(np.sqrt(w.D))
    return to_storage(q, w.dtype)
