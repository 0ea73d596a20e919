"""Seeded synthetic inputs for RocketKV's hot path (shared by the oracle tests and the GPU path).

Holds no arithmetic of the method: only random draws, the planting of needle keys, and
round-to-nearest-even narrowing to bfloat16 storage.

Recipe (per layer, per sequence b, per KV head h; every (layer, b, h) has its own sub-seed, so
any head can be generated alone and equals the same head of a full draw):
  * Q_win of the group's G query heads [G,W,D], K [L,D], V [L,D] and each decode query of the
    group [G,D] are i.i.d. N(0,1) in float32.
  * K is multiplied channel-wise by exp(N(0,1)) factors, one per (layer, b, h, channel).
  * Needles: u_h = unit vector along the sum of the group's window queries sum_{g,i} Q_win[g,i];
    n_needles distinct positions drawn uniformly from the prefix [0, L-W); each needle key is
    replaced by NEEDLE_GAIN * ||K||_rms * u_h, where ||K||_rms is the root-mean-square norm of the
    head's scaled keys: a key three times as long as a typical key of the head, pointing along
    the query direction.
  * bf16 workloads round every tensor to bfloat16 (round to nearest even) after planting.
Sub-seeds: numpy SeedSequence([seed, cfg_id, layer, tensor_id, b, h(, step)]).

`device_prompt_layer` draws the same distributions with torch's generator on the GPU (different
values); it serves the timed runs of the large workloads, where host generation would dominate.
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


def prompt_head(w: Workload, layer: int, b: int, h: int) -> dict:
    """One (layer, b, KV head): q_win [G,W,D], k [L,D], v [L,D] (float32, before rounding),
    needle positions [n] and direction [D]."""
    G, D, L, W = w.G, w.D, w.L, w.W
    q_win = _rng(w, layer, _T_QWIN, b, h).standard_normal((G, W, D), dtype=np.float32)
    k = _rng(w, layer, _T_K, b, h).standard_normal((L, D), dtype=np.float32)
    v = _rng(w, layer, _T_V, b, h).standard_normal((L, D), dtype=np.float32)
    k *= np.exp(_rng(w, layer, _T_SCALE, b, h).standard_normal(D)).astype(np.float32)
    n = min(w.n_needles, max(L - W, 0))
    s = q_win.astype(np.float64).sum(axis=(0, 1))
    u = (s / np.linalg.norm(s)).astype(np.float32)
    pos = np.sort(_rng(w, layer, _T_NEEDLE, b, h).choice(L - W, size=n, replace=False)) \
        if n else np.zeros(0, dtype=np.int64)
    if n:
        rms = np.sqrt(np.mean(np.sum(k.astype(np.float64) ** 2, axis=1)))
        k[pos] = (NEEDLE_GAIN * rms) * u
    return dict(q_win=q_win, k=k, v=v, needle_pos=pos.astype(np.int64), needle_dir=u)


def prompt_layer(w: Workload, layer: int = 0) -> dict:
    """One layer's prefill inputs in storage form: q_win [B,Hq,W,D], k/v [B,Hkv,L,D], plus
    needle_pos [B,Hkv,n] and needle_dir [B,Hkv,D]."""
    B, Hq, Hkv, D, L, W, G = w.B, w.Hq, w.Hkv, w.D, w.L, w.W, w.G
    n = min(w.n_needles, max(L - W, 0))
    q_win = np.empty((B, Hq, W, D), dtype=np.float32)
    k = np.empty((B, Hkv, L, D), dtype=np.float32)
    v = np.empty((B, Hkv, L, D), dtype=np.float32)
    needle_pos = np.zeros((B, Hkv, n), dtype=np.int64)
    needle_dir = np.zeros((B, Hkv, D), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            d = prompt_head(w, layer, b, h)
            q_win[b, h * G:(h + 1) * G] = d["q_win"]
            k[b, h], v[b, h] = d["k"], d["v"]
            needle_pos[b, h], needle_dir[b, h] = d["needle_pos"], d["needle_dir"]
    return dict(q_win=to_storage(q_win, w.dtype), k=to_storage(k, w.dtype),
                v=to_storage(v, w.dtype), needle_pos=needle_pos, needle_dir=needle_dir)


def decode_queries(w: Workload, layer: int = 0, steps: int | None = None) -> np.ndarray:
    """Decode queries [steps, B, Hq, D] in storage form, one independent draw per step and group."""
    steps = w.steps if steps is None else steps
    out = np.empty((steps, w.B, w.Hq, w.D), dtype=np.float32)
    G = w.G
    for s in range(steps):
        for b in range(w.B):
            for h in range(w.Hkv):
                out[s, b, h * G:(h + 1) * G] = _rng(w, layer, _T_QDEC, b, h, s).standard_normal(
                    (G, w.D), dtype=np.float32)
    return to_storage(out, w.dtype)


def needle_queries(w: Workload, needle_dir: np.ndarray) -> np.ndarray:
    """Decode queries [B, Hq, D] aimed at the needles: q_g = sqrt(D) * u_h for every g in group h."""
    q = np.repeat(needle_dir, w.G, axis=1) * np.float32(np.sqrt(w.D))
    return to_storage(q, w.dtype)


def storage_to_torch(x: np.ndarray, device="cuda"):
    """Storage array -> torch tensor on `device` (uint16 bf16 bits become torch.bfloat16)."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def torch_to_storage(t) -> np.ndarray:
    """torch tensor -> host storage array (bfloat16 becomes uint16 bits)."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def device_prompt_layer(w: Workload, layer: int, device="cuda"):
    """The recipe above drawn with torch's generator on `device`: dict of torch tensors
    q_win [B,Hq,W,D], k/v [B,Hkv,L,D] in the workload dtype, needle_pos [B,Hkv,n] (int64) and
    needle_dir [B,Hkv,D] (float32)."""
    import torch
    B, Hq, Hkv, D, L, W, G = w.B, w.Hq, w.Hkv, w.D, w.L, w.W, w.G
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed * 1_000_003 + w.cfg_id * 10_007 + layer) & 0x7FFFFFFFFFFFFFFF)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    q_win = torch.randn((B, Hq, W, D), **f32)
    k = torch.randn((B, Hkv, L, D), **f32)
    k.mul_(torch.randn((B, Hkv, 1, D), **f32).exp_())
    v = torch.randn((B, Hkv, L, D), **f32).to(dt)
    n = min(w.n_needles, max(L - W, 0))
    s = q_win.view(B, Hkv, G * W, D).double().sum(dim=2)
    u = (s / s.norm(dim=-1, keepdim=True)).float()
    pos = torch.zeros((B, Hkv, n), dtype=torch.int64, device=device)
    if n:
        rms = k.double().square().sum(-1).mean(-1).sqrt().float()  # [B,Hkv]
        for b in range(B):
            for h in range(Hkv):
                p = torch.randperm(L - W, generator=gen, device=device)[:n].sort().values
                pos[b, h] = p
                k[b, h, p] = (NEEDLE_GAIN * rms[b, h]) * u[b, h]
    return dict(q_win=q_win.to(dt), k=k.to(dt), v=v, needle_pos=pos, needle_dir=u)


def device_decode_queries(w: Workload, layer: int, steps: int, device="cuda"):
    """Decode queries [steps, B, Hq, D] drawn on `device` (same distribution, torch values)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed * 1_000_003 + w.cfg_id * 10_007 + layer + 7_777_777) & 0x7FFFFFFF)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    return torch.randn((steps, w.B, w.Hq, w.D), device=device, dtype=torch.float32,
                       generator=gen).to(dt)
