"""Synthetic end-to-end runs of the RocketKV path through the package's C-ABI binding.

Orchestration only (no arithmetic of the method): draw each layer's prompt on the GPU, evict it
with SnapKV++, keep the compressed cache, and fold layers into the batch axis (batch index
layer * B + b), as a multi-layer decode step processes every layer's heads in one launch.
Host copies of a few (layer, b, KV head) inputs can be kept for the oracle.
"""
from __future__ import annotations

import math

import torch

from . import generate as gen
from .configs import Workload


def _dtype(w: Workload):
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def compressed_stack(rkv, w: Workload, layers: int, sample=(), device="cuda", on_layer=None):
    """Evicts `layers` independently drawn layers (on_layer(layer), if given, after each one).
    Returns dict with
    k_c, v_c [layers*B, Hkv, Lc, D], kept [layers*B, Hkv, Lc] int32,
    needles_ok (bool: every planted needle survived in every head) and
    host: {(layer, b, h): dict(q_win [G,W,D], k [L,D], v [L,D], needle_pos)} storage arrays."""
    B, Hkv, Lc, D, G = w.B, w.Hkv, w.Lc, w.D, w.G
    dt = _dtype(w)
    k_c = torch.empty((layers * B, Hkv, Lc, D), dtype=dt, device=device)
    v_c = torch.empty_like(k_c)
    kept = torch.empty((layers * B, Hkv, Lc), dtype=torch.int32, device=device)
    nbytes = rkv.snapkvpp_workspace_bytes(B, w.Hq, Hkv, w.L, D, w.W, w.keep, 0 if w.dtype == "fp32" else 1)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    host = {}
    needles_ok = True
    scale = 1.0 / math.sqrt(D)
    for layer in range(layers):
        d = gen.device_prompt_layer(w, layer, device)
        for (sl, b, h) in sample:
            if sl == layer:
                host[(sl, b, h)] = dict(
                    q_win=gen.torch_to_storage(d["q_win"][b, h * G:(h + 1) * G]),
                    k=gen.torch_to_storage(d["k"][b, h]), v=gen.torch_to_storage(d["v"][b, h]),
                    needle_pos=d["needle_pos"][b, h].cpu().numpy())
        sl_ = slice(layer * B, (layer + 1) * B)
        rkv.rkv_snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, "avg", scale,
                               kept_idx=kept[sl_], k_out=k_c[sl_], v_out=v_c[sl_], workspace=ws)
        if d["needle_pos"].shape[-1] and w.keep < w.L:
            hit = (kept[sl_].unsqueeze(-1).long() == d["needle_pos"].unsqueeze(-2)).any(dim=-2)
            needles_ok = needles_ok and bool(hit.all())
        del d
        if on_layer is not None:
            on_layer(layer)
    return dict(k_c=k_c, v_c=v_c, kept=kept, needles_ok=needles_ok, host=host)
