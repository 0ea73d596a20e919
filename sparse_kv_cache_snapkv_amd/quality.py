"""Selection quality of the hybrid approximation against Exact-TopK, from the library's calls.

Exact-TopK (rebuttal, "Measurement of Exact-TopK") is the reference selection that ranks tokens by
their true scores, separately per query head and per step. Its recall and the share of the exact
softmax mass that a selection covers are the two measures used here. "Novelty: RocketKV is
SnapKV + QUEST" argues that one compression ratio is better spent on both the sequence and the
head dimension than on either alone (QUEST-like: whole-channel pages; SparQ-like: one-token
pages); the same measures compare those settings on synthetic data, with no dataset.

The heavy work runs in librkv. Exact per-head scores are the approximate scores of one-token
pages over all D channels, on a copy of K per query head: for one-token pages Kmin = Kmax = K, and
with one query head per group the bound is the dot product itself. The top-k calls pick both sets.
Only the set intersections and the attention mass are computed on the host.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from .api import rkv_build_page_summaries, rkv_hybrid_approx_scores, rkv_topk_select


def exact_scores(q: torch.Tensor, k_c: torch.Tensor) -> torch.Tensor:
    """q [B,Hq,D], k_c [B,Hkv,Lc,D] -> float32 [B,Hq,Lc]: q_g . k_t for every query head."""
    G = q.shape[1] // k_c.shape[1]
    k_rep = k_c.repeat_interleave(G, dim=1).contiguous()
    k_t, _ = rkv_build_page_summaries(k_rep, 1)  # one-token pages: Kmin = Kmax = K^T
    return rkv_hybrid_approx_scores(q, k_t, k_t, q.shape[2])


def hybrid_tokens(q: torch.Tensor, k_c: torch.Tensor, page_size: int, r: int,
                  topk: int) -> np.ndarray:
    """Token slots [B,Hkv,n_pages*page_size] the hybrid selection attends (slots past the cache
    end, in a partial last page, are -1)."""
    Lc = k_c.shape[2]
    kmin, kmax = rkv_build_page_summaries(k_c, page_size)
    n_pages = min(topk // page_size, kmin.shape[-1])
    pages = rkv_topk_select(rkv_hybrid_approx_scores(q, kmin, kmax, r), n_pages)
    pg = pages.cpu().numpy().astype(np.int64)
    toks = (pg[..., :, None] * page_size + np.arange(page_size)).reshape(*pg.shape[:-1], -1)
    return np.where(toks < Lc, toks, -1)


def selection_quality(q: torch.Tensor, k_c: torch.Tensor, page_size: int, r: int, topk: int,
                      scale: Optional[float] = None,
                      exact: Optional[torch.Tensor] = None) -> dict:
    """Against Exact-TopK (topk tokens per query head): token recall and the share of the exact
    softmax mass that the hybrid selection covers, averaged over (b, query head); mass_exact is
    the Exact-TopK ceiling of the latter."""
    B, Hq, D = q.shape
    G = Hq // k_c.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if exact is None:
        exact = exact_scores(q, k_c)
    top = rkv_topk_select(exact, topk).cpu().numpy()
    s = exact.cpu().numpy().astype(np.float64) * scale
    hyb = hybrid_tokens(q, k_c, page_size, r, topk)
    recall, mass, mass_exact = [], [], []
    for b in range(B):
        for g in range(Hq):
            p = np.exp(s[b, g] - s[b, g].max())
            p /= p.sum()
            h = hyb[b, g // G]
            h = h[h >= 0]
            recall.append(len(np.intersect1d(h, top[b, g])) / top.shape[-1])
            mass.append(p[h].sum())
            mass_exact.append(p[top[b, g]].sum())
    return dict(recall=float(np.mean(recall)), mass=float(np.mean(mass)),
                mass_exact=float(np.mean(mass_exact)))
