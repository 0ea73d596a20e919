"""Plain CPU oracle of RocketKV's hot path: SnapKV++ eviction and hybrid sparse decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never does. It shares no code with the HIP kernels.

Everything is computed in float64 on the exact input values (bfloat16 inputs are widened exactly).
Every selection is the head of a full stable sort: higher score first, lower index on ties.

Sources (RocketKV, arXiv 2502.14051; pages: the summarizepaper.com summary, the paperhub.cn
authors' rebuttal, the pith.science abstract):
  * stage 1, SnapKV++: one-time top-k filtering of the prompt driven by the queries at the end of
    the prompt (rebuttal, "Measurement of Exact-TopK" and "SCBench Results"), with a GQA
    enhancement (summary, key points; rebuttal, "Novelty of SnapKV++") and a pooling kernel whose
    size is a parameter (rebuttal, "Potential Sensitivity to Kernel Size in SnapKV++"); eviction
    is independent per KV head and layer (rebuttal, "Is Needle Among Evicted Tokens").
  * stage 2, hybrid attention: per-page element-wise Kmin/Kmax, the bound max(q*Kmin, q*Kmax)
    taken only on the channels where |q| is large, one of Kmin/Kmax fetched per channel by the
    sign of q, GQA-consistent selection from the group sums of q and |q|, then pages with the
    highest scores are selected (rebuttal, "Explanation of Calculating Approximate Attention
    Scores", paper Figure 3); exact attention runs on the selected tokens (rebuttal, "Lack of
    Direct Latency Comparison", Step 3; "Are Different KV Tokens Retrieved at Each Decoding
    Step?").

Readings where the pages are silent (each listed with its reason in the design notes):
  scale is a parameter (1/sqrt(D) by default); the window softmax is causal over all keys up to
  the row's own position; only prefix columns [0, L-W) are scored; pooling is a zero-padded,
  same-size box over the prefix (average by default, max optional), applied after the group sum;
  `keep` counts the W window tokens, which are always kept; kept tokens stay in ascending
  position order; query head g belongs to KV head g // G; pages are ps consecutive slots of the
  compressed cache and a partial last page covers only its valid slots (a token appended during
  decoding extends the last page, or starts a new one at a page boundary); channels are chosen from
  sum_g |q_g| and the bound uses qbar = sum_g q_g; k tokens mean k/ps whole pages.

Parity pins: every function here is pinned by tests/test_oracle_pins.py against closed forms,
brute force, invariants or library routines; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- input decoding

def widen(x: np.ndarray) -> np.ndarray:
    """Storage array -> float64. uint16 arrays are bfloat16 bit patterns (widened exactly)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------- selection

def stable_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best scores, best first; ties go to the lower index.

    The three selections of the method (kept prompt tokens, top-|q| channels, top pages) all use
    this rule; the pages do not state a tie-break, so the lower index wins.
    """
    scores = np.asarray(scores, dtype=np.float64)
    k = max(0, min(int(k), scores.shape[0]))
    order = np.argsort(-scores, kind="stable")
    return order[:k].astype(np.int64)


def topk_ascending(scores: np.ndarray, k: int) -> np.ndarray:
    """The same selected set as stable_topk, listed in ascending index order."""
    return np.sort(stable_topk(scores, k))


# ----------------------------------------------------------------------------- stage 1: SnapKV++

def window_attention(q_win_grp: np.ndarray, k_head: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of the window queries of one GQA group over the whole prompt.

    q_win_grp [G, W, D] are the queries of the last W prompt positions; k_head [L, D].
    Window row i sits at position L-W+i and sees keys 0..L-W+i (causal).
    Returns A [G, W, L] with every row summing to 1 (masked entries are exactly 0).
    """
    G, W, D = q_win_grp.shape
    L = k_head.shape[0]
    s = scale * (q_win_grp @ k_head.T)
    pos = np.arange(L)[None, :]
    row_pos = (L - W + np.arange(W))[:, None]
    s = np.where((pos <= row_pos)[None], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def group_column_sums(A: np.ndarray) -> np.ndarray:
    """c[j] = sum over the group's heads g and window rows i of A[g, i, j], for every column j."""
    return A.sum(axis=(0, 1))


def pool1d(c: np.ndarray, kernel: int, kind: str = "avg") -> np.ndarray:
    """Same-size 1D pooling with zero padding of kernel//2 on each side (kernel odd).

    avg: sum of the kernel-wide box divided by kernel (padding counted). max: box maximum.
    """
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pooling kernel must be odd and positive")
    h = kernel // 2
    padded = np.concatenate([np.zeros(h), np.asarray(c, dtype=np.float64), np.zeros(h)])
    boxes = np.lib.stride_tricks.sliding_window_view(padded, kernel)
    if kind == "avg":
        return boxes.sum(axis=1) / kernel
    if kind == "max":
        return boxes.max(axis=1)
    raise ValueError(kind)


def snapkvpp_head(q_win_grp, k_head, keep: int, kernel: int, scale: float, kind: str = "avg"):
    """SnapKV++ for one KV head: returns (kept [Lc] ascending, colsum [L-W], pooled [L-W]).

    Score of prefix token j: the group's window attention to j summed over heads and rows, then
    pooled. The keep-W best prefix tokens are kept together with all W window tokens.
    If keep >= L nothing is evicted.
    """
    G, W, D = q_win_grp.shape
    L = k_head.shape[0]
    n_prefix = L - W
    A = window_attention(q_win_grp, k_head, scale)
    colsum = group_column_sums(A)[:n_prefix]
    pooled = pool1d(colsum, kernel, kind) if n_prefix > 0 else np.zeros(0)
    if keep >= L:
        kept = np.arange(L, dtype=np.int64)
    else:
        if keep < W:
            raise ValueError("keep must be at least the window size")
        chosen = topk_ascending(pooled, keep - W)
        kept = np.concatenate([chosen, np.arange(n_prefix, L, dtype=np.int64)])
    return kept, colsum, pooled


def snapkvpp_evict(q_win, k, v, keep: int, kernel: int, scale: float, kind: str = "avg"):
    """SnapKV++ over a batch: q_win [B,Hq,W,D], k/v [B,Hkv,L,D] (storage arrays or float64).

    Returns dict(kept [B,Hkv,Lc], k_c/v_c [B,Hkv,Lc,D] float64, colsum/pooled [B,Hkv,L-W]).
    """
    q_win, k, v = widen(q_win), widen(k), widen(v)
    B, Hq, W, D = q_win.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    Lc = min(keep, L)
    kept = np.zeros((B, Hkv, Lc), dtype=np.int64)
    colsum = np.zeros((B, Hkv, L - W))
    pooled = np.zeros((B, Hkv, L - W))
    for b in range(B):
        for h in range(Hkv):
            kept[b, h], colsum[b, h], pooled[b, h] = snapkvpp_head(
                q_win[b, h * G:(h + 1) * G], k[b, h], keep, kernel, scale, kind)
    bi = np.arange(B)[:, None, None]
    hi = np.arange(Hkv)[None, :, None]
    return dict(kept=kept, k_c=k[bi, hi, kept], v_c=v[bi, hi, kept], colsum=colsum, pooled=pooled)


# ----------------------------------------------------------------------------- stage 2: hybrid

def page_summaries(k_c_head: np.ndarray, page_size: int):
    """Element-wise min and max of K over each page of page_size consecutive slots.

    k_c_head [Lc, D] -> (kmin_t, kmax_t) [D, P] channel-major, P = ceil(Lc / page_size); a partial
    last page covers only its valid slots.
    """
    Lc, D = k_c_head.shape
    P = -(-Lc // page_size)
    kmin = np.empty((D, P))
    kmax = np.empty((D, P))
    for p in range(P):
        page = k_c_head[p * page_size:min((p + 1) * page_size, Lc)]
        kmin[:, p] = page.min(axis=0)
        kmax[:, p] = page.max(axis=0)
    return kmin, kmax


def kv_append(k_c_head: np.ndarray, v_c_head: np.ndarray, kmin_t: np.ndarray,
               kmax_t: np.ndarray, Lc: int, k_new: np.ndarray, v_new: np.ndarray,
               page_size: int):
    """Decode-time append of one token to a compressed cache that grows (rebuttal, "SCBench
    Results": plain SnapKV compresses only the prompt, generated tokens join the cache; the page
    summaries of "Explanation of Calculating Approximate Attention Scores").

    k_c_head, v_c_head [cap, D] hold Lc valid slots; kmin_t, kmax_t [D, ceil(cap/ps)] summarise
    the first ceil(Lc/ps) pages. Slot Lc takes (k_new, v_new), and the summary of page
    Lc // page_size is recomputed from that page's slots up to and including Lc. Returns new
    arrays (the inputs are not modified).
    """
    k = np.array(k_c_head, dtype=np.float64)
    v = np.array(v_c_head, dtype=np.float64)
    kmin = np.array(kmin_t, dtype=np.float64)
    kmax = np.array(kmax_t, dtype=np.float64)
    k[Lc] = k_new
    v[Lc] = v_new
    p = Lc // page_size
    page = k[p * page_size:Lc + 1]
    kmin[:, p] = page.min(axis=0)
    kmax[:, p] = page.max(axis=0)
    return k, v, kmin, kmax


def select_channels(q_grp: np.ndarray, r: int):
    """Head-dim reduction for one GQA group: q_grp [G, D] -> (channels ascending [r], qbar [D]).

    Channels are the r largest of sum_g |q_g[c]|; qbar = sum_g q_g is the group query whose signs
    pick Kmin or Kmax, so every head of the group makes the same selection.
    """
    a = np.abs(q_grp).sum(axis=0)
    return topk_ascending(a, r), q_grp.sum(axis=0)


def approx_page_scores(qbar: np.ndarray, chans: np.ndarray, kmin_t: np.ndarray,
                       kmax_t: np.ndarray) -> np.ndarray:
    """Upper estimate of each page's best score on the chosen channels.

    s_hat[p] = sum_{c in chans} max(qbar[c] * kmin_t[c, p], qbar[c] * kmax_t[c, p]).
    """
    qc = qbar[chans][:, None]
    return np.maximum(qc * kmin_t[chans], qc * kmax_t[chans]).sum(axis=0)


def select_pages(scores: np.ndarray, n_pages: int) -> np.ndarray:
    """The n_pages highest-scoring pages, ascending (all pages when n_pages >= P)."""
    return topk_ascending(scores, n_pages)


def page_tokens(pages: np.ndarray, page_size: int, Lc: int) -> np.ndarray:
    """Valid compressed-cache slots of the given pages, in page order."""
    t = (np.asarray(pages, dtype=np.int64)[:, None] * page_size + np.arange(page_size)[None]).ravel()
    return t[t < Lc]


def sparse_attention(q_grp: np.ndarray, k_c_head: np.ndarray, v_c_head: np.ndarray,
                     tokens: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax attention of each query of the group over the given slots only.

    q_grp [G, D]; returns [G, D]: o_g = sum_t softmax_t(scale * <q_g, K[t]>) V[t].
    """
    ks = k_c_head[tokens]
    vs = v_c_head[tokens]
    s = scale * (q_grp @ ks.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vs


def hybrid_decode_step(q, k_c, v_c, kmin_t, kmax_t, page_size: int, r: int, topk: int,
                       scale: float):
    """One decode step over a batch.

    q [B,Hq,D]; k_c/v_c [B,Hkv,Lc,D]; kmin_t/kmax_t [B,Hkv,D,P] (storage arrays or float64).
    Returns dict(chans [B,Hkv,r], scores [B,Hkv,P], pages [B,Hkv,min(topk/ps, P)], out [B,Hq,D]).
    """
    if topk % page_size:
        raise ValueError("topk must be a multiple of the page size")
    q, k_c, v_c = widen(q), widen(k_c), widen(v_c)
    kmin_t, kmax_t = widen(kmin_t), widen(kmax_t)
    B, Hq, D = q.shape
    Hkv, Lc = k_c.shape[1], k_c.shape[2]
    P = kmin_t.shape[-1]
    G = Hq // Hkv
    r = min(r, D)
    n_pages = min(topk // page_size, P)
    chans = np.zeros((B, Hkv, r), dtype=np.int64)
    scores = np.zeros((B, Hkv, P))
    pages = np.zeros((B, Hkv, n_pages), dtype=np.int64)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hkv):
            qg = q[b, h * G:(h + 1) * G]
            chans[b, h], qbar = select_channels(qg, r)
            scores[b, h] = approx_page_scores(qbar, chans[b, h], kmin_t[b, h], kmax_t[b, h])
            pages[b, h] = select_pages(scores[b, h], n_pages)
            toks = page_tokens(pages[b, h], page_size, Lc)
            out[b, h * G:(h + 1) * G] = sparse_attention(qg, k_c[b, h], v_c[b, h], toks, scale)
    return dict(chans=chans, scores=scores, pages=pages, out=out)


def mt_view(k, v, kept):
    """RocketKV-MT (rebuttal, "SCBench Results"): SnapKV++ keeps every prompt token in memory and
    decoding selects only among the tokens it kept. The compressed cache is the view whose slot t
    of (b, h) is row kept[b, h, t] of the full caches k, v [B,Hkv,L,D]; the hybrid step then runs
    on that view unchanged. Returns the gathered (k_c, v_c) [B,Hkv,Lc,D] in float64."""
    k, v = widen(k), widen(v)
    kept = np.asarray(kept, dtype=np.int64)
    B, Hkv = kept.shape[:2]
    k_c = np.stack([np.stack([k[b, h, kept[b, h]] for h in range(Hkv)]) for b in range(B)])
    v_c = np.stack([np.stack([v[b, h, kept[b, h]] for h in range(Hkv)]) for b in range(B)])
    return k_c, v_c


def selection_quality(q, k_c, page_size: int, r: int, topk: int, scale: float) -> dict:
    """Hybrid selection against Exact-TopK (rebuttal, "Measurement of Exact-TopK": the top tokens
    by true importance for each head and decoding step). Per (b, query head g): Exact-TopK is the
    stable top-topk of the exact scores q_g . k_t; the hybrid tokens are those of its group's
    selected pages. recall = |hybrid & exact| / topk; mass = the share of softmax(scale * scores)
    on the hybrid tokens; mass_exact = the same on Exact-TopK. Means over (b, g)."""
    q, k_c = widen(q), widen(k_c)
    B, Hq, D = q.shape
    Hkv, Lc = k_c.shape[1], k_c.shape[2]
    G = Hq // Hkv
    recall, mass, mass_exact = [], [], []
    for b in range(B):
        for h in range(Hkv):
            kmin, kmax = page_summaries(k_c[b, h], page_size)
            qg = q[b, h * G:(h + 1) * G]
            chans, qbar = select_channels(qg, min(r, D))
            sc = approx_page_scores(qbar, chans, kmin, kmax)
            pages = select_pages(sc, min(topk // page_size, kmin.shape[1]))
            hyb = page_tokens(pages, page_size, Lc)
            for g in range(G):
                s = k_c[b, h] @ qg[g]
                exact = stable_topk(s, topk)
                p = np.exp(scale * (s - s.max()))
                p /= p.sum()
                recall.append(len(np.intersect1d(hyb, exact)) / len(exact))
                mass.append(p[hyb].sum())
                mass_exact.append(p[exact].sum())
    return dict(recall=float(np.mean(recall)), mass=float(np.mean(mass)),
                mass_exact=float(np.mean(mass_exact)))


def plan_budget(L: int, D: int, W: int, token_budget: int) -> dict:
    """Both stages' settings for a token budget (rebuttal, "Is Page Always Divided Into 4?": the
    ratio L / budget splits evenly between the two stages, and the second stage's share evenly
    between page size and channel reduction; "Lack of Direct Latency Comparison": the budget
    counts the approximation's reads, the rest is attended; "Potential Sensitivity to Kernel Size
    in SnapKV++": longer inputs take larger pooling kernels). Rounding: nearest integer for keep,
    page size and channels, approximation tokens rounded up, the attended tokens rounded down to
    whole pages."""
    import math
    if L <= 4096:
        pool = 7
    elif L <= 16384:
        pool = 15
    elif L <= 65536:
        pool = 31
    else:
        pool = 63
    if token_budget >= L:
        return dict(keep=L, page_size=1, r=D, topk=L, pool_kernel=pool, approx_tokens=0)
    per_stage = math.sqrt(L / token_budget)
    per_dim = math.sqrt(per_stage)
    keep = min(max(int(math.floor(L / per_stage + 0.5)), W), L)
    page_size = max(1, int(math.floor(per_dim + 0.5)))
    r = min(max(int(math.floor(D / per_dim + 0.5)), 1), D)
    approx = -(-(keep * r) // (page_size * 2 * D))
    pages_kept = -(-keep // page_size)
    topk = (token_budget - approx) // page_size * page_size if token_budget > approx else 0
    topk = min(max(topk, page_size), pages_kept * page_size)
    return dict(keep=keep, page_size=page_size, r=r, topk=topk, pool_kernel=pool,
                approx_tokens=approx)


def summaries(k_c, page_size: int):
    """page_summaries over a batch: k_c [B,Hkv,Lc,D] -> (kmin_t, kmax_t) [B,Hkv,D,P]."""
    k_c = widen(k_c)
    B, Hkv, Lc, D = k_c.shape
    P = -(-Lc // page_size)
    kmin = np.zeros((B, Hkv, D, P))
    kmax = np.zeros((B, Hkv, D, P))
    for b in range(B):
        for h in range(Hkv):
            kmin[b, h], kmax[b, h] = page_summaries(k_c[b, h], page_size)
    return kmin, kmax
