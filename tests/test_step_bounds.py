"""Host emulation of the address arithmetic of the fused decode step (k_decode_step), of the
page-summary kernel (k_page_minmax) and of the eviction's pooling (k_pool_count), at the shapes the
benchmark runs: the 128K 8B-shaped layer
over the compressed cache and over the multi-turn view of the full 131072-token cache (row map,
cache pitch L), the batch-16 layer (128 heads) and the 80-layer 70B-shaped stack (640 heads).

The plan and workspace layout below restate the library's host plan (rkv_step.hpp: step::plan,
step::layout); the layout's size is checked against rkv_hybrid_decode_workspace_bytes, which pins
the restatement to the library. Every global index the kernels form is then evaluated for every
role and thread, on the extents of the buffers the C ABI documents, for several CU counts.
CPU only: nothing here launches a kernel.
"""
import numpy as np
import pytest

import sparse_kv_cache_snapkv_amd as rkv
from workloads import configs

THREADS = 512
MAX_ATT, MAX_SCORE, TARGET = 16, 64, 256
SOLO_TOKENS, TOKENS_PER_BLOCK = 256, 64
SYNC_HEADER, HEAD_WORDS = 16, 4
MAX_PAGES_PER_WINDOW = 1024
MIN_SCORE_PAGES = 128
XCDS = 8
PREFETCH_TOKENS, PREFETCH_SHARE, PREFETCH_PAGES = 512, 256, 8


def prefetch_pages(BH, P, ps, n_pages, pl):
    # pages of its share that a block which only scores touches ahead (rkv_step.hip)
    ok = (pl["nb"] > 1 and BH % XCDS == 0 and n_pages < P and n_pages * ps <= PREFETCH_TOKENS
          and pl["ppb1"] <= PREFETCH_SHARE)
    return min(PREFETCH_PAGES, 2 * -(-n_pages // pl["ns"])) if ok else 0


def plan(BH, P, ps, n_pages, ncu, vmax):
    nb0 = max(min(ncu // BH, MAX_SCORE), 1)
    ntok = n_pages * ps
    na = 1 if ntok <= SOLO_TOKENS else max(min(MAX_ATT, nb0, -(-ntok // TOKENS_PER_BLOCK)), 1)
    pps = -(-n_pages // na)
    na = -(-n_pages // pps)
    ppb1 = max(-(-P // nb0), MIN_SCORE_PAGES)
    ppb1 = -(-ppb1 // vmax) * vmax
    ns = -(-P // ppb1)
    return dict(ns=ns, na=na, nb=max(ns, na), ppb1=ppb1, pps=pps)


def align256(x):
    return (x + 255) & ~255


def attend_splits_bound(BH, Pcap):
    return min(256, max(-(-2 * TARGET // BH), -(-Pcap // MAX_PAGES_PER_WINDOW)))


def layout(B, Hq, Hkv, D, Pcap):
    BH, G = B * Hkv, Hq // Hkv
    budget = 0 if BH >= TARGET else TARGET // BH
    lo = dict(off_sync=0, off_xscores=align256((SYNC_HEADER + HEAD_WORDS * BH) * 4))
    if BH > TARGET:  # three launches: scores, pages and attention partials in the workspace
        lo.update(pipe=True, cap_a=1, off_xpart=lo["off_xscores"], off_pscores=lo["off_xscores"])
        lo["off_ppages"] = align256(lo["off_pscores"] + BH * Pcap * 4)
        lo["off_ppart"] = align256(lo["off_ppages"] + BH * Pcap * 4)
        lo["total"] = align256(lo["off_ppart"]
                               + BH * attend_splits_bound(BH, Pcap) * G * (D + 2) * 4)
        return lo
    if budget < 2:
        lo.update(cap_a=1, off_xpart=lo["off_xscores"], total=lo["off_xscores"])
        return lo
    lo["cap_a"] = min(budget, MAX_ATT)
    lo["off_xpart"] = align256(lo["off_xscores"] + BH * Pcap * 8)
    lo["total"] = align256(lo["off_xpart"] + BH * lo["cap_a"] * (G * D + 2 * G) * 8)
    return lo


SHAPES = [
    # name, B (layers folded), Hq, Hkv, D, Lc, kv_pitch (L with a row map), ps, r, budgets, dtype
    ("128K", 1, 32, 8, 128, 16384, 16384, 4, 32, (128, 512, 2048), "bf16"),
    ("128K-MT", 1, 32, 8, 128, 16384, 131072, 4, 32, (128, 512, 2048), "bf16"),
    ("32K-b16", 16, 32, 8, 128, 4096, 4096, 4, 32, (256,), "bf16"),
    ("70B-80L", 80, 64, 8, 128, 32768, 32768, 4, 32, (1024,), "bf16"),
    ("tiny", 1, 4, 2, 64, 512, 512, 4, 16, (128,), "fp32"),
    ("grown", 1, 32, 8, 128, 16384 + 100, 16384 + 256, 4, 32, (128, 2048), "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_layout_matches_the_library(shape):
    name, B, Hq, Hkv, D, Lc, pitch, ps, r, budgets, dtype = shape
    code = 1 if dtype == "bf16" else 0
    cap = pitch if name == "grown" else Lc
    for tk in budgets:
        n_pages = min(tk // ps, -(-Lc // ps))
        nbytes = rkv.hybrid_decode_workspace_bytes(B, Hq, Hkv, cap, D, ps, n_pages, code)
        assert nbytes == layout(B, Hq, Hkv, D, -(-cap // ps))["total"]


def attend_plan(BH, ps, n_pages, D, e):
    """The standalone attention's split plan (rkv_attend.hip: plan_attend)."""
    V = 16 // e
    chunk = 4 * 4 * (64 // (D // V))  # waves x slots x tokens per load
    ntok = n_pages * ps
    ns = -(-2 * TARGET // BH)
    ns = 1 if ntok <= SOLO_TOKENS else min(ns, -(-ntok // chunk))
    ns = max(ns, -(-n_pages // MAX_PAGES_PER_WINDOW))
    ns = max(min(ns, 256), 1)
    pps = -(-n_pages // ns)
    return -(-n_pages // pps), pps


def approx_span(BH, P, pitch, V):
    """Pages per block of the approximate-score launch (rkv_approx.hip: launch_g)."""
    vec = pitch % V == 0
    pas = 16 * (V if vec else 1)
    span = max(1, min(8, BH * (-(-P // pas)) // 4096))
    return pas * span, vec


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_pipelined_step_indices_stay_in_their_buffers(shape):
    name, B, Hq, Hkv, D, Lc, pitch, ps, r, budgets, dtype = shape
    e = 2 if dtype == "bf16" else 4
    V = 16 // e
    BH, G = B * Hkv, Hq // Hkv
    if BH <= TARGET:
        pytest.skip("one launch")
    P = -(-Lc // ps)
    cap = pitch if name == "grown" else Lc
    Pcap = -(-cap // ps)
    lo = layout(B, Hq, Hkv, D, Pcap)
    # page scores: grid (ceil(P/per_block), BH); block bx reads pages [p0, min(P, p0+per_block))
    # of summary rows Pcap apart, in whole vectors when Pcap is a multiple of V
    per_block, vec = approx_span(BH, P, Pcap, V)
    for bx in (0, -(-P // per_block) - 1):
        p0, p1 = bx * per_block, min(P, bx * per_block + per_block)
        last = p0 + -(-(p1 - p0) // V) * V - 1 if vec else p1 - 1
        assert last < Pcap
        assert (BH - 1) * D * Pcap + (D - 1) * Pcap + last < BH * D * Pcap
        assert (BH - 1) * P + p1 - 1 < BH * Pcap  # scores, rows of P inside the [BH, Pcap] area
    for tk in budgets:
        n_pages = min(tk // ps, P)
        assert (BH - 1) * n_pages + n_pages - 1 < BH * Pcap  # pages, rows of n_pages
        ns, pps = attend_plan(BH, ps, n_pages, D, e)
        part = 0 if ns == 1 else BH * ns * G * (D + 2) * 4
        assert lo["off_ppart"] + part <= lo["total"]
        assert rkv.sparse_attend_workspace_bytes(B, Hq, Hkv, D, ps, n_pages, 1 if e == 2 else 0) \
            == part
        # the last split's pages and the token rows they cover
        assert (ns - 1) * pps < n_pages and ns * pps >= n_pages
        assert (BH - 1) * pitch * D + (pitch - 1) * D + D - 1 < BH * pitch * D


@pytest.mark.parametrize("ncu", [256, 304, 120, 8])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fused_step_indices_stay_in_their_buffers(shape, ncu):
    name, B, Hq, Hkv, D, Lc, pitch, ps, r, budgets, dtype = shape
    if B * Hkv > TARGET:
        pytest.skip("three launches (see the pipelined test)")
    ncu = min(ncu, TARGET)  # the library caps the CU count at 256
    e = 2 if dtype == "bf16" else 4
    V = 16 // e  # elements per 16-byte vector
    BH, G = B * Hkv, Hq // Hkv
    P = -(-Lc // ps)
    cap = pitch if name == "grown" else Lc
    Pcap = -(-cap // ps)
    s_pitch = Pcap
    rows_mapped = name.endswith("MT")
    kv_rows = pitch  # token rows per head of k_c / v_c (the full cache with a row map)
    lo = layout(B, Hq, Hkv, D, Pcap)
    tid = np.arange(THREADS)
    for tk in budgets:
        n_pages = min(tk // ps, P)
        pl = plan(BH, P, ps, n_pages, ncu, V)
        ns, na, nb, ppb1, pps = pl["ns"], pl["na"], pl["nb"], pl["ppb1"], pl["pps"]
        assert nb * BH <= max(ncu, BH), "a waiting plan fits one block per CU"
        assert ns <= nb and na <= nb
        if nb > 1:
            assert ns <= MAX_SCORE and na <= lo["cap_a"]
        # control words: kSyncHeader + kHeadWords * bh + 2 < words before the score area
        assert (SYNC_HEADER + HEAD_WORDS * (BH - 1) + 2) * 4 < max(lo["off_xscores"], 4 * (SYNC_HEADER + HEAD_WORDS * BH))
        E = 8 if P <= 8 * THREADS else 16
        assert P <= E * THREADS
        for bh in (0, BH - 1):
            for y in range(nb):
                # scorer: summary rows of the chosen channels (c < D), 16-byte vectors of pages
                if y < ns:
                    pb_lo, pb_hi = y * ppb1, min(P, y * ppb1 + ppb1)
                    assert 0 <= pb_lo < pb_hi <= P
                    vec = Pcap % V == 0
                    last = (pb_lo + (-(-(pb_hi - pb_lo) // V) - 1) * V + V - 1) if vec else pb_hi - 1
                    assert last < s_pitch
                    top = (bh * D * s_pitch) + (D - 1) * s_pitch + last
                    assert top < BH * D * s_pitch
                    if nb > 1:
                        assert bh * P + pb_hi - 1 < BH * Pcap  # tagged scores
                        assert (bh * P + pb_hi - 1) * 8 + lo["off_xscores"] < lo["off_xpart"]
                pf = prefetch_pages(BH, P, ps, n_pages, pl)
                if pf > 0 and na <= y < ns:
                    # touch ahead: the share's scores in LDS (E * THREADS floats, padded to a
                    # multiple of four), the ranks'
                    # page list in the merge area (G * D + MAX_ATT words), then the 16-byte
                    # pieces of the K/V rows of pages p in [pb_lo, pb_lo + nsh), slots t < Lc
                    nsh = min(P, y * ppb1 + ppb1) - y * ppb1
                    assert nsh <= PREFETCH_SHARE and nsh + 3 <= E * THREADS  # with its -inf padding
                    assert min(nsh, pf) <= G * D + MAX_ATT
                    chunks = D // V
                    i = np.arange(ps * chunks)
                    t = ((y * ppb1 + nsh - 1) * ps + i // chunks)
                    t = t[t < Lc] if (t < Lc).any() else np.array([0])
                    row = np.full_like(t, kv_rows - 1) if rows_mapped else t
                    assert ((bh * kv_rows + row) * D + (i[: len(row)] % chunks) * V + V - 1).max() < BH * kv_rows * D
                if y >= na:
                    continue
                # attender: every score word; a stale one marks share (page / ppb1) < ns
                j = np.arange(E)[:, None]
                idx = np.minimum(j * THREADS + tid[None, :], P - 1)
                assert idx.max() < P and bh * P + idx.max() < BH * Pcap
                assert (idx // ppb1).max() < ns <= 64
                # its slice of the page list and the token rows of those pages
                p_lo, p_hi = y * pps, min(y * pps + pps, n_pages)
                assert 0 <= p_lo and p_hi <= n_pages
                # a listed page p < P covers slots p*ps + u < Lc; with a row map the slot indexes
                # rows[bh*Lc + t] (t < Lc), whose value is clamped into [0, kv_pitch)
                t_max = Lc - 1
                assert bh * Lc + t_max < BH * Lc
                row_max = (kv_rows - 1) if rows_mapped else t_max
                assert (bh * kv_rows + row_max) * D + (D - V) + V - 1 < BH * kv_rows * D
                if na > 1:
                    # its partial, and the words of its merge range: o of (slice, element) at
                    # i < na*ne (three per thread), (max, sum) of (slice, head) at t < 2*na*G
                    stride = G * D + 2 * G
                    assert ((bh * lo["cap_a"] + y) * stride + stride - 1) * 8 + lo["off_xpart"] < lo["total"]
                    cpb = -(-(G * D) // na)
                    e0, ne = y * cpb, min(cpb, G * D - y * cpb)
                    no = na * ne if ne > 0 else 0
                    NO = -(-(G * D + MAX_ATT) // THREADS)
                    assert no <= NO * THREADS and no <= G * D + MAX_ATT
                    for k in range(NO):
                        i = np.minimum(tid + k * THREADS, max(no - 1, 0))
                        sl = i // ne if ne > 0 else 0 * i
                        e = i - sl * ne if ne > 0 else 0 * i
                        word = (bh * lo["cap_a"] + sl) * stride + np.minimum(e0 + e, G * D - 1)
                        assert (sl < na).all() and word.max() * 8 + lo["off_xpart"] < lo["total"]
                    t = np.minimum(tid, 2 * na * G - 1)
                    which, rem = t // (na * G), t % (na * G)
                    word = (bh * lo["cap_a"] + rem // G) * stride + G * D + which * G + rem % G
                    assert word.max() * 8 + lo["off_xpart"] < lo["total"]
                # outputs
                assert bh * G * D + G * D - 1 < BH * G * D
                assert bh * n_pages + n_pages - 1 < BH * n_pages
                assert bh * r + r - 1 < BH * r


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_page_minmax_indices_stay_in_their_buffers(shape):
    # grid (ceil(P/32), BH) of 256 threads; each thread folds kItems (page, chunk) items over
    # the page's valid slots, reading row r(t) of the cache, then writes channel rows of s_pitch
    name, B, Hq, Hkv, D, Lc, pitch, ps, r, budgets, dtype = shape
    e = 2 if dtype == "bf16" else 4
    V = 16 // e
    CH = D // V
    BH = B * Hkv
    P = -(-Lc // ps)
    cap = pitch if name == "grown" else Lc
    s_pitch = -(-cap // ps)
    kv_rows = pitch
    pages_per_block = 32
    items = pages_per_block * CH // 256
    tid = np.arange(256)
    for bx in (0, -(-P // pages_per_block) - 1):
        p0 = bx * pages_per_block
        for i in range(items):
            idx = i * 256 + tid
            p = p0 + idx // CH
            t0 = p * ps
            nt = np.where(p < P, np.minimum(ps, Lc - t0), 0)
            assert (nt >= 0).all()
            valid = nt > 0
            t_last = t0 + nt - 1
            assert (t_last[valid] < Lc).all()
            ch = idx % CH
            row = np.minimum(t_last, kv_rows - 1)
            assert ((BH - 1) * kv_rows * D + row[valid] * D + ch[valid] * V + V - 1
                    < BH * kv_rows * D).all()
        np_ = min(pages_per_block, P - p0)
        assert (BH - 1) * D * s_pitch + p0 + (D - 1) * s_pitch + np_ - 1 < BH * D * s_pitch


@pytest.mark.parametrize("kernel", [1, 3, 15, 31, 63, 127])
@pytest.mark.parametrize("n", [8193, 9001, 131040, 262080])
def test_pool_count_indices_stay_in_their_buffers(kernel, n):
    # k_pool_count (rkv_evict.hip): blocks of SPAN positions, THREADS_P threads of PER consecutive
    # outputs; the LDS tile holds SPAN + 128 floats, staged from position j0 - h for SPAN + 2h
    # entries. The sliding window reads tile[jb + m + kernel] after output m; only the reads that
    # feed an output must be staged, the last one only has to stay inside the tile.
    THREADS_P, PER = 1024, 4
    SPAN = THREADS_P * PER
    TILE = SPAN + 128
    h = kernel // 2
    staged = SPAN + 2 * h
    assert staged <= TILE
    jb = PER * np.arange(THREADS_P)
    first = jb[:, None] + np.arange(kernel)[None, :]  # the first window
    assert first.max() < staged
    for m in range(PER):
        out_in, out_out = jb + m + kernel, jb + m  # the slide after output m
        assert out_in.max() < TILE and out_out.max() < staged
        if m < PER - 1:  # feeds output m + 1
            assert out_in.max() < staged
    # global reads: positions j0 - h + i clamped into [0, n); writes: positions below n only
    nblk = -(-n // SPAN)
    for bx in (0, nblk - 1):
        j0 = bx * SPAN
        j = j0 - h + np.arange(staged)
        assert (np.clip(j, 0, n - 1) < n).all()
        nv = np.minimum(PER, n - (j0 + jb))
        assert ((j0 + jb + np.maximum(nv, 0) - 1)[nv > 0] < n).all()


def test_library_plans_of_the_benchmarked_workloads():
    # the plans the benchmark runs on a 256-CU device, written out
    assert plan(8, 4096, 4, 32, 256, 8) == dict(ns=32, na=1, nb=32, ppb1=128, pps=32)
    assert plan(8, 4096, 4, 128, 256, 8) == dict(ns=32, na=8, nb=32, ppb1=128, pps=16)
    assert plan(8, 4096, 4, 512, 256, 8) == dict(ns=32, na=16, nb=32, ppb1=128, pps=32)
    assert plan(128, 1024, 4, 64, 256, 8) == dict(ns=2, na=1, nb=2, ppb1=512, pps=64)
    assert plan(640, 8192, 4, 256, 256, 8) == dict(ns=1, na=1, nb=1, ppb1=8192, pps=256)
    # (the 80-layer stack's 640 heads run as three launches; these are their split plans)
    assert approx_span(640, 8192, 8192, 8) == (1024, True)
    assert attend_plan(640, 4, 256, 128, 2) == (1, 256)
    # the 2K fp32 workload's two heads of 128 pages: one block per head, nothing exchanged
    assert plan(2, 128, 4, 32, 256, 4) == dict(ns=1, na=1, nb=1, ppb1=128, pps=32)
    assert plan(8, 1024, 4, 32, 256, 8) == dict(ns=8, na=1, nb=8, ppb1=128, pps=32)
    assert configs.LLAMA8B_128K.P == 4096 and configs.LLAMA70B_256K_80L.P == 8192
