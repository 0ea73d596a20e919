"""Pins of the CPU oracle to facts outside itself (closed forms, brute force, invariants, library
routines and the pages' planted-needle claim). CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import rocketkv as O
from workloads import configs, generate


def _order_ok(scores, sel):
    """Brute force: sel (best first) is a valid stable top-k of scores."""
    sel = list(sel)
    assert len(set(sel)) == len(sel)
    chosen = set(sel)
    for i in sel:
        for j in range(len(scores)):
            if j in chosen:
                continue
            assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)
    for a, b in zip(sel, sel[1:]):
        assert scores[a] > scores[b] or (scores[a] == scores[b] and a < b)


# ----------------------------------------------------------------------------- selection

@pytest.mark.parametrize("seed", range(6))
def test_stable_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 24))
    scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
    if seed % 2:
        scores += rng.standard_normal(n) * 1e-3 * (rng.random(n) < 0.5)
    for k in range(0, n + 2):
        sel = O.stable_topk(scores, k)
        assert len(sel) == min(k, n)
        _order_ok(scores, sel)
        asc = O.topk_ascending(scores, k)
        assert list(asc) == sorted(sel)


def test_stable_topk_signed_zero_ties():
    s = np.array([0.0, -0.0, 0.0, -1.0, -0.0])
    assert list(O.stable_topk(s, 2)) == [0, 1]
    assert list(O.stable_topk(s, 4)) == [0, 1, 2, 4]


# ----------------------------------------------------------------------------- stage 1

def _rand_group(rng, G=2, W=5, L=23, D=8):
    return rng.standard_normal((G, W, D)), rng.standard_normal((L, D))


def test_window_rows_are_causal_distributions():
    rng = np.random.default_rng(1)
    q, k = _rand_group(rng)
    G, W, _ = q.shape
    L = k.shape[0]
    A = O.window_attention(q, k, 0.7)
    np.testing.assert_allclose(A.sum(-1), 1.0, rtol=0, atol=1e-13)
    for i in range(W):
        assert np.all(A[:, i, L - W + i + 1:] == 0.0)
        assert np.all(A[:, i, :L - W + i + 1] > 0.0)
    # the column sums over every key therefore total G*W
    assert O.group_column_sums(A).sum() == pytest.approx(G * W, abs=1e-12)


def test_window_uniform_keys_closed_form():
    # identical keys -> every row is uniform over the keys it sees: 1 / (L-W+i+1)
    rng = np.random.default_rng(2)
    G, W, L, D = 3, 4, 19, 6
    q = rng.standard_normal((G, W, D))
    k = np.tile(rng.standard_normal((1, D)), (L, 1))
    c = O.group_column_sums(O.window_attention(q, k, 0.5))
    expect_prefix = G * sum(1.0 / (L - W + i + 1) for i in range(W))
    np.testing.assert_allclose(c[:L - W], expect_prefix, rtol=1e-13)
    # window column L-W+t is seen by rows t..W-1
    for t in range(W):
        np.testing.assert_allclose(c[L - W + t], G * sum(1.0 / (L - W + i + 1) for i in range(t, W)),
                                   rtol=1e-13)


def test_window_softmax_hand_example():
    # one query [1, 0]; prefix keys [2, 0], [0, 0]; window key [1, 0]; scale 0.5
    # logits 1, 0, 0.5 -> softmax weights e^1, e^0, e^0.5 over their sum
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[2.0, 0.0], [0.0, 0.0], [1.0, 0.0]])
    A = O.window_attention(q, k, 0.5)[0, 0]
    z = math.e + 1.0 + math.sqrt(math.e)
    np.testing.assert_allclose(A, [math.e / z, 1.0 / z, math.sqrt(math.e) / z], rtol=1e-15)
    kept, colsum, pooled = O.snapkvpp_head(q, k, keep=2, kernel=1, scale=0.5)
    assert list(kept) == [0, 2]
    np.testing.assert_allclose(colsum, [math.e / z, 1.0 / z], rtol=1e-15)


def test_window_future_key_is_masked():
    rng = np.random.default_rng(3)
    q, k = _rand_group(rng)
    L, W = k.shape[0], q.shape[1]
    k2 = k.copy()
    k2[L - 1] = 50.0 * q[:, -1].mean(0)  # only the last window row may see it
    A1 = O.window_attention(q, k, 1.0)
    A2 = O.window_attention(q, k2, 1.0)
    assert np.array_equal(A1[:, :W - 1], A2[:, :W - 1])
    assert np.all(A2[:, W - 1, L - 1] > 0.99)


def test_window_dominant_prefix_key_takes_all_mass():
    rng = np.random.default_rng(4)
    G, W, L, D = 2, 6, 40, 16
    direction = rng.standard_normal(D)
    q = direction[None, None] + 0.01 * rng.standard_normal((G, W, D))
    k = 0.01 * rng.standard_normal((L, D))
    j0 = 11
    k[j0] = 40.0 * direction
    c = O.group_column_sums(O.window_attention(q, k, 1.0))
    assert c[j0] == pytest.approx(G * W, rel=1e-9)


def test_gqa_group_mapping_and_group_sum():
    # heads 0,1 look along e0, heads 2,3 along e1; KV head 0 must be scored by heads 0,1 only
    B, Hq, Hkv, W, L, D = 1, 4, 2, 4, 64, 8
    rng = np.random.default_rng(5)
    q = 0.01 * rng.standard_normal((B, Hq, W, D))
    q[0, :2, :, 0] += 3.0
    q[0, 2:, :, 1] += 3.0
    k = 0.01 * rng.standard_normal((B, Hkv, L, D))
    k[0, :, 10, 0] = 10.0   # matches the first group's direction
    k[0, :, 20, 1] = 10.0   # matches the second group's direction
    v = rng.standard_normal((B, Hkv, L, D))
    r = O.snapkvpp_evict(q, k, v, keep=W + 1, kernel=1, scale=1.0)
    assert list(r["kept"][0, 0, :1]) == [10]
    assert list(r["kept"][0, 1, :1]) == [20]
    # group sum = sum of single-head sums (linearity over the group's heads)
    per_head = sum(O.group_column_sums(O.window_attention(q[0, g:g + 1], k[0, 0], 1.0))
                   for g in range(2))
    np.testing.assert_allclose(r["colsum"][0, 0], per_head[:L - W], rtol=1e-12)


def test_pool_identity_impulse_constant():
    rng = np.random.default_rng(6)
    c = rng.random(30)
    assert np.array_equal(O.pool1d(c, 1), c)
    n, p = 30, 7
    h = p // 2
    for j0 in (0, 2, 15, 29):
        imp = np.zeros(n)
        imp[j0] = 1.0
        expect = np.array([1.0 / p if abs(j - j0) <= h else 0.0 for j in range(n)])
        np.testing.assert_allclose(O.pool1d(imp, p), expect, rtol=0, atol=1e-16)
        expect_max = np.array([1.0 if abs(j - j0) <= h else 0.0 for j in range(n)])
        assert np.array_equal(O.pool1d(imp, p, "max"), expect_max)
    ones = O.pool1d(np.ones(n), p)
    expect = np.array([(min(j + h, n - 1) - max(j - h, 0) + 1) / p for j in range(n)])
    np.testing.assert_allclose(ones, expect, rtol=1e-15)
    with pytest.raises(ValueError):
        O.pool1d(c, 4)


def test_snapkvpp_structure_and_selection_rule():
    w = configs.TINY_FP32
    d = generate.prompt_layer(w)
    scale = 1.0 / math.sqrt(w.D)
    r = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, scale)
    L, W, keep = w.L, w.W, w.keep
    for b in range(w.B):
        for h in range(w.Hkv):
            kept = r["kept"][b, h]
            assert len(kept) == keep and np.all(np.diff(kept) > 0)
            assert list(kept[-W:]) == list(range(L - W, L))
            chosen = kept[:-W]
            pooled = r["pooled"][b, h]
            rest = np.setdiff1d(np.arange(L - W), chosen)
            worst_in = min(pooled[chosen])
            best_out = max(pooled[rest])
            assert worst_in >= best_out
            if worst_in == best_out:  # ties resolved to the lower index
                assert max(chosen[pooled[chosen] == worst_in]) < min(rest[pooled[rest] == best_out])
            # planted needles survive (needle keys are never evicted at this budget)
            assert set(d["needle_pos"][b, h]) <= set(kept.tolist())
            # compaction gathers the kept rows
            assert np.array_equal(r["k_c"][b, h], O.widen(d["k"])[b, h, kept])
            assert np.array_equal(r["v_c"][b, h], O.widen(d["v"])[b, h, kept])


def test_snapkvpp_no_eviction_when_budget_covers_prompt():
    w = configs.TINY_FP32.replace(L=300, keep=300)
    d = generate.prompt_layer(w)
    r = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], 300, 7, 0.125)
    assert np.array_equal(r["kept"][0, 0], np.arange(300))
    r = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], 1000, 7, 0.125)
    assert np.array_equal(r["kept"][0, 1], np.arange(300))
    with pytest.raises(ValueError):
        O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.W - 1, 7, 0.125)


@pytest.mark.parametrize("w", [configs.SMALL[1], configs.SMALL[3]], ids=lambda w: w.name)
def test_snapkvpp_keeps_needles_small_bf16(w):
    d = generate.prompt_layer(w)
    r = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, 1 / math.sqrt(w.D))
    for b in range(w.B):
        for h in range(w.Hkv):
            assert set(d["needle_pos"][b, h]) <= set(r["kept"][b, h].tolist())


# ----------------------------------------------------------------------------- stage 2

def test_page_summaries_bounds_attained_partial_page():
    rng = np.random.default_rng(7)
    Lc, D, ps = 23, 5, 4
    k = rng.standard_normal((Lc, D))
    kmin, kmax = O.page_summaries(k, ps)
    assert kmin.shape == (D, 6)
    for t in range(Lc):
        p = t // ps
        assert np.all(kmin[:, p] <= k[t]) and np.all(k[t] <= kmax[:, p])
    for p in range(6):
        rows = k[p * ps:min(p * ps + ps, Lc)]
        for c in range(D):
            assert kmin[c, p] in rows[:, c] and kmax[c, p] in rows[:, c]
    k1min, k1max = O.page_summaries(k, 1)
    assert np.array_equal(k1min, k.T) and np.array_equal(k1max, k.T)


@pytest.mark.parametrize("ps", [1, 3, 4])
def test_kv_append_grows_pages_by_brute_force(ps):
    # appending one slot at a time from an empty cache: every written page's (min, max) bounds
    # each of its valid rows and is attained by one of them (brute force), pages are started at
    # page boundaries, unwritten slots and pages stay untouched, and the end state is the batch
    # summary of the grown cache
    rng = np.random.default_rng(30 + ps)
    cap, D, n = 14, 5, 11
    k_all = rng.standard_normal((n, D))
    v_all = rng.standard_normal((n, D))
    pcap = -(-cap // ps)
    k = np.full((cap, D), 7.0)
    v = np.full((cap, D), 7.0)
    kmin = np.full((D, pcap), 9.0)
    kmax = np.full((D, pcap), 9.0)
    for Lc in range(n):
        k, v, kmin, kmax = O.kv_append(k, v, kmin, kmax, Lc, k_all[Lc], v_all[Lc], ps)
        L1 = Lc + 1
        assert np.array_equal(k[:L1], k_all[:L1]) and np.array_equal(v[:L1], v_all[:L1])
        assert np.all(k[L1:] == 7.0) and np.all(v[L1:] == 7.0)
        np_ = -(-L1 // ps)
        for p in range(np_):
            rows = k_all[p * ps:min(p * ps + ps, L1)]
            assert np.all(kmin[:, p] <= rows.min(axis=0)) and np.all(rows.max(axis=0) <= kmax[:, p])
            for c in range(D):
                assert kmin[c, p] in rows[:, c] and kmax[c, p] in rows[:, c]
        assert np.all(kmin[:, np_:] == 9.0) and np.all(kmax[:, np_:] == 9.0)
        if Lc % ps == 0:  # a page boundary: the new page is the row itself
            assert np.array_equal(kmin[:, Lc // ps], k_all[Lc])
            assert np.array_equal(kmax[:, Lc // ps], k_all[Lc])
    bmin, bmax = O.page_summaries(k_all, ps)
    assert np.array_equal(kmin[:, :bmin.shape[1]], bmin)
    assert np.array_equal(kmax[:, :bmax.shape[1]], bmax)


def test_mt_view_identity_and_eviction_equivalence():
    # the multi-turn view with every row kept is the full cache, and with SnapKV++'s kept rows it
    # is exactly the cache that permanent eviction compacts (so the decode steps agree)
    rng = np.random.default_rng(41)
    B, Hq, Hkv, L, D, W, keep, ps = 1, 4, 2, 40, 8, 4, 16, 4
    q_win = rng.standard_normal((B, Hq, W, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    ident = np.broadcast_to(np.arange(L), (B, Hkv, L))
    kc, vc = O.mt_view(k, v, ident)
    assert np.array_equal(kc, k) and np.array_equal(vc, v)
    ev = O.snapkvpp_evict(q_win, k, v, keep, 3, 1 / math.sqrt(D))
    kc, vc = O.mt_view(k, v, ev["kept"])
    assert np.array_equal(kc, ev["k_c"]) and np.array_equal(vc, ev["v_c"])
    q = rng.standard_normal((B, Hq, D))
    kmin, kmax = O.summaries(kc, ps)
    a = O.hybrid_decode_step(q, kc, vc, kmin, kmax, ps, 4, 8, 0.3)
    kmin2, kmax2 = O.summaries(ev["k_c"], ps)
    b = O.hybrid_decode_step(q, ev["k_c"], ev["v_c"], kmin2, kmax2, ps, 4, 8, 0.3)
    assert np.array_equal(a["pages"], b["pages"]) and np.array_equal(a["out"], b["out"])


def test_bound_is_box_maximum_by_vertex_enumeration():
    rng = np.random.default_rng(8)
    D, P, r = 7, 9, 4
    a, b = rng.standard_normal((D, P)), rng.standard_normal((D, P))
    kmin, kmax = np.minimum(a, b), np.maximum(a, b)
    q = rng.standard_normal(D)
    q[2] = 0.0
    chans = np.array([0, 2, 3, 6])
    s = O.approx_page_scores(q, chans, kmin, kmax)
    for p in range(P):
        best = max(sum(q[c] * (kmax[c, p] if hi else kmin[c, p]) for c, hi in zip(chans, bits))
                   for bits in itertools.product((0, 1), repeat=r))
        assert s[p] == pytest.approx(best, rel=1e-14, abs=1e-14)


def test_bound_dominates_true_page_max_and_is_exact_for_single_token_pages():
    rng = np.random.default_rng(9)
    Lc, D, ps = 64, 16, 4
    k = rng.standard_normal((Lc, D)) * np.exp(rng.standard_normal(D))
    qg = rng.standard_normal((3, D))
    kmin, kmax = O.page_summaries(k, ps)
    chans_all, qbar = O.select_channels(qg, D)
    assert list(chans_all) == list(range(D))
    s_full = O.approx_page_scores(qbar, chans_all, kmin, kmax)
    exact = k @ qbar
    for p in range(Lc // ps):
        assert s_full[p] >= exact[p * ps:(p + 1) * ps].max() - 1e-12
    chans, _ = O.select_channels(qg, 5)
    s_r = O.approx_page_scores(qbar, chans, kmin, kmax)
    part = k[:, chans] @ qbar[chans]
    for p in range(Lc // ps):
        assert s_r[p] >= part[p * ps:(p + 1) * ps].max() - 1e-12
    k1min, k1max = O.page_summaries(k, 1)
    np.testing.assert_allclose(O.approx_page_scores(qbar, chans_all, k1min, k1max), exact,
                               rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_select_channels_brute_force(seed):
    rng = np.random.default_rng(seed)
    G, D, r = 4, 12, 5
    q = np.round(rng.standard_normal((G, D)), 1)  # coarse values -> ties in sum |q|
    chans, qbar = O.select_channels(q, r)
    a = np.abs(q).sum(0)
    _order_ok(a, sorted(chans, key=lambda c: (-a[c], c)))
    assert np.all(np.diff(chans) > 0)
    np.testing.assert_allclose(qbar, q.sum(0), rtol=0, atol=0)


def test_hybrid_reduces_to_exact_topk():
    # G = 1, one-token pages, all channels: the approximate score is the exact q.k
    rng = np.random.default_rng(10)
    B, Hq, Hkv, Lc, D, k = 1, 2, 2, 50, 8, 9
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Lc, D))
    vc = rng.standard_normal((B, Hkv, Lc, D))
    kmin, kmax = O.summaries(kc, 1)
    res = O.hybrid_decode_step(q, kc, vc, kmin, kmax, page_size=1, r=D, topk=k, scale=0.3)
    for h in range(Hkv):
        exact = [float(np.dot(q[0, h], kc[0, h, t])) for t in range(Lc)]
        ranked = sorted(range(Lc), key=lambda t: (-exact[t], t))[:k]
        assert list(res["pages"][0, h]) == sorted(ranked)


def test_decode_channels_come_from_each_group():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, Lc, D, r, ps = 2, 6, 3, 16, 10, 3, 4
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Lc, D))
    kmin, kmax = O.summaries(kc, ps)
    res = O.hybrid_decode_step(q, kc, kc, kmin, kmax, ps, r, topk=8, scale=0.3)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            a = [sum(abs(q[b, g, c]) for g in range(h * G, h * G + G)) for c in range(D)]
            top = sorted(sorted(range(D), key=lambda c: (-a[c], c))[:r])
            assert list(res["chans"][b, h]) == top
            qbar = q[b, h * G:h * G + G].sum(0)
            s = [sum(max(qbar[c] * kmin[b, h, c, p], qbar[c] * kmax[b, h, c, p]) for c in top)
                 for p in range(Lc // ps)]
            np.testing.assert_allclose(res["scores"][b, h], s, rtol=1e-13)


def _sdpa_gqa(q, k, v, scale):
    """Dense attention via torch's scaled_dot_product_attention (float64, CPU)."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    kk = torch.from_numpy(np.repeat(k, G, axis=1))
    vv = torch.from_numpy(np.repeat(v, G, axis=1))
    qq = torch.from_numpy(q)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("ps,Lc", [(4, 64), (4, 62), (1, 33), (8, 100)])
def test_full_budget_is_dense_attention(ps, Lc):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D = 2, 6, 2, 16
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Lc, D)) * 2
    vc = rng.standard_normal((B, Hkv, Lc, D))
    kmin, kmax = O.summaries(kc, ps)
    topk = ps * (-(-Lc // ps)) + 4 * ps
    res = O.hybrid_decode_step(q, kc, vc, kmin, kmax, ps, r=5, topk=topk, scale=0.25)
    np.testing.assert_allclose(res["out"], _sdpa_gqa(q, kc, vc, 0.25), rtol=1e-12, atol=1e-12)


def test_sparse_attention_convex_and_equal_keys():
    rng = np.random.default_rng(12)
    G, Lc, D = 3, 40, 8
    q = rng.standard_normal((G, D))
    k = rng.standard_normal((Lc, D))
    v = rng.standard_normal((Lc, D))
    toks = np.array([1, 2, 3, 17, 18, 19, 20, 39])
    o = O.sparse_attention(q, k, v, toks, 0.9)
    assert np.all(o <= v[toks].max(0) + 1e-12) and np.all(o >= v[toks].min(0) - 1e-12)
    keq = np.tile(k[:1], (Lc, 1))
    np.testing.assert_allclose(O.sparse_attention(q, keq, v, toks, 0.9),
                               np.tile(v[toks].mean(0), (G, 1)), rtol=1e-13)


def test_needle_query_selects_every_needle_page():
    w = configs.TINY_FP32
    d = generate.prompt_layer(w)
    scale = 1.0 / math.sqrt(w.D)
    ev = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, scale)
    kmin, kmax = O.summaries(ev["k_c"], w.page_size)
    q = generate.needle_queries(w, d["needle_dir"])
    res = O.hybrid_decode_step(q, ev["k_c"], ev["v_c"], kmin, kmax, w.page_size, w.r,
                               w.topk[0], scale)
    for b in range(w.B):
        for h in range(w.Hkv):
            slots = np.searchsorted(ev["kept"][b, h], d["needle_pos"][b, h])
            assert np.array_equal(ev["kept"][b, h][slots], d["needle_pos"][b, h])
            assert set((slots // w.page_size).tolist()) <= set(res["pages"][b, h].tolist())


def test_widen_bf16_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, -0.0, 65504.0], dtype=np.float32)
    bits = generate.bf16_bits(x)
    back = O.widen(bits)
    # bfloat16 keeps 8 significant bits: these values are exact or rounded to nearest even
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    assert abs(back[3] - 1e-3) <= 1e-3 * 2 ** -8
    assert np.signbit(back[4])
    assert bits[5] == 0x4780  # 65504 rounds to 65536 in bfloat16


# ----------------------------------------------------------------------------- budget planner

def test_plan_budget_rebuttal_worked_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "budget_rebuttal_example.json")))
    e = g["expect"]
    L, D, W, budget = g["L"], g["D"], g["W"], g["token_budget"]
    assert L // budget == e["compression_ratio"]
    assert math.isclose(math.sqrt(L / budget), e["per_stage_ratio"])
    assert math.isclose(math.sqrt(e["per_stage_ratio"]), e["per_dimension_ratio"])
    plan = O.plan_budget(L, D, W, budget)
    for key in ("keep", "page_size", "r", "approx_tokens", "topk"):
        assert plan[key] == e[key], key
    assert plan["approx_tokens"] + plan["topk"] == budget  # half approximates, half attends


@pytest.mark.parametrize("L,budget", [(2048, 128), (32768, 256), (131072, 1024), (262144, 2048)])
def test_plan_budget_spends_about_the_budget_and_balances_the_stages(L, budget):
    # the approximation and the attended tokens add up to the budget (up to rounding to whole
    # pages), and the first stage's ratio equals the second's (up to rounding)
    D, W = 128, 32
    p = O.plan_budget(L, D, W, budget)
    assert p["topk"] % p["page_size"] == 0
    assert abs(p["approx_tokens"] + p["topk"] - budget) <= 2 * p["page_size"] + 1
    s1 = L / p["keep"]
    s2 = (p["page_size"] * D / p["r"])
    assert 0.6 < s1 / s2 < 1.7
    assert O.plan_budget(L, D, W, L)["keep"] == L and O.plan_budget(L, D, W, L)["topk"] == L


# ----------------------------------------------------------------------------- selection quality

def test_selection_quality_exact_topk_maximises_mass_by_brute_force():
    # Exact-TopK's softmax mass is the largest of every topk-subset (enumerated), and the hybrid
    # with single-token pages, every channel and one head per group is Exact-TopK itself
    rng = np.random.default_rng(51)
    B, Hq, Hkv, Lc, D, topk = 1, 2, 2, 8, 4, 3
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, Lc, D))
    res = O.selection_quality(q, k, 1, D, topk, 0.7)
    assert res["recall"] == 1.0 and math.isclose(res["mass"], res["mass_exact"])
    for h in range(Hkv):
        s = k[0, h] @ q[0, h]
        p = np.exp(0.7 * (s - s.max()))
        p /= p.sum()
        best = max(p[list(c)].sum() for c in itertools.combinations(range(Lc), topk))
        assert math.isclose(p[O.stable_topk(s, topk)].sum(), best)
    coarse = O.selection_quality(q, k, 4, 1, topk + 1, 0.7)
    assert 0.0 <= coarse["recall"] <= 1.0 and coarse["mass"] <= 1.0 + 1e-12
    assert O.selection_quality(q, k, 2, D, Lc, 0.7)["mass"] > 1 - 1e-12  # every token selected


def test_selection_quality_hand_computed_mass_and_recall():
    # Worked by hand (rebuttal, "Measurement of Exact-TopK": the best tokens of each head and
    # step; "Explanation of Calculating Approximate Attention Scores": channels by the group sum
    # of |q|, bound from the group sum of q). D = 2, one KV head, one-token pages, one channel,
    # top-1, scale = ln 2 so that every softmax weight is a power of two.
    #   keys k0 = (1, 0), k1 = (0, 3), k2 = (0, 0), k3 = (-1, 0)
    # Case G = 1, q = (2, 1): |q| picks channel 0, qbar_0 = 2 > 0 reads the page maxima (the keys
    # themselves), so the bound is (2, 0, 0, -2) and the hybrid keeps k0. Exact scores are
    # (2, 3, 0, -2): Exact-TopK keeps k1, recall 0. Weights 2^s = (4, 8, 1, 1/4), total 53/4:
    # mass = 4 / (53/4) = 16/53, mass_exact = 32/53.
    k = np.array([[[[1.0, 0.0], [0.0, 3.0], [0.0, 0.0], [-1.0, 0.0]]]])
    q1 = np.array([[[2.0, 1.0]]])
    res = O.selection_quality(q1, k, 1, 1, 1, math.log(2.0))
    assert res["recall"] == 0.0
    assert math.isclose(res["mass"], 16 / 53, rel_tol=1e-12)
    assert math.isclose(res["mass_exact"], 32 / 53, rel_tol=1e-12)
    # Case G = 2, heads q0 = (2, 1), q1 = (1, -3): sum |q| = (3, 4) picks channel 1 with
    # qbar_1 = -2 < 0, which reads the page minima: bound (0, -6, 0, 0); the tie at 0 goes to the
    # lowest page, so the hybrid keeps k0 for both heads.
    #   head 0: as above, recall 0, mass 16/53, mass_exact 32/53.
    #   head 1: exact scores (1, -9, 0, -1), Exact-TopK keeps k0 (recall 1); weights
    #   (2, 2^-9, 1, 1/2), total 1793/512, so mass = mass_exact = 1024/1793.
    # Means over the two heads: recall 1/2, mass (16/53 + 1024/1793)/2,
    # mass_exact (32/53 + 1024/1793)/2.
    q2 = np.array([[[2.0, 1.0], [1.0, -3.0]]])
    res = O.selection_quality(q2, k, 1, 1, 1, math.log(2.0))
    assert res["recall"] == 0.5
    assert math.isclose(res["mass"], (16 / 53 + 1024 / 1793) / 2, rel_tol=1e-12)
    assert math.isclose(res["mass_exact"], (32 / 53 + 1024 / 1793) / 2, rel_tol=1e-12)
    # a dropped or doubled scale moves the mass off the hand-computed value
    for wrong in (1.0, 2 * math.log(2.0)):
        assert not math.isclose(O.selection_quality(q1, k, 1, 1, 1, wrong)["mass"], 16 / 53,
                                rel_tol=1e-3)


@pytest.mark.parametrize("L,kernel", [(2048, 7), (32768, 31), (131072, 63), (262144, 63)])
def test_plan_budget_pooling_kernel_at_the_configured_lengths(L, kernel):
    # The pages give only the trend of the pooling kernel with input length ("Potential
    # Sensitivity to Kernel Size in SnapKV++": longer inputs, larger kernels). The four evaluated
    # workloads pair these context lengths with these kernels (2K: 7, 32K: 31, 128K and 256K: 63),
    # and the planner's table must reproduce them.
    assert O.plan_budget(L, 128, 32, 256)["pool_kernel"] == kernel


def test_plan_budget_pooling_kernel_grows_with_length():
    lengths = [64, 2048, 4096, 4097, 16384, 16385, 65536, 65537, 131072, 1 << 20]
    ks = [O.plan_budget(L, 128, 32, 64)["pool_kernel"] for L in lengths]
    assert ks == sorted(ks) and all(k % 2 == 1 for k in ks)
    assert ks[0] == 7 and ks[-1] == 63
