"""GPU parity of each C-ABI call against the CPU oracle on seeded inputs (small and ragged
shapes, edge cases). Marked gpu: needs an MI355X and the built librkv.so."""
import math

import numpy as np
import pytest
import torch

from _parity import TOL_OUT, assert_rows_close, selection_matches
from oracle import rocketkv as O
from workloads import configs, generate as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rkv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_kv_cache_snapkv_amd as rkv
    rkv._lib.load()
    return rkv


def T(x):
    return gen.storage_to_torch(x, "cuda")


def H(t):
    return gen.torch_to_storage(t)


def _wid(w):
    return w.name


# ----------------------------------------------------------------------------- top-k

TOPK_CASES = [(1, 1), (7, 0), (7, 3), (7, 7), (7, 9), (100, 10), (4096, 32), (4097, 128),
              (8192, 512), (8193, 1000), (16384, 16), (16385, 4000), (20000, 1234),
              (131040, 16352)]


@pytest.mark.parametrize("n,k", TOPK_CASES)
def test_topk_select_equals_stable_sort(rkv, n, k):
    rng = np.random.default_rng(n * 31 + k)
    s = rng.standard_normal((4, n)).astype(np.float32)
    s[0, ::3] = 0.5                                  # a large block of exact ties
    s[1, : n // 2] = 0.0
    s[1, n // 2::2] = -0.0                           # signed zeros tie
    s[2] = np.round(s[2], 1)                         # many small tie groups
    s[3] = np.abs(s[3]) * 1e-3 + 1.0                 # positives sharing the top bits
    gpu = rkv.rkv_topk_select(torch.from_numpy(s).cuda(), k).cpu().numpy()
    assert gpu.shape == (4, min(k, n))
    for r in range(4):
        assert np.array_equal(gpu[r], O.topk_ascending(s[r].astype(np.float64), k)), r


def test_topk_select_all_equal_and_rows_layout(rkv):
    s = np.full((3, 5000), 2.0, dtype=np.float32)
    gpu = rkv.rkv_topk_select(torch.from_numpy(s).cuda(), 777).cpu().numpy()
    assert np.array_equal(gpu, np.tile(np.arange(777), (3, 1)))
    # rows spread over several blocks: all ties, and every element but one
    s = np.full((2, 20000), -3.0, dtype=np.float32)
    gpu = rkv.rkv_topk_select(torch.from_numpy(s).cuda(), 7777).cpu().numpy()
    assert np.array_equal(gpu, np.tile(np.arange(7777), (2, 1)))
    s = np.random.default_rng(9).standard_normal((2, 12289)).astype(np.float32)
    gpu = rkv.rkv_topk_select(torch.from_numpy(s).cuda(), 12288).cpu().numpy()
    for r in range(2):
        assert np.array_equal(gpu[r], O.topk_ascending(s[r].astype(np.float64), 12288))
    s3 = np.random.default_rng(5).standard_normal((2, 3, 300)).astype(np.float32)
    g3 = rkv.rkv_topk_select(torch.from_numpy(s3).cuda(), 20).cpu().numpy()
    for b in range(2):
        for h in range(3):
            assert np.array_equal(g3[b, h], O.topk_ascending(s3[b, h], 20))


# ----------------------------------------------------------------------------- summaries

SUMMARY_CASES = [("fp32", 64, 512, 4), ("bf16", 128, 702, 4), ("fp32", 128, 333, 4),
                 ("bf16", 64, 640, 8), ("bf16", 64, 129, 1), ("bf16", 128, 4100, 4),
                 ("bf16", 128, 5, 8), ("fp32", 64, 1001, 3)]


@pytest.mark.parametrize("dtype,D,Lc,ps", SUMMARY_CASES)
def test_page_summaries_bit_exact(rkv, dtype, D, Lc, ps):
    w = configs.SMALL[1].replace(dtype=dtype, D=D, L=Lc, keep=Lc, W=min(8, Lc), n_needles=0,
                                 B=2, Hq=4, Hkv=2, cfg_id=100 + Lc)
    k = gen.prompt_layer(w)["k"]
    kmin, kmax = rkv.rkv_build_page_summaries(T(k), ps)
    omin, omax = O.summaries(k, ps)
    assert np.array_equal(O.widen(H(kmin)), omin)
    assert np.array_equal(O.widen(H(kmax)), omax)


# ----------------------------------------------------------------------------- decode calls

def _cache(w, steps=2):
    """A synthetic compressed cache of Lc slots (drawn like a prompt of length Lc)."""
    wc = w.replace(L=w.Lc, keep=w.Lc)
    d = gen.prompt_layer(wc)
    return wc, d, gen.decode_queries(wc, steps=steps)


DECODE_CASES = list(configs.SMALL) + [
    configs.SMALL[1].replace(name="bf16-P-not-multiple-of-8", keep=1001, cfg_id=20),
    configs.SMALL[2].replace(name="fp32-P-not-multiple-of-4", keep=501, cfg_id=21, topk=(8, 104)),
    configs.SMALL[1].replace(name="bf16-g8-d128", Hq=16, Hkv=2, W=16, cfg_id=22),
]


@pytest.mark.parametrize("w", DECODE_CASES, ids=_wid)
def test_hybrid_approx_scores(rkv, w):
    wc, d, qs = _cache(w)
    kmin, kmax = rkv.rkv_build_page_summaries(T(d["k"]), w.page_size)
    omin, omax = O.summaries(d["k"], w.page_size)
    G = w.G
    for s in range(qs.shape[0]):
        scores, chans = rkv.rkv_hybrid_approx_scores(T(qs[s]), kmin, kmax, w.r,
                                                     return_channels=True)
        scores, chans = scores.cpu().numpy(), chans.cpu().numpy()
        q = O.widen(qs[s])
        for b in range(w.B):
            for h in range(w.Hkv):
                qg = q[b, h * G:(h + 1) * G]
                selection_matches(chans[b, h], np.abs(qg).sum(0), w.r)
                # bound over the GPU's channel set (equal to the oracle's up to exact ties)
                ref = O.approx_page_scores(qg.sum(0), chans[b, h].astype(np.int64), omin[b, h],
                                           omax[b, h])
                assert_rows_close(scores[b, h], ref, 1e-5, f"scores b{b} h{h}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_hybrid_approx_scores_wide_grid(rkv, dtype):
    # enough (b, h) rows x pages that the launch picks the fewest channel groups per block
    B, Hq, Hkv, D, P, r = 8, 32, 8, 128, 8200, 32
    rng = np.random.default_rng(41)
    a = rng.standard_normal((B, Hkv, D, P), dtype=np.float32)
    b = a + np.abs(rng.standard_normal((B, Hkv, D, P), dtype=np.float32))
    kmin, kmax = gen.to_storage(a, dtype), gen.to_storage(b, dtype)
    q = gen.to_storage(rng.standard_normal((B, Hq, D), dtype=np.float32), dtype)
    scores, chans = rkv.rkv_hybrid_approx_scores(T(q), T(kmin), T(kmax), r, return_channels=True)
    scores, chans = scores.cpu().numpy(), chans.cpu().numpy()
    q64, mn, mx = O.widen(q), O.widen(kmin), O.widen(kmax)
    G = Hq // Hkv
    for bb in range(B):
        for h in range(Hkv):
            qg = q64[bb, h * G:(h + 1) * G]
            selection_matches(chans[bb, h], np.abs(qg).sum(0), r)
            ref = O.approx_page_scores(qg.sum(0), chans[bb, h].astype(np.int64), mn[bb, h],
                                       mx[bb, h])
            assert_rows_close(scores[bb, h], ref, 1e-5, f"scores b{bb} h{h}")


def _random_pages(rng, P, n, force_last=False):
    if force_last and n < P:
        sel = np.append(rng.choice(P - 1, size=n - 1, replace=False), P - 1)
    else:
        sel = rng.choice(P, size=n, replace=False)
    return np.sort(sel).astype(np.int32)


@pytest.mark.parametrize("w", DECODE_CASES, ids=_wid)
def test_sparse_attend_decode(rkv, w):
    wc, d, qs = _cache(w)
    rng = np.random.default_rng(w.cfg_id)
    P = w.P
    kc, vc = O.widen(d["k"]), O.widen(d["v"])
    scale = 1.0 / math.sqrt(w.D)
    for n_pages in sorted({1, min(P, 3), min(P, 33), max(1, P // 2), P}):
        # the first head always lists the (possibly partial) last page
        pages = np.stack([np.stack([_random_pages(rng, P, n_pages, force_last=(b == 0 and h == 0))
                                    for h in range(w.Hkv)]) for b in range(w.B)])
        out = rkv.rkv_sparse_attend_decode(T(qs[0]), T(d["k"]), T(d["v"]),
                                           torch.from_numpy(pages).cuda(), w.page_size, scale)
        got = O.widen(H(out))
        q = O.widen(qs[0])
        G = w.G
        ref = np.zeros_like(got)
        for b in range(w.B):
            for h in range(w.Hkv):
                toks = O.page_tokens(pages[b, h], w.page_size, w.Lc)
                ref[b, h * G:(h + 1) * G] = O.sparse_attention(q[b, h * G:(h + 1) * G], kc[b, h],
                                                               vc[b, h], toks, scale)
        assert_rows_close(got, ref, TOL_OUT[w.dtype], f"attend n_pages={n_pages}")


@pytest.mark.parametrize("G,ps", [(1, 1), (3, 4), (5, 2), (6, 3), (7, 4), (8, 5)])
def test_sparse_attend_matrix_core_group_sizes(rkv, G, ps):
    # bf16 rows of 128 go through the matrix-core wave, whose 16 columns hold the G heads and
    # zero padding; odd page sizes and partial chunks of 32 tokens at the end of the list
    w = configs.SMALL[1].replace(name=f"mfma-g{G}", B=2, Hq=2 * G, Hkv=2, L=1037, keep=1037,
                                 page_size=ps, cfg_id=70 + G)
    wc, d, qs = _cache(w, steps=1)
    rng = np.random.default_rng(70 + G)
    P = w.P
    kc, vc = O.widen(d["k"]), O.widen(d["v"])
    q = O.widen(qs[0])
    for n_pages in sorted({1, min(P, 7), min(P, 45), P}):
        pages = np.stack([np.stack([_random_pages(rng, P, n_pages, force_last=(b == 1))
                                    for _ in range(w.Hkv)]) for b in range(w.B)])
        out = rkv.rkv_sparse_attend_decode(T(qs[0]), T(d["k"]), T(d["v"]),
                                           torch.from_numpy(pages).cuda(), ps)
        got = O.widen(H(out))
        for b in range(w.B):
            for h in range(w.Hkv):
                toks = O.page_tokens(pages[b, h], ps, w.Lc)
                ref = O.sparse_attention(q[b, h * G:(h + 1) * G], kc[b, h], vc[b, h], toks,
                                         1 / math.sqrt(w.D))
                assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT["bf16"],
                                  f"G={G} n_pages={n_pages} b{b} h{h}")


def test_sparse_attend_many_splits_bf16(rkv):
    # a long page list per head exercises the split + log-sum-exp merge path
    w = configs.SMALL[1].replace(name="long", B=1, Hq=8, Hkv=2, L=12500, keep=12000, cfg_id=30)
    wc, d, qs = _cache(w, steps=1)
    rng = np.random.default_rng(3)
    pages = np.stack([_random_pages(rng, w.P, 2500) for _ in range(w.Hkv)])[None]
    out = rkv.rkv_sparse_attend_decode(T(qs[0]), T(d["k"]), T(d["v"]),
                                       torch.from_numpy(pages).cuda(), w.page_size)
    got = O.widen(H(out))
    q, kc, vc = O.widen(qs[0]), O.widen(d["k"]), O.widen(d["v"])
    for h in range(w.Hkv):
        toks = O.page_tokens(pages[0, h], w.page_size, w.Lc)
        ref = O.sparse_attention(q[0, h * 4:(h + 1) * 4], kc[0, h], vc[0, h], toks,
                                 1 / math.sqrt(w.D))
        assert_rows_close(got[0, h * 4:(h + 1) * 4], ref, TOL_OUT["bf16"])


def test_full_budget_is_dense_attention(rkv):
    w = configs.SMALL[2]
    wc, d, qs = _cache(w, steps=1)
    pages = np.tile(np.arange(w.P, dtype=np.int32), (w.B, w.Hkv, 1))
    out = rkv.rkv_sparse_attend_decode(T(qs[0]), T(d["k"]), T(d["v"]),
                                       torch.from_numpy(pages).cuda(), w.page_size)
    q, kc, vc = O.widen(qs[0]), O.widen(d["k"]), O.widen(d["v"])
    G = w.G
    kk = torch.from_numpy(np.repeat(kc, G, axis=1))
    vv = torch.from_numpy(np.repeat(vc, G, axis=1))
    dense = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], kk, vv, scale=1 / math.sqrt(w.D))[:, :, 0].numpy()
    assert_rows_close(O.widen(H(out)), dense, TOL_OUT["fp32"])


# ----------------------------------------------------------------------------- eviction

def _evict_check(rkv, w, d, pool="avg", rtol_pooled=1e-4, needles=True):
    scale = 1.0 / math.sqrt(w.D)
    pooled = torch.empty((w.B, w.Hkv, max(w.L - w.W, 1)), dtype=torch.float32, device="cuda")
    kept, kc, vc = rkv.rkv_snapkvpp_evict(T(d["q_win"]), T(d["k"]), T(d["v"]), w.keep,
                                          w.pool_kernel, pool, scale, pooled_out=pooled)
    kept = kept.cpu().numpy()
    ref = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, scale, pool)
    k64, v64 = O.widen(d["k"]), O.widen(d["v"])
    assert kept.shape == ref["kept"].shape
    exact = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            kp = kept[b, h].astype(np.int64)
            if w.keep < w.L:
                assert_rows_close(pooled[b, h].cpu().numpy(), ref["pooled"][b, h], rtol_pooled,
                                  f"pooled b{b} h{h}")
                assert list(kp[w.keep - w.W:]) == list(range(w.L - w.W, w.L))
                exact += selection_matches(kp[:w.keep - w.W], ref["pooled"][b, h], w.keep - w.W)
                if needles:
                    assert set(d["needle_pos"][b, h].tolist()) <= set(kp.tolist()), "needle evicted"
            else:
                assert np.array_equal(kp, np.arange(w.L))
            assert np.array_equal(O.widen(H(kc[b, h])), k64[b, h, kp])
            assert np.array_equal(O.widen(H(vc[b, h])), v64[b, h, kp])
    return exact


@pytest.mark.parametrize("w", configs.SMALL, ids=_wid)
def test_snapkvpp_evict(rkv, w):
    d = gen.prompt_layer(w)
    _evict_check(rkv, w, d)


def test_snapkvpp_evict_max_pool_and_limits(rkv):
    w = configs.SMALL[1]
    d = gen.prompt_layer(w)
    _evict_check(rkv, w, d, pool="max")
    _evict_check(rkv, w.replace(keep=w.W), d, needles=False)  # only the window survives
    _evict_check(rkv, w.replace(keep=w.L), d)          # nothing evicted
    _evict_check(rkv, w.replace(keep=w.L + 5), d)      # budget above the prompt


def test_snapkvpp_evict_odd_key_groups_multiblock_topk(rkv):
    # 32 heads over 10000 keys: three key groups per block in both window passes (the last one
    # unpaired in the double buffer, chunks of different group counts), and a prefix above 8192
    # scores, so the kept-set top-k spreads each row over blocks with histograms that the
    # log-sum-exp launch cleared
    w = configs.SMALL[1].replace(name="odd-groups", B=16, Hq=4, Hkv=2, D=64, L=10000, W=16,
                                 keep=2000, pool_kernel=15, cfg_id=31)
    d = gen.prompt_layer(w)
    _evict_check(rkv, w, d)
    _evict_check(rkv, w.replace(keep=w.W), d, needles=False)  # nothing to select
    # the fp32 passes ahead of the same multi-block top-k
    wf = w.replace(name="odd-groups-fp32", dtype="fp32", B=2, L=9000, cfg_id=32)
    _evict_check(rkv, wf, gen.prompt_layer(wf))
    # a prefix of 9001 scores: the pooling that counts the top-k's first digit level ends in a
    # partial block, and the second row's scores start off a 16-byte boundary
    wr = w.replace(name="odd-groups-ragged", B=2, L=9017, keep=1500, cfg_id=34)
    _evict_check(rkv, wr, gen.prompt_layer(wr))


# (G, W, D): window rows G*W from one 32-row tile to 16 tiles; 120 rows end in a partial tile,
# and above 256 rows the rows split into parts of unequal size (288 and 480 rows).
ROW_TILE_CASES = [(1, 32, 128), (2, 32, 64), (3, 32, 128), (5, 24, 128), (5, 32, 64),
                  (6, 32, 128), (7, 32, 128), (8, 32, 64), (9, 32, 128), (15, 32, 64),
                  (16, 32, 128)]


@pytest.mark.parametrize("G,W,D", ROW_TILE_CASES, ids=[f"g{g}-w{w}-d{d}" for g, w, d in ROW_TILE_CASES])
def test_snapkvpp_evict_row_tiles(rkv, G, W, D):
    w = configs.SMALL[1].replace(name=f"tiles-g{G}-w{W}-d{D}", B=1, Hq=2 * G, Hkv=2, D=D, L=2111,
                                 W=W, keep=530, pool_kernel=15, n_needles=4, cfg_id=60 + G)
    _evict_check(rkv, w, gen.prompt_layer(w))


def test_snapkvpp_evict_logit_jump_in_a_later_key_group(rkv):
    # 70000 keys over 2 KV heads: every pass-1 block takes two key groups. A key planted in the
    # second group of its block scores about 90 nats above the rest for one window row, so that
    # row's running maximum jumps there and the first group's sum is rescaled to almost nothing.
    w = configs.SMALL[1].replace(name="jump", B=1, Hq=8, Hkv=2, D=128, L=70000, W=32, keep=9000,
                                 pool_kernel=15, n_needles=4, cfg_id=70)
    d = gen.prompt_layer(w)
    nchunk = -(-((w.L + 255) // 256) // 2)  # chunks of two 256-key groups
    pos = (1 * nchunk + 5) * 256 + 10       # group 1 of chunk 5
    for h in range(w.Hkv):
        q = O.widen(d["q_win"][0, h * w.G, 3]) * 8.0  # exact in bf16: a power-of-two multiple
        d["k"][0, h, pos] = gen.to_storage(q.astype(np.float32), w.dtype)
    _evict_check(rkv, w, d)


def test_evict_indices_only(rkv):
    w = configs.TINY_FP32
    d = gen.prompt_layer(w)
    kept, kc, vc = rkv.rkv_snapkvpp_evict(T(d["q_win"]), T(d["k"]), T(d["v"]), w.keep,
                                          w.pool_kernel, indices_only=True)
    assert kc is None and vc is None
    ref = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, 1 / math.sqrt(w.D))
    for h in range(w.Hkv):
        selection_matches(kept[0, h, :w.keep - w.W].cpu().numpy(), ref["pooled"][0, h],
                          w.keep - w.W)


def test_error_codes_leave_outputs_untouched(rkv):
    q = torch.zeros((1, 4, 64), device="cuda")
    kc = torch.zeros((1, 2, 10, 64), device="cuda")
    pages = torch.zeros((1, 2, 4), dtype=torch.int32, device="cuda")  # 4 > ceil(10/4)=3 pages
    out = torch.full((1, 4, 64), 7.0, device="cuda")
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_sparse_attend_decode(q, kc, kc, pages, 4, out=out)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ----------------------------------------------------------------------------- fused step

def _fused_vs_calls(rkv, w, q, k_c, v_c, kmin, kmax, topk, ws=None):
    """Runs the fused step and the three separate calls; checks identical selections."""
    n_pages = min(topk // w.page_size, w.P)
    B, Hq, D = q.shape
    Hkv = k_c.shape[1]
    chans = torch.empty((B, Hkv, w.r), dtype=torch.int32, device="cuda")
    scores = torch.empty((B, Hkv, w.P), dtype=torch.float32, device="cuda")
    pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device="cuda")
    if ws is None:
        ws = rkv.rkv_hybrid_decode_workspace(q, Hkv, w.Lc, w.page_size, n_pages)
    out = rkv.rkv_hybrid_decode_step(q, kmin, kmax, k_c, v_c, w.page_size, w.r, n_pages,
                                     chan_idx=chans, page_scores=scores, page_idx=pages,
                                     workspace=ws)
    s2, c2 = rkv.rkv_hybrid_approx_scores(q, kmin, kmax, w.r, return_channels=True)
    p2 = rkv.rkv_topk_select(s2, n_pages)
    o2 = rkv.rkv_sparse_attend_decode(q, k_c, v_c, p2, w.page_size)
    torch.cuda.synchronize()
    assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0
    assert torch.equal(chans, c2)
    assert torch.equal(scores.view(torch.int32), s2.view(torch.int32)), "scores differ in bits"
    assert torch.equal(pages, p2)
    return out, pages, o2


@pytest.mark.parametrize("w", DECODE_CASES, ids=_wid)
def test_fused_decode_step(rkv, w):
    wc, d, qs = _cache(w)
    kc_t, vc_t = T(d["k"]), T(d["v"])
    kmin, kmax = rkv.rkv_build_page_summaries(kc_t, w.page_size)
    kc, vc = O.widen(d["k"]), O.widen(d["v"])
    G = w.G
    for s in range(qs.shape[0]):
        for topk in sorted(set(w.topk) | {w.page_size, w.P * w.page_size}):
            out, pages, o2 = _fused_vs_calls(rkv, w, T(qs[s]), kc_t, vc_t, kmin, kmax, topk)
            got, pg = O.widen(H(out)), pages.cpu().numpy()
            q = O.widen(qs[s])
            ref = np.zeros_like(got)
            for b in range(w.B):
                for h in range(w.Hkv):
                    toks = O.page_tokens(pg[b, h], w.page_size, w.Lc)
                    ref[b, h * G:(h + 1) * G] = O.sparse_attention(
                        q[b, h * G:(h + 1) * G], kc[b, h], vc[b, h], toks, 1 / math.sqrt(w.D))
            assert_rows_close(got, ref, TOL_OUT[w.dtype], f"fused step topk={topk}")
            assert_rows_close(O.widen(H(o2)), ref, TOL_OUT[w.dtype], f"three calls topk={topk}")


def test_fused_decode_step_windows_one_block_per_head(rkv):
    # enough heads that every head gets one block, and more pages than the LDS page buffer
    w = configs.SMALL[4].replace(name="wide", B=64, Hq=4, Hkv=4, D=64, L=5000, keep=5000,
                                 page_size=1, r=16, cfg_id=40)
    g = torch.Generator(device="cuda").manual_seed(7)
    k_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    v_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((w.B, w.Hq, w.D), device="cuda", generator=g).to(torch.bfloat16)
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, 1)
    out, pages, _ = _fused_vs_calls(rkv, w, q, k_c, v_c, kmin, kmax, 2100)
    got, pg = O.widen(H(out)), pages.cpu().numpy()
    q64 = O.widen(H(q))
    for (b, h) in [(0, 0), (17, 2), (63, 3)]:
        kc = O.widen(H(k_c[b, h]))
        vc = O.widen(H(v_c[b, h]))
        ref = O.sparse_attention(q64[b, h:h + 1], kc, vc, pg[b, h].astype(np.int64), 0.125)
        assert_rows_close(got[b, h:h + 1], ref, TOL_OUT["bf16"], f"b{b} h{h}")


def _check_fused_heads(rkv, w, q, k_c, v_c, topk, heads, scale):
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, w.page_size)
    out, pages, _ = _fused_vs_calls(rkv, w, q, k_c, v_c, kmin, kmax, topk)
    got, pg = O.widen(H(out)), pages.cpu().numpy()
    q64 = O.widen(H(q))
    G = w.Hq // w.Hkv
    for (b, h) in heads:
        toks = O.page_tokens(pg[b, h], w.page_size, w.Lc)
        ref = O.sparse_attention(q64[b, h * G:(h + 1) * G], O.widen(H(k_c[b, h])),
                                 O.widen(H(v_c[b, h])), toks, scale)
        assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT["bf16"], f"b{b} h{h} k{topk}")


def test_fused_decode_step_rows_over_4096_pages(rkv):
    # a head spread over many blocks, with more pages than 8 per thread of a block
    w = configs.SMALL[1].replace(name="p6000", B=1, Hq=4, Hkv=2, D=64, L=6000, keep=6000,
                                 page_size=1, r=16, cfg_id=41)
    g = torch.Generator(device="cuda").manual_seed(11)
    k_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    v_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((w.B, w.Hq, w.D), device="cuda", generator=g).to(torch.bfloat16)
    for topk in (1, 64, 3000, 5999):
        _check_fused_heads(rkv, w, q, k_c, v_c, topk, [(0, 0), (0, 1)], 0.125)


def test_limits_at_their_maximum(rkv):
    # the largest sizes the header accepts: a fused step over 8192 pages (16 per thread of the
    # ranking block), and an fp32 eviction with G*W = 2048 window rows and the widest pooling
    w = configs.SMALL[1].replace(name="p8192", B=1, Hq=4, Hkv=2, D=64, L=8192, keep=8192,
                                 page_size=1, r=16, cfg_id=43)
    g = torch.Generator(device="cuda").manual_seed(12)
    k_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    v_c = torch.randn((w.B, w.Hkv, w.Lc, w.D), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((w.B, w.Hq, w.D), device="cuda", generator=g).to(torch.bfloat16)
    for topk in (1, 100, 8191, 8192):
        _check_fused_heads(rkv, w, q, k_c, v_c, topk, [(0, 0), (0, 1)], 0.125)
    we = configs.SMALL[2].replace(name="gw2048", dtype="fp32", B=1, Hq=16, Hkv=2, D=64,
                                  L=700, W=256, keep=400, pool_kernel=127, cfg_id=44)
    # a 127-wide box over a 444-token prefix smears the planted needles away: the oracle evicts
    # them too, so only parity is checked here
    _evict_check(rkv, we, gen.prompt_layer(we), needles=False)


# Shapes whose plans cover the fused step's role mixes on a 256-CU device: one attender with 32
# scorers (B*Hkv = 8, top-k 128, the 128K workload's plan), 8 and 16 attenders merged by the last
# to arrive, one scorer that also attends beside a second attender (B*Hkv = 128, the batch-16
# workload's plan), ragged page counts, a group of 8 with two merge rounds, fp32, and one block
# per head (B*Hkv >= 256).
PLAN_CASES = [
    # name, dtype, B, Hq, Hkv, D, P, ps, top-k budgets
    ("bh8-p4096", "bf16", 1, 32, 8, 128, 4096, 4, (128, 512, 1024, 2048)),
    ("bh128-p1024", "bf16", 16, 32, 8, 128, 1024, 4, (256, 64, 1024)),
    ("bh9-ragged", "bf16", 3, 12, 3, 64, 777, 3, (3, 300, 1500)),
    ("g8-bh1", "bf16", 1, 8, 1, 128, 2000, 2, (1200, 130)),
    ("fp32-bh4", "fp32", 2, 4, 2, 64, 500, 2, (200, 998)),
    ("bh320-solo", "bf16", 40, 32, 8, 64, 300, 4, (512,)),
    # over 256 heads (the three-launch form): fp32 rows on the VALU attention wave, and bf16 rows
    # of 128 on the matrix-core wave with a top-k row of more than 4096 pages (512-thread rows)
    ("bh264-fp32", "fp32", 66, 8, 4, 64, 700, 2, (64, 1400)),
    ("bh264-p5000", "bf16", 33, 64, 8, 128, 5000, 1, (700, 5000)),
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_fused_decode_step_plans(rkv, case):
    name, dtype, B, Hq, Hkv, D, P, ps, budgets = case
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Lc = P * ps - (1 if ps > 1 else 0)  # a partial last page
    w = configs.SMALL[1].replace(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, L=Lc, keep=Lc,
                                 page_size=ps, r=D // 4, cfg_id=45)
    g = torch.Generator(device="cuda").manual_seed(21)
    k_c = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(dt)
    v_c = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(dt)
    q = torch.randn((B, Hq, D), device="cuda", generator=g).to(dt)
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, ps)
    G = Hq // Hkv
    q64 = O.widen(H(q))
    heads = sorted({(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)})
    for topk in budgets:
        out, pages, _ = _fused_vs_calls(rkv, w, q, k_c, v_c, kmin, kmax, topk)
        got, pg = O.widen(H(out)), pages.cpu().numpy()
        for (b, h) in heads:
            toks = O.page_tokens(pg[b, h], ps, Lc)
            ref = O.sparse_attention(q64[b, h * G:(h + 1) * G], O.widen(H(k_c[b, h])),
                                     O.widen(H(v_c[b, h])), toks, 1 / math.sqrt(D))
            assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT[dtype],
                              f"{name} b{b} h{h} k{topk}")


def test_fused_decode_step_beside_a_busy_stream(rkv):
    # A block that still misses another block's scores or slice at the steal deadline does that
    # work itself, so fused steps finish with correct results while another stream's kernels
    # hold CUs at the same time. The outputs equal those of the same steps run alone.
    w = configs.SMALL[1].replace(name="busy", B=1, Hq=32, Hkv=8, D=128, L=8192, keep=8192,
                                 page_size=4, r=32, cfg_id=46)
    g = torch.Generator(device="cuda").manual_seed(23)
    k_c = torch.randn((1, 8, w.Lc, 128), device="cuda", generator=g).to(torch.bfloat16)
    v_c = torch.randn((1, 8, w.Lc, 128), device="cuda", generator=g).to(torch.bfloat16)
    qs = torch.randn((12, 1, 32, 128), device="cuda", generator=g).to(torch.bfloat16)
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, 4)
    n_pages = 256
    ws = rkv.rkv_hybrid_decode_workspace(qs[0], 8, w.Lc, 4, n_pages)
    alone = [rkv.rkv_hybrid_decode_step(qs[s], kmin, kmax, k_c, v_c, 4, 32, n_pages, workspace=ws)
             for s in range(12)]
    torch.cuda.synchronize()
    a = torch.randn((4096, 4096), device="cuda", generator=g).to(torch.bfloat16)
    busy = torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    with torch.cuda.stream(busy):
        acc = a
        for _ in range(6):
            acc = torch.mm(acc, a) * 1e-3
    for s in range(12):
        outs.append(rkv.rkv_hybrid_decode_step(qs[s], kmin, kmax, k_c, v_c, 4, 32, n_pages,
                                               workspace=ws))
    torch.cuda.synchronize()
    assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0
    for s in range(12):
        assert torch.equal(outs[s], alone[s]), f"step {s}"
    del acc


@pytest.mark.parametrize("case", [PLAN_CASES[0], PLAN_CASES[1], PLAN_CASES[3]],
                         ids=[PLAN_CASES[i][0] for i in (0, 1, 3)])
def test_fused_decode_step_stealing(rkv, case, monkeypatch):
    # With a negative steal deadline (a test mode), every attender scores every share and
    # attends every slice itself: the work is done several times over, and the results must
    # still equal the three calls' bit for bit (scores, pages) and the oracle.
    monkeypatch.setenv("RKV_STEAL_US", "-1")
    name, dtype, B, Hq, Hkv, D, P, ps, budgets = case
    Lc = P * ps
    w = configs.SMALL[1].replace(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, L=Lc, keep=Lc,
                                 page_size=ps, r=D // 4, cfg_id=47)
    g = torch.Generator(device="cuda").manual_seed(29)
    k_c = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(torch.bfloat16)
    v_c = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((B, Hq, D), device="cuda", generator=g).to(torch.bfloat16)
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, ps)
    G = Hq // Hkv
    q64 = O.widen(H(q))
    stole = 0
    for topk in budgets:
        n_pages = min(topk // ps, P)
        ws = rkv.rkv_hybrid_decode_workspace(q, Hkv, Lc, ps, n_pages)
        for rep in range(3):  # repeated calls on one workspace: the epochs stay consistent
            out, pages, _ = _fused_vs_calls(rkv, w, q, k_c, v_c, kmin, kmax, topk, ws=ws)
        stole |= rkv.decode_workspace_status(ws)
        got, pg = O.widen(H(out)), pages.cpu().numpy()
        for (b, h) in [(0, 0), (B - 1, Hkv - 1)]:
            toks = O.page_tokens(pg[b, h], ps, Lc)
            ref = O.sparse_attention(q64[b, h * G:(h + 1) * G], O.widen(H(k_c[b, h])),
                                     O.widen(H(v_c[b, h])), toks, 1 / math.sqrt(D))
            assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT[dtype], f"{name} k{topk}")
    # informational bits: 16 = an attender scored a share, 32 = an attender attended a slice
    assert stole & 16, "no share was scored by an attender"
    assert stole & 32 or all(min(tk // ps, P) * ps <= 256 for tk in budgets), "no slice redone"


def _tied_keys(B, Hkv, P, ps, D, mode, seed):
    """K caches whose pages repeat, so that page scores tie exactly: every page the same, half
    of the pages the same, or pages in groups of three."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, P, ps, D)).astype(np.float32)
    if mode == "all":
        k[:] = k[:, :, :1]
    elif mode == "half":
        sel = rng.permutation(P)[: P // 2]
        k[:, :, sel] = k[:, :, sel[:1]]
    elif mode == "triples":
        k = k[:, :, (np.arange(P) // 3) * 3]
    return torch.from_numpy(np.ascontiguousarray(k).reshape(B, Hkv, P * ps, D)).to(
        "cuda", torch.bfloat16)


@pytest.mark.parametrize("mode", ["all", "half", "triples"])
@pytest.mark.parametrize("B,P", [(1, 4096), (128, 256)], ids=["many-blocks", "one-block"])
def test_fused_decode_step_tied_scores(rkv, mode, B, P):
    # exact ties in the page scores: the lower page index wins in the fused step as in the
    # separate top-k call (all equal, a crowded bin, and small tied groups)
    ps, D = 4, 128
    w = configs.SMALL[1].replace(name=f"ties-{mode}", B=B, Hq=8, Hkv=2, D=D, L=P * ps,
                                 keep=P * ps, page_size=ps, r=32, cfg_id=42)
    k_c = _tied_keys(B, w.Hkv, P, ps, D, mode, 5)
    g = torch.Generator(device="cuda").manual_seed(6)
    v_c = torch.randn((B, w.Hkv, w.Lc, D), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((B, w.Hq, D), device="cuda", generator=g).to(torch.bfloat16)
    heads = [(0, 0), (B - 1, 1)]
    for n in (1, P // 4, P // 2, 3 * P // 4, P - 1):
        _check_fused_heads(rkv, w, q, k_c, v_c, n * ps, heads, 1 / math.sqrt(D))


GRAPH_CASES = [configs.SMALL[1],
               # 264 heads: the step's three launches (scores, top-k, attention) in one graph
               configs.SMALL[1].replace(name="graph-264-heads", B=132, L=600, keep=600, W=16,
                                        n_needles=2, cfg_id=48)]


@pytest.mark.parametrize("w", GRAPH_CASES, ids=_wid)
def test_fused_decode_step_graph_replays(rkv, w):
    wc, d, qs = _cache(w, steps=3)
    kc_t, vc_t = T(d["k"]), T(d["v"])
    kmin, kmax = rkv.rkv_build_page_summaries(kc_t, w.page_size)
    n_pages = w.topk[-1] // w.page_size
    q_in = T(qs[0]).clone()
    out = torch.empty_like(q_in)
    pages = torch.empty((w.B, w.Hkv, n_pages), dtype=torch.int32, device="cuda")
    ws = rkv.rkv_hybrid_decode_workspace(q_in, w.Hkv, w.Lc, w.page_size, n_pages)

    def step():
        rkv.rkv_hybrid_decode_step(q_in, kmin, kmax, kc_t, vc_t, w.page_size, w.r, n_pages,
                                   page_idx=pages, out=out, workspace=ws)

    eager = []
    for s in range(3):
        q_in.copy_(T(qs[s]))
        step()
        eager.append((out.clone(), pages.clone()))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(6):
        s = rep % 3
        q_in.copy_(T(qs[s]))
        _ = (kc_t.float().sum() + 1.0).item()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[s][0]), f"replay {rep} output"
        assert torch.equal(pages, eager[s][1]), f"replay {rep} pages"
    assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0


# ----------------------------------------------------------------------------- growing cache

def _randn(shape, g, dt):
    return torch.randn(shape, device="cuda", generator=g).to(dt)


@pytest.mark.parametrize("dtype,D,ps", [("bf16", 128, 4), ("fp32", 64, 3), ("bf16", 64, 1)])
def test_kv_append_bit_exact(rkv, dtype, D, ps):
    # tokens appended one at a time into caches of fixed capacity: rows and page summaries equal
    # the oracle's append chain, and the batch summaries of the grown cache, bit for bit
    B, Hkv, cap, L0, n = 2, 3, 61, 17, 30
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(21)
    k_all, v_all = _randn((B, Hkv, L0 + n, D), g, dt), _randn((B, Hkv, L0 + n, D), g, dt)
    k_c = torch.zeros((B, Hkv, cap, D), dtype=dt, device="cuda")
    v_c = torch.zeros_like(k_c)
    k_c[:, :, :L0] = k_all[:, :, :L0]
    v_c[:, :, :L0] = v_all[:, :, :L0]
    kmin, kmax = rkv.rkv_build_page_summaries_cap(k_c, L0, ps)
    pcap = -(-cap // ps)
    assert kmin.shape == (B, Hkv, D, pcap)
    ka, va = O.widen(H(k_all)), O.widen(H(v_all))
    ref = {}
    for b in range(B):
        for h in range(Hkv):
            kk = np.zeros((cap, D))
            vv = np.zeros((cap, D))
            kk[:L0], vv[:L0] = ka[b, h, :L0], va[b, h, :L0]
            mn, mx = np.zeros((D, pcap)), np.zeros((D, pcap))
            p0 = -(-L0 // ps)
            mn[:, :p0], mx[:, :p0] = O.page_summaries(ka[b, h, :L0], ps)
            ref[b, h] = [kk, vv, mn, mx]
    Lc = L0
    for _ in range(n):
        for (b, h), st in ref.items():
            ref[b, h] = list(O.kv_append(*st, Lc, ka[b, h, Lc], va[b, h, Lc], ps))
        Lc = rkv.rkv_kv_append(k_all[:, :, Lc].contiguous(), v_all[:, :, Lc].contiguous(), k_c, v_c,
                               kmin, kmax, Lc, ps)
    torch.cuda.synchronize()
    P = -(-Lc // ps)
    gk, gv = O.widen(H(k_c)), O.widen(H(v_c))
    gmin, gmax = O.widen(H(kmin[..., :P])), O.widen(H(kmax[..., :P]))  # pages past P unwritten
    for (b, h), (kk, vv, mn, mx) in ref.items():
        assert np.array_equal(gk[b, h, :Lc], kk[:Lc]) and np.array_equal(gv[b, h, :Lc], vv[:Lc])
        assert np.array_equal(gmin[b, h], mn[:, :P]), f"kmin b{b} h{h}"
        assert np.array_equal(gmax[b, h], mx[:, :P]), f"kmax b{b} h{h}"
    bmin, bmax = rkv.rkv_build_page_summaries_cap(k_c, Lc, ps)
    torch.cuda.synchronize()
    assert torch.equal(bmin[..., :P].view(torch.int16 if dtype == "bf16" else torch.int32),
                       kmin[..., :P].view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(bmax[..., :P].view(torch.int16 if dtype == "bf16" else torch.int32),
                       kmax[..., :P].view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("cap", [1104, 1152], ids=["pitch-not-vector-multiple", "pitch-vector-multiple"])
def test_decode_step_cap_on_growing_cache(rkv, cap):
    # decode steps between appends on caches laid out for a capacity, one workspace for every
    # length: channels, scores and pages equal the three calls on a dense copy, outputs the oracle
    B, Hq, Hkv, D, ps, r, L0 = 1, 8, 2, 128, 4, 32, 1001
    dt = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(23)
    k_c = _randn((B, Hkv, cap, D), g, dt)
    v_c = _randn((B, Hkv, cap, D), g, dt)
    kmin, kmax = rkv.rkv_build_page_summaries_cap(k_c, L0, ps)
    Lc = L0
    for n_pages in (16, 64):
        q0 = _randn((B, Hq, D), g, dt)
        ws = rkv.rkv_hybrid_decode_workspace(q0, Hkv, cap, ps, n_pages)
        for step in range(3):
            for _ in range(7):
                Lc = rkv.rkv_kv_append(_randn((B, Hkv, D), g, dt), _randn((B, Hkv, D), g, dt), k_c,
                                       v_c, kmin, kmax, Lc, ps)
            q = _randn((B, Hq, D), g, dt)
            P = -(-Lc // ps)
            chans = torch.empty((B, Hkv, r), dtype=torch.int32, device="cuda")
            scores = torch.empty((B, Hkv, P), dtype=torch.float32, device="cuda")
            pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device="cuda")
            out = rkv.rkv_hybrid_decode_step_cap(q, kmin, kmax, k_c, v_c, Lc, ps, r, n_pages,
                                                 chan_idx=chans, page_scores=scores,
                                                 page_idx=pages, workspace=ws)
            kd, vd = k_c[:, :, :Lc].contiguous(), v_c[:, :, :Lc].contiguous()
            dmin, dmax = rkv.rkv_build_page_summaries(kd, ps)
            s2, c2 = rkv.rkv_hybrid_approx_scores(q, dmin, dmax, r, return_channels=True)
            p2 = rkv.rkv_topk_select(s2, n_pages)
            torch.cuda.synchronize()
            assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0
            assert torch.equal(chans, c2)
            assert torch.equal(scores.view(torch.int32), s2.view(torch.int32)), "scores differ"
            assert torch.equal(pages, p2), f"pages differ at Lc={Lc}"
            got, pg, q64 = O.widen(H(out)), pages.cpu().numpy(), O.widen(H(q))
            G = Hq // Hkv
            for h in range(Hkv):
                toks = O.page_tokens(pg[0, h], ps, Lc)
                ref = O.sparse_attention(q64[0, h * G:(h + 1) * G], O.widen(H(kd[0, h])),
                                         O.widen(H(vd[0, h])), toks, 1 / math.sqrt(D))
                assert_rows_close(got[0, h * G:(h + 1) * G], ref, TOL_OUT["bf16"],
                                  f"Lc={Lc} n_pages={n_pages} h{h}")


# ----------------------------------------------------------------------------- multi-turn variant

@pytest.mark.parametrize("dtype,D,Lc,ps", [("bf16", 128, 702, 4), ("fp32", 64, 333, 3)])
def test_mt_indexed_step_equals_step_on_gathered_cache(rkv, dtype, D, Lc, ps):
    # the view through kept rows of the full cache: summaries and every output of the fused step
    # are bit-identical to those on the gathered cache, and the outputs match the oracle's view
    B, Hq, Hkv, L, r = 2, 8, 2, 3001, 24
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(31)
    k, v = _randn((B, Hkv, L, D), g, dt), _randn((B, Hkv, L, D), g, dt)
    rng = np.random.default_rng(31)
    kept_np = np.stack([np.stack([np.sort(rng.choice(L, Lc, replace=False)) for _ in range(Hkv)])
                        for _ in range(B)]).astype(np.int32)
    kept = torch.from_numpy(kept_np).cuda()
    bi = torch.arange(B, device="cuda")[:, None, None]
    hi = torch.arange(Hkv, device="cuda")[None, :, None]
    kg, vg = k[bi, hi, kept.long()].contiguous(), v[bi, hi, kept.long()].contiguous()
    kmin, kmax = rkv.rkv_build_page_summaries_indexed(k, kept, ps)
    gmin, gmax = rkv.rkv_build_page_summaries(kg, ps)
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(kmin.view(iv), gmin.view(iv)) and torch.equal(kmax.view(iv), gmax.view(iv))
    P = kmin.shape[-1]
    ka, va = O.mt_view(H(k), H(v), kept_np)
    for topk in (ps, 64 * ps, 128 * ps, P * ps):
        n_pages = min(topk // ps, P)
        q = _randn((B, Hq, D), g, dt)
        res = []
        for fn, args in ((rkv.rkv_hybrid_decode_step_indexed, (q, kmin, kmax, k, v, kept)),
                         (rkv.rkv_hybrid_decode_step, (q, gmin, gmax, kg, vg))):
            chans = torch.empty((B, Hkv, r), dtype=torch.int32, device="cuda")
            scores = torch.empty((B, Hkv, P), dtype=torch.float32, device="cuda")
            pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device="cuda")
            out = fn(*args, ps, r, n_pages, chan_idx=chans, page_scores=scores, page_idx=pages)
            res.append((chans, scores, pages, out))
        torch.cuda.synchronize()
        (c1, s1, p1, o1), (c2, s2, p2, o2) = res
        assert torch.equal(c1, c2) and torch.equal(p1, p2), f"topk={topk}"
        assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
        assert torch.equal(o1.view(iv), o2.view(iv)), f"outputs differ at topk={topk}"
        got, pg, q64 = O.widen(H(o1)), p1.cpu().numpy(), O.widen(H(q))
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hkv):
                toks = O.page_tokens(pg[b, h], ps, Lc)
                ref = O.sparse_attention(q64[b, h * G:(h + 1) * G], ka[b, h], va[b, h], toks,
                                         1 / math.sqrt(D))
                assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT[dtype],
                                  f"topk={topk} b{b} h{h}")


def test_many_head_variants_run_as_three_launches(rkv):
    # 260 KV heads (more than the 256 the single-launch step serves): the multi-turn view and the
    # capacity layout go through the three-launch form, with their row map and pitches. Channels,
    # scores and pages equal the plain step on gathered / dense copies bit for bit, and sampled
    # heads match the oracle.
    B, Hq, Hkv, D, L, Lc, ps, r = 130, 8, 2, 128, 1500, 333, 4, 32
    dt = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(37)
    k, v = _randn((B, Hkv, L, D), g, dt), _randn((B, Hkv, L, D), g, dt)
    kept = torch.sort(torch.rand((B, Hkv, L), device="cuda", generator=g).argsort(-1)[..., :Lc],
                      -1).values.to(torch.int32).contiguous()
    bi = torch.arange(B, device="cuda")[:, None, None]
    hi = torch.arange(Hkv, device="cuda")[None, :, None]
    kg, vg = k[bi, hi, kept.long()].contiguous(), v[bi, hi, kept.long()].contiguous()
    kmin, kmax = rkv.rkv_build_page_summaries_indexed(k, kept, ps)
    gmin, gmax = rkv.rkv_build_page_summaries(kg, ps)
    P = kmin.shape[-1]
    # a capacity layout holding the gathered cache in its first Lc of cap slots
    cap = 400
    kc = torch.zeros((B, Hkv, cap, D), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :Lc] = kg
    vc[:, :, :Lc] = vg
    cmin, cmax = rkv.rkv_build_page_summaries_cap(kc, Lc, ps)
    q64s = []
    for n_pages in (16, 60):
        q = _randn((B, Hq, D), g, dt)
        res = []
        for fn, args in ((rkv.rkv_hybrid_decode_step_indexed, (q, kmin, kmax, k, v, kept)),
                         (rkv.rkv_hybrid_decode_step, (q, gmin, gmax, kg, vg))):
            chans = torch.empty((B, Hkv, r), dtype=torch.int32, device="cuda")
            scores = torch.empty((B, Hkv, P), dtype=torch.float32, device="cuda")
            pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device="cuda")
            out = fn(*args, ps, r, n_pages, chan_idx=chans, page_scores=scores, page_idx=pages)
            res.append((chans, scores, pages, out))
        chans = torch.empty((B, Hkv, r), dtype=torch.int32, device="cuda")
        scores = torch.empty((B, Hkv, P), dtype=torch.float32, device="cuda")
        pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device="cuda")
        out = rkv.rkv_hybrid_decode_step_cap(q, cmin, cmax, kc, vc, Lc, ps, r, n_pages,
                                             chan_idx=chans, page_scores=scores, page_idx=pages)
        res.append((chans, scores, pages, out))
        torch.cuda.synchronize()
        (c1, s1, p1, o1) = res[1]
        for c2, s2, p2, o2 in (res[0], res[2]):
            assert torch.equal(c1, c2) and torch.equal(p1, p2), f"n_pages={n_pages}"
            assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        got, pg, q64 = O.widen(H(o1)), p1.cpu().numpy(), O.widen(H(q))
        G = Hq // Hkv
        for b, h in ((0, 0), (64, 1), (B - 1, Hkv - 1)):
            toks = O.page_tokens(pg[b, h], ps, Lc)
            ref = O.sparse_attention(q64[b, h * G:(h + 1) * G], O.widen(H(kg[b, h])),
                                     O.widen(H(vg[b, h])), toks, 1 / math.sqrt(D))
            assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT["bf16"],
                              f"n_pages={n_pages} b{b} h{h}")


# ----------------------------------------------------------------------------- selection quality

@pytest.mark.parametrize("ps,r", [(4, 32), (16, 128), (1, 8)],
                         ids=["hybrid", "quest-like", "sparq-like"])
def test_selection_quality_matches_oracle(rkv, ps, r):
    # exact per-head scores from the library equal the oracle's dot products (fp32 sum of exact
    # bf16 products), and recall / attention mass against Exact-TopK equal the oracle's up to
    # near-tie flips of the fp32 scores
    from sparse_kv_cache_snapkv_amd import quality as Q
    B, Hq, Hkv, D, Lc = 1, 8, 2, 128, 2048
    g = torch.Generator(device="cuda").manual_seed(61)
    scale_c = torch.randn((B, Hkv, 1, D), device="cuda", generator=g).exp()
    k_c = (torch.randn((B, Hkv, Lc, D), device="cuda", generator=g) * scale_c).to(torch.bfloat16)
    q = _randn((B, Hq, D), g, torch.bfloat16)
    ex = Q.exact_scores(q, k_c)
    torch.cuda.synchronize()
    q64, k64 = O.widen(H(q)), O.widen(H(k_c))
    G = Hq // Hkv
    ref = np.stack([np.stack([k64[0, gi // G] @ q64[0, gi] for gi in range(Hq)])])
    got = ex.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref)), "exact scores"
    for topk in (64, 256):
        a = Q.selection_quality(q, k_c, ps, r, topk, exact=ex)
        b = O.selection_quality(H(q), H(k_c), ps, r, topk, 1 / math.sqrt(D))
        assert abs(a["recall"] - b["recall"]) <= 1.0 / topk, (topk, a, b)
        assert abs(a["mass"] - b["mass"]) <= 1e-3 and abs(a["mass_exact"] - b["mass_exact"]) <= 1e-3
