"""End-to-end GPU parity: SnapKV++ eviction -> page summaries -> decode steps (approximate
scores, page top-k, sparse attention), against the oracle run on the same seeded inputs.

Small workloads are checked on every head; the full-size workloads run on the GPU at their real
shapes and launch configuration, and the oracle checks sampled (layer, sequence, KV head) slots.
Where a selection differs from the oracle's only at a score tie (within 1e-5 relative), the
downstream GPU result is checked against the oracle applied to the GPU's own valid selection.
"""
import math

import numpy as np
import pytest
import torch

from _parity import TOL_OUT, assert_rows_close, selection_matches
from oracle import rocketkv as O
from workloads import configs, generate as gen, runs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rkv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_kv_cache_snapkv_amd as rkv
    rkv._lib.load()
    return rkv


def _decode_gpu(rkv, w, q, k_c, v_c, kmin, kmax, topk, fused=False):
    """The three calls; with fused, also the fused step on the same inputs, whose channels,
    scores and pages must equal the three calls' bit for bit (its output is returned too)."""
    scores, chans = rkv.rkv_hybrid_approx_scores(q, kmin, kmax, w.r, return_channels=True)
    n_pages = min(topk // w.page_size, w.P)
    pages = rkv.rkv_topk_select(scores, n_pages)
    out = rkv.rkv_sparse_attend_decode(q, k_c, v_c, pages, w.page_size)
    res = dict(scores=scores.cpu().numpy(), chans=chans.cpu().numpy(),
               pages=pages.cpu().numpy(), out=gen.torch_to_storage(out))
    if fused:
        B, Hkv = k_c.shape[:2]
        fc = torch.empty_like(chans)
        fs = torch.empty_like(scores)
        fp = torch.empty_like(pages)
        ws = rkv.rkv_hybrid_decode_workspace(q, Hkv, k_c.shape[2], w.page_size, n_pages)
        fo = rkv.rkv_hybrid_decode_step(q, kmin, kmax, k_c, v_c, w.page_size, w.r, n_pages,
                                        chan_idx=fc, page_scores=fs, page_idx=fp, workspace=ws)
        assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0
        assert torch.equal(fc, chans), "fused step channels"
        assert torch.equal(fs.view(torch.int32), scores.view(torch.int32)), "fused step scores"
        assert torch.equal(fp, pages), "fused step pages"
        res["fused_out"] = gen.torch_to_storage(fo)
        del ws
    return res


def check_head(w, kept_gpu, pooled_ref, k_head, v_head, kmin_gpu, kmax_gpu, steps):
    """One (layer, b, KV head). kept_gpu [Lc]; pooled_ref [L-W] oracle scores (None if keep>=L);
    k_head/v_head [L, D] float64 inputs; kmin/kmax_gpu [D, P] float64; steps: list of
    (qg [G,D] float64, topk, gpu dict sliced to this head). Returns counts of exact matches."""
    stats = dict(kept_exact=1, pages_exact=0, pages_total=0)
    if pooled_ref is not None:
        ok = selection_matches(kept_gpu[:w.keep - w.W], pooled_ref, w.keep - w.W)
        stats["kept_exact"] = int(ok)
        assert list(kept_gpu[w.keep - w.W:]) == list(range(w.L - w.W, w.L))
    # the compressed cache the GPU holds: generator rows at its (valid) kept positions; equal to
    # the oracle's own cache whenever the kept sets are equal
    kc, vc = k_head[kept_gpu], v_head[kept_gpu]
    omin, omax = O.page_summaries(kc, w.page_size)
    assert np.array_equal(kmin_gpu, omin) and np.array_equal(kmax_gpu, omax), "summaries"
    scale = 1.0 / math.sqrt(w.D)
    for qg, topk, g in steps:
        chans_o, qbar = O.select_channels(qg, w.r)
        selection_matches(g["chans"], np.abs(qg).sum(0), w.r)
        scores_o = O.approx_page_scores(qbar, g["chans"].astype(np.int64), omin, omax)
        assert_rows_close(g["scores"], scores_o, 1e-5, "page scores")
        n_pages = min(topk // w.page_size, w.P)
        stats["pages_total"] += 1
        stats["pages_exact"] += int(selection_matches(g["pages"], scores_o, n_pages))
        toks = O.page_tokens(g["pages"].astype(np.int64), w.page_size, w.Lc)
        ref = O.sparse_attention(qg, kc, vc, toks, scale)
        assert_rows_close(O.widen(g["out"]), ref, TOL_OUT[w.dtype], "attention output")
        if "fused_out" in g:
            assert_rows_close(O.widen(g["fused_out"]), ref, TOL_OUT[w.dtype], "fused step output")
    return stats


@pytest.mark.parametrize("w", configs.SMALL, ids=lambda w: w.name)
def test_pipeline_small(rkv, w):
    d = gen.prompt_layer(w)
    qs = gen.decode_queries(w)
    scale = 1.0 / math.sqrt(w.D)
    T = lambda x: gen.storage_to_torch(x, "cuda")  # noqa: E731
    kept, k_c, v_c = rkv.rkv_snapkvpp_evict(T(d["q_win"]), T(d["k"]), T(d["v"]), w.keep,
                                            w.pool_kernel, "avg", scale)
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, w.page_size)
    gpu_steps = [(s, tk, _decode_gpu(rkv, w, T(qs[s]), k_c, v_c, kmin, kmax, tk))
                 for s in range(qs.shape[0]) for tk in w.topk]
    ref = O.snapkvpp_evict(d["q_win"], d["k"], d["v"], w.keep, w.pool_kernel, scale)
    kept = kept.cpu().numpy().astype(np.int64)
    kmin64, kmax64 = O.widen(gen.torch_to_storage(kmin)), O.widen(gen.torch_to_storage(kmax))
    k64, v64, q64 = O.widen(d["k"]), O.widen(d["v"]), O.widen(qs)
    G = w.G
    for b in range(w.B):
        for h in range(w.Hkv):
            steps = [(q64[s, b, h * G:(h + 1) * G], tk,
                      dict(chans=g["chans"][b, h], scores=g["scores"][b, h], pages=g["pages"][b, h],
                           out=g["out"][b, h * G:(h + 1) * G])) for s, tk, g in gpu_steps]
            check_head(w, kept[b, h], ref["pooled"][b, h] if w.keep < w.L else None, k64[b, h],
                       v64[b, h], kmin64[b, h], kmax64[b, h], steps)


FULL = [
    (configs.LLAMA8B_32K, 1, [(0, 0, 0), (0, 0, 7)]),
    (configs.LLAMA8B_128K, 1, [(0, 0, 3)]),
    (configs.LLAMA8B_32K_B16, 1, [(0, 5, 1), (0, 15, 6)]),
    (configs.LLAMA70B_256K_80L, 80, [(0, 0, 0), (79, 0, 5)]),
]


@pytest.mark.parametrize("w,layers,sample", FULL, ids=[f[0].name for f in FULL])
def test_pipeline_full_size_sampled(rkv, w, layers, sample):
    torch.cuda.empty_cache()
    st = runs.compressed_stack(rkv, w, layers, sample=sample)
    assert st["needles_ok"], "a planted needle was evicted"
    k_c, v_c = st["k_c"], st["v_c"]
    kmin, kmax = rkv.rkv_build_page_summaries(k_c, w.page_size)
    wl = w.replace(B=layers * w.B)
    steps = 2
    qs = gen.device_decode_queries(wl, 0, steps)
    # the fused step (the kernel the benchmark times) runs at the workload's own shape and plan
    gpu_steps = [(s, tk, _decode_gpu(rkv, wl, qs[s], k_c, v_c, kmin, kmax, tk, fused=True))
                 for s in range(steps) for tk in w.topk]
    kept = st["kept"]
    G = w.G
    scale = 1.0 / math.sqrt(w.D)
    for (layer, b, h), hd in st["host"].items():
        bb = layer * w.B + b
        kept_g, _, pooled_ref = O.snapkvpp_head(O.widen(hd["q_win"]), O.widen(hd["k"]), w.keep,
                                                w.pool_kernel, scale)
        q64 = O.widen(gen.torch_to_storage(qs[:, bb, h * G:(h + 1) * G]))
        hs = [(q64[s], tk, dict(chans=g["chans"][bb, h], scores=g["scores"][bb, h],
                                pages=g["pages"][bb, h], out=g["out"][bb, h * G:(h + 1) * G],
                                fused_out=g["fused_out"][bb, h * G:(h + 1) * G]))
              for s, tk, g in gpu_steps]
        k_slot = kept[bb, h].cpu().numpy().astype(np.int64)
        check_head(w, k_slot, pooled_ref, O.widen(hd["k"]), O.widen(hd["v"]),
                   O.widen(gen.torch_to_storage(kmin[bb, h])),
                   O.widen(gen.torch_to_storage(kmax[bb, h])), hs)
        assert set(hd["needle_pos"].tolist()) <= set(k_slot.tolist())
        del kept_g
    del st, k_c, v_c, kmin, kmax
    torch.cuda.empty_cache()
