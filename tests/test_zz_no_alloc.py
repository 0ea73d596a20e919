"""The allocation-free fused decode step (rkv_hybrid_decode_step_noalloc, the library's own
per-GPU scratch in place of a workspace) against the workspace entry point rkv_hybrid_decode_step
on the same seeded inputs: channels, page scores and selected pages bit-equal, outputs within the
attention tolerance, and a sampled head against the oracle. Calls run back to back on one stream:
a 128K-shaped layer (8 KV heads, 4096 pages), then a smaller ragged shape (the scratch is cleared
for the new layout), then the first shape again twice (the second time its counters carry over)."""
import math

import pytest
import torch

from _parity import TOL_OUT, assert_rows_close
from oracle import rocketkv as O
from workloads import generate as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rkv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_kv_cache_snapkv_amd as rkv
    rkv._lib.load()
    return rkv


def _inputs(rkv, B, Hq, Hkv, Lc, D, ps, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(dtype)
    v = torch.randn((B, Hkv, Lc, D), device="cuda", generator=g).to(dtype)
    q = torch.randn((B, Hq, D), device="cuda", generator=g).to(dtype)
    kmin, kmax = rkv.rkv_build_page_summaries(k, ps)
    return q, k, v, kmin, kmax


def _outputs(q, Hkv, P, r, n_pages):
    B = q.shape[0]
    return (torch.full((B, Hkv, r), -1, dtype=torch.int32, device="cuda"),
            torch.full((B, Hkv, P), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((B, Hkv, n_pages), -1, dtype=torch.int32, device="cuda"),
            torch.full_like(q, float("nan")))


def _compare(rkv, q, k, v, kmin, kmax, ps, r, n_pages):
    B, Hq, D = q.shape
    Hkv, Lc = k.shape[1], k.shape[2]
    P = -(-Lc // ps)
    ch_n, sc_n, pg_n, out_n = _outputs(q, Hkv, P, r, n_pages)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    print(f"noalloc step B={B} Hq={Hq} Hkv={Hkv} Lc={Lc} D={D} ps={ps} n_pages={n_pages} "
          f"{q.dtype}", flush=True)
    rkv.rkv_hybrid_decode_step_noalloc(q, kmin, kmax, k, v, ps, r, n_pages, chan_idx=ch_n,
                                       page_scores=sc_n, page_idx=pg_n, out=out_n, status=status)
    ch_w, sc_w, pg_w, out_w = _outputs(q, Hkv, P, r, n_pages)
    ws = rkv.rkv_hybrid_decode_workspace(q, Hkv, Lc, ps, n_pages)
    rkv.rkv_hybrid_decode_step(q, kmin, kmax, k, v, ps, r, n_pages, chan_idx=ch_w,
                               page_scores=sc_w, page_idx=pg_w, out=out_w, workspace=ws)
    torch.cuda.synchronize()
    assert int(status.item()) & rkv.DECODE_STATUS_INVALID == 0
    assert rkv.decode_workspace_status(ws) & rkv.DECODE_STATUS_INVALID == 0
    assert torch.equal(ch_n, ch_w)
    assert torch.equal(sc_n.view(torch.int32), sc_w.view(torch.int32)), "scores differ in bits"
    assert torch.equal(pg_n, pg_w)
    dt = "bf16" if q.dtype == torch.bfloat16 else "fp32"
    got = O.widen(gen.torch_to_storage(out_n))
    assert_rows_close(got, O.widen(gen.torch_to_storage(out_w)), TOL_OUT[dt], "noalloc vs ws")
    # one head against the oracle's attention over the pages both selected
    b, h, G = B - 1, Hkv - 1, Hq // Hkv
    toks = O.page_tokens(pg_n.cpu().numpy()[b, h], ps, Lc)
    ref = O.sparse_attention(O.widen(gen.torch_to_storage(q))[b, h * G:(h + 1) * G],
                             O.widen(gen.torch_to_storage(k[b, h])),
                             O.widen(gen.torch_to_storage(v[b, h])), toks, 1 / math.sqrt(D))
    assert_rows_close(got[b, h * G:(h + 1) * G], ref, TOL_OUT[dt], "noalloc vs oracle")
    return out_n


def test_noalloc_step_matches_the_workspace_step(rkv):
    big = dict(B=1, Hq=32, Hkv=8, Lc=16384, D=128, ps=4)
    small = dict(B=1, Hq=8, Hkv=2, Lc=3001, D=64, ps=4)
    x_big = _inputs(rkv, **big, dtype=torch.bfloat16, seed=101)
    x_small = _inputs(rkv, **small, dtype=torch.bfloat16, seed=102)
    _compare(rkv, *x_big, big["ps"], 32, 128)
    _compare(rkv, *x_small, small["ps"], 16, 40)     # smaller: a new layout, cleared first
    first = _compare(rkv, *x_big, big["ps"], 32, 512)
    again = _compare(rkv, *x_big, big["ps"], 32, 512)  # same layout: counters carried over
    assert_rows_close(O.widen(gen.torch_to_storage(again)), O.widen(gen.torch_to_storage(first)),
                      TOL_OUT["bf16"], "repeated call")


def test_noalloc_step_fp32_and_one_block_per_head(rkv):
    many = dict(B=40, Hq=16, Hkv=4, Lc=2048, D=128, ps=2)   # 160 heads: no exchange area
    x = _inputs(rkv, **many, dtype=torch.float32, seed=103)
    _compare(rkv, *x, many["ps"], 32, 64)
    tiny = dict(B=2, Hq=4, Hkv=2, Lc=200, D=64, ps=4)
    x = _inputs(rkv, **tiny, dtype=torch.float32, seed=104)
    _compare(rkv, *x, tiny["ps"], 16, 20)


def test_noalloc_step_refuses_a_shape_beyond_its_scratch(rkv):
    # 128 KV heads of 8192 pages need about 10.5 MB of exchange words, more than the 8 MiB
    # scratch; the call is refused on the host and nothing runs
    B, Hq, Hkv, Lc, D = 16, 32, 8, 32768, 128
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, 64, D), dtype=torch.bfloat16, device="cuda")
    assert rkv.hybrid_decode_workspace_bytes(B, Hq, Hkv, Lc, D, 4, 256, 1) > 8 << 20
    lib = rkv._lib.load()
    p = k.data_ptr()
    st = lib.rkv_hybrid_decode_step_noalloc(q.data_ptr(), p, p, p, p, B, Hq, Hkv, Lc, D, 4, 32,
                                            256, 0.088, 1, None, None, None, q.data_ptr(), None,
                                            None)
    assert st == -7
