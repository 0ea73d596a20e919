"""CPU checks of the C ABI: the library loads, exports every function include/rkv.h declares,
and rejects bad arguments on the host before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

from sparse_kv_cache_snapkv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("librkv.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("rkv_snapkvpp_evict", "rkv_build_page_summaries", "rkv_hybrid_approx_scores",
              "rkv_topk_select", "rkv_sparse_attend_decode"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES), "binding and header disagree"


def _prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(?:int|const char\*)\s+(rkv_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        args = [a.strip() for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        protos[m.group(1)] = args
    return protos


def test_binding_argument_types_match_header():
    protos = _prototypes()
    assert set(protos) == set(_lib.SIGNATURES)
    kinds = {ctypes.c_int: "int", ctypes.c_float: "float", ctypes.c_size_t: "size_t"}
    for name, args in protos.items():
        _, argtypes = _lib.SIGNATURES[name]
        assert len(args) == len(argtypes), (name, len(args), len(argtypes))
        for decl, ct in zip(args, argtypes):
            if "*" in decl:
                assert ct in (ctypes.c_void_p,) or hasattr(ct, "_type_"), (name, decl, ct)
            else:
                base = decl.rsplit(" ", 1)[0]
                assert kinds.get(ct) == base, (name, decl, ct)


def test_version_and_status_strings(lib):
    assert lib.rkv_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        s = lib.rkv_status_string(code)
        assert isinstance(s, bytes) and len(s) > 3


def _sz(lib, fn, *args):
    out = ctypes.c_size_t(12345)
    st = getattr(lib, fn)(*args, ctypes.byref(out))
    return st, out.value


def test_workspace_queries(lib):
    st, n = _sz(lib, "rkv_snapkvpp_workspace_bytes", 1, 32, 8, 131072, 128, 32, 16384, 1)
    assert st == 0 and n > 8 * 131040 * 4  # holds at least the column sums
    st, n = _sz(lib, "rkv_snapkvpp_workspace_bytes", 1, 32, 8, 1000, 128, 32, 2000, 1)
    assert st == 0 and n == 0                # nothing to score when keep >= L
    assert _sz(lib, "rkv_snapkvpp_workspace_bytes", 1, 32, 7, 1000, 128, 32, 200, 1)[0] == -2
    assert _sz(lib, "rkv_snapkvpp_workspace_bytes", 1, 32, 8, 1000, 96, 32, 200, 1)[0] == -5
    assert _sz(lib, "rkv_snapkvpp_workspace_bytes", 1, 32, 8, 1000, 128, 32, 200, 7)[0] == -3
    assert _sz(lib, "rkv_topk_workspace_bytes", 8, 4096, 32) == (0, 0)
    st, n = _sz(lib, "rkv_sparse_attend_workspace_bytes", 1, 32, 8, 128, 4, 1, 1)
    assert st == 0 and n == 0                # one page per head fits one block: no merge
    st, n = _sz(lib, "rkv_sparse_attend_workspace_bytes", 1, 32, 8, 128, 4, 512, 1)
    assert st == 0 and n > 0
    assert lib.rkv_topk_workspace_bytes(8, 4096, 32, None) == -1
    st, n = _sz(lib, "rkv_hybrid_decode_workspace_bytes", 1, 32, 8, 16384, 128, 4, 512, 1)
    assert st == 0 and n >= 8 * 4096 * 4     # holds the page scores
    assert _sz(lib, "rkv_hybrid_decode_workspace_bytes", 1, 32, 8, 65536, 128, 4, 512, 1)[0] == -5
    assert _sz(lib, "rkv_hybrid_decode_workspace_bytes", 1, 32, 8, 16384, 128, 4, 4097, 1)[0] == -2
    assert lib.rkv_hybrid_decode_workspace_init(None, 1024, None) == -1


FAKE = 0x10000  # a non-NULL, 16-byte aligned address that is never dereferenced


def test_evict_rejects_bad_arguments(lib):
    ev = lib.rkv_snapkvpp_evict
    ok = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=4, Hkv=2, L=2048, D=64, W=16, keep=512, p=7, pt=0,
              scale=0.125, dt=0, kept=FAKE, ko=FAKE, vo=FAKE, pooled=None, ws=FAKE,
              wsb=1 << 30, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return ev(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["D"], a["W"],
                  a["keep"], a["p"], a["pt"], a["scale"], a["dt"], a["kept"], a["ko"], a["vo"],
                  a["pooled"], a["ws"], a["wsb"], a["stream"])

    assert call(q=None) == -1
    assert call(kept=None) == -1
    assert call(ko=None) == -1                      # k_out and v_out come together
    assert call(dt=3) == -3
    assert call(Hkv=3) == -2                        # Hq not a multiple of Hkv
    assert call(W=0) == -2
    assert call(keep=8) == -2                       # keep below the window
    assert call(p=4) == -2                          # even pooling kernel
    assert call(pt=2) == -2
    assert call(scale=0.0) == -2
    assert call(scale=float("nan")) == -2
    assert call(D=96) == -5
    assert call(p=129) == -5
    assert call(k=FAKE + 4) == -2                   # misaligned
    assert call(ws=None) == -4
    assert call(wsb=16) == -4


def test_decode_calls_reject_bad_arguments(lib):
    att = lib.rkv_sparse_attend_decode
    base = [FAKE, FAKE, FAKE, FAKE, 1, 32, 8, 16384, 128, 4, 32, 0.088, 1, FAKE, None, 0, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return att(*a)

    assert call(0, None) == -1
    assert call(10, 4097) == -2                     # more pages than the cache has
    assert call(10, 0) == -2
    assert call(5, 33) == -2
    assert call(8, 256) == -5
    assert call(5, 8 * 9) == -5                     # group of 9 query heads
    assert call(12, 2) == -3
    assert call(11, float("inf")) == -2
    # a split plan needs a workspace
    a = list(base)
    a[10] = 512
    assert att(*a) == -4
    ap = lib.rkv_hybrid_approx_scores
    assert ap(FAKE, FAKE, FAKE, 1, 32, 8, 128, 4096, 0, 1, None, FAKE, None) == -2    # r = 0
    assert ap(FAKE, FAKE, FAKE, 1, 32, 8, 128, 4096, 129, 1, None, FAKE, None) == -2  # r > D
    assert ap(FAKE, FAKE, FAKE, 1, 32, 8, 128, 4096, 32, 1, None, None, None) == -1
    ps = lib.rkv_build_page_summaries
    assert ps(FAKE, 1, 8, 16384, 128, 0, 1, FAKE, FAKE, None) == -2
    assert ps(FAKE, 1, 8, 16384, 100, 4, 1, FAKE, FAKE, None) == -5
    tk = lib.rkv_topk_select
    assert tk(FAKE, 0, 10, 3, FAKE, None, 0, None) == -2
    assert tk(FAKE, 1, 10, -1, FAKE, None, 0, None) == -2
    assert tk(None, 1, 10, 3, FAKE, None, 0, None) == -1


def test_decode_status_and_scratch_step_reject_bad_arguments(lib):
    st = ctypes.c_uint32(7)
    assert lib.rkv_hybrid_decode_status(None, 4096, 0, ctypes.byref(st), None) == -1
    assert lib.rkv_hybrid_decode_status(FAKE, 4096, 0, None, None) == -1
    assert lib.rkv_hybrid_decode_status(FAKE, 16, 0, ctypes.byref(st), None) == -4
    assert st.value == 7
    na = lib.rkv_hybrid_decode_step_noalloc
    # q kmin kmax k v, B Hq Hkv Lc D ps r n_pages, scale dtype, chan scores pages out status stream
    base = [FAKE] * 5 + [1, 32, 8, 16384, 128, 4, 32, 128, 0.088, 1, None, None, None, FAKE,
                         None, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return na(*a)

    assert call(a0=None) == -1
    assert call(a18=None) == -1                     # out
    assert call(a12=4097) == -2                     # more pages than the cache has
    assert call(a14=5) == -3
    assert call(a9=96) == -5
    assert call(a19=FAKE + 4) == -2                 # misaligned status word
    # 16 x 8 = 128 KV heads of 8192 pages need more than the fixed scratch: refused before any
    # HIP call
    assert call(a5=16, a8=32768, a12=256) == -7
    assert lib.rkv_status_string(-7).startswith(b"the shape needs more")
    assert _sz(lib, "rkv_hybrid_decode_workspace_bytes", 16, 32, 8, 32768, 128, 4, 256, 1)[1] \
        > 8 << 20


def test_plan_budget_matches_the_oracle(lib):
    # a host-only call: the library's planner equals the oracle's over a grid of shapes
    from oracle import rocketkv as O
    from sparse_kv_cache_snapkv_amd import rkv_plan_budget
    for L in (1, 7, 100, 2048, 5000, 32768, 131072, 262144):
        for D in (64, 128):
            for budget in (1, 16, 128, 256, 512, 1000, 4096, 300000):
                W = min(32, L)
                assert rkv_plan_budget(L, D, W, budget) == O.plan_budget(L, D, W, budget), \
                    (L, D, budget)
    outs = [ctypes.c_int(-7) for _ in range(6)]
    assert lib.rkv_plan_budget(100, 64, 101, 10, *[ctypes.byref(o) for o in outs]) == -2
    assert all(o.value == -7 for o in outs)  # nothing written on error


def test_binding_refuses_misshaped_buffers():
    # the kernels index every buffer by the sizes a call passes: a tensor of another shape is
    # refused before any pointer reaches the library (checked with host tensors: no GPU call)
    import torch
    import sparse_kv_cache_snapkv_amd as rkv
    bf = torch.bfloat16
    q = torch.zeros((1, 4, 64), dtype=bf)
    k_c = torch.zeros((1, 2, 40, 64), dtype=bf)
    kmin = torch.zeros((1, 2, 64, 10), dtype=bf)
    with pytest.raises(ValueError, match="out"):
        rkv.rkv_hybrid_decode_step(q, kmin, kmin, k_c, k_c, 4, 16, 4,
                                   out=torch.zeros((1, 4, 32), dtype=bf))
    with pytest.raises(ValueError, match="page_idx"):
        rkv.rkv_hybrid_decode_step(q, kmin, kmin, k_c, k_c, 4, 16, 4,
                                   page_idx=torch.zeros((1, 2, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="kmin_t"):
        rkv.rkv_hybrid_decode_step(q, kmin[..., :9], kmin, k_c, k_c, 4, 16, 4)
    with pytest.raises(ValueError, match="page_scores"):
        rkv.rkv_hybrid_approx_scores(q, kmin, kmin, 16, page_scores=torch.zeros((1, 2, 9)))
    with pytest.raises(ValueError, match="idx_out"):
        rkv.rkv_topk_select(torch.zeros((2, 100)), 5, idx_out=torch.zeros((2, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="kept_idx"):
        rkv.rkv_snapkvpp_evict(torch.zeros((1, 4, 8, 64), dtype=bf), k_c, k_c, 16, 3,
                               kept_idx=torch.zeros((1, 2, 15), dtype=torch.int32))
    with pytest.raises(ValueError, match="v_c"):
        rkv.rkv_sparse_attend_decode(q, k_c, k_c[:, :, :20].contiguous(),
                                     torch.zeros((1, 2, 4), dtype=torch.int32), 4)
