"""Synthetic workload shapes for RocketKV's hot path.

Five named workloads (tiny fp32, Llama3.1-8B-shaped at 32K and 128K, a batch-16 8B decode, and a
70B-shaped 80-layer GQA stack at 256K), plus small ragged shapes that the CPU oracle finishes in
seconds. Shapes only: no arithmetic of the method lives here.

The page size (4), the top-32-of-128 channel reduction and the 256-token budget follow the
RocketKV rebuttal page (paperhub.cn), sections "Is Page Always Divided Into 4?" and "Lack of
Direct Latency Comparison"; the model shapes are Llama3.1-8B (32 query / 8 KV heads) and a
70B-class GQA layer (64 / 8), the models the pages evaluate on.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # batch (independent sequences)
    Hq: int           # query heads
    Hkv: int          # KV heads; query head g uses KV head g // (Hq // Hkv)
    D: int            # head dim
    L: int            # prompt (context) length before eviction
    W: int            # SnapKV++ observation window (last W prompt positions)
    pool_kernel: int  # 1D pooling kernel size (odd)
    keep: int         # tokens kept per KV head, window included
    page_size: int    # tokens per page of the compressed cache
    r: int            # channels kept by the head-dim reduction
    topk: Tuple[int, ...]  # decode token budgets for exact attention (multiples of page_size)
    dtype: str        # "fp32" or "bf16"
    steps: int        # decode steps (fresh random q each)
    layers: int       # independent layers (folded into the batch axis on the GPU)
    n_needles: int    # planted needle keys per (layer, b, KV head)
    seed: int = 0
    cfg_id: int = 0   # sub-seed namespace

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def Lc(self) -> int:
        return min(self.keep, self.L)

    @property
    def P(self) -> int:
        return -(-self.Lc // self.page_size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY_FP32 = Workload("tiny-fp32-L2048", B=1, Hq=4, Hkv=2, D=64, L=2048, W=16, pool_kernel=7,
                     keep=512, page_size=4, r=16, topk=(128,), dtype="fp32", steps=8, layers=1,
                     n_needles=4, cfg_id=0)
LLAMA8B_32K = Workload("llama8b-L32768-bf16", B=1, Hq=32, Hkv=8, D=128, L=32768, W=32,
                       pool_kernel=31, keep=4096, page_size=4, r=32, topk=(128,), dtype="bf16",
                       steps=128, layers=1, n_needles=64, cfg_id=1)
LLAMA8B_128K = Workload("llama8b-L131072-bf16", B=1, Hq=32, Hkv=8, D=128, L=131072, W=32,
                        pool_kernel=63, keep=16384, page_size=4, r=32, topk=(128, 512, 2048),
                        dtype="bf16", steps=256, layers=1, n_needles=64, cfg_id=2)
# Window and pool kernel are not stated for the batched workload; the 32K ones are reused.
LLAMA8B_32K_B16 = Workload("llama8b-L32768-b16-bf16", B=16, Hq=32, Hkv=8, D=128, L=32768, W=32,
                           pool_kernel=31, keep=4096, page_size=4, r=32, topk=(256,),
                           dtype="bf16", steps=64, layers=1, n_needles=64, cfg_id=3)
LLAMA70B_256K_80L = Workload("llama70b-L262144-80layer-bf16", B=1, Hq=64, Hkv=8, D=128, L=262144,
                             W=64, pool_kernel=63, keep=32768, page_size=4, r=32, topk=(1024,),
                             dtype="bf16", steps=16, layers=80, n_needles=64, cfg_id=4)

NAMED = (TINY_FP32, LLAMA8B_32K, LLAMA8B_128K, LLAMA8B_32K_B16, LLAMA70B_256K_80L)

# Small shapes for oracle-vs-GPU parity: several tiles and a ragged tail each.
SMALL = (
    TINY_FP32,
    Workload("small-bf16-ragged", B=2, Hq=8, Hkv=2, D=128, L=3001, W=32, pool_kernel=31,
             keep=702, page_size=4, r=32, topk=(64, 256), dtype="bf16", steps=3, layers=1,
             n_needles=8, cfg_id=10),
    Workload("small-fp32-d128-ragged", B=1, Hq=6, Hkv=2, D=128, L=1531, W=24, pool_kernel=9,
             keep=333, page_size=4, r=24, topk=(40, 400), dtype="fp32", steps=2, layers=1,
             n_needles=4, cfg_id=11),
    Workload("small-bf16-d64-g8", B=1, Hq=16, Hkv=2, D=64, L=2500, W=64, pool_kernel=15,
             keep=640, page_size=8, r=16, topk=(96,), dtype="bf16", steps=2, layers=1,
             n_needles=4, cfg_id=12),
    Workload("small-bf16-g1-ps1", B=1, Hq=3, Hkv=3, D=64, L=777, W=8, pool_kernel=1,
             keep=129, page_size=1, r=64, topk=(17,), dtype="bf16", steps=2, layers=1,
             n_needles=2, cfg_id=13),
)


def by_name(name: str) -> Workload:
    for w in NAMED + SMALL:
        if w.name == name:
            return w
    raise KeyError(name)
