"""Seeded synthetic attention inputs, shared by the tests, the smoke check and
the benchmark.

This module only draws numbers and names workloads; it holds none of the
attention arithmetic, and neither the GPU library nor the oracle imports it.

Recipe: the pages' workloads are all fp16 (or bf16) tensors filled with
standard-normal draws («ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Сравнить Hyena vs FlashAttention
на 128k», stage 2, the FlashAttention benchmark function; «Оптимизация
внимания Flash», Quick start and Workflow 1, Steps 3-4).  Here q, then k, then
v are drawn as fp32 N(0,1) from one CPU generator seeded with `seed`, then
rounded to the 16-bit type (round to nearest even).  The same bits go to the
GPU and to the oracle.
"""
from __future__ import annotations

import dataclasses

import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    L: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    window: int         # -1: no window; else keys at most `window` before (and, non-causal, after)
    scale: float        # the fp32 softmax scale passed to the library
    seed: int
    note: str = ""

    def key(self) -> str:
        return self.name


# The workloads the pages measure (sizes, masks and dtypes), by name.
#   causal_4k:    stage 1 of «ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Сравнить Hyena vs FlashAttention на
#                 128k»: batch 1, head_dim 64, 4 heads, causal, fp16; shortest length.
#   noncausal_2k: «Оптимизация внимания Flash», Workflow 1, Step 3 (speed check):
#                 batch 2, 8 heads, 2048 tokens, head_dim 64, scale 1/8, no mask.
#   causal_sweep: the same technical assignment's length list, 8k ... 64k.
#   causal_128k:  its longest length, 131072, at 4 heads (the headline) and 8 heads.
#   swa_gqa_16k:  «Оптимизация внимания Flash», Workflow 2, Step 3: fewer K/V heads
#                 plus a causal sliding window; here 32 query heads over 8 K/V heads,
#                 head_dim 128, bf16, window 4096 keys back.
#   p2_accuracy:  «Оптимизация внимания Flash», Workflow 1, Step 4 (accuracy check):
#                 batch 1, 8 heads, 512 tokens, head_dim 64, scale 1/8, no mask,
#                 fp16, max difference below 1e-3.
_INV_SQRT_128 = float(torch.tensor(1.0 / 128 ** 0.5, dtype=torch.float32))

WORKLOADS = {
    w.name: w for w in [
        Workload("causal_4k", 1, 4, 4, 4096, 64, "f16", True, -1, 0.125, 1000),
        Workload("noncausal_2k_f16", 2, 8, 8, 2048, 64, "f16", False, -1, 0.125, 1001),
        Workload("noncausal_2k_bf16", 2, 8, 8, 2048, 64, "bf16", False, -1, 0.125, 1001),
        Workload("causal_8k", 1, 4, 4, 8192, 64, "f16", True, -1, 0.125, 1002),
        Workload("causal_16k", 1, 4, 4, 16384, 64, "f16", True, -1, 0.125, 1002),
        Workload("causal_32k", 1, 4, 4, 32768, 64, "f16", True, -1, 0.125, 1002),
        Workload("causal_64k", 1, 4, 4, 65536, 64, "f16", True, -1, 0.125, 1002),
        Workload("causal_128k_h4", 1, 4, 4, 131072, 64, "f16", True, -1, 0.125, 1003),
        Workload("causal_128k_h8", 1, 8, 8, 131072, 64, "f16", True, -1, 0.125, 1003),
        Workload("swa_gqa_16k", 1, 32, 8, 16384, 128, "bf16", True, 4096, _INV_SQRT_128, 1004),
        Workload("p2_accuracy", 1, 8, 8, 512, 64, "f16", False, -1, 0.125, 1005),
    ]
}


def make_qkv(B: int, H: int, H_kv: int, L: int, d: int, dtype: str, seed: int):
    """q [B,H,L,d], k and v [B,H_kv,L,d]: CPU tensors of iid N(0,1) rounded to `dtype`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    tdt = TORCH_DTYPES[dtype]
    q = torch.randn((B, H, L, d), generator=gen, dtype=torch.float32).to(tdt)
    k = torch.randn((B, H_kv, L, d), generator=gen, dtype=torch.float32).to(tdt)
    v = torch.randn((B, H_kv, L, d), generator=gen, dtype=torch.float32).to(tdt)
    return q, k, v


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.H, w.H_kv, w.L, w.d, w.dtype, w.seed)


def sample_rows(B: int, H: int, L: int, n_random: int, seed: int, tile: int = 64):
    """Flat row ids (b*H + h)*L + i to check at sizes the oracle cannot do whole.

    Per (b, h): the first and last 64 rows, rows on both sides of every
    `tile`-th boundary among the first and last 16 boundaries, and `n_random`
    seeded random rows.  Returned sorted and unique.
    """
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    picks = set()
    edge = min(L, 64)
    for i in list(range(edge)) + list(range(L - edge, L)):
        picks.add(i)
    boundaries = list(range(tile, L, tile))
    for bnd in boundaries[:16] + boundaries[-16:]:
        for i in (bnd - 1, bnd):
            if 0 <= i < L:
                picks.add(i)
    base = sorted(picks)
    out = []
    for bh in range(B * H):
        rnd = torch.randint(0, L, (n_random,), generator=gen).tolist() if n_random else []
        for i in sorted(set(base) | set(rnd)):
            out.append(bh * L + i)
    return out
