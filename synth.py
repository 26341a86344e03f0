"""Seeded synthetic attention inputs, shared by the tests, the smoke check and
the benchmark.

This module only draws numbers and names workloads; it holds none of the
attention arithmetic, and neither the GPU library nor the oracle imports it.

Recipe: the pages' workloads are all fp16 (or bf16) tensors filled with
standard-normal draws («ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Сравнить Hyena vs FlashAttention
на 128k», stage 2, the FlashAttention benchmark function; «Оптимизация
внимания Flash», Quick start and Workflow 1, Steps 3-4).  Here q, then k, then
v are drawn as fp32 N(0,1) from one CPU generator seeded with `seed`, then
rounded to the input type (round to nearest even; fp8 inputs are drawn the
same way and cast to float8_e4m3fn, as «Оптимизация внимания Flash»,
Workflow 3, Step 3 casts its fp16 inputs).  The same bits go to the GPU and
to the oracle.
"""
from __future__ import annotations

import dataclasses

import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f8": torch.float8_e4m3fn}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    L: int
    d: int
    dtype: str          # "f16", "bf16" or "f8" (OCP fp8 E4M3 inputs, bf16 output)
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
#   fp8_fa3_4k:   «Оптимизация внимания Flash», Workflow 3, Steps 3-4: fp16 randn
#                 inputs of [batch 2, 4096 tokens, 32 heads, head_dim 64] cast to
#                 float8_e4m3fn, default scale, no mask.
#   fa3_4k_f16:   the same shape and draws in fp16 (the page's fp16 reference).
#   fp8_causal_128k_h4: the headline shape with fp8 inputs.
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
        Workload("fp8_fa3_4k", 2, 32, 32, 4096, 64, "f8", False, -1, 0.125, 1006),
        Workload("fa3_4k_f16", 2, 32, 32, 4096, 64, "f16", False, -1, 0.125, 1006),
        Workload("fp8_causal_128k_h4", 1, 4, 4, 131072, 64, "f8", True, -1, 0.125, 1003),
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


def randn_device(shape, dtype: str, gen: torch.Generator):
    """A tensor of iid N(0,1) rounded to `dtype`, drawn on gen's device one
    index of the first dimension at a time (bounding the fp32 temporary): for
    tensors too large to draw on the host."""
    t = torch.empty(shape, dtype=TORCH_DTYPES[dtype], device=gen.device)
    for i in range(shape[0]):
        t[i] = torch.randn(tuple(shape[1:]), generator=gen, device=gen.device, dtype=torch.float32).to(t.dtype)
    return t


def make_qkv_device(B: int, H: int, H_kv: int, L: int, d: int, dtype: str, seed: int, device):
    """As make_qkv, drawn on `device` by its own seeded generator (so the
    values differ from make_qkv's for the same seed)."""
    gen = torch.Generator(device=device).manual_seed(int(seed))
    return (randn_device((B, H, L, d), dtype, gen), randn_device((B, H_kv, L, d), dtype, gen),
            randn_device((B, H_kv, L, d), dtype, gen))


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


# ---------------------------------------------------------------- decode over a paged KV cache
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Lq new queries per sequence against a paged KV cache.

    Sequence lengths are drawn uniformly from [len_min, len_max] (seeded), so
    a batch is ragged as a serving batch is; each sequence's cache is cut into
    `block_size`-token blocks placed at seeded random physical blocks of one
    pool, as PagedAttention places them («Что такое memory-efficient attention
    для long context на 8x H100?», section 3: fixed-size blocks, e.g. 16
    tokens, behind a page table)."""
    name: str
    B: int
    H: int
    H_kv: int
    d: int
    dtype: str
    Lq: int
    len_min: int
    len_max: int
    block_size: int
    window: int
    scale: float
    seed: int


#   decode_128k_gqa: the long-context case of «Что такое memory-efficient attention
#                    для long context на 8x H100?» (section 1: every generated token
#                    reads the whole KV cache): 8 sequences of 64k-128k tokens, 32
#                    query heads over 8 K/V heads, head_dim 128, bf16, 16-token blocks.
#   decode_128k_h4:  one decode step of the headline shape (causal, 4 heads, head_dim
#                    64, fp16) at 131072 tokens.
#   decode_32k_spec: 32 sequences of 8k-32k tokens, 4 new queries each (several tokens
#                    per step), GQA 32/8, head_dim 128, bf16, 32-token blocks.
#   decode_64k_swa:  sliding-window decode (window 4096, «Оптимизация внимания
#                    Flash», Workflow 2, Step 3) over 4 sequences of 32k-64k tokens.
DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("decode_128k_gqa", 8, 32, 8, 128, "bf16", 1, 65536, 131072, 16, -1, _INV_SQRT_128, 2000),
        DecodeWorkload("decode_128k_h4", 1, 4, 4, 64, "f16", 1, 131072, 131072, 16, -1, 0.125, 2001),
        DecodeWorkload("decode_32k_spec", 32, 32, 8, 128, "bf16", 4, 8192, 32768, 32, -1, _INV_SQRT_128, 2002),
        DecodeWorkload("decode_64k_swa", 4, 32, 8, 128, "bf16", 1, 32768, 65536, 16, 4096, _INV_SQRT_128, 2003),
    ]
}


def make_paged(B: int, H: int, H_kv: int, d: int, dtype: str, Lq: int, lens, block_size: int, seed: int,
               spare_blocks: int = 3):
    """Inputs of a decode step: q [B,H,Lq,d]; k_cache, v_cache
    [num_blocks, H_kv, block_size, d] of iid N(0,1) rounded to `dtype` (blocks
    no sequence uses hold draws too); block_table int32 [B, max_blocks] with
    each sequence's blocks at seeded random distinct physical blocks (unused
    entries -1); seq_lens int32 [B]."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    tdt = TORCH_DTYPES[dtype]
    lens = [int(n) for n in lens]
    per_seq = [(n + block_size - 1) // block_size for n in lens]
    num_blocks = sum(per_seq) + spare_blocks
    q = torch.randn((B, H, Lq, d), generator=gen, dtype=torch.float32).to(tdt)
    k_cache = torch.empty((num_blocks, H_kv, block_size, d), dtype=tdt)
    v_cache = torch.empty((num_blocks, H_kv, block_size, d), dtype=tdt)
    step = max(1, (1 << 24) // (H_kv * block_size * d))  # draw in bounded chunks
    for cache in (k_cache, v_cache):
        for s in range(0, num_blocks, step):
            e = min(num_blocks, s + step)
            cache[s:e] = torch.randn((e - s, H_kv, block_size, d), generator=gen, dtype=torch.float32).to(tdt)
    perm = torch.randperm(num_blocks, generator=gen)
    width = max(per_seq)
    table = torch.full((B, width), -1, dtype=torch.int32)
    used = 0
    for b, nb in enumerate(per_seq):
        table[b, :nb] = perm[used:used + nb].to(torch.int32)
        used += nb
    return q, k_cache, v_cache, table, torch.tensor(lens, dtype=torch.int32)


def decode_lens(w: DecodeWorkload):
    """The workload's seeded sequence lengths (each >= Lq)."""
    gen = torch.Generator(device="cpu").manual_seed(int(w.seed) + 1)
    if w.len_min == w.len_max:
        return [w.len_max] * w.B
    return torch.randint(w.len_min, w.len_max + 1, (w.B,), generator=gen).tolist()


def decode_inputs(w: DecodeWorkload):
    return make_paged(w.B, w.H, w.H_kv, w.d, w.dtype, w.Lq, decode_lens(w), w.block_size, w.seed)
