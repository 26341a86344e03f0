"""GPU parity beyond 2^31 elements per tensor (4.4 GB per 16-bit tensor).

Every kernel addresses global memory with 64-bit offsets; these cases put
the checked heads (and KV-cache blocks) on both sides of element 2^31 of
their tensors, at the forward's own L = 65536, d = 64, causal:

* forward fp16, backward fp16 and forward fp8 over B=2, H=260 (2.18e9
  elements per tensor; flat head 511 ends at element 2^31 exactly, head 512
  starts there);
* paged decode over a pool of 140000 blocks (8 K/V heads x 16 tokens x 128,
  bf16: 2.29e9 elements per cache), with one sequence's blocks taken from
  above block 131072 (element 2^31) and the other's from both sides.

Inputs are drawn on the GPU (seeded; N(0,1) rounded to the input type, as
everywhere else); only the heads or blocks under test are copied back, so the
oracle sees exactly the bits the kernel saw.  Bounds: the same as the
smaller cases (the forward's fp16 bars, the backward's derived bound, the
fp8 bound, the forward's bf16 bars for decode).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_25_amd as attn
import oracle
from oracle import paged
from synth import make_qkv_device, randn_device, sample_rows
from test_gpu_backward import check_all
from test_gpu_fp8 import check_fp8, fp8_bound_inputs
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
B, H, L, D = 2, 260, 65536, 64
SCALE = 0.125
HEADS = [0, 511, 512, B * H - 1]  # flat b*H + h


@pytest.fixture(scope="module")
def big16():
    announce(f"large inputs: B={B} H={H} L={L} d={D} f16 ({B * H * L * D / 2 ** 31:.3f} x 2^31 elements each)")
    q, k, v = make_qkv_device(B, H, H, L, D, "f16", 9100, DEV)
    out, lse = attn.forward(q, k, v, causal=True, scale=SCALE)
    torch.cuda.synchronize(DEV)
    yield q, k, v, out, lse
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def head(t, bh):
    b, h = divmod(bh, H)
    return t[b:b + 1, h:h + 1].cpu()


def test_forward_beyond_2_31(big16):
    q, k, v, out, lse = big16
    for bh in HEADS:
        case = f"large forward, head {bh} (elements {bh * L * D / 2 ** 31:.3f}..{(bh + 1) * L * D / 2 ** 31:.3f} x 2^31)"
        announce(case)
        rows = sample_rows(1, 1, L, 24, seed=bh)
        ref_o, ref_l = oracle.attention(head(q, bh), head(k, bh), head(v, bh), "f16", True, -1, SCALE, rows=rows)
        check(head(out, bh).reshape(-1, D)[rows], head(lse, bh).reshape(-1)[rows], (ref_o, ref_l), "f16", case)


def test_backward_beyond_2_31(big16):
    q, k, v, out, lse = big16
    announce("large backward")
    gen = torch.Generator(device=DEV).manual_seed(9101)
    dout = randn_device((B, H, L, D), "f16", gen)
    ws = torch.empty(attn.attn_bwd_workspace_size(B, H, L), dtype=torch.uint8, device=DEV)
    dq, dk, dv = attn.backward(q, k, v, out, lse, dout, causal=True, scale=SCALE, workspace=ws)
    torch.cuda.synchronize(DEV)
    for bh in HEADS:
        case = f"large backward, head {bh}"
        announce(case)
        rows = sample_rows(1, 1, L, 8, seed=bh)
        # keys near the end: a causal key's gradient needs every row after it
        keys = [L - 1, L - 2, L - 31, L - 32, L - 33, L - 64, L - 65, L - 128, L - 129, L - 200]
        ref = oracle.attention_bwd(head(q, bh), head(k, bh), head(v, bh), head(dout, bh), "f16", True, -1, SCALE,
                                   q_rows=rows, kv_rows=keys, with_abs=True)
        res = {"dq": head(dq, bh), "dk": head(dk, bh), "dv": head(dv, bh)}
        check_all(res, ref, "f16", L, case, q_rows=rows, kv_rows=keys)
    del dout, ws, dq, dk, dv
    torch.cuda.empty_cache()


def test_fp8_forward_beyond_2_31():
    announce("large fp8 forward")
    q, k, v = make_qkv_device(B, H, H, L, D, "f8", 9102, DEV)
    out, lse = attn.forward(q, k, v, causal=True, scale=SCALE)
    torch.cuda.synchronize(DEV)
    for bh in HEADS:
        case = f"large fp8 forward, head {bh}"
        announce(case)
        rows = sample_rows(1, 1, L, 16, seed=bh)
        ref_o, ref_l, r, se = fp8_bound_inputs(head(q, bh), head(k, bh), head(v, bh), True, -1, SCALE, rows=rows)
        check_fp8(head(out, bh).reshape(-1, D)[rows], head(lse, bh).reshape(-1)[rows], ref_o, ref_l, r, case, se)
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_decode_cache_beyond_2_31():
    nb, hk, bs, d, hq = 140000, 8, 16, 128, 32
    high = 2 ** 31 // (hk * bs * d)  # first block at element 2^31
    announce(f"large decode: pool of {nb} blocks ({nb * hk * bs * d / 2 ** 31:.3f} x 2^31 elements per cache)")
    gen = torch.Generator(device=DEV).manual_seed(9103)
    kc = randn_device((nb, hk, bs, d), "bf16", gen)
    vc = randn_device((nb, hk, bs, d), "bf16", gen)
    q = randn_device((2, hq, 1, d), "bf16", gen)
    lens = [5000, 3001]
    per = [(n + bs - 1) // bs for n in lens]
    pick = torch.Generator().manual_seed(9104)
    above = high + torch.randperm(nb - high, generator=pick)  # every block past element 2^31, shuffled
    n_hi = per[1] - per[1] // 2
    seq1 = torch.cat([torch.randperm(high, generator=pick)[:per[1] // 2], above[per[0]:per[0] + n_hi]])
    table = torch.full((2, max(per)), -1, dtype=torch.int32)
    table[0, :per[0]] = above[:per[0]].to(torch.int32)
    table[1, :per[1]] = seq1[torch.randperm(per[1], generator=pick)].to(torch.int32)
    assert int(table.max()) < nb and (table[0, :per[0]] >= high).all() and (table[1, :per[1]] >= high).any()
    out, lse = attn.decode(q, kc, vc, table.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens))
    torch.cuda.synchronize(DEV)
    # the oracle gets only the blocks in use, renumbered
    used = torch.unique(table[table >= 0]).long()
    remap = torch.full((nb,), -1, dtype=torch.int32)
    remap[used] = torch.arange(used.numel(), dtype=torch.int32)
    small = torch.where(table >= 0, remap[table.clamp(min=0).long()], table)
    idx = used.to(DEV)
    ref_o, ref_l = paged.decode_attention(q.cpu(), kc[idx].cpu(), vc[idx].cpu(), small, lens, "bf16")
    check(out.cpu(), lse.cpu(), (ref_o, ref_l), "bf16", "large decode")
