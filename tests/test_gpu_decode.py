"""GPU parity of paged decode: the HIP path against the fp64 paged oracle.

Decode is the forward definition for the last Lq positions of each sequence,
so the forward's bars apply to the decode workloads (fp16 2e-3 / 2e-4, bf16
1e-2 / 1e-3 max / mean over O, 1e-3 over lse), and the forward's per-element
bound derived from the arithmetic (weights rounded to the 16-bit type before
the product, fp32 sums) to the grid of small ragged batches.  Cases: a grid of small ragged batches
(several chunks per sequence, more than 32 query rows per K/V head, every
block size and mask kind), the decode workloads at full size against the
whole oracle, invariants (block placement, lengths clamped to max_seq_len,
sequences shorter than Lq), and the partial kernel's even split of the tile
list (more than 64 sequences, empty sequences among them, all empty).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_25_amd as attn
from oracle import paged
from synth import DECODE_WORKLOADS, decode_inputs, decode_lens, make_paged
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def gpu_decode(q, kc, vc, bt, lens, max_len, window, scale):
    out, lse = attn.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), lens.to(DEV), max_len,
                           window=window, scale=scale)
    torch.cuda.synchronize(DEV)
    return out.cpu(), lse.cpu()


GRID = [
    # (B, H, H_kv, Lq, d, dtype, lens, block_size, window)
    (1, 4, 4, 1, 64, "f16", [1], 16, -1),
    (3, 8, 2, 2, 128, "bf16", [2, 17, 33], 16, -1),
    (2, 4, 1, 4, 64, "f16", [31, 32], 32, 5),
    (4, 32, 8, 1, 128, "bf16", [100, 1000, 3000, 257], 16, -1),
    (2, 16, 1, 4, 64, "bf16", [700, 2049], 64, 100),          # 64 query rows per K/V head
    (1, 8, 8, 16, 128, "f16", [4000], 16, 0),
    (3, 32, 4, 3, 64, "f16", [300, 5, 1500], 128, 37),        # 24 rows, block 128
    (2, 2, 2, 1, 128, "bf16", [6000, 2500], 16, 2048),
    (5, 8, 2, 1, 64, "f16", [1, 64, 65, 1023, 1024], 16, -1),
]


@pytest.mark.parametrize("case", GRID, ids=lambda c: f"B{c[0]}-H{c[1]}/{c[2]}-Lq{c[3]}-d{c[4]}-{c[5]}-bs{c[7]}-w{c[8]}")
def test_decode_grid(case):
    B, H, H_kv, Lq, d, dtype, lens, bs, window = case
    announce(f"decode grid {case}")
    q, kc, vc, bt, sl = make_paged(B, H, H_kv, d, dtype, Lq, lens, bs, seed=sum(lens) + H)
    scale = 0.125 if d == 64 else None
    max_len = max(lens) + 7  # larger than every length: the grid covers chunks no sequence reaches
    max_len = min(max_len, bt.shape[1] * bs)
    out, lse = gpu_decode(q, kc, vc, bt, sl, max_len, window, scale)
    ref = paged.decode_attention(q, kc, vc, bt, lens, dtype, window, 0.0 if scale is None else scale,
                                 with_abs=True)
    check(out, lse, ref, dtype, f"decode {case}", vmax=float(vc.abs().max()))


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workload(name):
    w = DECODE_WORKLOADS[name]
    announce(f"decode workload {name}")
    q, kc, vc, bt, sl = decode_inputs(w)
    max_len = max(decode_lens(w))
    out, lse = gpu_decode(q, kc, vc, bt, sl, max_len, w.window, w.scale)
    ref_o, ref_l = paged.decode_attention(q, kc, vc, bt, decode_lens(w), w.dtype, w.window, w.scale)
    check(out, lse, (ref_o, ref_l), w.dtype, name)


def test_decode_block_placement_is_invisible():
    """The same sequences in a different physical block order give bitwise
    the same result."""
    B, H, H_kv, Lq, d, bs = 2, 8, 2, 2, 128, 16
    lens = [900, 1300]
    announce("decode block placement")
    q, kc, vc, bt, sl = make_paged(B, H, H_kv, d, "bf16", Lq, lens, bs, seed=5)
    perm = torch.randperm(kc.shape[0], generator=torch.Generator().manual_seed(9))
    inv = torch.argsort(perm)
    kc2, vc2 = kc[perm], vc[perm]
    bt2 = torch.where(bt >= 0, inv[bt.clamp(min=0).long()].to(torch.int32), bt)
    a = gpu_decode(q, kc, vc, bt, sl, 1300, -1, None)
    b = gpu_decode(q, kc2, vc2, bt2, sl, 1300, -1, None)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_decode_lengths_clamped_and_short_sequences():
    """seq_lens above max_seq_len count as max_seq_len; rows of a sequence
    shorter than Lq whose position is negative see no key (O = 0, lse = -inf)."""
    B, H, H_kv, Lq, d, bs = 3, 4, 2, 4, 64, 16
    lens = [500, 2, 300]
    announce("decode clamp / short")
    q, kc, vc, bt, sl = make_paged(B, H, H_kv, d, "f16", Lq, lens, bs, seed=6)
    sl_big = sl.clone()
    sl_big[0] = 10 ** 6  # clamped to max_seq_len = 400
    out, lse = gpu_decode(q, kc, vc, bt, sl_big, 400, -1, 0.125)
    ref_o, ref_l = paged.decode_attention(q[0:1], kc, vc, bt[0:1], [400], "f16", -1, 0.125)
    check(out[0:1], lse[0:1], (ref_o, ref_l), "f16", "clamped length")
    # sequence 1 has 2 tokens and Lq = 4: positions -2, -1, 0, 1
    assert torch.all(out[1, :, :2] == 0) and torch.all(torch.isneginf(lse[1, :, :2]))
    q1 = q[1:2, :, 2:]
    ref_o, ref_l = paged.decode_attention(q1, kc, vc, bt[1:2], [2], "f16", -1, 0.125)
    check(out[1:2, :, 2:], lse[1:2, :, 2:], (ref_o, ref_l), "f16", "short sequence")
    ref_o, ref_l = paged.decode_attention(q[2:3], kc, vc, bt[2:3], [300], "f16", -1, 0.125)
    check(out[2:3], lse[2:3], (ref_o, ref_l), "f16", "third sequence")


def test_decode_rejects_bad_workspace_and_outputs():
    """A strided or short workspace, and outputs of the wrong shape, are
    refused before any launch (ValueError), never written past."""
    B, H, H_kv, Lq, d, bs = 1, 4, 2, 1, 64, 16
    announce("decode argument checks")
    q, kc, vc, bt, sl = (t.to(DEV) for t in make_paged(B, H, H_kv, d, "f16", Lq, [100], bs, seed=3))
    need = attn.attn_decode_workspace_size(B, H, H_kv, Lq, d, 100)
    strided = torch.empty(2 * need + 32, dtype=torch.uint8, device=DEV)[::2]
    with pytest.raises(ValueError):
        attn.decode(q, kc, vc, bt, sl, 100, workspace=strided)
    with pytest.raises(ValueError):
        attn.decode(q, kc, vc, bt, sl, 100, workspace=torch.empty(max(need - 1, 1), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        attn.decode(q, kc, vc, bt, sl, 100, out=torch.empty(B, H, Lq + 1, d, dtype=torch.float16, device=DEV))
    out, lse = attn.decode(q, kc, vc, bt, sl, 100)  # and the defaults still work
    torch.cuda.synchronize(DEV)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("case", [(150, 8, 2, 1, 64, "f16", 16), (70, 16, 1, 3, 128, "bf16", 32)],
                         ids=["B150-H8/2-Lq1-d64-f16", "B70-H16/1-Lq3-d128-bf16"])
def test_decode_many_sequences_with_empty_ones(case):
    """More than 64 sequences (the partial kernel's prefix sum over the
    lengths takes several 64-lane passes), every fifth one empty, the rest of
    seeded ragged lengths: the waves' equal runs of the tile list cross many
    sequence (and row-block) boundaries.  Empty sequences give O = 0 and
    lse = -inf; the others match the oracle within the derived bound."""
    B, H, H_kv, Lq, d, dtype, bs = case
    announce(f"decode many sequences {case}")
    gen = torch.Generator().manual_seed(B + d)
    lens = torch.randint(Lq, 900, (B,), generator=gen).tolist()
    for b in range(0, B, 5):
        lens[b] = 0
    q, kc, vc, bt, sl = make_paged(B, H, H_kv, d, dtype, Lq, lens, bs, seed=B * 7 + d)
    scale = 0.125 if d == 64 else None
    out, lse = gpu_decode(q, kc, vc, bt, sl, max(lens), -1, scale)
    empty = [b for b in range(B) if lens[b] == 0]
    live = [b for b in range(B) if lens[b] > 0]
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
    ref = paged.decode_attention(q[live], kc, vc, bt[live], [lens[b] for b in live], dtype, -1,
                                 0.0 if scale is None else scale, with_abs=True)
    check(out[live], lse[live], ref, dtype, f"decode many sequences {case}", vmax=float(vc.abs().max()))


def test_decode_all_sequences_empty():
    """No sequence holds a token: no wave of the partial kernel has work, and
    every row comes out as O = 0, lse = -inf."""
    B, H, H_kv, Lq, d, bs = 3, 4, 2, 2, 64, 16
    announce("decode all empty")
    q, kc, vc, _, _ = make_paged(B, H, H_kv, d, "f16", Lq, [16] * B, bs, seed=4)
    bt = torch.full((B, 1), -1, dtype=torch.int32)
    sl = torch.zeros(B, dtype=torch.int32)
    out, lse = gpu_decode(q, kc, vc, bt, sl, 16, -1, 0.125)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
