"""GPU parity where the online softmax must move its reference mid-row.

With N(0,1) inputs a row's scores never climb far above the first tile's, so
the kernels' sum-checked fast path keeps the reference of the first tile and
the rescale of O and the running sum (by 2^(m_old - m_new), strictly between
0 and 1) never runs.  Here one direction of every key row carries a ramp that
query rows lean on with row-dependent slopes: scores rise by up to ~60
(natural log units) along a row, so the reference moves several times, at
different tiles for different rows of one wave (lanes that move beside lanes
that do not), and later keys dominate O.  A saw-tooth variant drops the
ramp back mid-row.  All values are exact in the input type (drawn in fp32,
rounded once); the oracle sees the same bits.  Bounds: the forward's
per-element bound derived from its arithmetic (16-bit), and the fp8 bound.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_25_amd as attn
import oracle
from synth import TORCH_DTYPES
from test_gpu_fp8 import check_fp8, fp8_bound_inputs
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def ramp_inputs(B, H, H_kv, L, d, dtype, seed, saw=False):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, L, d), generator=gen) * 0.25
    k = torch.randn((B, H_kv, L, d), generator=gen) * 0.25
    v = torch.randn((B, H_kv, L, d), generator=gen)
    j = torch.arange(L, dtype=torch.float32)
    ramp = 120.0 * j / max(L - 1, 1)
    if saw:
        ramp = torch.where(j < L // 2, ramp * 2, ramp * 2 - 120.0)
    k[..., 0] = ramp  # keys: the ramp in component 0
    # queries: slope 2..6 (row dependent) on that component; scale 1/8 makes
    # the scores of a row span 0 .. 120 * slope / 8 = up to 90
    slope = 2.0 + (torch.arange(L) % 5).float()
    q[..., 0] = slope
    tdt = TORCH_DTYPES[dtype]
    return q.to(tdt), k.to(tdt), v.to(tdt)


CASES = [
    # (dtype, d, causal, window, saw)
    ("f16", 64, True, -1, False),
    ("f16", 64, False, -1, True),
    ("f16", 128, True, 100, False),
    ("bf16", 64, True, -1, True),
    ("bf16", 128, False, -1, False),
    ("bf16", 64, False, 200, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-d{c[1]}-c{int(c[2])}-w{c[3]}-saw{int(c[4])}")
def test_reference_moves_mid_row(case):
    dtype, d, causal, window, saw = case
    B, H, H_kv, L = 1, 4, 2, 777
    announce(f"rescale {case}")
    q, k, v = ramp_inputs(B, H, H_kv, L, d, dtype, seed=40 + d + int(causal), saw=saw)
    out, lse = attn.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, scale=0.125)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, dtype, causal, window, 0.125, with_abs=True)
    # the rows' score ranges really are wide (the reference had to move)
    assert float(ref[1].max()) > 40.0
    check(out.cpu(), lse.cpu(), ref, dtype, f"rescale {case}", vmax=float(v.abs().max()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("saw", [False, True])
def test_fp8_reference_moves_mid_row(d, saw):
    B, H, H_kv, L = 1, 4, 2, 777
    announce(f"fp8 rescale d={d} saw={saw}")
    q, k, v = ramp_inputs(B, H, H_kv, L, d, "f8", seed=90 + d, saw=saw)
    out, lse = attn.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.125)
    torch.cuda.synchronize()
    ref_o, ref_lse, r, se = fp8_bound_inputs(q, k, v, True, -1, 0.125)
    assert float(np.max(ref_lse)) > 40.0
    check_fp8(out.cpu(), lse.cpu(), ref_o, ref_lse, r, f"fp8 rescale d={d} saw={saw}", se)


BWD_CASES = [("f16", 64, True, -1), ("bf16", 128, True, 100), ("bf16", 64, False, -1), ("f16", 128, False, 50)]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[0]}-d{c[1]}-c{int(c[2])}-w{c[3]}")
def test_backward_with_wide_score_ranges(case):
    """The backward on the same inputs (weights spread over ~60 natural-log
    units within a row, so P is far from uniform and dP - D cancels hard),
    against the fp64 oracle with the backward's derived bound."""
    from test_gpu_backward import check_all, gpu_fwd_bwd, make_dout

    dtype, d, causal, window = case
    B, H, H_kv, L = 1, 4, 2, 300
    announce(f"rescale backward {case}")
    q, k, v = ramp_inputs(B, H, H_kv, L, d, dtype, seed=120 + d)
    dout = make_dout(B, H, L, d, dtype, 121 + d)
    res = gpu_fwd_bwd(q, k, v, dout, causal, window, 0.125)
    ref = oracle.attention_bwd(q, k, v, dout, dtype, causal, window, 0.125, with_abs=True)
    check_all(res, ref, dtype, L * (H // H_kv), f"rescale backward {case}")
