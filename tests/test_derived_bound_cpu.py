"""The per-element bound of the GPU parity tests (``derived_bounds``) against
a CPU model of the arithmetic it describes, so the bound is checked without a
GPU and cannot be vacuous.

The model: scores as fp32 sums of exact products of the 16-bit inputs, the
exp2-domain shift by the row maximum, weights exp2 in fp32 rounded to the
input type, the second product accumulated in fp32, the row sum of the
rounded weights (fp16) or of the fp32 weights (bf16), O/l rounded once to the
input type.  Every element of that model must lie inside the bound; a model
with a real defect (weights rounded to 8 bits where fp16 keeps 11, or a
dropped key) must fall outside it somewhere.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import TORCH_DTYPES, make_qkv

from bounds import derived_bounds


def _f32(x):
    return np.asarray(x, np.float32)


def model_forward(q, k, v, dtype, causal, window, scale, weight_bits=None, drop_last_key=False):
    """fp32/16-bit model of one attention forward on the CPU (numpy)."""
    qd, kd, vd = (t.float().numpy() for t in (q, k, v))
    B, H, L, d = qd.shape
    H_kv = kd.shape[1]
    c = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    out = np.zeros((B, H, L, d), np.float64)
    lse = np.zeros((B, H, L), np.float64)
    tdt = TORCH_DTYPES[dtype]
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            for i in range(L):
                js = [j for j in range(L) if oracle_visible(i, j, causal, window)]
                if drop_last_key and len(js) > 1:
                    js = js[:-1]
                s = np.zeros(len(js), np.float32)
                for t, j in enumerate(js):
                    acc = np.float32(0)
                    for cc in range(d):
                        acc = np.float32(acc + np.float32(qd[b, h, i, cc] * kd[b, g, j, cc]))
                    s[t] = acc
                x = _f32(s * c)
                m = np.float32(x.max())
                p32 = _f32(np.exp2(_f32(x - m)))
                if weight_bits is None:
                    p16 = torch.from_numpy(p32).to(tdt).float().numpy()
                else:
                    mant, ex = np.frexp(p32)
                    p16 = _f32(np.ldexp(np.round(mant * 2.0 ** weight_bits) / 2.0 ** weight_bits, ex))
                o = np.zeros(d, np.float32)
                for t, j in enumerate(js):
                    o = _f32(o + _f32(p16[t] * vd[b, g, j]))
                lsum = np.float32(0)
                for t in range(len(js)):
                    lsum = np.float32(lsum + (p16[t] if dtype == "f16" else p32[t]))
                out[b, h, i] = torch.from_numpy(_f32(o / lsum)).to(tdt).double().numpy()
                lse[b, h, i] = float(np.float32((m + np.float32(np.log2(lsum))) * np.float32(0.6931471805599453)))
    return out, lse


def oracle_visible(i, j, causal, window):
    if causal and j > i:
        return False
    if window >= 0 and (i - j > window or (not causal and j - i > window)):
        return False
    return True


CASES = [("f16", 64, True, -1, 17), ("f16", 64, False, 3, 40), ("bf16", 64, True, -1, 33),
         ("bf16", 128, False, -1, 12), ("f16", 128, True, 5, 25)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-d{c[1]}-c{int(c[2])}-w{c[3]}-L{c[4]}")
def test_model_arithmetic_within_bound(case):
    dtype, d, causal, window, L = case
    q, k, v = make_qkv(1, 2, 1, L, d, dtype, 500 + L)
    scale = 0.125 if d == 64 else float(np.float32(1 / np.sqrt(d)))
    o, l = model_forward(q, k, v, dtype, causal, window, scale)
    ref = oracle.attention(q, k, v, dtype, causal, window, scale, with_abs=True)
    ob, lb = derived_bounds(*ref, dtype, float(v.abs().max()))
    assert (np.abs(o - ref[0]) <= ob).all()
    assert (np.abs(l - ref[1]) <= lb).all()


def test_bound_catches_defects():
    """Weights rounded to 8 bits in an fp16 kernel, or a key dropped, fall
    outside the bound."""
    q, k, v = make_qkv(1, 2, 1, 40, 64, "f16", 77)
    ref = oracle.attention(q, k, v, "f16", True, -1, 0.125, with_abs=True)
    ob, lb = derived_bounds(*ref, "f16", float(v.abs().max()))
    o, l = model_forward(q, k, v, "f16", True, -1, 0.125, weight_bits=8)
    assert (np.abs(o - ref[0]) > ob).any() or (np.abs(l - ref[1]) > lb).any()
    o, l = model_forward(q, k, v, "f16", True, -1, 0.125, drop_last_key=True)
    assert (np.abs(o - ref[0]) > ob).any()
