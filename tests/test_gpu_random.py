"""GPU parity on seeded random configurations, against the fp64 oracles.

The fixed grids of the other GPU tests walk the sizes and masks that matter
one axis at a time; here every argument varies at once, drawn from a seeded
generator: batch, head counts with K/V groups of 1, 2, 3, 4, 6 and 8 (the
odd ones included), lengths log-uniform from 1 to a few thousand, causal or
not, windows from 0 to beyond the length, scales log-uniform across 30x
(wide score ranges make the online softmax move its reference often), both
head sizes and both 16-bit types; for decode also the block size, the
number of new tokens, empty sequences and sequences shorter than the new
tokens.  Each case is held to the same per-element bound as the grid tests
of its entry point (derived from the kernels' arithmetic: forward and decode
in test_gpu_parity.check, backward in test_gpu_backward.check_all, fp8 in
test_gpu_fp8.check_fp8).  The draws depend only on the seed, so a failing
case is reproduced by its printed description.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_25_amd as attn
import oracle
from oracle import paged
from synth import make_paged, make_qkv
from test_gpu_backward import check_all, gpu_fwd_bwd, make_dout
from test_gpu_fp8 import check_fp8, fp8_bound_inputs
from test_gpu_parity import announce, check, gpu_forward

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GROUPS = [1, 2, 3, 4, 6, 8]


def draw_shape(rng, max_len, budget, dtypes=("f16", "bf16"), scale_range=(0.02, 0.6)):
    """One forward/backward configuration; B*H*L*L stays within `budget`
    so that the oracle finishes in about a second."""
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(list(dtypes)))
    causal = bool(rng.random() < 0.6)
    H_kv = int(rng.integers(1, 4))
    group = int(rng.choice(GROUPS))
    L = max(1, int(np.exp(rng.uniform(0.0, np.log(max_len)))))
    B = int(rng.integers(1, 4))
    while B > 1 and B * H_kv * group * L * L > budget:
        B -= 1
    while group > 1 and B * H_kv * group * L * L > budget:
        group = max(g for g in GROUPS if g < group)
    while H_kv > 1 and B * H_kv * group * L * L > budget:
        H_kv -= 1
    window = int(rng.integers(0, L + 40)) if rng.random() < 0.4 else -1
    scale = float(np.exp(rng.uniform(np.log(scale_range[0]), np.log(scale_range[1]))))
    return dict(B=B, H=H_kv * group, H_kv=H_kv, L=L, d=d, dtype=dtype, causal=causal, window=window,
                scale=scale)


def describe(c):
    return (f"B={c['B']} H={c['H']}/{c['H_kv']} L={c['L']} d={c['d']} {c['dtype']} causal={c['causal']} "
            f"window={c['window']} scale={c['scale']:.4f}")


@pytest.mark.parametrize("block", range(4))
def test_forward_random(block):
    rng = np.random.default_rng(7100 + block)
    for i in range(25):
        c = draw_shape(rng, 2600, 3e7)
        case = f"random forward {block}.{i}: {describe(c)}"
        announce(case)
        q, k, v = make_qkv(c["B"], c["H"], c["H_kv"], c["L"], c["d"], c["dtype"], 7100 + 37 * block + i)
        out, lse = gpu_forward(q, k, v, c["causal"], c["window"], c["scale"])
        ref = oracle.attention(q, k, v, c["dtype"], c["causal"], c["window"], c["scale"], with_abs=True)
        check(out, lse, ref, c["dtype"], case, vmax=float(v.abs().max()))


@pytest.mark.parametrize("block", range(2))
def test_backward_random(block):
    rng = np.random.default_rng(7200 + block)
    for i in range(16):
        c = draw_shape(rng, 700, 4e6)
        case = f"random backward {block}.{i}: {describe(c)}"
        announce(case)
        seed = 7200 + 37 * block + i
        q, k, v = make_qkv(c["B"], c["H"], c["H_kv"], c["L"], c["d"], c["dtype"], seed)
        dout = make_dout(c["B"], c["H"], c["L"], c["d"], c["dtype"], seed)
        res = gpu_fwd_bwd(q, k, v, dout, c["causal"], c["window"], c["scale"])
        ref = oracle.attention_bwd(q, k, v, dout, c["dtype"], c["causal"], c["window"], c["scale"],
                                   with_abs=True)
        check_all(res, ref, c["dtype"], c["L"] * (c["H"] // c["H_kv"]), case)


def test_fp8_random():
    rng = np.random.default_rng(7300)
    for i in range(24):
        c = draw_shape(rng, 1500, 1e7, dtypes=("f8",), scale_range=(0.03, 0.3))
        case = f"random fp8 {i}: {describe(c)}"
        announce(case)
        q, k, v = make_qkv(c["B"], c["H"], c["H_kv"], c["L"], c["d"], "f8", 7300 + i)
        out, lse = attn.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=c["causal"], window=c["window"],
                                scale=c["scale"])
        torch.cuda.synchronize(DEV)
        ref_o, ref_l, r, se = fp8_bound_inputs(q, k, v, c["causal"], c["window"], c["scale"])
        check_fp8(out.cpu(), lse.cpu(), ref_o, ref_l, r, case, se)


def draw_decode(rng):
    """One paged-decode batch: lengths up to 5000 with empty ones and ones
    shorter than the new tokens among them, at least one non-empty."""
    B = int(rng.integers(1, 7))
    H_kv = int(rng.integers(1, 5))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    Lq = int(rng.integers(1, 6))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    lens = []
    for _ in range(B):
        kind = rng.random()
        lens.append(0 if kind < 0.1 else int(rng.integers(1, Lq + 1)) if kind < 0.2
                    else int(np.exp(rng.uniform(0.0, np.log(5000)))))
    if max(lens) == 0:
        lens[0] = 1
    window = int(rng.integers(0, 3000)) if rng.random() < 0.3 else -1
    scale = float(np.exp(rng.uniform(np.log(0.03), np.log(0.4))))
    return dict(B=B, H=H_kv * group, H_kv=H_kv, Lq=Lq, d=d, dtype=dtype, bs=bs, lens=lens, window=window,
                scale=scale)


def test_decode_random():
    rng = np.random.default_rng(7400)
    for i in range(30):
        c = draw_decode(rng)
        case = (f"random decode {i}: B={c['B']} H={c['H']}/{c['H_kv']} Lq={c['Lq']} d={c['d']} {c['dtype']} "
                f"block={c['bs']} lens={c['lens']} window={c['window']} scale={c['scale']:.4f}")
        announce(case)
        q, kc, vc, bt, sl = make_paged(c["B"], c["H"], c["H_kv"], c["d"], c["dtype"], c["Lq"], c["lens"],
                                       c["bs"], seed=7400 + i)
        max_len = min(max(c["lens"]) + int(rng.integers(0, 8)), bt.shape[1] * c["bs"])
        out, lse = attn.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), sl.to(DEV), max_len,
                               window=c["window"], scale=c["scale"])
        torch.cuda.synchronize(DEV)
        out, lse = out.cpu(), lse.cpu()
        vmax = float(vc.abs().max())
        for b, n in enumerate(c["lens"]):
            # rows whose position n - Lq + t is negative see no key: O = 0, lse = -inf
            k0 = max(0, c["Lq"] - n)
            assert torch.all(out[b, :, :k0] == 0) and torch.all(torch.isneginf(lse[b, :, :k0])), \
                f"{case}: rows without keys of sequence {b}"
            if n == 0:
                continue
            ref = paged.decode_attention(q[b:b + 1, :, k0:], kc, vc, bt[b:b + 1], [n], c["dtype"], c["window"],
                                         c["scale"], with_abs=True)
            check(out[b:b + 1, :, k0:], lse[b:b + 1, :, k0:], ref, c["dtype"], f"{case}, sequence {b}", vmax=vmax)
