"""Pins of the fp64 oracle to facts other than itself.

Each pin is a function of a loaded oracle library (the real one, or a
variant with a planted mistake built by the mutation test) and raises
AssertionError when the oracle disagrees with what the pages or mathematics
fix.  The checks are:

* exhaustive 16-bit decoders against NumPy's binary16 and torch's bfloat16;
* whole-matrix NumPy brute force on tiny inputs;
* torch's CPU fp64 scaled_dot_product_attention (a library routine the plain
  definition reduces to) with an explicit mask;
* closed forms: one visible key returns its value; K = 0 gives the mean of
  the visible values and lse = ln(number of visible keys); identical value
  rows return that row; all-ones values return ones (softmax rows sum to 1);
  two visible keys give a sigmoid mix;
* the per-element weights applied to |v|, visible-key counts and score bounds
  (what the GPU tests derive rounding bounds from) against brute force and
  closed forms (one key, two keys, nonnegative values, |O| bound);
* invariances: adding a constant vector to every key, permuting keys and
  values together, doubling q vs doubling the scale, GQA vs K/V heads
  repeated to H, batch elements computed apart;
* the default scale equals fp32(1/sqrt(d)).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import brute
from synth import make_qkv


def _run(lib, q, k, v, dtype, causal, window, scale, rows=None):
    return oracle.attention(q, k, v, dtype, causal, window, scale, rows=rows, lib=lib)


def _f64(t):
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- decoders
def pin_decoders_exhaustive(lib):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, "f16", lib=lib)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "fp16 NaN patterns"
    assert np.array_equal(got[~nan], want[~nan]), "fp16 values"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "fp16 signed zeros"
    got = oracle.decode(bits, "bf16", lib=lib)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN patterns"
    assert np.array_equal(got[~nan], want[~nan]), "bf16 values"


def pin_f8_decoder_exhaustive(lib):
    """OCP fp8 E4M3 (float8_e4m3fn): all 256 patterns against torch's own
    conversion (values, the two NaN patterns, signed zero)."""
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.decode(bits, "f8", lib=lib)
    want = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "fp8 NaN patterns"
    assert np.array_equal(got[~nan], want[~nan]), "fp8 values"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "fp8 signed zeros"


def pin_f8_inputs_equal_their_f16_widening(lib):
    """Every fp8 E4M3 value is exactly a binary16 value, so attention of fp8
    inputs equals attention of the same values widened to fp16 (bitwise), and
    matches the NumPy brute force."""
    for (L, H, H_kv, causal, window, seed) in [(40, 4, 2, True, -1, 51), (33, 2, 2, False, 5, 52)]:
        q, k, v = make_qkv(1, H, H_kv, L, 64, "f8", seed)
        o8, l8 = _run(lib, q, k, v, "f8", causal, window, 0.125)
        o16, l16 = _run(lib, q.to(torch.float16), k.to(torch.float16), v.to(torch.float16), "f16", causal,
                        window, 0.125)
        assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
        bo, bl = brute.attention(_f64(q), _f64(k), _f64(v), causal, window, 0.125)
        assert np.max(np.abs(o8 - bo)) <= 1e-12 and np.max(np.abs(l8 - bl)) <= 1e-12


# ---------------------------------------------------------------- brute force
BRUTE_GRID_FULL = dict(L=[1, 2, 3, 7, 17, 64, 130], d=[64, 128], heads=[(1, 1), (4, 2), (4, 1)],
                       causal=[False, True], window=[-1, 0, 1, 5], dtype=["f16", "bf16"])
BRUTE_GRID_QUICK = dict(L=[3, 17, 70], d=[64], heads=[(4, 2)], causal=[False, True],
                        window=[-1, 0, 5], dtype=["f16", "bf16"])


def _brute_cases(grid):
    seed = 0
    for L in grid["L"]:
        for d in grid["d"]:
            for H, H_kv in grid["heads"]:
                for causal in grid["causal"]:
                    for window in grid["window"]:
                        for dtype in grid["dtype"]:
                            seed += 1
                            yield L, d, H, H_kv, causal, window, dtype, seed


def pin_brute_force(lib, grid=BRUTE_GRID_QUICK):
    for L, d, H, H_kv, causal, window, dtype, seed in _brute_cases(grid):
        B = 2 if L <= 17 else 1
        q, k, v = make_qkv(B, H, H_kv, L, d, dtype, seed)
        scale = 1.0 / math.sqrt(d) if d != 64 else 0.125
        scale = float(np.float32(scale))
        o, lse = _run(lib, q, k, v, dtype, causal, window, scale)
        bo, blse = brute.attention(_f64(q), _f64(k), _f64(v), causal, window, scale)
        case = f"L={L} d={d} H={H}/{H_kv} causal={causal} window={window} {dtype}"
        assert np.max(np.abs(o - bo)) <= 1e-12, case
        assert np.max(np.abs(lse - blse)) <= 1e-12, case


def pin_brute_force_full(lib):
    pin_brute_force(lib, BRUTE_GRID_FULL)


# ---------------------------------------------------------------- torch SDPA
def _torch_mask(L, causal, window):
    i = torch.arange(L).view(L, 1)
    j = torch.arange(L).view(1, L)
    ok = torch.ones(L, L, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window >= 0:
        ok &= (i - j) <= window
        if not causal:
            ok &= (j - i) <= window
    return ok


def pin_torch_sdpa(lib):
    import torch.nn.functional as F
    for (L, d, H, H_kv, causal, window, dtype, seed) in [
        (33, 64, 4, 2, True, -1, "f16", 11), (33, 64, 4, 1, False, 6, "bf16", 12),
        (96, 128, 2, 2, True, 17, "f16", 13), (50, 64, 8, 8, False, -1, "bf16", 14),
    ]:
        q, k, v = make_qkv(1, H, H_kv, L, d, dtype, seed)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        o, lse = _run(lib, q, k, v, dtype, causal, window, scale)
        qd, kd, vd = (t.to(torch.float64) for t in (q, k, v))
        mask = _torch_mask(L, causal, window)
        ref = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=scale,
                                             enable_gqa=(H != H_kv))
        kr = kd.repeat_interleave(H // H_kv, dim=1)
        scores = (qd @ kr.transpose(-1, -2)) * scale
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
        case = f"L={L} d={d} H={H}/{H_kv} causal={causal} window={window}"
        assert np.max(np.abs(o - ref.numpy())) <= 1e-12, case
        assert np.max(np.abs(lse - ref_lse.numpy())) <= 1e-12, case


# ---------------------------------------------------------------- closed forms
def pin_single_visible_key(lib):
    """window = 0 leaves only the diagonal key: O_i = v_i, lse_i = scale q_i.k_i."""
    for causal in (False, True):
        for dtype in ("f16", "bf16"):
            q, k, v = make_qkv(1, 4, 2, 40, 64, dtype, 21)
            o, lse = _run(lib, q, k, v, dtype, causal, 0, 0.125)
            vd = np.repeat(_f64(v), 2, axis=1)
            assert np.array_equal(o, vd), f"O != V, causal={causal} {dtype}"
            qd, kd = _f64(q), np.repeat(_f64(k), 2, axis=1)
            want = 0.125 * np.einsum("bhid,bhid->bhi", qd, kd)
            assert np.max(np.abs(lse - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def pin_causal_row0(lib):
    """Causal row 0 sees only key 0: O_0 = v_0, lse_0 = scale q_0.k_0."""
    q, k, v = make_qkv(2, 2, 1, 37, 128, "f16", 22)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, lse = _run(lib, q, k, v, "f16", True, -1, scale)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(o[b, h, 0], vd[b, 0, 0])
            want = scale * float(np.dot(qd[b, h, 0], kd[b, 0, 0]))
            assert abs(lse[b, h, 0] - want) <= 1e-13


def visible_count(i, L, causal, window):
    """Number of keys row i sees, written from the window's geometry."""
    before = i if window < 0 else min(i, window)                       # keys j < i
    after = 0 if causal else ((L - 1 - i) if window < 0 else min(L - 1 - i, window))
    return before + 1 + after


def pin_zero_keys(lib, L=300, d=64):
    """K = 0: all visible scores are 0, so O_i is the mean of the visible values
    and lse_i = ln |V(i)|.  The mean uses prefix sums over the visible range."""
    for causal, window in [(True, -1), (False, -1), (True, 9), (False, 9), (True, 0), (False, 200)]:
        q, _, v = make_qkv(1, 2, 1, L, d, "f16", 23)
        k = torch.zeros(1, 1, L, d, dtype=torch.float16)
        o, lse = _run(lib, q, k, v, "f16", causal, window, 0.125)
        vd = _f64(v)[0, 0]
        prefix = np.vstack([np.zeros((1, d)), np.cumsum(vd, axis=0)])
        for i in range(L):
            n = visible_count(i, L, causal, window)
            lo = i - (i if window < 0 else min(i, window))
            hi = lo + n                                   # visible keys are the range [lo, hi)
            mean = (prefix[hi] - prefix[lo]) / n
            for h in range(2):
                assert abs(lse[0, h, i] - math.log(n)) <= 1e-13, (causal, window, i)
                assert np.max(np.abs(o[0, h, i] - mean)) <= 1e-12, (causal, window, i)


def pin_identical_values(lib):
    """Identical value rows u give O_i = u for every row."""
    for causal, window in [(True, -1), (False, 7)]:
        q, k, v = make_qkv(1, 2, 2, 90, 64, "bf16", 24)
        v = v[:, :, :1, :].expand(1, 2, 90, 64).contiguous()
        o, _ = _run(lib, q, k, v, "bf16", causal, window, 0.125)
        u = _f64(v)[:, :, :1, :]
        assert np.max(np.abs(o - u)) <= 1e-13 * max(1.0, np.max(np.abs(u)))


def pin_ones(lib):
    """All-ones values give ones: each row's softmax weights sum to 1."""
    q, k, _ = make_qkv(1, 2, 1, 77, 64, "f16", 25)
    v = torch.ones(1, 1, 77, 64, dtype=torch.float16)
    for causal, window in [(True, -1), (False, -1), (True, 5)]:
        o, _ = _run(lib, q, k, v, "f16", causal, window, 0.125)
        assert np.max(np.abs(o - 1.0)) <= 1e-14


def pin_two_keys(lib):
    """Causal row 1 sees keys 0 and 1: O_1 = w v_0 + (1 - w) v_1 with
    w = 1 / (1 + exp(s_1 - s_0)), lse_1 = s_0 + ln(1 + exp(s_1 - s_0))."""
    q, k, v = make_qkv(1, 1, 1, 2, 64, "f16", 26)
    o, lse = _run(lib, q, k, v, "f16", True, -1, 0.125)
    qd, kd, vd = _f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0]
    s0 = 0.125 * float(qd[1] @ kd[0])
    s1 = 0.125 * float(qd[1] @ kd[1])
    w = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.max(np.abs(o[0, 0, 1] - (w * vd[0] + (1 - w) * vd[1]))) <= 1e-13
    assert abs(lse[0, 0, 1] - (s0 + math.log1p(math.exp(s1 - s0)))) <= 1e-13


# ---------------------------------------------------------------- weights applied to |v|
def _run_abs(lib, q, k, v, dtype, causal, window, scale):
    return oracle.attention(q, k, v, dtype, causal, window, scale, lib=lib, with_abs=True)


def pin_abs_outputs_brute_force(lib):
    """The weights applied to |v|, the visible-key count and the largest
    scale * sum_c |q_ic k_jc| against whole-matrix NumPy on tiny shapes."""
    for (B, H, H_kv, L, d, causal, window, dtype, seed) in [
        (2, 4, 2, 17, 64, True, -1, "f16", 61), (1, 4, 1, 40, 128, False, 5, "bf16", 62),
        (1, 2, 2, 65, 64, True, 9, "f16", 63), (2, 1, 1, 3, 64, False, -1, "bf16", 64),
    ]:
        q, k, v = make_qkv(B, H, H_kv, L, d, dtype, seed)
        scale = 0.125 if d == 64 else float(np.float32(1 / math.sqrt(d)))
        o, lse, oabs, count, sabs = _run_abs(lib, q, k, v, dtype, causal, window, scale)
        bo, blse, boabs, bcount, bsabs = brute.attention(_f64(q), _f64(k), _f64(v), causal, window, scale,
                                                         with_abs=True)
        case = f"L={L} d={d} H={H}/{H_kv} causal={causal} window={window} {dtype}"
        assert np.max(np.abs(oabs - boabs)) <= 1e-12, case
        assert np.array_equal(count, bcount), case
        assert np.max(np.abs(sabs - bsabs)) <= 1e-12 * max(1.0, float(np.max(bsabs))), case
        o2, lse2 = _run(lib, q, k, v, dtype, causal, window, scale)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2), case


def pin_abs_outputs_closed_forms(lib):
    """One visible key: the weights applied to |v| give |v_i|, one key is
    counted and the score bound is scale * sum_c |q_ic k_ic|.  Two visible
    keys (causal row 1): w |v_0| + (1 - w) |v_1| with the sigmoid weight w.
    Nonnegative values: the weights applied to |v| equal O itself, and in
    general they bound |O| (triangle inequality)."""
    q, k, v = make_qkv(1, 4, 2, 40, 64, "f16", 65)
    _, _, oabs, count, sabs = _run_abs(lib, q, k, v, "f16", True, 0, 0.125)
    vd = np.repeat(_f64(v), 2, axis=1)
    kd = np.repeat(_f64(k), 2, axis=1)
    assert np.array_equal(oabs, np.abs(vd))
    assert np.array_equal(count, np.ones_like(count))
    want = 0.125 * np.einsum("bhid,bhid->bhi", np.abs(_f64(q)), np.abs(kd))
    assert np.max(np.abs(sabs - want)) <= 1e-13 * np.max(want)

    q, k, v = make_qkv(1, 1, 1, 2, 64, "bf16", 66)
    o, _, oabs, count, sabs = _run_abs(lib, q, k, v, "bf16", True, -1, 0.125)
    qd, kd, vd = _f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0]
    s0, s1 = 0.125 * float(qd[1] @ kd[0]), 0.125 * float(qd[1] @ kd[1])
    w = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.max(np.abs(oabs[0, 0, 1] - (w * np.abs(vd[0]) + (1 - w) * np.abs(vd[1])))) <= 1e-13
    assert count[0, 0, 1] == 2 and count[0, 0, 0] == 1
    want = 0.125 * max(float(np.abs(qd[1]) @ np.abs(kd[0])), float(np.abs(qd[1]) @ np.abs(kd[1])))
    assert abs(sabs[0, 0, 1] - want) <= 1e-13 * want

    q, k, v = make_qkv(1, 2, 1, 70, 64, "f16", 67)
    for causal, window in [(True, -1), (False, 8)]:
        o, _, oabs, count, _ = _run_abs(lib, q, k, v.abs().contiguous(), "f16", causal, window, 0.125)
        assert np.max(np.abs(oabs - o)) <= 1e-13 * np.max(o)
        o, _, oabs, _, _ = _run_abs(lib, q, k, v, "f16", causal, window, 0.125)
        assert (oabs >= np.abs(o) * (1 - 1e-13)).all()
        assert all(count[0, h, i] == visible_count(i, 70, causal, window) for h in range(2) for i in range(70))


# ---------------------------------------------------------------- invariances
def pin_key_shift(lib):
    """Adding c to every key row adds scale*q_i.c to every visible score of row i:
    O is unchanged and lse_i grows by scale*q_i.c.  Inputs are multiples of 1/8
    so the shifted keys are exact in fp16."""
    gen = torch.Generator().manual_seed(27)
    L, d = 60, 64
    q = (torch.randint(-8, 9, (1, 2, L, d), generator=gen) / 8).to(torch.float16)
    k = (torch.randint(-8, 9, (1, 1, L, d), generator=gen) / 8).to(torch.float16)
    v = torch.randn(1, 1, L, d, generator=gen).to(torch.float16)
    c = (torch.randint(-8, 9, (d,), generator=gen) / 8).to(torch.float16)
    for causal, window in [(True, -1), (False, 11)]:
        o1, lse1 = _run(lib, q, k, v, "f16", causal, window, 0.125)
        o2, lse2 = _run(lib, q, (k + c).contiguous(), v, "f16", causal, window, 0.125)
        shift = 0.125 * (_f64(q) @ _f64(c))
        assert np.max(np.abs(o1 - o2)) <= 1e-12
        assert np.max(np.abs((lse2 - lse1) - shift)) <= 1e-12


def pin_permutation(lib):
    """Without a mask, permuting keys and values together leaves O and lse unchanged."""
    q, k, v = make_qkv(1, 2, 2, 50, 64, "bf16", 28)
    perm = torch.randperm(50, generator=torch.Generator().manual_seed(29))
    o1, lse1 = _run(lib, q, k, v, "bf16", False, -1, 0.125)
    o2, lse2 = _run(lib, q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), "bf16", False, -1, 0.125)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(lse1 - lse2)) <= 1e-13


def pin_scale_vs_query(lib):
    """Doubling the scale equals doubling q (exact in fp16 at these magnitudes)."""
    q, k, v = make_qkv(1, 2, 1, 45, 64, "f16", 30)
    o1, lse1 = _run(lib, (q * 2).contiguous(), k, v, "f16", True, 6, 0.0625)
    o2, lse2 = _run(lib, q, k, v, "f16", True, 6, 0.125)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(lse1 - lse2)) <= 1e-13


def pin_gqa_equals_repeated_heads(lib):
    """H_kv < H equals the same run with each K/V head repeated over its group."""
    for H, H_kv in [(4, 1), (6, 3), (8, 2)]:
        q, k, v = make_qkv(1, H, H_kv, 41, 64, "f16", 31 + H)
        o1, lse1 = _run(lib, q, k, v, "f16", True, 9, 0.125)
        kr = k.repeat_interleave(H // H_kv, dim=1).contiguous()
        vr = v.repeat_interleave(H // H_kv, dim=1).contiguous()
        o2, lse2 = _run(lib, q, kr, vr, "f16", True, 9, 0.125)
        assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2), (H, H_kv)


def pin_batch_independence(lib):
    q, k, v = make_qkv(3, 2, 1, 35, 64, "bf16", 40)
    o, lse = _run(lib, q, k, v, "bf16", False, 4, 0.125)
    for b in range(3):
        ob, lseb = _run(lib, q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                        v[b:b + 1].contiguous(), "bf16", False, 4, 0.125)
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(lse[b:b + 1], lseb), b


def pin_default_scale(lib):
    """scale <= 0 or NaN selects fp32(1/sqrt(d))."""
    for d in (64, 128):
        want = float(np.float32(1.0 / np.sqrt(np.float64(d))))
        for s in (0.0, -1.0, float("nan")):
            assert oracle.resolve_scale(s, d, lib=lib) == want
    assert oracle.resolve_scale(0.3, 64, lib=lib) == float(np.float32(0.3))
    q, k, v = make_qkv(1, 1, 1, 20, 128, "f16", 41)
    o1, l1 = _run(lib, q, k, v, "f16", True, -1, 0.0)
    o2, l2 = _run(lib, q, k, v, "f16", True, -1, float(np.float32(1 / math.sqrt(128))))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_row_subset(lib):
    """Rows requested one by one equal the same rows of the full result."""
    q, k, v = make_qkv(2, 4, 2, 70, 64, "f16", 42)
    o, lse = _run(lib, q, k, v, "f16", True, 13, 0.125)
    rows = [0, 5, 69, 70, 139, 280, 559, 333]
    os_, lses = _run(lib, q, k, v, "f16", True, 13, 0.125, rows=rows)
    flat_o, flat_lse = o.reshape(-1, 64), lse.reshape(-1)
    assert np.array_equal(os_, flat_o[rows]) and np.array_equal(lses, flat_lse[rows])


ALL_PINS = [
    pin_decoders_exhaustive, pin_f8_decoder_exhaustive, pin_f8_inputs_equal_their_f16_widening, pin_brute_force, pin_torch_sdpa, pin_single_visible_key,
    pin_causal_row0, pin_zero_keys, pin_identical_values, pin_ones, pin_two_keys,
    pin_abs_outputs_brute_force, pin_abs_outputs_closed_forms, pin_key_shift, pin_permutation, pin_scale_vs_query, pin_gqa_equals_repeated_heads,
    pin_batch_independence, pin_default_scale, pin_row_subset,
]
