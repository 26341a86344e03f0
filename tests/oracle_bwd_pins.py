"""Pins of the fp64 backward-pass oracle to facts other than itself.

Each pin takes a loaded oracle library (the real one or a variant with a
planted mistake) and raises AssertionError when the oracle's gradients
disagree with what mathematics fixes:

* central finite differences of the whole-matrix NumPy forward (a different
  implementation of the forward definition, differentiated numerically: it
  knows nothing of the gradient formulas);
* torch's CPU fp64 autograd through scaled_dot_product_attention with an
  explicit mask (a library routine the definition reduces to);
* exact sums: the keys' gradients sum to zero (adding one vector to every
  key leaves every output unchanged), the values' gradients sum to the
  upstream gradient (softmax rows sum to one), sum_i q_i.dq_i equals
  sum_j k_j.dk_j (scores are bilinear in q and k), and sum_j v_j.dv_j equals
  sum_i dO_i.O_i;
* closed forms: one visible key gives dq = dk = 0 and dv = dO; K = 0 gives
  dq = 0 and dv_j = sum over rows seeing j of dO_i / |V(i)|; two visible keys
  give the derivative of a sigmoid mix (and the sum of |terms| of dq);
* relations: doubling the scale vs doubling q, GQA vs K/V heads repeated to
  H, rows requested one by one vs all at once;
* the sums of |terms| returned beside the gradients bound them, and equal
  them where every term has one sign; they and the sensitivities to the row
  terms D are pinned in closed form by the two-key case.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import brute
from synth import make_qkv

from oracle_pins import _torch_mask, visible_count


def _inputs(B, H, H_kv, L, d, dtype, seed):
    q, k, v = make_qkv(B, H, H_kv, L, d, dtype, seed)
    dout, _, _ = make_qkv(B, H, H_kv, L, d, dtype, seed + 1000)
    return q, k, v, dout


def _f64(t):
    return t.to(torch.float64).numpy()


def _bwd(lib, q, k, v, dout, dtype, causal, window, scale, **kw):
    return oracle.attention_bwd(q, k, v, dout, dtype, causal, window, scale, lib=lib, **kw)


# ---------------------------------------------------------------- finite differences
FD_CASES = [
    # (B, H, H_kv, L, d, causal, window, dtype, seed)
    (1, 2, 1, 5, 4, True, -1, "f16", 1),
    (1, 2, 2, 6, 3, False, 1, "bf16", 2),
    (2, 2, 1, 4, 5, False, -1, "f16", 3),
    (1, 1, 1, 7, 2, True, 2, "f16", 4),
    (1, 3, 1, 3, 64, False, 0, "f16", 5),
]


def pin_bwd_finite_differences(lib):
    """Each gradient element equals the central difference of sum(dO * O)
    computed with the NumPy forward, perturbing that one input element."""
    h = 1e-5
    for B, H, H_kv, L, d, causal, window, dtype, seed in FD_CASES:
        q, k, v, dout = _inputs(B, H, H_kv, L, d, dtype, seed)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        dq, dk, dv = _bwd(lib, q, k, v, dout, dtype, causal, window, scale)
        x = {"q": _f64(q), "k": _f64(k), "v": _f64(v)}
        g = _f64(dout)
        grads = {"q": dq, "k": dk, "v": dv}

        def loss(args):
            o, _ = brute.attention(args["q"], args["k"], args["v"], causal, window, scale)
            return float(np.sum(g * o))

        case = f"B={B} H={H}/{H_kv} L={L} d={d} causal={causal} window={window}"
        for name in ("q", "k", "v"):
            fd = np.zeros_like(x[name])
            for idx in np.ndindex(x[name].shape):
                plus = {kk: vv.copy() for kk, vv in x.items()}
                minus = {kk: vv.copy() for kk, vv in x.items()}
                plus[name][idx] += h
                minus[name][idx] -= h
                fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
            err = np.max(np.abs(fd - grads[name]))
            assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), f"d{name} vs finite differences {err:.3e}: {case}"


# ---------------------------------------------------------------- torch autograd
def pin_bwd_torch_autograd(lib):
    import torch.nn.functional as F
    for (B, L, d, H, H_kv, causal, window, dtype, seed) in [
        (1, 33, 64, 4, 2, True, -1, "f16", 21), (1, 40, 64, 4, 1, False, 6, "bf16", 22),
        (1, 70, 128, 2, 2, True, 17, "f16", 23), (2, 17, 64, 2, 2, False, -1, "bf16", 24),
        (1, 65, 64, 8, 2, True, 0, "f16", 25),
    ]:
        q, k, v, dout = _inputs(B, H, H_kv, L, d, dtype, seed)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        dq, dk, dv = _bwd(lib, q, k, v, dout, dtype, causal, window, scale)
        qd, kd, vd = (t.to(torch.float64).requires_grad_() for t in (q, k, v))
        o = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=_torch_mask(L, causal, window),
                                           scale=scale, enable_gqa=(H != H_kv))
        o.backward(dout.to(torch.float64))
        case = f"B={B} L={L} d={d} H={H}/{H_kv} causal={causal} window={window} {dtype}"
        for name, mine, ref in (("dq", dq, qd.grad), ("dk", dk, kd.grad), ("dv", dv, vd.grad)):
            err = np.max(np.abs(mine - ref.numpy()))
            assert err <= 1e-12 * max(1.0, float(ref.abs().max())), f"{name} {err:.3e}: {case}"


# ---------------------------------------------------------------- exact sums
def pin_bwd_sums(lib):
    for (B, H, H_kv, L, d, causal, window, dtype, seed) in [
        (2, 4, 2, 90, 64, True, -1, "f16", 31), (1, 4, 1, 77, 128, False, 9, "bf16", 32),
        (1, 2, 2, 64, 64, True, 20, "f16", 33),
    ]:
        q, k, v, dout = _inputs(B, H, H_kv, L, d, dtype, seed)
        scale = 0.125
        dq, dk, dv = _bwd(lib, q, k, v, dout, dtype, causal, window, scale)
        o, _ = oracle.attention(q, k, v, dtype, causal, window, scale, lib=lib)
        qf, kf, vf, gf = _f64(q), _f64(k), _f64(v), _f64(dout)
        group = H // H_kv
        case = f"B={B} H={H}/{H_kv} L={L} d={d} causal={causal} window={window}"
        for b in range(B):
            for g in range(H_kv):
                heads = slice(g * group, (g + 1) * group)
                mag = np.abs(dk[b, g]).sum(axis=0).max() + 1.0
                assert np.max(np.abs(dk[b, g].sum(axis=0))) <= 1e-12 * mag, f"sum_j dk_j = 0: {case}"
                want = gf[b, heads].sum(axis=(0, 1))
                assert np.allclose(dv[b, g].sum(axis=0), want, rtol=0, atol=1e-11), f"sum_j dv_j: {case}"
                lhs = float(np.sum(qf[b, heads] * dq[b, heads]))
                rhs = float(np.sum(kf[b, g] * dk[b, g]))
                assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), f"q.dq = k.dk: {case}"
                lhs = float(np.sum(vf[b, g] * dv[b, g]))
                rhs = float(np.sum(gf[b, heads] * o[b, heads]))
                assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), f"v.dv = dO.O: {case}"


# ---------------------------------------------------------------- closed forms
def pin_bwd_single_visible_key(lib):
    """window = 0: O_i = v_i whatever q and k are, so dq = dk = 0 and dv_j is
    the upstream gradient of row j summed over the heads sharing the K/V head."""
    for causal in (False, True):
        q, k, v, dout = _inputs(2, 4, 2, 37, 64, "f16", 41)
        dq, dk, dv = _bwd(lib, q, k, v, dout, "f16", causal, 0, 0.125)
        assert np.all(dq == 0) and np.all(dk == 0), "dq, dk with one visible key"
        want = _f64(dout).reshape(2, 2, 2, 37, 64).sum(axis=2)
        assert np.max(np.abs(dv - want)) <= 1e-14, "dv with one visible key"


def pin_bwd_causal_row0(lib):
    """Causal row 0 sees only key 0: its dq is zero."""
    q, k, v, dout = _inputs(1, 2, 2, 50, 128, "bf16", 42)
    dq, _, _ = _bwd(lib, q, k, v, dout, "bf16", True, -1, 0.09)
    assert np.all(dq[:, :, 0] == 0)
    assert np.max(np.abs(dq[:, :, 1:])) > 0


def pin_bwd_zero_keys(lib, L=200, d=64):
    """K = 0: every visible score is 0, so dq = 0 and dv_j is the sum over
    the rows i that see j of dO_i / |V(i)|."""
    for causal, window in ((True, -1), (True, 13), (False, 7), (False, -1)):
        q, k, v, dout = _inputs(1, 2, 1, L, d, "f16", 43)
        k = torch.zeros_like(k)
        dq, _, dv = _bwd(lib, q, k, v, dout, "f16", causal, window, 0.125)
        assert np.all(dq == 0), f"dq with K = 0, causal={causal} window={window}"
        g = _f64(dout)[0]  # [H, L, d]
        counts = np.array([visible_count(i, L, causal, window) for i in range(L)], np.float64)
        want = np.zeros((L, d))
        for i in range(L):
            if window >= 0:
                lo = max(0, i - window)
                hi = i if causal else min(L - 1, i + window)
            else:
                lo, hi = 0, (i if causal else L - 1)
            want[lo:hi + 1] += (g[0, i] + g[1, i]) / counts[i]
        assert np.max(np.abs(dv[0, 0] - want)) <= 1e-12, f"dv with K = 0, causal={causal} window={window}"


def pin_bwd_two_keys(lib):
    """Causal window 1: row i >= 1 sees keys i-1 and i with weight
    sigma = 1/(1+exp(s_{i,i-1} - s_{i,i})) on key i, so
    dS_{i,i} = -dS_{i,i-1} = sigma (1-sigma) (dO_i.(v_i - v_{i-1})) and
    dq_i = scale dS_{i,i} (k_i - k_{i-1}); each key is seen by two rows, which
    gives dk, dv and all the sums of |terms| in closed form too."""
    q, k, v, dout = _inputs(1, 1, 1, 40, 64, "f16", 44)
    scale = 0.125
    (dq, dk, dv), (dq_abs, dk_abs, dv_abs), (dq_sens, dk_sens) = _bwd(lib, q, k, v, dout, "f16", True, 1,
                                                                     scale, with_abs=True)
    qf, kf, vf, gf = (_f64(t)[0, 0] for t in (q, k, v, dout))
    sig_of, ds_of = {0: 1.0}, {0: 0.0, 40: 0.0}  # row 0 sees key 0 only; row 40 does not exist
    rho_of = {0: np.linalg.norm(gf[0] * vf[0]), 40: 0.0}  # root-sum-square of the terms of D_i
    for i in range(1, 40):
        s_new, s_old = scale * qf[i] @ kf[i], scale * qf[i] @ kf[i - 1]
        sig = 1.0 / (1.0 + math.exp(s_old - s_new))
        ds = sig * (1 - sig) * (gf[i] @ (vf[i] - vf[i - 1]))  # dS of key i; key i-1 gets -ds
        want = scale * ds * (kf[i] - kf[i - 1])
        assert np.max(np.abs(dq[0, 0, i] - want)) <= 1e-12, f"row {i}"
        want_abs = scale * abs(ds) * (np.abs(kf[i]) + np.abs(kf[i - 1]))
        assert np.max(np.abs(dq_abs[0, 0, i] - want_abs)) <= 1e-12, f"|terms| of row {i}"
        rho = np.linalg.norm(gf[i] * (sig * vf[i] + (1 - sig) * vf[i - 1]))
        want_sens = scale * rho * (sig * np.abs(kf[i]) + (1 - sig) * np.abs(kf[i - 1]))
        assert np.max(np.abs(dq_sens[0, 0, i] - want_sens)) <= 1e-12, f"D sensitivity of row {i}"
        sig_of[i], ds_of[i], rho_of[i] = sig, ds, rho
    # key j is seen by rows j (weight sigma_j, dS = ds_j) and j+1 (weight
    # 1 - sigma_{j+1}, dS = -ds_{j+1})
    for j in range(40):
        s_next = sig_of.get(j + 1, 1.0)
        want = sig_of[j] * gf[j] + (1 - s_next) * (gf[j + 1] if j + 1 < 40 else 0)
        assert np.max(np.abs(dv[0, 0, j] - want)) <= 1e-12, f"dv of key {j}"
        want = sig_of[j] * np.abs(gf[j]) + (1 - s_next) * (np.abs(gf[j + 1]) if j + 1 < 40 else 0)
        assert np.max(np.abs(dv_abs[0, 0, j] - want)) <= 1e-12, f"|terms| of dv of key {j}"
        q_next = qf[j + 1] if j + 1 < 40 else 0 * qf[j]
        want = scale * (ds_of[j] * qf[j] - ds_of[j + 1] * q_next)
        assert np.max(np.abs(dk[0, 0, j] - want)) <= 1e-12, f"dk of key {j}"
        want = scale * (abs(ds_of[j]) * np.abs(qf[j]) + abs(ds_of[j + 1]) * np.abs(q_next))
        assert np.max(np.abs(dk_abs[0, 0, j] - want)) <= 1e-12, f"|terms| of dk of key {j}"
        want = scale * (sig_of[j] * rho_of[j] * np.abs(qf[j]) + (1 - s_next) * rho_of[j + 1] * np.abs(q_next))
        assert np.max(np.abs(dk_sens[0, 0, j] - want)) <= 1e-12, f"D sensitivity of dk of key {j}"


# ---------------------------------------------------------------- relations
def pin_bwd_scale_vs_query(lib):
    """O depends on scale * q only: dq(2s, q) = 2 dq(s, 2q); dk and dv agree."""
    q, k, v, dout = _inputs(1, 2, 1, 45, 64, "f16", 45)
    a = _bwd(lib, q, k, v, dout, "f16", True, 11, 0.25)
    b = _bwd(lib, q * 2, k, v, dout, "f16", True, 11, 0.125)
    assert np.max(np.abs(a[0] - 2 * b[0])) <= 1e-12 * (1 + np.max(np.abs(a[0])))
    assert np.max(np.abs(a[1] - b[1])) <= 1e-12 * (1 + np.max(np.abs(a[1])))
    assert np.max(np.abs(a[2] - b[2])) <= 1e-12


def pin_bwd_gqa_equals_repeated_heads(lib):
    """With K/V repeated to H heads, dq is unchanged and the GQA dk, dv are
    the sums of the repeated heads' dk, dv over each group."""
    q, k, v, dout = _inputs(1, 6, 2, 33, 64, "bf16", 46)
    dq, dk, dv = _bwd(lib, q, k, v, dout, "bf16", False, 4, 0.125)
    kr, vr = k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1)
    rq, rk, rv = _bwd(lib, q, kr, vr, dout, "bf16", False, 4, 0.125)
    assert np.array_equal(dq, rq)
    assert np.max(np.abs(dk - rk.reshape(1, 2, 3, 33, 64).sum(axis=2))) <= 1e-13
    assert np.max(np.abs(dv - rv.reshape(1, 2, 3, 33, 64).sum(axis=2))) <= 1e-13


def pin_bwd_row_subsets(lib):
    """Rows requested one by one equal the same rows of the full result."""
    q, k, v, dout = _inputs(2, 4, 2, 70, 64, "f16", 47)
    dq, dk, dv = _bwd(lib, q, k, v, dout, "f16", True, 13, 0.125)
    qr = [0, 5, 69, 70, 139, 280, 559, 333]
    kr = [0, 1, 69, 70, 200, 279, 140]
    sq, sk, sv = _bwd(lib, q, k, v, dout, "f16", True, 13, 0.125, q_rows=qr, kv_rows=kr)
    assert np.array_equal(sq, dq.reshape(-1, 64)[qr])
    assert np.array_equal(sk, dk.reshape(-1, 64)[kr])
    assert np.array_equal(sv, dv.reshape(-1, 64)[kr])
    eq, ek, ev = _bwd(lib, q, k, v, dout, "f16", True, 13, 0.125, q_rows=[], kv_rows=kr)
    assert eq.shape == (0, 64) and np.array_equal(ek, sk) and np.array_equal(ev, sv)


ALL_BWD_PINS = [
    pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_sums, pin_bwd_single_visible_key,
    pin_bwd_causal_row0, pin_bwd_zero_keys, pin_bwd_two_keys, pin_bwd_scale_vs_query,
    pin_bwd_gqa_equals_repeated_heads, pin_bwd_row_subsets,
]


def pin_bwd_abs_sums(lib):
    """The sums of |terms| bound their sums, reduce to them where every term
    has one sign (dv with non-negative dO: P >= 0), and do not change the
    gradients."""
    q, k, v, dout = _inputs(1, 4, 2, 60, 64, "f16", 48)
    g, a, _ = _bwd(lib, q, k, v, dout, "f16", True, 9, 0.125, with_abs=True)
    plain = _bwd(lib, q, k, v, dout, "f16", True, 9, 0.125)
    for x, y, s in zip(g, plain, a):
        assert np.array_equal(x, y)
        assert np.all(np.abs(x) <= s * (1 + 1e-12))
    pos = dout.abs()
    g, a, _ = _bwd(lib, q, k, v, pos, "f16", True, 9, 0.125, with_abs=True)
    assert np.max(np.abs(g[2] - a[2])) <= 1e-12 * (1 + np.max(a[2]))
    gs, as_, ss = _bwd(lib, q, k, v, dout, "f16", True, 9, 0.125, q_rows=[3, 100], kv_rows=[7, 64],
                       with_abs=True)
    full, full_abs, full_sens = _bwd(lib, q, k, v, dout, "f16", True, 9, 0.125, with_abs=True)
    assert np.array_equal(ss[0], full_sens[0].reshape(-1, 64)[[3, 100]])
    assert np.array_equal(ss[1], full_sens[1].reshape(-1, 64)[[7, 64]])
    assert np.array_equal(as_[0], full_abs[0].reshape(-1, 64)[[3, 100]])
    assert np.array_equal(as_[1], full_abs[1].reshape(-1, 64)[[7, 64]])
    assert np.array_equal(as_[2], full_abs[2].reshape(-1, 64)[[7, 64]])


ALL_BWD_PINS.append(pin_bwd_abs_sums)
