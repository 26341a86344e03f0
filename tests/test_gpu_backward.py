"""GPU parity of the backward pass: dq, dk, dv of the HIP path against the
fp64 oracle, element by element, through the C ABI.

Tolerance (no bar is given for gradients; this one follows the arithmetic).
Each gradient element is a sum of terms t = a * b in which one factor, the
softmax weight P or the score gradient dS, is rounded to the 16-bit input
type before the product (relative error <= u: 2^-11 fp16, 2^-8 bf16, so
<= u sum|t|, with 2u allowed for the weights' own fp32 evaluation); P is
recomputed from the forward's fp32 lse, whose error (tested to 1e-3)
multiplies P by exp(error); the sum runs in fp32 over n terms (random-walk
error ~ sqrt(n) 2^-24 relative to sum|t|); and the result is rounded once to
the 16-bit type.  The row terms D_i = dO_i.O_i are formed from the 16-bit
forward output: O_i carries its rounding (<= u |O|) and the forward's own
rounding of the weights (of the same size), so D_i is off by a random sum
of d such errors, std ~ 0.8 u rho_i with rho_i = ||dO_i * O_i||_2; 4u rho_i
is 5 standard deviations.  So, per element,

    |gpu - exact| <= floor + (2u + 1e-3 + 3 sqrt(n) 2^-24) sum|t| + 4u sens_D + 1e-4

where floor = |round(exact) - exact|, and sum|t| and sens_D (the element's
sensitivity to D, per unit of rho) come from the oracle; the absolute 1e-4
covers the fp32 evaluation of dP - D (d-term dot products, ~2^-24 d |dO| |v|),
which does not scale with sum|t| where dS is ~0.
"""
import math
import sys

import numpy as np
import pytest
import torch

import exact_io_aware_25_amd as attn
import oracle
from synth import TORCH_DTYPES, WORKLOADS, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
LSE_TOL = 1e-3
ABS_SLACK = 1e-4
LOG2E = 1.4426950408889634


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def make_dout(B, H, L, d, dtype, seed):
    g, _, _ = make_qkv(B, H, H, L, d, dtype, seed + 5000)
    return g


def gpu_fwd_bwd(q, k, v, dout, causal, window, scale, keep_device=False):
    """Forward then backward on the GPU; returns a dict of CPU tensors."""
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = attn.forward(qd, kd, vd, causal=causal, window=window, scale=scale)
    B, H, L, _ = q.shape
    ws = torch.empty(max(attn.attn_bwd_workspace_size(B, H, L), 16), dtype=torch.uint8, device=DEV)
    dq, dk, dv = attn.backward(qd, kd, vd, out, lse, gd, causal=causal, window=window, scale=scale,
                               workspace=ws)
    torch.cuda.synchronize(DEV)
    res = dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws)
    return res if keep_device else {n: t.cpu() for n, t in res.items()}


def round_to(x, dtype):
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype]).double().numpy()


def check_grad(name, got, ref, ref_abs, dtype, n_terms, case, ref_sens=None):
    """got: torch tensor (any shape with ref.size elements); ref, ref_abs,
    ref_sens (None for dv, which D does not enter): fp64 arrays."""
    g = got.double().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{case}: non-finite {name}"
    err = np.abs(g - ref)
    floor = np.abs(round_to(ref, dtype) - ref)
    u = UNIT_ROUNDOFF[dtype]
    rel = 2 * u + LSE_TOL + 3 * math.sqrt(max(n_terms, 1)) * 2.0 ** -24
    bound = floor + rel * ref_abs + ABS_SLACK
    if ref_sens is not None:
        bound = bound + 4 * u * ref_sens
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (
        f"{case}: {name} error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
        f"(exact {ref[worst]:.4e}, sum|t| {ref_abs[worst]:.3e}); max err {err.max():.3e}")
    return float(err.max()), float((err / bound).max())


def check_all(res, oracle_out, dtype, n_terms, case, q_rows=None, kv_rows=None):
    ref, ref_abs, ref_sens = oracle_out
    d = res["dq"].shape[-1]
    out = {}
    for name, rows, i in (("dq", q_rows, 0), ("dk", kv_rows, 1), ("dv", kv_rows, 2)):
        t = res[name]
        if rows is not None:
            t = t.reshape(-1, d)[torch.as_tensor(rows)]
        out[name] = check_grad(name, t, ref[i], ref_abs[i], dtype, n_terms, case,
                               ref_sens[i] if i < 2 else None)
    return out


# ------------------------------------------------------------------ small grid
GRID_L = [1, 2, 17, 63, 64, 65, 129, 300]
GRID_WINDOW = [-1, 0, 1, 37, 200]
GRID_HEADS = [(1, 1), (4, 1), (4, 2), (3, 3)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_grid(dtype, d, causal):
    seed = 300 + 10 * d + (5 if causal else 0)
    for L in GRID_L:
        for window in GRID_WINDOW:
            seed += 1
            H, H_kv = GRID_HEADS[seed % len(GRID_HEADS)]
            B = 2 if (L + seed) % 3 == 0 else 1
            case = f"bwd B={B} H={H}/{H_kv} L={L} d={d} causal={causal} window={window} {dtype}"
            announce(case)
            q, k, v = make_qkv(B, H, H_kv, L, d, dtype, seed)
            dout = make_dout(B, H, L, d, dtype, seed)
            scale = 0.125 if d == 64 else None
            res = gpu_fwd_bwd(q, k, v, dout, causal, window, scale)
            ref = oracle.attention_bwd(q, k, v, dout, dtype, causal, window,
                                       0.0 if scale is None else scale, with_abs=True)
            check_all(res, ref, dtype, L * (H // H_kv), case)


# ------------------------------------------------------------------ workloads
FULL_ORACLE = ["causal_4k", "noncausal_2k_f16", "noncausal_2k_bf16", "p2_accuracy"]


@pytest.mark.parametrize("name", FULL_ORACLE)
def test_bwd_workload_full(name):
    w = WORKLOADS[name]
    announce(f"bwd workload {name} (whole oracle)")
    q, k, v = workload_inputs(w)
    dout = make_dout(w.B, w.H, w.L, w.d, w.dtype, 7)
    res = gpu_fwd_bwd(q, k, v, dout, w.causal, w.window, w.scale)
    ref = oracle.attention_bwd(q, k, v, dout, w.dtype, w.causal, w.window, w.scale, with_abs=True)
    check_all(res, ref, w.dtype, w.L * (w.H // w.H_kv), name)


def sampled_rows(w, heads, extra_seed):
    """Flat dq row ids (b*H + h)*L + i and dk/dv row ids (b*H_kv + g)*L + j:
    tile and block edges, the last rows, and seeded random rows; keys are
    taken where few rows see them (the last ones) and, with a window, around
    the middle too."""
    L = w.L
    rng = np.random.default_rng(extra_seed)
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, L // 2, L - 129, L - 65, L - 64, L - 2, L - 1}
    q_rows = []
    for h in heads:
        rows = sorted((edges | set(rng.integers(0, L, 24).tolist())) & set(range(L)))
        q_rows += [h * L + i for i in rows]
    keys = {L - 1, L - 2, L - 31, L - 32, L - 33, L - 64, L - 65, L - 128, L - 129, L - 200}
    if w.window >= 0:
        keys |= set(range(L // 2 - 8, L // 2 + 8)) | {w.window, w.window + 1, 0, 1}
    kv_heads = sorted({h // (w.H // w.H_kv) for h in heads})
    kv_rows = [g * L + j for g in kv_heads for j in sorted(keys & set(range(L)))]
    return q_rows, kv_rows


@pytest.mark.parametrize("name", ["causal_128k_h4", "swa_gqa_16k", "causal_16k"])
def test_bwd_workload_sampled(name):
    w = WORKLOADS[name]
    announce(f"bwd workload {name} (sampled rows and keys)")
    q, k, v = workload_inputs(w)
    dout = make_dout(w.B, w.H, w.L, w.d, w.dtype, 8)
    res = gpu_fwd_bwd(q, k, v, dout, w.causal, w.window, w.scale)
    heads = sorted({0, w.H // 2, w.H - 1})
    q_rows, kv_rows = sampled_rows(w, heads, 11)
    ref = oracle.attention_bwd(q, k, v, dout, w.dtype, w.causal, w.window, w.scale,
                               q_rows=q_rows, kv_rows=kv_rows, with_abs=True)
    check_all(res, ref, w.dtype, w.L * (w.H // w.H_kv), name, q_rows=q_rows, kv_rows=kv_rows)


# ------------------------------------------------------------------ closed forms at full size
def visible_range(i, L, causal, window):
    lo = max(0, i - window) if window >= 0 else 0
    hi = i if causal else (min(L - 1, i + window) if window >= 0 else L - 1)
    return lo, hi


@pytest.mark.parametrize("name", ["causal_128k_h4", "swa_gqa_16k", "noncausal_2k_bf16"])
def test_bwd_zero_keys_full_size(name):
    """K = 0: every visible score is 0, so dq = 0 exactly (every term has a
    zero factor) and dv_j = sum over the rows i that see j of dO_i / |V(i)|,
    with sum|t| = the same sum of |dO_i| / |V(i)|: every key of every head
    is checked, at the workload's full size."""
    w = WORKLOADS[name]
    announce(f"bwd K=0 closed form {name}")
    q, k, v = workload_inputs(w)
    k = torch.zeros_like(k)
    dout = make_dout(w.B, w.H, w.L, w.d, w.dtype, 9)
    res = gpu_fwd_bwd(q, k, v, dout, w.causal, w.window, w.scale)
    assert torch.all(res["dq"] == 0), "dq must be exactly 0 when K = 0"
    L, group = w.L, w.H // w.H_kv
    i = np.arange(L)
    lo = np.maximum(0, i - w.window) if w.window >= 0 else np.zeros(L, np.int64)
    if w.causal:
        hi = i
    else:
        hi = np.minimum(L - 1, i + w.window) if w.window >= 0 else np.full(L, L - 1)
    count = (hi - lo + 1).astype(np.float64)
    g = dout.double().numpy()  # [B, H, L, d]
    for b in range(w.B):
        for kvh in range(w.H_kv):
            heads = g[b, kvh * group:(kvh + 1) * group]              # [group, L, d]
            contrib = (heads / count[None, :, None]).sum(axis=0)      # per row i
            contrib_abs = (np.abs(heads) / count[None, :, None]).sum(axis=0)
            # dv_j = sum over i with lo_i <= j <= hi_i: difference array over j
            diff = np.zeros((L + 1, w.d))
            diff_abs = np.zeros((L + 1, w.d))
            np.add.at(diff, lo, contrib)
            np.add.at(diff, hi + 1, -contrib)
            np.add.at(diff_abs, lo, contrib_abs)
            np.add.at(diff_abs, hi + 1, -contrib_abs)
            ref = np.cumsum(diff, axis=0)[:L]
            ref_abs = np.cumsum(diff_abs, axis=0)[:L]
            check_grad("dv", res["dv"][b, kvh], ref, np.abs(ref_abs), w.dtype, L * group,
                       f"{name} K=0 b={b} kv head {kvh}")


# ------------------------------------------------------------------ invariants
def test_bwd_deterministic_and_overwrites():
    """No atomics: repeated runs are bitwise equal, and every output element
    is written (outputs prefilled with NaN)."""
    B, H, H_kv, L, d = 1, 4, 2, 700, 64
    announce("bwd determinism")
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, H_kv, L, d, "f16", 21))
    g = make_dout(B, H, L, d, "f16", 21).to(DEV)
    out, lse = attn.forward(q, k, v, causal=True)
    first = None
    for _ in range(3):
        dq = torch.full_like(q, float("nan"))
        dk = torch.full_like(k, float("nan"))
        dv = torch.full_like(v, float("nan"))
        attn.backward(q, k, v, out, lse, g, causal=True, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize(DEV)
        cur = [t.cpu() for t in (dq, dk, dv)]
        assert all(torch.isfinite(t).all() for t in cur)
        if first is None:
            first = cur
        else:
            assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(first, cur))


def test_bwd_batch_independence():
    """A B=2 call equals two B=1 calls, bitwise."""
    B, H, H_kv, L, d = 2, 4, 1, 333, 128
    announce("bwd batch independence")
    q, k, v = make_qkv(B, H, H_kv, L, d, "bf16", 22)
    g = make_dout(B, H, L, d, "bf16", 22)
    both = gpu_fwd_bwd(q, k, v, g, True, 50, None)
    for b in range(B):
        one = gpu_fwd_bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], True, 50, None)
        for name in ("dq", "dk", "dv"):
            assert torch.equal(both[name][b:b + 1].view(torch.int16), one[name].view(torch.int16)), name


def test_bwd_workspace_contents():
    """The workspace holds -lse*log2(e) (fp32, bitwise) and -D = -dout.out
    per row (fp32 sum of 16-bit products), with zeros in the padding rows."""
    B, H, H_kv, L, d = 2, 3, 3, 100, 64
    announce("bwd workspace")
    q, k, v = make_qkv(B, H, H_kv, L, d, "f16", 23)
    g = make_dout(B, H, L, d, "f16", 23)
    res = gpu_fwd_bwd(q, k, v, g, False, -1, None)
    Lp = 128
    ws = res["ws"][:attn.attn_bwd_workspace_size(B, H, L)].view(torch.float32).reshape(B * H, 2, Lp)
    lse = res["lse"].reshape(B * H, L)
    want = -(lse * torch.tensor(LOG2E, dtype=torch.float32))
    assert torch.equal(ws[:, 0, :L], want)
    dsum = (res["out"].double() * g.double()).sum(-1).reshape(B * H, L)
    assert torch.allclose(-ws[:, 1, :L].double(), dsum, rtol=1e-5, atol=1e-5)
    assert torch.all(ws[:, :, L:] == 0)


def test_bwd_single_visible_key():
    """window = 0: P = 1 on the diagonal only, so dv = dO summed over the
    group's heads, and dq, dk vanish up to the fp32 evaluation of dP - D."""
    B, H, H_kv, L, d = 1, 4, 2, 300, 64
    announce("bwd one visible key")
    q, k, v = make_qkv(B, H, H_kv, L, d, "f16", 24)
    g = make_dout(B, H, L, d, "f16", 24)
    res = gpu_fwd_bwd(q, k, v, g, True, 0, 0.125)
    want_dv = g.double().reshape(B, H_kv, 2, L, d).sum(2).numpy()
    err = np.abs(res["dv"].double().numpy() - want_dv)
    floor = np.abs(round_to(want_dv, "f16") - want_dv)
    assert (err <= floor + 1e-3 * np.abs(want_dv) + ABS_SLACK).all()
    assert res["dq"].abs().max() <= ABS_SLACK and res["dk"].abs().max() <= ABS_SLACK


def test_bwd_side_stream_and_errors():
    B, H, L, d = 1, 2, 130, 64
    announce("bwd side stream / errors")
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, H, L, d, "f16", 25))
    g = make_dout(B, H, L, d, "f16", 25).to(DEV)
    out, lse = attn.forward(q, k, v, causal=True)
    ref = attn.backward(q, k, v, out, lse, g, causal=True)
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        side = attn.backward(q, k, v, out, lse, g, causal=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize(DEV)
    assert all(torch.equal(a, b) for a, b in zip(ref, side))
    with pytest.raises(ValueError):
        attn.backward(q, k, v, out, lse, g, causal=True, dq=q)          # dq aliases q
    with pytest.raises(ValueError):
        attn.backward(q, k, v, out, lse, g, window=-5)
    small = torch.empty(8, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        attn.backward(q, k, v, out, lse, g, workspace=small)


def test_bwd_rejects_strided_workspace():
    """A workspace view with enough elements but not contiguous is refused."""
    announce("bwd argument checks")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 2, 2, 100, 64, "f16", 5))
    out, lse = attn.forward(q, k, v, causal=True)
    need = attn.attn_bwd_workspace_size(1, 2, 100)
    strided = torch.empty(2 * need + 32, dtype=torch.uint8, device=DEV)[::2]
    with pytest.raises(ValueError):
        attn.backward(q, k, v, out, lse, torch.randn_like(out), causal=True, workspace=strided)
