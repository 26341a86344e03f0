"""Error bounds the GPU parity tests hold the kernels to (no GPU needed).

``derived_bounds`` states, per element, how far the kernels' fp32/16-bit
arithmetic can move O and lse from the exact fp64 values, given the oracle's
softmax weights applied to |v|, visible-key counts and score sizes.  It is
checked against a CPU model of that arithmetic in
``test_derived_bound_cpu.py``.
"""
import numpy as np
import torch

from synth import TORCH_DTYPES


def round_to(x, dtype):
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype]).double().numpy()


# unit roundoff of the 16-bit types (the softmax weights are rounded to the
# input type before the second product)
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
EPS32 = 2.0 ** -24


def derived_bounds(ref_o, ref_lse, oabs, count, sabs, dtype, vmax, rel_extra=None):
    """Per-element bound on |O_gpu - O| and per-row bound on |lse_gpu - lse|,
    derived from the arithmetic of the kernels.

    The kernels form every score as an fp32 sum of d exact products of 16-bit
    inputs (error at most d * 2^-24 * sabs_i in natural-log units, sabs_i =
    max_j scale * sum_c |q_ic k_jc| from the oracle), take each weight with
    fp32 exp2 (2^-22 covers it and the fp32 shift), round it to the input type
    for the second product (unit roundoff u; fp16 weights below 2^-14 are
    subnormal, an absolute error of at most 2^-25 against a row sum >= 1,
    since the key that set the reference has weight 1), and accumulate O and
    the row sum in fp32 over n_i keys (n_i * 2^-24 relative).  A relative
    error delta_j of every weight moves O_ic by at most
    max|delta| * sum_j P_ij |v_jc - O_ic| <= max|delta| (A_ic + |O_ic|), with
    A_ic = sum_j P_ij |v_jc| from the oracle, whether the row sum uses the
    rounded weights (fp16) or the fp32 ones (bf16, decode).  So the kernel's
    fp32 value x has |x - O| <= e_ic with

        e_ic = (u + 2^-22 + (n_i + d sabs_i) 2^-24) (A_ic + |O_ic|) + n_i 2^-25 (vmax + |O_ic|),

    and rounding x to the output type gives |round(x) - O| <= floor + 2 e_ic
    (round(x) is at least as close to x as round(O) is).  lse moves by the
    relative error of the row sum plus the fp32 evaluation of
    (m + log2 l) ln 2.  ``rel_extra`` (per row) adds a computation's own
    score error, e.g. scores rounded to 16 bits.  A 1 % margin covers
    second-order terms.
    """
    u = UNIT_ROUNDOFF[dtype]
    d = ref_o.shape[-1]
    n = np.asarray(count, np.float64)[..., None]
    sa = np.asarray(sabs, np.float64)[..., None]
    rel = u + 2.0 ** -22 + (n + d * sa) * EPS32
    if rel_extra is not None:
        rel = rel + np.asarray(rel_extra, np.float64)[..., None]
    o_abs = np.abs(ref_o)
    e = 1.01 * (rel * (oabs + o_abs) + n * 2.0 ** -25 * (vmax + o_abs))
    floor = np.abs(round_to(ref_o, dtype) - ref_o)
    o_bound = floor + 2 * e + 1e-12
    eta = rel[..., 0] + count * 2.0 ** -25
    lse_bound = 1.01 * (eta + 2.0 ** -22 * (1.5 * np.abs(ref_lse) + 1))
    return o_bound, lse_bound
