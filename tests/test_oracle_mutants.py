"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, changes one line into a plausible
mistake (a dropped term, a wrong sign or bound, a wrong index or operand),
compiles the copy into a temporary directory and runs the pins against it.
At least one pin must fail for every mistake.  Runs on the CPU only.
"""
import os

import pytest

import oracle
import oracle_bwd_pins
import oracle_pins

MUTANTS = {
    "causal_excludes_diagonal": ("if (causal && j > i)", "if (causal && j >= i)"),
    "window_off_by_one": ("if (i - j > window)", "if (i - j >= window)"),
    "window_ignores_right_side": ("if (!causal && j - i > window)", "if (0 && j - i > window)"),
    "gqa_interleaved_heads": ("return h / (H / H_kv);", "return h % H_kv;"),
    "lse_without_max": ("lse[t] = m + log(l);", "lse[t] = log(l);"),
    "scale_dropped": ("s[j] = sc * dot;", "s[j] = dot;"),
    "key_transposed": ("dot += qd[c] * kd[j * d + c];", "dot += qd[c] * kd[c * L + j];"),
    "value_row_reversed": ("acc[c] += p * vd[j * d + c];", "acc[c] += p * vd[(L - 1 - j) * d + c];"),
    "no_normalisation": ("out[t * d + c] = acc[c] / l;", "out[t * d + c] = acc[c];"),
    "f16_subnormal_exponent": ("mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    "f16_bias": ("expo - 25); /*", "expo - 24); /*"),
    "bf16_shift": ("(uint32_t)bits << 16;", "(uint32_t)bits << 15;"),
    "default_scale_wrong": ("return (float)(1.0 / sqrt((double)d));", "return (float)(1.0 / (double)d);"),
    "max_not_subtracted_from_lse_side": ("double p = exp(s[j] - m);", "double p = exp(s[j]);"),
    "sum_over_one_row_only": ("l += p;", "l = p;"),
    "f8_bias": ("mag = ldexp((double)(8 + frac), expo - 10);", "mag = ldexp((double)(8 + frac), expo - 9);"),
    "f8_subnormal_exponent": ("mag = ldexp((double)frac, -9);", "mag = ldexp((double)frac, -10);"),
    "f8_top_exponent_is_nan": ("else if (expo == 15 && frac == 7)", "else if (expo == 15)"),
    "abs_weights_signed": ("acc_abs[c] += p * fabs(vd[j * d + c]);", "acc_abs[c] += p * vd[j * d + c];"),
    "abs_weights_unnormalised": ("oabs[t * d + c] = acc_abs[c] / l;", "oabs[t * d + c] = acc_abs[c];"),
    "score_abs_signed": ("dot_abs += fabs(qd[c] * kd[j * d + c]);", "dot_abs += qd[c] * kd[j * d + c];"),
    "visible_count_off_by_one": ("aux[0] = (double)count;", "aux[0] = (double)(count - 1);"),
    # backward pass
    "bwd_dq_uses_values": ("acc[c] += dS * kd[j * d + c];", "acc[c] += dS * vd[j * d + c];"),
    "bwd_dq_scale_dropped": ("dq[t * d + c] = sc * acc[c];", "dq[t * d + c] = acc[c];"),
    "bwd_dk_scale_dropped": ("dk[t * d + c] = sc * ak[c];", "dk[t * d + c] = ak[c];"),
    "bwd_dv_unnormalised": ("av[c] += P * doi[c];", "av[c] += P * l[gr] * doi[c];"),
    "bwd_delta_unnormalised": ("D += dod[c] * (acc[c] / l);", "D += dod[c] * acc[c];"),
    "bwd_dk_sign": ("ak[c] += dS * qi[c];", "ak[c] -= dS * qi[c];"),
    "bwd_dk_reads_first_head": ("const int64_t gr = hh * L + i;", "const int64_t gr = i;"),
    "bwd_group_heads_dropped": ("for (int hh = 0; hh < group; ++hh) {", "for (int hh = 0; hh < 1; ++hh) {"),
    "bwd_stats_rows_skipped": ("needed[hh * L + i] = 1;", "needed[hh * L + i] = needed[hh * L + i];"),
    "bwd_dq_row_of_first_head": ("const int64_t gr = (bh % H - h0) * L + r % L;", "const int64_t gr = r % L;"),
    "bwd_abs_dv_signed": ("av_abs[c] += fabs(P * doi[c]);", "av_abs[c] += P * doi[c];"),
    "bwd_abs_dq_without_key": ("acc_abs[c] += fabs(dS * kd[j * d + c]);", "acc_abs[c] += fabs(dS);"),
    "bwd_abs_dk_unscaled": ("dk_abs[t * d + c] = sc * ak_abs[c];", "dk_abs[t * d + c] = ak_abs[c];"),
    "bwd_rho_not_rooted": ("*rho_out = sqrt(R);", "*rho_out = R;"),
    "bwd_dsens_dk_without_weight": ("ak_P[c] += P * rho[gr] * fabs(qi[c]);", "ak_P[c] += rho[gr] * fabs(qi[c]);"),
    "bwd_dsens_dq_without_rho": ("dq_dsens[t * d + c] = sc * rho[gr] * acc_P[c];", "dq_dsens[t * d + c] = sc * acc_P[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load_library(oracle.compile_library(path, os.path.join(tmp_path, "mutant.so")))
    caught = []
    for pin in oracle_pins.ALL_PINS + oracle_bwd_pins.ALL_BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as exc:
            caught.append(pin.__name__)
            if len(caught) >= 1:
                break
    assert caught, f"no pin caught the planted mistake {name}"


PAGED_MUTANTS = {
    "paged_top_left_alignment": ("p = n - Lq + i", "p = i"),
    "paged_page_index": ("cache[block_table[b, j // block_size], g, j % block_size]",
                         "cache[block_table[b, j % block_size], g, j // block_size]"),
    "paged_window_off_by_one": ("lo = 0 if window < 0 else max(0, p - window)",
                                "lo = 0 if window < 0 else max(0, p - window + 1)"),
    "paged_scale_dropped": ("s = sc * (keys[lo:p + 1] @ qd[b, h, i])", "s = keys[lo:p + 1] @ qd[b, h, i]"),
    "paged_last_key_dropped": ("s = sc * (keys[lo:p + 1] @ qd[b, h, i])", "s = sc * (keys[lo:p] @ qd[b, h, i])"),
    "paged_no_normalisation": ("out[b, h, i] = (w @ vals[lo:p + 1]) / w.sum()", "out[b, h, i] = w @ vals[lo:p + 1]"),
    "paged_lse_without_max": ("lse[b, h, i] = m + np.log(w.sum())", "lse[b, h, i] = np.log(w.sum())"),
    "paged_gqa_interleaved": ("for h in range(g * group, (g + 1) * group):", "for h in range(g, H, H_kv):"),
    "paged_abs_weights_signed": ("oabs[b, h, i] = (w @ np.abs(vals[lo:p + 1])) / w.sum()",
                                 "oabs[b, h, i] = (w @ vals[lo:p + 1]) / w.sum()"),
    "paged_count_whole_sequence": ("count[b, h, i] = p + 1 - lo", "count[b, h, i] = n"),
    "paged_score_abs_unscaled": ("sabs[b, h, i] = sc * (np.abs(keys[lo:p + 1]) @ np.abs(qd[b, h, i])).max()",
                                 "sabs[b, h, i] = (np.abs(keys[lo:p + 1]) @ np.abs(qd[b, h, i])).max()"),
}


@pytest.mark.parametrize("name", sorted(PAGED_MUTANTS))
def test_planted_paged_mistake_is_caught(name, tmp_path):
    import importlib.util

    import oracle_paged_pins
    from oracle import paged
    old, new = PAGED_MUTANTS[name]
    src = open(paged.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    path = os.path.join(tmp_path, "paged_mutant.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("paged_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in oracle_paged_pins.ALL_PAGED_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
