"""The workloads the tests and the benchmark use are the pages' own shapes,
and the oracle meets the pages' accuracy check against standard attention."""
import json
import os

import numpy as np
import torch

import oracle
from synth import WORKLOADS, workload_inputs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_cases.json")))


def _shape(w):
    return dict(B=w.B, H=w.H, L=w.L, d=w.d, dtype=w.dtype, causal=w.causal, window=w.window,
                scale=w.scale)


def test_workloads_follow_the_pages():
    acc = GOLDEN["p2_accuracy"]
    assert _shape(WORKLOADS["p2_accuracy"]) == {k: acc[k] for k in _shape(WORKLOADS["p2_accuracy"])}
    speed = GOLDEN["p2_speed_shape"]
    for name in ("noncausal_2k_f16", "noncausal_2k_bf16"):
        w = WORKLOADS[name]
        assert (w.B, w.H, w.L, w.d, w.causal, w.scale) == (
            speed["B"], speed["H"], speed["L"], speed["d"], speed["causal"], speed["scale"])
    sweep = GOLDEN["p1_length_sweep"]
    swept = sorted(w.L for w in WORKLOADS.values()
                   if w.causal and w.window < 0 and w.d == sweep["d"] and w.B == sweep["B"])
    assert sorted(set(swept)) == sweep["lengths"]
    assert {w.H for w in WORKLOADS.values() if w.L == 131072} == set(sweep["H"])
    fp8 = GOLDEN["p2_fp8_shape"]
    assert _shape(WORKLOADS["fp8_fa3_4k"]) == {k: fp8[k] for k in _shape(WORKLOADS["fp8_fa3_4k"])}


def test_oracle_meets_page_accuracy_bound(oracle_lib):
    """Standard attention in fp32 (materialised scores, softmax, @V) lies within
    the page's 1e-3 bound of the fp64 oracle at the page's accuracy shape."""
    w = WORKLOADS["p2_accuracy"]
    q, k, v = workload_inputs(w)
    o, _ = oracle.attention(q, k, v, w.dtype, w.causal, w.window, w.scale, lib=oracle_lib)
    qf, kf, vf = (t.float() for t in (q, k, v))
    std = torch.softmax(qf @ kf.transpose(-1, -2) * w.scale, dim=-1) @ vf
    assert np.max(np.abs(std.double().numpy() - o)) < GOLDEN["p2_accuracy"]["max_abs_bound"]
