"""The standard-attention comparator of bench.py --compare, on the GPU.

«Оптимизация внимания Flash», Workflow 1, Step 4 checks FlashAttention
against standard attention (matmul, softmax, matmul) in fp16 at batch 1, 8
heads, 512 tokens, head_dim 64, scale 1/8, and expects a max difference below
1e-3; the same check is made here with the comparator the benchmark times.
The comparator itself is first checked against the fp64 oracle, so the speed
and memory figures it produces are figures of a correct computation.
"""
import numpy as np
import pytest
import torch

import bench
import exact_io_aware_25_amd as attn
import oracle
from synth import WORKLOADS, workload_inputs
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_comparator_matches_oracle():
    announce("standard-attention comparator vs oracle")
    w = WORKLOADS["p2_accuracy"]
    q, k, v = workload_inputs(w)
    o = bench.standard_attention(q.to(DEV), k.to(DEV), v.to(DEV), True, w.scale)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, "f16", True, -1, w.scale, with_abs=True)
    # the comparator's own arithmetic: its fp16 product rounds each score
    # q.k once (relative 2^-11, at most 2^-11 * sabs_i in natural-log units;
    # the scale 1/8 is exact), and its softmax rounds each weight to fp16 (the
    # u of the bound); lse is not produced: pass the oracle's own
    check(o.cpu(), torch.from_numpy(ref[1]), ref, "f16", "comparator", vmax=float(v.abs().max()),
          rel_extra=2.0 ** -11 * ref[4])


def test_page_accuracy_check():
    """The page's own check: kernel vs fp16 standard attention, max |diff| < 1e-3."""
    announce("page accuracy check vs standard attention")
    w = WORKLOADS["p2_accuracy"]
    q, k, v = (t.to(DEV) for t in workload_inputs(w))
    flash, _ = attn.forward(q, k, v, causal=False, scale=w.scale)
    std = bench.standard_attention(q, k, v, False, w.scale)
    torch.cuda.synchronize()
    diff = float((flash.float() - std.float()).abs().max())
    print(f"max |flash - standard| = {diff:.3e}", flush=True)
    assert diff < 1e-3
