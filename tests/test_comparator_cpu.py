"""The standard-attention comparator of bench.py against the oracle, on the
CPU in fp32: the plain three-step version and the version split into
(batch, head, row block) operations that long sequences use."""
import numpy as np

import bench
import oracle
from synth import make_qkv


def test_comparator_plain_and_split(oracle_lib):
    q, k, v = make_qkv(2, 3, 3, 70, 64, "f16", 11)
    for causal in (False, True):
        ref, _ = oracle.attention(q, k, v, "f16", causal, -1, 0.125, lib=oracle_lib)
        plain = bench.standard_attention(q.float(), k.float(), v.float(), causal, 0.125)
        assert np.max(np.abs(plain.double().numpy() - ref)) < 1e-5
        split = bench.standard_attention(q.float(), k.float(), v.float(), causal, 0.125, rows_per_step=16,
                                         split_above=0)
        assert np.max(np.abs(split.double().numpy() - ref)) < 1e-5
