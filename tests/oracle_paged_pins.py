"""Pins of the paged-KV decode oracle (oracle/paged.py) to facts other than
itself.  Each pin takes the module (the real one or a copy with a planted
mistake) and raises AssertionError on disagreement:

* contiguous pages: the last Lq rows of the C forward oracle (itself pinned)
  for the same sequence, so the bottom-right position of the new queries,
  the causal rule and the window are fixed by an independent implementation;
* invariances: shuffling the physical blocks together with the page table,
  changing the block size, and computing a ragged batch one sequence at a
  time leave every output bitwise unchanged; GQA equals K/V heads repeated;
* closed forms: with one visible key (window 0) O is that key's value and
  lse = scale q.k; with K = 0, O is the mean of the visible values and
  lse = ln(number of visible keys).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from synth import make_qkv


def paged_cache(k, v, block_size, seed=None, extra_blocks=0):
    """Pack contiguous k, v [1, H_kv, n, d] into [num_blocks, H_kv, block_size, d]
    caches; with a seed the physical blocks are shuffled (and the table says
    where each logical block went).  Returns (k_cache, v_cache, table [1, nb])."""
    _, H_kv, n, d = k.shape
    nb = (n + block_size - 1) // block_size
    total = nb + extra_blocks
    phys = np.arange(total)
    if seed is not None:
        phys = np.random.default_rng(seed).permutation(total)
    kc = torch.zeros(total, H_kv, block_size, d, dtype=k.dtype)
    vc = torch.zeros_like(kc)
    for lb in range(nb):
        rows = slice(lb * block_size, min(n, (lb + 1) * block_size))
        cnt = rows.stop - rows.start
        kc[phys[lb], :, :cnt] = k[0, :, rows]
        vc[phys[lb], :, :cnt] = v[0, :, rows]
    return kc, vc, phys[:nb][None].astype(np.int32)


def pin_paged_vs_forward(mod):
    for (H, H_kv, n, d, Lq, window, dtype, bs, seed) in [
        (4, 2, 100, 64, 3, -1, "f16", 16, 1), (4, 4, 70, 128, 1, -1, "bf16", 32, 2),
        (8, 2, 129, 64, 5, 7, "f16", 16, 3), (2, 1, 40, 64, 16, 0, "bf16", 64, 4),
        (4, 1, 17, 64, 16, 3, "f16", 16, 5), (1, 1, 1, 64, 1, -1, "f16", 16, 6),
    ]:
        q, k, v = make_qkv(1, H, H_kv, n, d, dtype, seed)
        kc, vc, bt = paged_cache(k, v, bs, seed=seed)
        scale = float(np.float32(1 / math.sqrt(d)))
        o, l = mod.decode_attention(q[:, :, n - Lq:], kc, vc, bt, [n], dtype, window, scale)
        fo, fl = oracle.attention(q, k, v, dtype, True, window, scale)
        case = f"H={H}/{H_kv} n={n} d={d} Lq={Lq} window={window} {dtype} block={bs}"
        assert np.max(np.abs(o - fo[:, :, n - Lq:])) <= 1e-12, case
        assert np.max(np.abs(l - fl[:, :, n - Lq:])) <= 1e-12, case
        # the weights applied to |v|, the visible-key count and the score bound
        # against the C oracle's (themselves pinned against brute force)
        _, _, oabs, cnt, sabs = mod.decode_attention(q[:, :, n - Lq:], kc, vc, bt, [n], dtype, window, scale,
                                                     with_abs=True)
        _, _, foabs, fcnt, fsabs = oracle.attention(q, k, v, dtype, True, window, scale, with_abs=True)
        assert np.max(np.abs(oabs - foabs[:, :, n - Lq:])) <= 1e-12, case
        assert np.array_equal(cnt, fcnt[:, :, n - Lq:]), case
        assert np.max(np.abs(sabs - fsabs[:, :, n - Lq:])) <= 1e-12 * max(1.0, float(fsabs.max())), case


def pin_paged_invariances(mod):
    H, H_kv, d, Lq = 4, 2, 64, 2
    lens = [33, 100, 2, 64]
    seqs = [make_qkv(1, H, H_kv, n, d, "f16", 20 + i) for i, n in enumerate(lens)]
    # one sequence at a time, contiguous pages, block size 16
    alone = []
    for q, k, v in seqs:
        kc, vc, bt = paged_cache(k, v, 16)
        alone.append(mod.decode_attention(q[:, :, -Lq:], kc, vc, bt, [k.shape[2]], "f16", 9, 0.125))
    for bs in (16, 32):
        # the whole ragged batch in one shuffled pool
        parts = [paged_cache(k, v, bs) for _, k, v in seqs]
        offs = np.cumsum([0] + [p[0].shape[0] for p in parts])
        kc = torch.cat([p[0] for p in parts])
        vc = torch.cat([p[1] for p in parts])
        perm = np.random.default_rng(bs).permutation(kc.shape[0])
        inv = np.argsort(perm)
        kc, vc = kc[perm], vc[perm]
        width = max(p[2].shape[1] for p in parts)
        bt = np.zeros((len(seqs), width), np.int32)
        for i, p in enumerate(parts):
            bt[i, :p[2].shape[1]] = inv[p[2][0] + offs[i]]
        q = torch.cat([s[0][:, :, -Lq:] for s in seqs])
        o, l = mod.decode_attention(q, kc, vc, bt, lens, "f16", 9, 0.125)
        for i, (ao, al) in enumerate(alone):
            assert np.array_equal(o[i:i + 1], ao) and np.array_equal(l[i:i + 1], al), f"block {bs} seq {i}"
    # GQA vs K/V heads repeated
    q, k, v = seqs[1]
    kc, vc, bt = paged_cache(k, v, 16, seed=3)
    o, l = mod.decode_attention(q[:, :, -Lq:], kc, vc, bt, [100], "f16", -1, 0.125)
    kr, vr, btr = paged_cache(k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1), 16, seed=3)
    o2, l2 = mod.decode_attention(q[:, :, -Lq:], kr, vr, btr, [100], "f16", -1, 0.125)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def pin_paged_closed_forms(mod):
    H, H_kv, n, d, Lq = 4, 2, 50, 64, 3
    q, k, v = make_qkv(1, H, H_kv, n, d, "bf16", 30)
    kc, vc, bt = paged_cache(k, v, 16, seed=30)
    o, l = mod.decode_attention(q[:, :, -Lq:], kc, vc, bt, [n], "bf16", 0, 0.1)
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    sc = float(np.float32(0.1))
    for h in range(H):
        for i in range(Lq):
            p = n - Lq + i
            assert np.array_equal(o[0, h, i], vd[0, h // 2, p])
            assert abs(l[0, h, i] - sc * qd[0, h, p] @ kd[0, h // 2, p]) <= 1e-12
    kz, vz, btz = paged_cache(torch.zeros_like(k), v, 16)
    for window in (-1, 5):
        o, l = mod.decode_attention(q[:, :, -Lq:], kz, vz, btz, [n], "bf16", window, 0.1)
        for i in range(Lq):
            p = n - Lq + i
            lo = 0 if window < 0 else max(0, p - window)
            mean = vd[0, :, lo:p + 1].mean(axis=1)          # [H_kv, d]
            for h in range(H):
                assert np.max(np.abs(o[0, h, i] - mean[h // 2])) <= 1e-12
                assert abs(l[0, h, i] - math.log(p + 1 - lo)) <= 1e-12


ALL_PAGED_PINS = [pin_paged_vs_forward, pin_paged_invariances, pin_paged_closed_forms]
