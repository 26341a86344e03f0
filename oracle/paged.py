"""fp64 oracle for attention of a few new queries over a paged KV cache.

TEST INFRASTRUCTURE ONLY (like the rest of this package).

Decoding reads the whole KV cache for every generated token, which makes HBM
bandwidth the limit («Что такое memory-efficient attention для long context
на 8x H100?», section 1, key limits); PagedAttention keeps that cache in
fixed-size blocks reached through a page table (same page, section 3).  The
operation is still the attention of the forward definition, for the last Lq
positions of each sequence:

* sequence b has n_b = seq_lens[b] tokens; its key/value j lives in physical
  block block_table[b, j // block_size], row j % block_size;
* its Lq new queries sit at positions p_i = n_b - Lq + i (i < Lq): the last
  query is aligned with the last key (reading: bottom-right alignment, the
  only one under which a generated token sees its whole context);
* query i of head h sees key j iff j <= p_i and, with a window, p_i - j <=
  window (the causal and sliding-window rules of «Оптимизация внимания
  Flash», Workflow 2, Steps 2-3, applied at position p_i), using K/V head
  h / (H / H_kv);
* O and the natural-log lse as in the forward definition.

Everything is fp64 after decoding the 16-bit inputs exactly; the page gather is
plain indexing and the softmax is written out row by row.
"""
from __future__ import annotations

import numpy as np

import oracle


def gather_sequence(cache: np.ndarray, block_table: np.ndarray, b: int, g: int, n: int,
                    block_size: int) -> np.ndarray:
    """Rows 0..n-1 of K/V head g of sequence b from a [num_blocks, H_kv,
    block_size, d] cache, in key order."""
    j = np.arange(n)
    return cache[block_table[b, j // block_size], g, j % block_size]


def decode_attention(q, k_cache, v_cache, block_table, seq_lens, dtype: str, window: int = -1,
                     scale: float = 0.0, lib=None, with_abs: bool = False):
    """q: [B, H, Lq, d]; caches: [num_blocks, H_kv, block_size, d] (16-bit
    patterns or torch tensors); block_table: int [B, max_blocks]; seq_lens:
    int [B] (each >= Lq).  Returns (out [B, H, Lq, d], lse [B, H, Lq]) fp64.
    With ``with_abs`` also (oabs, count, sabs): the softmax weights applied
    to |v| (shaped like out), and per query the number of visible keys and
    max_j scale * sum_c |q_c k_jc| (shaped like lse)."""
    qd = oracle.decode(q, dtype, lib=lib)
    kbits = oracle._bits(k_cache)
    vbits = oracle._bits(v_cache)
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B, H, Lq, d = qd.shape
    H_kv, block_size = kbits.shape[1], kbits.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    sc = oracle.resolve_scale(scale, d, lib=lib)
    group = H // H_kv
    out = np.zeros((B, H, Lq, d))
    lse = np.zeros((B, H, Lq))
    oabs = np.zeros((B, H, Lq, d))
    count = np.zeros((B, H, Lq))
    sabs = np.zeros((B, H, Lq))
    for b in range(B):
        n = int(lens[b])
        if n < Lq:
            raise ValueError("every sequence must hold at least its Lq new tokens")
        for g in range(H_kv):
            # gather the 16-bit rows in key order, then decode them exactly
            keys = oracle.decode(gather_sequence(kbits, bt, b, g, n, block_size), dtype, lib=lib)
            vals = oracle.decode(gather_sequence(vbits, bt, b, g, n, block_size), dtype, lib=lib)
            for h in range(g * group, (g + 1) * group):
                for i in range(Lq):
                    p = n - Lq + i
                    lo = 0 if window < 0 else max(0, p - window)
                    s = sc * (keys[lo:p + 1] @ qd[b, h, i])
                    m = s.max()
                    w = np.exp(s - m)
                    out[b, h, i] = (w @ vals[lo:p + 1]) / w.sum()
                    lse[b, h, i] = m + np.log(w.sum())
                    if with_abs:
                        oabs[b, h, i] = (w @ np.abs(vals[lo:p + 1])) / w.sum()
                        count[b, h, i] = p + 1 - lo
                        sabs[b, h, i] = sc * (np.abs(keys[lo:p + 1]) @ np.abs(qd[b, h, i])).max()
    if with_abs:
        return out, lse, oabs, count, sabs
    return out, lse
