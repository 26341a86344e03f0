"""Whole-matrix NumPy fp64 attention with an explicit mask.

TEST INFRASTRUCTURE ONLY: used to check the C oracle on tiny inputs.  It
builds the full L x L score matrix per head -- the "standard attention" the
pages compare FlashAttention against («Оптимизация внимания Flash», Workflow
1, Step 2 and Step 4) -- so it is only meant for small L.

The mask is built from whole-matrix conditions (lower triangle for causal, a
band for the window: «Оптимизация внимания Flash», Workflow 2, Step 3), and
fewer K/V heads are handled by repeating each K/V head over its group of
query heads, which is how grouped/multi-query attention shares them
(«Оптимизация внимания Flash», Workflow 2, Step 3).
"""
from __future__ import annotations

import numpy as np


def mask_matrix(L: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [L, L] matrix, True where query row i may attend key column j."""
    allowed = np.ones((L, L), dtype=bool)
    if causal:
        allowed &= np.tril(np.ones((L, L), dtype=bool))          # j <= i
    if window >= 0:
        band_below = np.triu(np.ones((L, L), dtype=bool), -window)  # j >= i - window
        allowed &= band_below
        if not causal:
            allowed &= np.tril(np.ones((L, L), dtype=bool), window)  # j <= i + window
    return allowed


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, window: int,
              scale: float, with_abs: bool = False):
    """fp64 attention. q: [B,H,L,d]; k, v: [B,H_kv,L,d] (float64 values).

    Returns (out [B,H,L,d], lse [B,H,L]); with ``with_abs`` also the weights
    applied to |v| ([B,H,L,d]), the number of visible keys per row and
    max_j scale * sum_c |q_ic k_jc| over the visible keys ([B,H,L] each).
    """
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    group = H // H_kv
    k_full = np.repeat(k, group, axis=1)
    v_full = np.repeat(v, group, axis=1)
    scores = scale * np.matmul(q, np.swapaxes(k_full, -1, -2))       # [B,H,L,L]
    scores = np.where(mask_matrix(L, causal, window), scores, -np.inf)
    row_max = scores.max(axis=-1, keepdims=True)
    weights = np.exp(scores - row_max)
    total = weights.sum(axis=-1, keepdims=True)
    out = np.matmul(weights, v_full) / total
    lse = (row_max + np.log(total))[..., 0]
    if not with_abs:
        return out, lse
    allowed = mask_matrix(L, causal, window)
    oabs = np.matmul(weights, np.abs(v_full)) / total
    count = np.broadcast_to(allowed.sum(axis=-1).astype(np.float64), (B, H, L))
    score_abs = scale * np.matmul(np.abs(q), np.swapaxes(np.abs(k_full), -1, -2))
    sabs = np.where(allowed, score_abs, -np.inf).max(axis=-1)
    return out, lse, oabs, count, sabs
