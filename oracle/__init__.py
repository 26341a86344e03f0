"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the GPU library and its Python
binding never do, and nothing here imports them.

Two independent implementations of the same plain definition live here:

* ``attn_oracle.c`` (loaded through ctypes): row-by-row fp64 attention that
  materialises each query row's scores, parallel over rows with OpenMP.  It
  is the oracle the GPU path is compared with.
* ``brute.py``: whole-matrix NumPy fp64 attention with an explicit boolean
  mask, used only to check the C oracle on tiny inputs.

``attn_oracle.c`` also holds the backward pass (``attention_bwd``): the
gradients of the same definition with respect to q, k and v for an upstream
gradient dO, in fp64.

The definition both follow is softmax(scale * Q K^T + mask) V with the
natural-log logsumexp of each row («Оптимизация внимания Flash», Workflow 1,
Steps 2 and 4; Workflow 2, Steps 2-3; «Что такое memory-efficient attention
для long context на 8x H100?», section 2).  The header of ``attn_oracle.c``
states the formula and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "_attn_oracle.so")

DTYPES = {"f16": 0, "fp16": 0, "float16": 0, "bf16": 1, "bfloat16": 1, "f8": 2, "f8e4m3": 2}

_lib = None


def compile_library(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the C oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           *extra_flags, "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def build(force: bool = False) -> str:
    """Build ``_attn_oracle.so`` next to its source if missing or stale."""
    stale = (not os.path.exists(LIBRARY)
             or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
    if force or stale:
        compile_library()
    return LIBRARY


def _bind(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_attn.restype = ctypes.c_int
    lib.oracle_attn.argtypes = [u16p, u16p, u16p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                i64p, ctypes.c_int64, f64p, f64p, f64p, f64p, ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [u16p, u16p, u16p, u16p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                    i64p, ctypes.c_int64, i64p, ctypes.c_int64,
                                    f64p, f64p, f64p, f64p, f64p, f64p, f64p, f64p, ctypes.c_int]
    lib.oracle_decode.restype = None
    lib.oracle_decode.argtypes = [u16p, f64p, ctypes.c_int64, ctypes.c_int]
    lib.oracle_f8e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_f8e4m3_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_resolve_scale.restype = ctypes.c_float
    lib.oracle_resolve_scale.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.oracle_visible.restype = ctypes.c_int
    lib.oracle_visible.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    return lib


def load_library(path: str):
    """Load a compiled oracle library (the default one or a test-built variant)."""
    return _bind(ctypes.CDLL(path))


def _default_lib():
    global _lib
    if _lib is None:
        _lib = load_library(build())
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits(a) -> np.ndarray:
    """16-bit patterns of a float16/bfloat16 torch tensor or a uint16/float16
    array; an fp8 (float8_e4m3fn) tensor or uint8 array gives its bytes
    widened to uint16 (the oracle's "f8" dtype reads the low byte)."""
    if hasattr(a, "detach"):  # torch tensor, CPU
        import torch
        a = a.detach().cpu().contiguous()
        a = a.view(torch.uint8).numpy() if a.element_size() == 1 else a.view(torch.int16).numpy()
    if isinstance(a, np.ndarray) and a.dtype == np.uint8:
        return np.ascontiguousarray(a).astype(np.uint16)
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit float patterns, got {a.dtype}")
    return a


def decode(bits, dtype: str, lib=None) -> np.ndarray:
    """Exact fp64 values of 16-bit float patterns (same shape)."""
    lib = lib or _default_lib()
    b = _bits(bits)
    out = np.empty(b.shape, np.float64)
    lib.oracle_decode(_ptr(b, ctypes.c_uint16), _ptr(out, ctypes.c_double), b.size, DTYPES[dtype])
    return out


def resolve_scale(scale: float, d: int, lib=None) -> float:
    """The fp32 scale the definition uses: ``scale`` or, if <= 0/NaN, fp32(1/sqrt(d))."""
    lib = lib or _default_lib()
    return float(lib.oracle_resolve_scale(float(scale), int(d)))


def attention(q, k, v, dtype: str, causal: bool, window: int = -1, scale: float = 0.0,
              rows=None, threads: int = 0, lib=None, with_abs: bool = False):
    """Exact attention of 16-bit inputs in fp64.

    q: [B,H,L,d]; k, v: [B,H_kv,L,d] (torch tensors or uint16 arrays of bit
    patterns).  ``rows``: optional flat row ids (b*H + h)*L + i; when given,
    the result holds those rows only, in that order.
    Returns (out, lse): fp64 [B,H,L,d] and [B,H,L], or [n, d] and [n].
    With ``with_abs``, returns (out, lse, oabs, count, sabs): oabs shaped like
    out holds sum_j P_ij |v_jc| (the softmax weights applied to |v|); count
    and sabs shaped like lse hold each row's number of visible keys and
    max_j scale * sum_c |q_ic k_jc|.
    """
    lib = lib or _default_lib()
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, H, L, d = qb.shape
    H_kv = kb.shape[1]
    if kb.shape != (B, H_kv, L, d) or vb.shape != kb.shape:
        raise ValueError(f"shape mismatch q{qb.shape} k{kb.shape} v{vb.shape}")
    if rows is None:
        n = B * H * L
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
        if n and (rows_arr.min() < 0 or rows_arr.max() >= B * H * L):
            raise ValueError("row id out of range")
        rows_ptr = _ptr(rows_arr, ctypes.c_int64)
    out = np.zeros((n, d), np.float64)
    lse = np.zeros((n,), np.float64)
    oabs = np.zeros((n, d), np.float64) if with_abs else None
    aux = np.zeros((n, 2), np.float64) if with_abs else None
    st = lib.oracle_attn(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                         DTYPES[dtype], B, H, H_kv, L, d, int(bool(causal)), int(window), float(scale),
                         rows_ptr, n, _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
                         _ptr(oabs, ctypes.c_double) if with_abs else None,
                         _ptr(aux, ctypes.c_double) if with_abs else None, int(threads))
    if st != 0:
        raise ValueError(f"oracle_attn failed with status {st}")
    if rows is None:
        out, lse = out.reshape(B, H, L, d), lse.reshape(B, H, L)
        if with_abs:
            oabs, aux = oabs.reshape(B, H, L, d), aux.reshape(B, H, L, 2)
    if with_abs:
        return out, lse, oabs, aux[..., 0].copy(), aux[..., 1].copy()
    return out, lse


def _row_ids(rows, total):
    if rows is None:
        return None, total, None
    arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if arr.size and (arr.min() < 0 or arr.max() >= total):
        raise ValueError("row id out of range")
    return arr, arr.size, _ptr(arr, ctypes.c_int64)


def attention_bwd(q, k, v, dout, dtype: str, causal: bool, window: int = -1, scale: float = 0.0,
                  q_rows=None, kv_rows=None, threads: int = 0, lib=None, with_abs: bool = False):
    """Gradients of exact attention of 16-bit inputs, in fp64.

    q, dout: [B,H,L,d]; k, v: [B,H_kv,L,d] (torch tensors or uint16 arrays of
    bit patterns).  ``q_rows``: optional flat ids (b*H + h)*L + i of the dq
    rows wanted; ``kv_rows``: optional flat ids (b*H_kv + g)*L + j of the
    dk/dv rows wanted (an empty list skips that part).
    Returns (dq, dk, dv): fp64 [B,H,L,d], [B,H_kv,L,d], [B,H_kv,L,d], or
    [n_q, d], [n_kv, d], [n_kv, d] for the requested rows.  With
    ``with_abs``, returns ((dq, dk, dv), (dq_abs, dk_abs, dv_abs),
    (dq_dsens, dk_dsens)): the second triple holds, for each element, the sum
    of the absolute values of the terms whose sum it is; the third, the
    sensitivity of dq and dk to the row terms D_i = dO_i.O_i (if each D_i
    moves by at most eps times the root-sum-square of its terms, the element
    moves by at most eps times this).
    """
    lib = lib or _default_lib()
    qb, kb, vb, gb = _bits(q), _bits(k), _bits(v), _bits(dout)
    B, H, L, d = qb.shape
    H_kv = kb.shape[1]
    if kb.shape != (B, H_kv, L, d) or vb.shape != kb.shape or gb.shape != qb.shape:
        raise ValueError(f"shape mismatch q{qb.shape} k{kb.shape} v{vb.shape} dout{gb.shape}")
    qa, nq, qp = _row_ids(q_rows, B * H * L)
    ka, nk, kp = _row_ids(kv_rows, B * H_kv * L)
    dq = np.zeros((nq, d), np.float64)
    dk = np.zeros((nk, d), np.float64)
    dv = np.zeros((nk, d), np.float64)
    absd = [np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)] if with_abs else [None] * 3
    sens = [np.zeros_like(dq), np.zeros_like(dk)] if with_abs else [None] * 2
    aptr = [_ptr(a, ctypes.c_double) if a is not None else None for a in absd + sens]
    st = lib.oracle_attn_bwd(_ptr(qb, ctypes.c_uint16), _ptr(kb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                             _ptr(gb, ctypes.c_uint16), DTYPES[dtype], B, H, H_kv, L, d,
                             int(bool(causal)), int(window), float(scale), qp, nq, kp, nk,
                             _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                             _ptr(dv, ctypes.c_double), *aptr, int(threads))
    if st != 0:
        raise ValueError(f"oracle_attn_bwd failed with status {st}")
    grads = [dq, dk, dv]
    if q_rows is None:
        grads[0] = dq.reshape(B, H, L, d)
        if with_abs:
            absd[0] = absd[0].reshape(B, H, L, d)
            sens[0] = sens[0].reshape(B, H, L, d)
    if kv_rows is None:
        for i in (1, 2):
            grads[i] = grads[i].reshape(B, H_kv, L, d)
            if with_abs:
                absd[i] = absd[i].reshape(B, H_kv, L, d)
        if with_abs:
            sens[1] = sens[1].reshape(B, H_kv, L, d)
    if with_abs:
        return tuple(grads), tuple(absd), tuple(sens)
    return tuple(grads)
