"""Exact IO-aware attention (forward, backward, paged decode) for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI declared in ``include/attn.h``.  The
names match the C entry points; this module only marshals arguments.  Every
step of the computation runs in the HIP kernels of ``libattn_gfx950.so``;
there is no fallback: if the library is missing, every call raises.

``forward`` and ``backward`` are conveniences for PyTorch users: they check
the tensors, allocate the outputs (and the backward's workspace) with torch
on the inputs' device and launch on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libattn_gfx950.so")

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_HEAD_DIM = 3
ATTN_ERR_WINDOW = 4
ATTN_ERR_ALIAS = 5
ATTN_ERR_LAUNCH = 6
ATTN_ERR_SIZE = 7
ATTN_ERR_FLAG = 8
ATTN_ERR_SCALE = 9
ATTN_ERR_ALIGN = 10
ATTN_ERR_SCRATCH = 11

EXPORTS = ("attn_fwd", "attn_fwd_bf16", "attn_fwd_fp8", "attn_bwd", "attn_bwd_bf16", "attn_bwd_workspace_size",
           "attn_decode", "attn_decode_bf16", "attn_decode_workspace_size", "attn_decode_noalloc",
           "attn_launch_shape", "attn_status_string", "attn_resolve_scale")

_lib = None


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def library():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIBRARY)
        sig = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
               ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        for name in ("attn_fwd", "attn_fwd_bf16", "attn_fwd_fp8"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = sig
        bsig = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_void_p]
        for name in ("attn_bwd", "attn_bwd_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = bsig
        dsig = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 10 + [ctypes.c_float, ctypes.c_void_p]
        for name in ("attn_decode", "attn_decode_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = dsig
        fn = lib.attn_decode_noalloc
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 10 + [ctypes.c_float, ctypes.c_void_p]
        lib.attn_decode_workspace_size.restype = ctypes.c_size_t
        lib.attn_decode_workspace_size.argtypes = [ctypes.c_int] * 6
        lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 3
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_resolve_scale.restype = ctypes.c_float
        lib.attn_resolve_scale.argtypes = [ctypes.c_float, ctypes.c_int]
        lib.attn_launch_shape.restype = ctypes.c_int
        lib.attn_launch_shape.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(ctypes.c_int)] * 2
        _lib = lib
    return _lib


def attn_fwd(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream) -> int:
    """fp16 entry point; pointers are integer device addresses, stream a hipStream_t address."""
    return library().attn_fwd(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream)


def attn_fwd_bf16(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream) -> int:
    """bf16 entry point; same arguments as ``attn_fwd``."""
    return library().attn_fwd_bf16(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream)


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, H_kv, L, d, causal, window, scale,
             stream) -> int:
    """fp16 backward entry point; pointers are integer device addresses."""
    return library().attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, H_kv, L, d, causal,
                              window, scale, stream)


def attn_bwd_bf16(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, H_kv, L, d, causal, window, scale,
                  stream) -> int:
    """bf16 backward entry point; same arguments as ``attn_bwd``."""
    return library().attn_bwd_bf16(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, H_kv, L, d, causal,
                                   window, scale, stream)


def attn_bwd_workspace_size(B, H, L) -> int:
    return int(library().attn_bwd_workspace_size(int(B), int(H), int(L)))


def attn_decode(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv, Lq, d, block_size,
                max_blocks_per_seq, num_blocks, max_seq_len, window, scale, stream) -> int:
    """fp16 decode entry point; pointers are integer device addresses."""
    return library().attn_decode(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv, Lq,
                                 d, block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale, stream)


def attn_decode_bf16(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv, Lq, d,
                     block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale, stream) -> int:
    """bf16 decode entry point; same arguments as ``attn_decode``."""
    return library().attn_decode_bf16(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv,
                                      Lq, d, block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale,
                                      stream)


def attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, out, lse, B, H, H_kv, Lq, d, block_size,
                        max_blocks_per_seq, num_blocks, max_seq_len, window, scale, stream) -> int:
    """fp16 decode into the library's static scratch (no workspace argument,
    nothing allocated); pointers are integer device addresses."""
    return library().attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, out, lse, B, H, H_kv, Lq, d,
                                         block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale,
                                         stream)


def attn_decode_workspace_size(B, H, H_kv, Lq, d, max_seq_len) -> int:
    return int(library().attn_decode_workspace_size(int(B), int(H), int(H_kv), int(Lq), int(d), int(max_seq_len)))


def attn_fwd_fp8(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream) -> int:
    """fp8 (E4M3) entry point; out is bf16."""
    return library().attn_fwd_fp8(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream)


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def attn_resolve_scale(scale: float, d: int) -> float:
    return float(library().attn_resolve_scale(float(scale), int(d)))


def attn_launch_shape(B, H, L, d, causal, window):
    """(waves per key-range group, key-range groups) attn_fwd would use; raises on bad arguments."""
    waves, splits = ctypes.c_int(), ctypes.c_int()
    B, H, L, d, window = _int32(B=B, H=H, L=L, d=d, window=window)
    st = library().attn_launch_shape(B, H, L, d, int(causal), window, ctypes.byref(waves), ctypes.byref(splits))
    if st != ATTN_OK:
        raise ValueError(attn_status_string(st))
    return waves.value, splits.value


def forward(q, k, v, causal: bool = False, window: int = -1, scale=None, out=None, lse=None,
            stream=None):
    """Attention of torch tensors q [B,H,L,d], k and v [B,H_kv,L,d] (fp16, bf16 or
    float8_e4m3fn, on the GPU).

    Returns (out [B,H,L,d] of q's dtype -- bf16 for fp8 inputs --, lse [B,H,L] fp32).  ``scale=None``
    selects 1/sqrt(d); an explicit scale must be finite and > 0 (ValueError
    otherwise).  ``out``/``lse`` may be given to write into existing
    tensors.  Launches on ``stream`` (default: torch's current stream).
    """
    import torch

    scale_value = _scale_arg(scale)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B, H, L, d] and [B, H_kv, L, d]")
    if (q.dtype not in (torch.float16, torch.bfloat16, torch.float8_e4m3fn) or k.dtype != q.dtype
            or v.dtype != q.dtype):
        raise ValueError("q, k, v must share one dtype: float16, bfloat16 or float8_e4m3fn")
    out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    if tuple(k.shape) != (B, H_kv, L, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if (tuple(out.shape) != tuple(q.shape) or out.dtype != out_dtype or not out.is_contiguous()
            or out.device != q.device):
        raise ValueError("out must be a contiguous tensor shaped like q (bf16 for fp8 inputs)")
    if (tuple(lse.shape) != (B, H, L) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, L]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = {torch.float16: attn_fwd, torch.bfloat16: attn_fwd_bf16, torch.float8_e4m3fn: attn_fwd_fp8}[q.dtype]
    B, H, H_kv, L, d, window = _int32(B=B, H=H, H_kv=H_kv, L=L, d=d, window=window)
    with torch.cuda.device(q.device):
        status = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, H_kv, L, d, int(bool(causal)), int(window),
                    scale_value, stream.cuda_stream)
    _check(status)
    return out, lse


def _scale_arg(scale):
    """The scale argument for the C ABI: None selects 1/sqrt(d) (passed as 0,
    the ABI's request for the default); an explicit scale must be a finite
    number > 0.  The ABI itself would silently replace a zero, negative or NaN
    scale by the default, which would compute a different function than the
    caller asked for, so the binding refuses them."""
    if scale is None:
        return 0.0
    value = float(scale)
    if not (value > 0.0 and value != float("inf")):
        raise ValueError(f"scale must be None (1/sqrt(d)) or a finite number > 0, got {scale!r}")
    return value


def _int32(**values):
    """The given integers, checked to fit the C ABI's 32-bit int arguments.

    ctypes would otherwise pass an out-of-range Python int wrapped modulo
    2^32, which could turn an invalid argument into a valid but different one.
    """
    for name, value in values.items():
        if not -2 ** 31 <= int(value) < 2 ** 31:
            raise ValueError(f"{name}={value} does not fit a 32-bit int argument")
    return tuple(int(v) for v in values.values())


def _check(status):
    if status != ATTN_OK:
        msg = attn_status_string(status)
        if status in (1, 2, 3, 4, 5, 8, 9, 10, 11):
            raise ValueError(msg)
        raise AttnError(status, msg)


def backward(q, k, v, out, lse, dout, causal: bool = False, window: int = -1, scale=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attention for the upstream gradient ``dout``.

    q, k, v, causal, window, scale as given to ``forward`` (``scale=None``
    selects 1/sqrt(d); an explicit scale must be finite and > 0); out and lse as it
    returned them; dout like out.  Outputs are allocated unless given;
    ``workspace`` (uint8, ``attn_bwd_workspace_size`` bytes) likewise.
    Launches on ``stream`` (default: torch's current stream).
    """
    import torch

    scale_value = _scale_arg(scale)
    tensors = (q, k, v, out, dout)
    if any(t.dim() != 4 for t in tensors):
        raise ValueError("q, k, v, out, dout must be 4-D")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in tensors):
        raise ValueError("q, k, v, out, dout must share one dtype, float16 or bfloat16")
    if not q.is_cuda or any(t.device != q.device for t in tensors + (lse,)):
        raise ValueError("all tensors must be on the same GPU device")
    if not all(t.is_contiguous() for t in tensors + (lse,)):
        raise ValueError("all tensors must be contiguous")
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    if (tuple(k.shape) != (B, H_kv, L, d) or tuple(v.shape) != tuple(k.shape)
            or tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape)):
        raise ValueError("shape mismatch between q, k, v, out, dout")
    if tuple(lse.shape) != (B, H, L) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 tensor [B, H, L]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if (tuple(t.shape) != tuple(like.shape) or t.dtype != like.dtype or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like {name[1:]}")
    need = attn_bwd_workspace_size(B, H, L)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if (workspace.numel() * workspace.element_size() < need or workspace.device != q.device
            or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = attn_bwd if q.dtype == torch.float16 else attn_bwd_bf16
    B, H, H_kv, L, d, window = _int32(B=B, H=H, H_kv=H_kv, L=L, d=d, window=window)
    with torch.cuda.device(q.device):
        status = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, H, H_kv, L, d,
                    int(bool(causal)), int(window), scale_value, stream.cuda_stream)
    _check(status)
    return dq, dk, dv


def decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, window: int = -1, scale=None,
           out=None, lse=None, workspace=None, stream=None):
    """Attention of the Lq newest tokens of each sequence over a paged KV cache.

    q [B,H,Lq,d]; k_cache, v_cache [num_blocks,H_kv,block_size,d] (fp16 or
    bf16, on the GPU); block_table int32 [B, max_blocks]; seq_lens int32 [B]
    on the GPU; ``max_seq_len`` bounds seq_lens (host int); ``scale=None``
    selects 1/sqrt(d), an explicit scale must be finite and > 0.  Returns (out
    [B,H,Lq,d], lse [B,H,Lq] fp32).  Launches on ``stream`` (default: torch's
    current stream).
    """
    import torch

    scale_value = _scale_arg(scale)
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B,H,Lq,d] and the caches [num_blocks,H_kv,block_size,d]")
    if q.dtype not in (torch.float16, torch.bfloat16) or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share one dtype, float16 or bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [B, max_blocks] and seq_lens int32 [B]")
    tensors = (q, k_cache, v_cache, block_table, seq_lens)
    if not q.is_cuda or any(t.device != q.device for t in tensors):
        raise ValueError("all tensors must be on the same GPU device")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous")
    B, H, Lq, d = q.shape
    num_blocks, H_kv, block_size, _ = k_cache.shape
    if (tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d or block_table.shape[0] != B
            or tuple(seq_lens.shape) != (B,)):
        raise ValueError("shape mismatch between q, caches, block_table and seq_lens")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    if (tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous()
            or out.device != q.device):
        raise ValueError("out must be a contiguous tensor like q, on q's device")
    if (tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Lq] on q's device")
    B, H, H_kv, Lq, d, block_size, max_blocks, num_blocks, max_seq_len, window = _int32(
        B=B, H=H, H_kv=H_kv, Lq=Lq, d=d, block_size=block_size, max_blocks=block_table.shape[1],
        num_blocks=num_blocks, max_seq_len=max_seq_len, window=window)
    need = attn_decode_workspace_size(B, H, H_kv, Lq, d, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if (workspace.numel() * workspace.element_size() < need or workspace.device != q.device
            or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = attn_decode if q.dtype == torch.float16 else attn_decode_bf16
    with torch.cuda.device(q.device):
        status = fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                    seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), B, H, H_kv, Lq, d,
                    block_size, max_blocks, num_blocks, max_seq_len, window,
                    scale_value, stream.cuda_stream)
    _check(status)
    return out, lse
