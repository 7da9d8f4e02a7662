"""rational_softmax_tiled_amd -- rational-softmax attention on AMD MI355X (gfx950).

A thin ctypes binding over ``libra_attn.so``.  The functions named like the C entry points
(``ra_attn_fwd``, ``ra_attn_fwd_counted``, ``ra_attn_bwd``, ``ra_attn_bwd_dq``,
``ra_attn_bwd_dkdv``, ``ra_attn_bwd_workspace_bytes``, ``ra_softmax_rows``,
``ra_softmax_rows_bwd``, ``ra_rope_neox``) only marshal arguments: tensors become device pointers, the stream
becomes a ``hipStream_t``.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and importing the compute functions without the built
library raises.

On top of them, ``ra_attention`` (a drop-in for ``scaled_dot_product_attention`` with
autograd) and ``ra_softmax`` allocate outputs with ``torch.empty`` and call the entry points
on the current stream.  Source of the operation: "Ra-Family: Rational Neural Architecture",
section 3 "Rational Attention & Softmax" (items ra_softmax and ra_attention).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "RA_F32", "RA_BF16", "RaError", "load_library", "library_path",
    "ra_status_string", "ra_attn_fwd", "ra_attn_fwd_counted", "ra_attn_bwd",
    "ra_attn_bwd_dq", "ra_attn_bwd_dkdv", "ra_attn_bwd_workspace_bytes", "ra_softmax_rows",
    "ra_softmax_rows_bwd", "ra_rope_neox", "ra_rope",
    "attn_fwd", "attn_bwd", "ra_attention", "ra_softmax",
]

RA_F32 = 0
RA_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libra_attn.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class RaError(RuntimeError):
    """A non-zero ra_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = ra_status_string(status)
        if status == 10:  # RA_ERR_HIP
            msg += f" (hipError {load_library().ra_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libra_attn.so (built by ``python -m rational_softmax_tiled_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built: run `python -m rational_softmax_tiled_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ra_status_string.argtypes = [ctypes.c_int]
    lib.ra_status_string.restype = ctypes.c_char_p
    lib.ra_last_hip_error.argtypes = []
    lib.ra_last_hip_error.restype = ctypes.c_int
    lib.ra_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp]
    lib.ra_attn_fwd.restype = ctypes.c_int
    lib.ra_attn_fwd_counted.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                        _i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp, _vp]
    lib.ra_attn_fwd_counted.restype = ctypes.c_int
    lib.ra_attn_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.ra_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ra_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                                ctypes.c_int, _vp]
    lib.ra_attn_bwd.restype = ctypes.c_int
    lib.ra_attn_bwd_dq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                   _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_int, _vp]
    lib.ra_attn_bwd_dq.restype = ctypes.c_int
    lib.ra_attn_bwd_dkdv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                     _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, _vp]
    lib.ra_attn_bwd_dkdv.restype = ctypes.c_int
    lib.ra_softmax_rows.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_int, _vp]
    lib.ra_softmax_rows.restype = ctypes.c_int
    lib.ra_softmax_rows_bwd.argtypes = [_vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp]
    lib.ra_softmax_rows_bwd.restype = ctypes.c_int
    lib.ra_rope_neox.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
                                 ctypes.c_int, _vp]
    lib.ra_rope_neox.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------ entry points (same names)

def ra_status_string(status: int) -> str:
    return load_library().ra_status_string(int(status)).decode()


def ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, stream=None) -> int:
    return load_library().ra_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(stats), B, Hq,
                                      Hkv, Nq, Nk, D, int(causal), float(scale), int(dtype),
                                      _stream(stream))


def ra_attn_fwd_counted(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, counters,
                        stream=None) -> int:
    return load_library().ra_attn_fwd_counted(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(stats), B,
                                              Hq, Hkv, Nq, Nk, D, int(causal), float(scale),
                                              int(dtype), _ptr(counters), _stream(stream))


def ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, dtype) -> int:
    return load_library().ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, int(dtype))


def ra_attn_bwd(q, k, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                Nk, D, causal, scale, dtype, stream=None) -> int:
    return load_library().ra_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(stats),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                      int(workspace_bytes), B, Hq, Hkv, Nq, Nk, D, int(causal),
                                      float(scale), int(dtype), _stream(stream))


def ra_attn_bwd_dq(q, k, v, o, d_o, stats, dq, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, D,
                   causal, scale, dtype, stream=None) -> int:
    return load_library().ra_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                                         _ptr(stats), _ptr(dq), _ptr(workspace),
                                         int(workspace_bytes), B, Hq, Hkv, Nq, Nk, D, int(causal),
                                         float(scale), int(dtype), _stream(stream))


def ra_attn_bwd_dkdv(q, k, v, d_o, stats, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk,
                     D, causal, scale, dtype, stream=None) -> int:
    return load_library().ra_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(stats),
                                           _ptr(dk), _ptr(dv), _ptr(workspace),
                                           int(workspace_bytes), B, Hq, Hkv, Nq, Nk, D,
                                           int(causal), float(scale), int(dtype), _stream(stream))


def ra_softmax_rows(x, p, rows, cols, dtype, stream=None) -> int:
    return load_library().ra_softmax_rows(_ptr(x), _ptr(p), rows, cols, int(dtype),
                                          _stream(stream))


def ra_softmax_rows_bwd(x, dp, dx, rows, cols, dtype, stream=None) -> int:
    return load_library().ra_softmax_rows_bwd(_ptr(x), _ptr(dp), _ptr(dx), rows, cols, int(dtype),
                                              _stream(stream))


# ------------------------------------------------------------ tensor-level helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check(status: int, where: str):
    if status != 0:
        raise RaError(status, where)


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("inconsistent q/k/v shapes")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    return B, Hq, Hkv, Nq, Nk, D


def attn_fwd(q, k, v, causal: bool, scale: Optional[float] = None, with_stats: bool = True):
    """Allocate O (and stats) and run ra_attn_fwd on the current stream."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device=q.device) if with_stats else None
    _check(ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, _dtype_code(q)),
           "ra_attn_fwd")
    return o, stats


def attn_bwd(q, k, v, o, d_o, stats, causal: bool, scale: Optional[float] = None):
    """Allocate dQ, dK, dV and a workspace and run ra_attn_bwd on the current stream."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    d_o = d_o.contiguous()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = _dtype_code(q)
    nbytes = ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(ra_attn_bwd(q, k, v, o, d_o, stats, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                       causal, scale, code), "ra_attn_bwd")
    return dq, dk, dv


def _autograd_fn():
    import torch

    class _RaAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            o, stats = attn_fwd(q, k, v, causal, scale, with_stats=True)
            ctx.save_for_backward(q, k, v, o, stats)
            ctx.causal, ctx.scale = causal, scale
            return o

        @staticmethod
        def backward(ctx, d_o):
            q, k, v, o, stats = ctx.saved_tensors
            dq, dk, dv = attn_bwd(q, k, v, o, d_o, stats, ctx.causal, ctx.scale)
            return dq, dk, dv, None, None

    return _RaAttentionFn


_FN = None


def ra_attention(q, k, v, is_causal: bool = False, scale: Optional[float] = None):
    """Rational-softmax attention, a drop-in for scaled_dot_product_attention (no attn_mask,
    no dropout).  q: [B, Hq, N, D], k, v: [B, Hkv, N, D] with Hq a multiple of Hkv; bf16 or
    fp32 contiguous device tensors; D in {64, 128}.  Differentiable."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return _FN.apply(q, k, v, bool(is_causal), scale)


def ra_rope_neox(x, y, positions, mats, N, D, theta, inverse, dtype, stream=None) -> int:
    return load_library().ra_rope_neox(_ptr(x), _ptr(y), _ptr(positions), mats, N, D,
                                       float(theta), int(bool(inverse)), int(dtype),
                                       _stream(stream))


def _rope_apply(x, theta, positions, inverse):
    import torch
    xc = x.contiguous()
    N, D = xc.shape[-2], xc.shape[-1]
    mats = xc.numel() // max(N * D, 1)
    pos = None
    if positions is not None:
        pos = torch.as_tensor(positions, dtype=torch.int32, device=xc.device).contiguous()
        if pos.numel() != N:
            raise ValueError("positions must have one entry per row (axis -2)")
    y = torch.empty_like(xc)
    _check(ra_rope_neox(xc, y, pos, mats, N, D, theta, inverse, _dtype_code(xc)), "ra_rope_neox")
    return y


class _RopeFn:
    _cls = None

    @classmethod
    def get(cls):
        if cls._cls is None:
            import torch

            class Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, x, theta, positions, inverse):
                    ctx.args = (theta, positions, inverse)
                    return _rope_apply(x, theta, positions, inverse)

                @staticmethod
                def backward(ctx, dy):
                    theta, positions, inverse = ctx.args
                    return _rope_apply(dy, theta, positions, not inverse), None, None, None

            cls._cls = Fn
        return cls._cls


def ra_rope(x, theta: float = 10000.0, positions=None, inverse: bool = False):
    """NEOX (split-halves) rotary embedding along the last axis of x [..., N, D], positions on
    axis -2 (default 0..N-1), with autograd (the gradient is the inverse rotation)."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("ra_rope supports float32 and bfloat16")
    return _RopeFn.get().apply(x, float(theta), positions, bool(inverse))


def _softmax_rows_2d(x):
    """x as a contiguous [rows, cols] view with the softmax axis last."""
    cols = x.shape[-1]
    return x.contiguous(), x.numel() // max(cols, 1), cols


class _RaSoftmaxFn:
    """autograd.Function over ra_softmax_rows / ra_softmax_rows_bwd (built lazily: torch is
    imported only when a tensor API is used)."""
    _cls = None

    @classmethod
    def get(cls):
        if cls._cls is None:
            import torch

            class Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, xt):
                    x2, rows, cols = _softmax_rows_2d(xt)
                    p = torch.empty_like(x2)
                    _check(ra_softmax_rows(x2, p, rows, cols, _dtype_code(x2)), "ra_softmax_rows")
                    ctx.save_for_backward(x2)
                    return p

                @staticmethod
                def backward(ctx, dp):
                    (x2,) = ctx.saved_tensors
                    dp2, rows, cols = _softmax_rows_2d(dp.to(x2.dtype))
                    dx = torch.empty_like(x2)
                    _check(ra_softmax_rows_bwd(x2, dp2, dx, rows, cols, _dtype_code(x2)),
                           "ra_softmax_rows_bwd")
                    return dx

            cls._cls = Fn
        return cls._cls


def ra_softmax(x, dim: int = -1):
    """ra_softmax along ``dim`` with autograd; -inf entries are masked (p = 0, dx = 0)."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("ra_softmax supports float32 and bfloat16")
    xt = x.movedim(dim, -1)
    return _RaSoftmaxFn.get().apply(xt).movedim(-1, dim)
