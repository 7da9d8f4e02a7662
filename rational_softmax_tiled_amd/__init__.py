"""rational_softmax_tiled_amd -- rational-softmax attention on AMD MI355X (gfx950).

A thin ctypes binding over ``libra_attn.so``.  The functions named like the C entry points
(``ra_attn_fwd``, ``ra_attn_fwd_masked``, ``ra_attn_fwd_counted``, ``ra_attn_bwd``,
``ra_attn_bwd_masked``, ``ra_attn_bwd_dq``, ``ra_attn_bwd_dkdv``, ``ra_attn_bwd_workspace_bytes``,
``ra_attn_bwd_noalloc``,
``ra_attn_decode``, ``ra_attn_decode_workspace_bytes``, ``ra_softmax_rows``,
``ra_softmax_rows_bwd``, ``ra_rope_neox``) only marshal arguments: tensors
become device pointers, a mask becomes an ``ra_mask`` descriptor, the stream becomes a
``hipStream_t``.  Every step of the computation runs in the library's HIP kernels;
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
    "RA_F32", "RA_BF16", "RA_CAUSAL_NONE", "RA_CAUSAL_TOP_LEFT", "RA_CAUSAL_BOTTOM_RIGHT",
    "RA_MASK_NONE", "RA_MASK_BOOL", "RA_MASK_ADD", "RaMask", "RaError", "load_library",
    "library_path", "ra_status_string", "ra_attn_fwd", "ra_attn_fwd_masked",
    "ra_attn_fwd_counted", "ra_attn_bwd", "ra_attn_bwd_masked",
    "ra_attn_bwd_dq", "ra_attn_bwd_dkdv", "ra_attn_bwd_workspace_bytes", "ra_attn_bwd_noalloc",
    "ra_attn_decode",
    "ra_attn_decode_workspace_bytes", "attn_decode", "ra_softmax_rows",
    "ra_softmax_rows_bwd", "ra_rope_neox", "ra_rope", "ra_attn_fwd_rope", "ra_attn_bwd_rope",
    "attn_fwd", "attn_bwd", "attn_fwd_rope", "attn_bwd_rope", "ra_attention", "ra_attention_rope",
    "ra_softmax",
]

RA_F32 = 0
RA_BF16 = 1
RA_CAUSAL_NONE, RA_CAUSAL_TOP_LEFT, RA_CAUSAL_BOTTOM_RIGHT = 0, 1, 2
RA_MASK_NONE, RA_MASK_BOOL, RA_MASK_ADD = 0, 1, 2


class RaMask(ctypes.Structure):
    """The C ``ra_mask`` descriptor: data pointer, kind, element strides over (b, h, i, j)."""
    _fields_ = [("data", ctypes.c_void_p), ("kind", ctypes.c_int),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64)]

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
    _mp = ctypes.POINTER(RaMask)
    lib.ra_attn_fwd_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_int, _mp, _vp]
    lib.ra_attn_fwd_masked.restype = ctypes.c_int
    lib.ra_attn_bwd_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_int, _mp, _vp]
    lib.ra_attn_bwd_masked.restype = ctypes.c_int
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
    lib.ra_attn_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                        _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_int, _vp]
    lib.ra_attn_bwd_noalloc.restype = ctypes.c_int
    lib.ra_attn_decode_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.ra_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.ra_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i64, _i64,
                                   _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                                   ctypes.c_int, _vp]
    lib.ra_attn_decode.restype = ctypes.c_int
    lib.ra_softmax_rows.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_int, _vp]
    lib.ra_softmax_rows.restype = ctypes.c_int
    lib.ra_softmax_rows_bwd.argtypes = [_vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp]
    lib.ra_softmax_rows_bwd.restype = ctypes.c_int
    lib.ra_rope_neox.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
                                 ctypes.c_int, _vp]
    lib.ra_rope_neox.restype = ctypes.c_int
    lib.ra_attn_fwd_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_double,
                                     _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, _mp, _vp]
    lib.ra_attn_fwd_rope.restype = ctypes.c_int
    lib.ra_attn_bwd_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp, _vp, ctypes.c_double, _i64, _i64, _i64,
                                     _i64, _i64, _i64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                     _mp, _vp]
    lib.ra_attn_bwd_rope.restype = ctypes.c_int
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


def _mask_struct(mask, kind, strides):
    """A pointer to an RaMask (None for kind RA_MASK_NONE).  A NULL ``mask`` with another kind
    is passed on, so the library reports it (RA_ERR_NULLPTR)."""
    if kind == RA_MASK_NONE:
        return None
    sb, sh, sq, sk = (int(x) for x in strides)
    return ctypes.pointer(RaMask(_ptr(mask), int(kind), sb, sh, sq, sk))


def ra_attn_fwd_masked(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, mask,
                       mask_kind, mask_strides, stream=None) -> int:
    """ra_attn_fwd_masked; ``mask`` (tensor or address), ``mask_kind`` (RA_MASK_*) and
    ``mask_strides`` (element strides over batch, query head, query row, key) form the
    ra_mask descriptor."""
    return load_library().ra_attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(stats), B,
                                             Hq, Hkv, Nq, Nk, D, int(causal), float(scale),
                                             int(dtype), _mask_struct(mask, mask_kind, mask_strides),
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


def ra_attn_bwd_masked(q, k, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                       Nq, Nk, D, causal, scale, dtype, mask, mask_kind, mask_strides,
                       stream=None) -> int:
    return load_library().ra_attn_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                                             _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _ptr(workspace), int(workspace_bytes), B, Hq, Hkv, Nq,
                                             Nk, D, int(causal), float(scale), int(dtype),
                                             _mask_struct(mask, mask_kind, mask_strides),
                                             _stream(stream))


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


def ra_attn_bwd_noalloc(q, k, v, o, d_o, stats, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D, causal, scale,
                        dtype, stream=None) -> int:
    return load_library().ra_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                                              _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq,
                                              Hkv, Nq, Nk, D, int(causal), float(scale),
                                              int(dtype), _stream(stream))


def ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, dtype) -> int:
    return load_library().ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, int(dtype))


def ra_attn_decode(q, k, v, o, stats, seqlens, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, D,
                   causal, scale, dtype, stream=None) -> int:
    return load_library().ra_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(stats),
                                         _ptr(seqlens), _ptr(workspace), int(workspace_bytes), B,
                                         Hq, Hkv, Nq, Nk, D, int(causal), float(scale),
                                         int(dtype), _stream(stream))


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


def attn_decode(q, k_cache, v_cache, seqlens=None, causal=False, scale: Optional[float] = None,
                with_stats: bool = False):
    """Decode step: q [B, Hq, Nq, D] (bf16 or fp32, (Hq / Hkv) * Nq <= 32) against the caches
    k_cache, v_cache [B, Hkv, Nk, D], sample b using its first seqlens[b] keys (int32 device
    tensor [B], or None for all).  ``causal``: see causal_code ("bottom_right": query i is
    position seqlens[b] - Nq + i).  Allocates O (and stats) and a workspace; runs
    ra_attn_decode on the current stream.  Forward only."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k_cache, v_cache)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device=q.device) if with_stats else None
    lens = None
    if seqlens is not None:
        lens = torch.as_tensor(seqlens, dtype=torch.int32, device=q.device).contiguous()
        if tuple(lens.shape) != (B,):
            raise ValueError(f"seqlens must be [B] = [{B}]")
    code = _dtype_code(q)
    nbytes = ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(ra_attn_decode(q, k_cache, v_cache, o, stats, lens, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                          causal_code(causal), scale, code), "ra_attn_decode")
    return (o, stats) if with_stats else o


def causal_code(is_causal) -> int:
    """RA_CAUSAL_* for False / True ("top_left", scaled_dot_product_attention's is_causal) /
    "bottom_right" (or the integer codes)."""
    if is_causal is None or is_causal is False or (isinstance(is_causal, int) and is_causal == 0):
        return RA_CAUSAL_NONE
    if is_causal is True or is_causal == "top_left" or (isinstance(is_causal, int) and is_causal == 1):
        return RA_CAUSAL_TOP_LEFT
    if is_causal == "bottom_right" or (isinstance(is_causal, int) and is_causal == 2):
        return RA_CAUSAL_BOTTOM_RIGHT
    raise ValueError(f"is_causal must be False, True, 'top_left' or 'bottom_right', not {is_causal!r}")


def mask_descriptor(q, k, attn_mask=None, key_padding_mask=None):
    """(tensor, RA_MASK_* kind, element strides) for the library, or None.

    ``attn_mask`` follows scaled_dot_product_attention: broadcastable to [B, Hq, Nq, Nk];
    boolean (True = attend) or of q's dtype (added to the scaled scores, -inf masks).  It is
    passed as a strided view (broadcast dimensions get stride 0), not copied.
    ``key_padding_mask``: [B, Nk], 1 / True = attend, 0 / False = ignore (the CrossAttention
    polarity, the inverse of torch's nn.MultiheadAttention key_padding_mask); a non-boolean
    one becomes a boolean [B, Nk] tensor.  At most one of the two."""
    import torch
    if attn_mask is not None and key_padding_mask is not None:
        raise ValueError("pass attn_mask or key_padding_mask, not both")
    B, Hq, Nq, _ = q.shape
    Nk = k.shape[2]
    if key_padding_mask is not None:
        kpm = key_padding_mask
        if tuple(kpm.shape) != (B, Nk):
            raise ValueError(f"key_padding_mask must be [B, Nk] = [{B}, {Nk}], got {tuple(kpm.shape)}")
        if kpm.dtype not in (torch.bool, torch.uint8):
            kpm = kpm != 0
        if kpm.device != q.device:
            raise ValueError("key_padding_mask must be on the device of q")
        return kpm, RA_MASK_BOOL, (kpm.stride(0), 0, 0, kpm.stride(1))
    if attn_mask is None:
        return None
    if attn_mask.device != q.device:
        raise ValueError("attn_mask must be on the device of q")
    if attn_mask.dtype == torch.bool:
        kind = RA_MASK_BOOL
    elif attn_mask.dtype == q.dtype:
        kind = RA_MASK_ADD
    else:
        raise TypeError(f"attn_mask must be bool or {q.dtype}, not {attn_mask.dtype}")
    m = attn_mask.expand(B, Hq, Nq, Nk)
    return m, kind, tuple(m.stride())


def attn_fwd(q, k, v, causal, scale: Optional[float] = None, with_stats: bool = True, mask=None):
    """Allocate O (and stats) and run ra_attn_fwd (ra_attn_fwd_masked with ``mask``, a
    mask_descriptor) on the current stream.  ``causal``: see causal_code."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device=q.device) if with_stats else None
    cc = causal_code(causal)
    if mask is None:
        _check(ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, cc, scale, _dtype_code(q)),
               "ra_attn_fwd")
    else:
        _check(ra_attn_fwd_masked(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, cc, scale,
                                  _dtype_code(q), *mask), "ra_attn_fwd_masked")
    return o, stats


def attn_bwd(q, k, v, o, d_o, stats, causal, scale: Optional[float] = None, mask=None):
    """Allocate dQ, dK, dV and a workspace and run ra_attn_bwd (ra_attn_bwd_masked with
    ``mask``) on the current stream."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    d_o = d_o.contiguous()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = _dtype_code(q)
    nbytes = ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    cc = causal_code(causal)
    if mask is None:
        _check(ra_attn_bwd(q, k, v, o, d_o, stats, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                           cc, scale, code), "ra_attn_bwd")
    else:
        _check(ra_attn_bwd_masked(q, k, v, o, d_o, stats, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq,
                                  Nk, D, cc, scale, code, *mask), "ra_attn_bwd_masked")
    return dq, dk, dv


def _autograd_fn():
    import torch

    class _RaAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, mask):
            o, stats = attn_fwd(q, k, v, causal, scale, with_stats=True, mask=mask)
            ctx.save_for_backward(q, k, v, o, stats)
            ctx.causal, ctx.scale, ctx.mask = causal, scale, mask
            return o

        @staticmethod
        def backward(ctx, d_o):
            q, k, v, o, stats = ctx.saved_tensors
            dq, dk, dv = attn_bwd(q, k, v, o, d_o, stats, ctx.causal, ctx.scale, mask=ctx.mask)
            return dq, dk, dv, None, None, None

    return _RaAttentionFn


_FN = None


def ra_attention(q, k, v, attn_mask=None, is_causal=False, scale: Optional[float] = None,
                 key_padding_mask=None):
    """Rational-softmax attention, a drop-in for scaled_dot_product_attention (no dropout).

    q: [B, Hq, Nq, D], k, v: [B, Hkv, Nk, D] with Hq a multiple of Hkv; bf16 or fp32
    contiguous device tensors; D in {64, 128}.  ``is_causal``: False, True (= "top_left", key
    j <= query i) or "bottom_right" (j <= i + Nk - Nq).  ``attn_mask`` / ``key_padding_mask``:
    see mask_descriptor; they combine with is_causal.  A query row with no allowed key gives a
    zero output.  Differentiable in q, k and v (the masks get no gradient)."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    for m in (attn_mask, key_padding_mask):
        if m is not None and getattr(m, "requires_grad", False):
            raise ValueError("ra_attention computes no gradient for a mask; detach it")
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mask = mask_descriptor(q, k, attn_mask, key_padding_mask)
    return _FN.apply(q, k, v, causal_code(is_causal), scale, mask)


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


def ra_attn_fwd_rope(q, k, v, o, stats, q_rot, k_rot, q_positions, k_positions, theta, B, Hq, Hkv,
                     Nq, Nk, D, causal, scale, dtype, mask=None, mask_kind=RA_MASK_NONE,
                     mask_strides=(0, 0, 0, 0), stream=None) -> int:
    """ra_attn_fwd_rope; ``mask``, ``mask_kind``, ``mask_strides`` as ra_attn_fwd_masked (none by
    default)."""
    return load_library().ra_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(stats),
                                           _ptr(q_rot), _ptr(k_rot), _ptr(q_positions),
                                           _ptr(k_positions), float(theta), B, Hq, Hkv, Nq, Nk, D,
                                           int(causal), float(scale), int(dtype),
                                           _mask_struct(mask, mask_kind, mask_strides),
                                           _stream(stream))


def ra_attn_bwd_rope(q_rot, k_rot, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes,
                     q_positions, k_positions, theta, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype,
                     mask=None, mask_kind=RA_MASK_NONE, mask_strides=(0, 0, 0, 0),
                     stream=None) -> int:
    """ra_attn_bwd_rope; the mask arguments as ra_attn_fwd_rope."""
    return load_library().ra_attn_bwd_rope(_ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(o), _ptr(d_o),
                                           _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv),
                                           _ptr(workspace), workspace_bytes, _ptr(q_positions),
                                           _ptr(k_positions), float(theta), B, Hq, Hkv, Nq, Nk, D,
                                           int(causal), float(scale), int(dtype),
                                           _mask_struct(mask, mask_kind, mask_strides),
                                           _stream(stream))


def _positions(p, n, device):
    import torch
    if p is None:
        return None
    t = torch.as_tensor(p, dtype=torch.int32, device=device).contiguous()
    if t.numel() != n:
        raise ValueError(f"positions must have {n} entries")
    return t


def attn_fwd_rope(q, k, v, causal, theta: float = 10000.0, scale: Optional[float] = None,
                  q_positions=None, k_positions=None, with_rotated: bool = True, mask=None):
    """Allocate O, stats, the rotated keys (and queries) and run ra_attn_fwd_rope on the current
    stream (``mask``: a mask_descriptor or None).  Returns (o, stats, q_rot or None, k_rot)."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device=q.device)
    q_rot = torch.empty_like(q) if with_rotated else None
    k_rot = torch.empty_like(k)
    qp, kp = _positions(q_positions, Nq, q.device), _positions(k_positions, Nk, q.device)
    _check(ra_attn_fwd_rope(q, k, v, o, stats, q_rot, k_rot, qp, kp, theta, B, Hq, Hkv, Nq, Nk, D,
                            causal_code(causal), scale, _dtype_code(q), *(mask or ())),
           "ra_attn_fwd_rope")
    return o, stats, q_rot, k_rot


def attn_bwd_rope(q_rot, k_rot, v, o, d_o, stats, causal, theta: float = 10000.0,
                  scale: Optional[float] = None, q_positions=None, k_positions=None, mask=None):
    """Allocate dQ, dK, dV and a workspace and run ra_attn_bwd_rope on the current stream: the
    gradients with respect to the unrotated q and k."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = _shapes(q_rot, k_rot, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    d_o = d_o.contiguous()
    dq, dk, dv = torch.empty_like(q_rot), torch.empty_like(k_rot), torch.empty_like(v)
    code = _dtype_code(q_rot)
    nbytes = ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q_rot.device)
    qp, kp = _positions(q_positions, Nq, q_rot.device), _positions(k_positions, Nk, q_rot.device)
    _check(ra_attn_bwd_rope(q_rot, k_rot, v, o, d_o, stats, dq, dk, dv, ws, nbytes, qp, kp, theta,
                            B, Hq, Hkv, Nq, Nk, D, causal_code(causal), scale, code, *(mask or ())),
           "ra_attn_bwd_rope")
    return dq, dk, dv


class _RopeAttentionFn:
    _cls = None

    @classmethod
    def get(cls):
        if cls._cls is None:
            import torch

            class Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, causal, theta, scale, q_positions, k_positions, mask):
                    o, stats, q_rot, k_rot = attn_fwd_rope(q, k, v, causal, theta, scale,
                                                           q_positions, k_positions, mask=mask)
                    ctx.save_for_backward(q_rot, k_rot, v, o, stats)
                    ctx.args = (causal, theta, scale, q_positions, k_positions, mask)
                    return o

                @staticmethod
                def backward(ctx, d_o):
                    q_rot, k_rot, v, o, stats = ctx.saved_tensors
                    causal, theta, scale, qp, kp, mask = ctx.args
                    dq, dk, dv = attn_bwd_rope(q_rot, k_rot, v, o, d_o, stats, causal, theta, scale,
                                               qp, kp, mask=mask)
                    return dq, dk, dv, None, None, None, None, None, None

            cls._cls = Fn
        return cls._cls


def ra_attention_rope(q, k, v, is_causal=False, theta: float = 10000.0,
                      scale: Optional[float] = None, q_positions=None, k_positions=None,
                      attn_mask=None, key_padding_mask=None):
    """ra_attention on q and k rotated by the NEOX rotary embedding (ra_rope), the query rotation
    fused into the attention kernel.  q, k unrotated, bf16 or fp32, shapes, causal modes and
    masks as ra_attention; positions default to 0..N-1.  Differentiable in q, k and v (the
    gradients are with respect to the unrotated q and k)."""
    import torch
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("ra_attention_rope supports bfloat16 and float32")
    for m in (attn_mask, key_padding_mask):
        if m is not None and getattr(m, "requires_grad", False):
            raise ValueError("ra_attention_rope computes no gradient for a mask; detach it")
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    mask = mask_descriptor(q, k, attn_mask, key_padding_mask)
    return _RopeAttentionFn.get().apply(q, k, v, causal_code(is_causal), float(theta), scale,
                                        q_positions, k_positions, mask)


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
