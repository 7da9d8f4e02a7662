"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws random tensors,
applies the host-side input preparation a workload names (NEOX rotary
embedding) and rounds to the storage dtype.  Both the oracle and the HIP path
consume exactly the arrays it returns.

Generation recipe (every workload):
* ``numpy.random.default_rng(seed)`` (PCG64); standard normals drawn in float32,
  C order, in the sequence Q, K, V, dO, each multiplied by its sigma.
* Optional NEOX split-halves rotary embedding on Q and K in float32 (pairs
  channel j with j + D/2; inv_freq_j = theta^(-2j/D); position = token index).
  Pairing from the noeira "Primitives" page (RoPE entry) and the nurl ``nn``
  page (nn_rope, NEOX half-split); the frequency schedule is the standard
  rotary one, which neither page spells out.
* Cast to the storage dtype with round-to-nearest-even (bf16) or kept (fp32).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    dtype: str          # "bf16" or "f32": storage and MFMA operand type
    causal: bool
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    rope_theta: Optional[float] = None
    with_grad: bool = False   # also draw dO

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to fp32, the value the library receives."""
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def counted_flops_fwd(self) -> float:
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.D
        return f / 2.0 if self.causal else f

    def counted_flops_fwd_bwd(self) -> float:
        return 3.5 * self.counted_flops_fwd()


# The five attention workloads the measurements and parity checks use.
WORKLOADS = {
    "fp32_noncausal_B1_H2_N128_D64": AttnWorkload(
        "fp32_noncausal_B1_H2_N128_D64", "f32", False, 1, 2, 2, 128, 128, 64, seed=0),
    "bf16_causal_B2_H12_N128_D64": AttnWorkload(
        "bf16_causal_B2_H12_N128_D64", "bf16", True, 2, 12, 12, 128, 128, 64, seed=1),
    "bf16_causal_B8_H16_N2048_D64_sigma2": AttnWorkload(
        "bf16_causal_B8_H16_N2048_D64_sigma2", "bf16", True, 8, 16, 16, 2048, 2048, 64,
        seed=2, sigma_qk=2.0),
    "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope": AttnWorkload(
        "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope", "bf16", True, 4, 32, 8, 4096, 4096,
        128, seed=3, rope_theta=10000.0),
    "bf16_causal_B4_H16_N8192_D128_fwd_bwd": AttnWorkload(
        "bf16_causal_B4_H16_N8192_D128_fwd_bwd", "bf16", True, 4, 16, 16, 8192, 8192, 128,
        seed=4, with_grad=True),
}
WORKLOAD_ORDER = list(WORKLOADS)

# A padded batch for the explicit-mask path: B sequences of different lengths padded to N, with a
# [B, N] key padding mask (1 = attend up to the sample's length), the CrossAttention key padding
# mask of the noeira "Primitives" page.  Inputs follow the recipe above; the lengths are fixed.
PADDED_BATCH = AttnWorkload("bf16_causal_keypad_B4_H16_N4096_D128", "bf16", True, 4, 16, 16,
                            4096, 4096, 128, seed=6, with_grad=True)
PADDED_LENGTHS = (4096, 3000, 2048, 1111)


def padded_batch_workload() -> AttnWorkload:
    return PADDED_BATCH


def padded_batch_lengths(w: AttnWorkload = PADDED_BATCH):
    """Per-sample valid lengths of the padded batch (keys at or past the length are masked)."""
    assert w == PADDED_BATCH
    return PADDED_LENGTHS


# A decode step: one new query row per head against per-sample K/V caches of different lengths
# (grouped-query heads, the cache capacity Nk).  Lengths are drawn uniformly from [Nk/4, Nk]
# with their own seeded generator; inputs follow the recipe above (Q [B, Hq, 1, D], caches
# [B, Hkv, Nk, D]).
DECODE = AttnWorkload("bf16_decode_gqa_B16_Hq32_Hkv8_Nq1_Nk16384_D128", "bf16", True, 16, 32, 8,
                      1, 16384, 128, seed=7)


# The same decode step with fp32 caches and queries (same seed, so the same cache lengths).
DECODE_F32 = dataclasses.replace(DECODE, name="fp32_decode_gqa_B16_Hq32_Hkv8_Nq1_Nk16384_D128",
                                 dtype="f32")


def decode_workload(dtype: str = "bf16") -> AttnWorkload:
    return DECODE if dtype == "bf16" else DECODE_F32


def decode_seqlens(w: AttnWorkload = DECODE) -> np.ndarray:
    """int32 [B] cache lengths of the decode workload."""
    rng = np.random.default_rng(w.seed + 1000)
    return rng.integers(w.Nk // 4, w.Nk + 1, size=w.B).astype(np.int32)


# Packed documents for the general explicit-mask path: each sample of N tokens holds several
# documents back to back, and a token attends to the tokens of its own document only (with the
# causal limit).  The mask is one [B, N, N] boolean array broadcast over heads; document lengths
# are drawn from [N/16, N/2] with their own seeded generator, the last one cut at N.  Most of its
# 64-key tiles are either wholly inside a document or wholly outside.
DOCUMENTS = AttnWorkload("bf16_causal_documents_B4_H16_N4096_D128", "bf16", True, 4, 16, 16,
                         4096, 4096, 128, seed=8, with_grad=True)


def documents_workload() -> AttnWorkload:
    return DOCUMENTS


def document_ids(B: int, N: int, seed: int, lo: int, hi: int) -> np.ndarray:
    """int32 [B, N]: the document of every token, documents of lengths drawn from [lo, hi]."""
    rng = np.random.default_rng(seed)
    ids = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        pos, d = 0, 0
        while pos < N:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    return ids


def documents_keep(w: AttnWorkload = DOCUMENTS) -> np.ndarray:
    """The [B, N, N] boolean mask of the documents workload: True where query and key share a
    document."""
    assert w.Nq == w.Nk
    ids = document_ids(w.B, w.Nq, w.seed + 2000, w.Nq // 16, w.Nq // 2)
    return ids[:, :, None] == ids[:, None, :]


def padded_batch_keep(w: AttnWorkload = PADDED_BATCH) -> np.ndarray:
    """The [B, Nk] boolean key padding mask: True where key j < length of sample b."""
    return np.arange(w.Nk)[None, :] < np.asarray(padded_batch_lengths(w))[:, None]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of ``x`` as stored in ``dtype``, returned as float32."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x))
    raise ValueError(dtype)


def neox_rope(x: np.ndarray, theta: float) -> np.ndarray:
    """Split-halves rotary embedding along the last axis; positions on axis -2."""
    D = x.shape[-1]
    N = x.shape[-2]
    half = D // 2
    j = np.arange(half, dtype=np.float32)
    inv_freq = (np.float32(theta) ** (-(2.0 * j) / np.float32(D))).astype(np.float32)
    ang = np.arange(N, dtype=np.float32)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(np.float32)
    sin = np.sin(ang).astype(np.float32)
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = x1 * cos - x2 * sin
    out[..., half:] = x2 * cos + x1 * sin
    return out


def make_attention_inputs(w: AttnWorkload, seed: Optional[int] = None) -> dict:
    """Q, K, V (and dO) of workload ``w`` as float32 arrays holding the exact
    storage-dtype values."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp_q = (w.B, w.Hq, w.Nq, w.D)
    shp_k = (w.B, w.Hkv, w.Nk, w.D)
    q = rng.standard_normal(shp_q, dtype=np.float32) * np.float32(w.sigma_qk)
    k = rng.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_qk)
    v = rng.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_v)
    out = {}
    if w.rope_theta is not None:
        q = neox_rope(q, w.rope_theta)
        k = neox_rope(k, w.rope_theta)
    out["q"] = round_to_dtype(q, w.dtype)
    out["k"] = round_to_dtype(k, w.dtype)
    out["v"] = round_to_dtype(v, w.dtype)
    if w.with_grad:
        do = rng.standard_normal(shp_q, dtype=np.float32)
        out["do"] = round_to_dtype(do, w.dtype)
    return out


def make_unrotated_inputs(w: AttnWorkload, seed: Optional[int] = None) -> dict:
    """The draws of make_attention_inputs for a workload with a rotary embedding, with Q and K
    left unrotated (for the kernels that rotate them on the device), each rounded to the
    storage dtype; dO as a seeded N(0, 1) draw when the workload has none."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp_q = (w.B, w.Hq, w.Nq, w.D)
    shp_k = (w.B, w.Hkv, w.Nk, w.D)
    q = rng.standard_normal(shp_q, dtype=np.float32) * np.float32(w.sigma_qk)
    k = rng.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_qk)
    v = rng.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_v)
    out = {"q": round_to_dtype(q, w.dtype), "k": round_to_dtype(k, w.dtype),
           "v": round_to_dtype(v, w.dtype)}
    do = rng.standard_normal(shp_q, dtype=np.float32)
    out["do"] = round_to_dtype(do, w.dtype)
    return out


def make_local_inputs(B=1, H=16, N=2048, D=64, amplitude=4.0, seed=7, dtype="bf16"):
    """Structured causal workload whose scores fall off sharply away from the
    diagonal, so whole tiles leave the compact support.  Q = K = RoPE(a*c + 0.5*e)
    with one shared c ~ N(0, I) per head and e ~ N(0, I) per token."""
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((B, H, 1, D), dtype=np.float32)
    eq = rng.standard_normal((B, H, N, D), dtype=np.float32)
    ek = rng.standard_normal((B, H, N, D), dtype=np.float32)
    v = rng.standard_normal((B, H, N, D), dtype=np.float32)
    q = neox_rope(np.float32(amplitude) * c + np.float32(0.5) * eq, 10000.0)
    k = neox_rope(np.float32(amplitude) * c + np.float32(0.5) * ek, 10000.0)
    return {"q": round_to_dtype(q, dtype), "k": round_to_dtype(k, dtype),
            "v": round_to_dtype(v, dtype)}


def make_rows(rows: int, cols: int, sigma: float = 4.0, seed: int = 11, dtype: str = "f32"):
    """Logit rows for the standalone row softmax, x ~ N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
    return round_to_dtype(x, dtype)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def storage_sha256(inp: dict, dtype: str) -> dict:
    """SHA-256 of each input buffer as the device stores it (bf16 bits or fp32 bytes)."""
    out = {}
    for name, a in inp.items():
        raw = f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)
        out[name] = sha256(raw)
    return out


# The structured workload that exercises tile skipping (make_local_inputs), at the size the
# measurements use, beside an i.i.d. workload of the same shape in which no tile skips.
LOCAL = dict(B=1, H=16, N=2048, D=64, amplitude=4.0, seed=7)
LOCAL_IID = AttnWorkload("bf16_causal_B1_H16_N2048_D64_iid", "bf16", True, 1, 16, 16, 2048, 2048,
                         64, seed=8)
