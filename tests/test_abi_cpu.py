"""The C-ABI library loads, exports every declared symbol and rejects bad arguments before any
launch.  No GPU is needed: every call here either fails validation or has nothing to do."""
import ctypes
import math
import os
import re

import pytest

import rational_softmax_tiled_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra_attn.h")

OK, NULLPTR, SHAPE, GQA, HEADDIM, DTYPE, SCALE, WORKSPACE, ALIGN, TOO_LARGE, HIP, MASK = range(12)

# Fake, 256-byte aligned "device" addresses: never dereferenced, since every call fails
# validation or is empty.
P = 0x7F0000000000
P2 = P + 0x100000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ra.library_path()):
        from rational_softmax_tiled_amd import build
        build.build()
    return ra.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"ra_attn_fwd", "ra_attn_bwd", "ra_softmax_rows", "ra_attn_bwd_workspace_bytes",
            "ra_attn_fwd_counted", "ra_status_string", "ra_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(12):
        s = ra.ra_status_string(code)
        assert s.startswith("RA_")
    assert "unknown" in ra.ra_status_string(99)


def fwd(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=64, causal=1, scale=0.125, dtype=ra.RA_BF16,
        q=P, k=P, v=P, o=P2, stats=None):
    return ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, 0)


def test_fwd_validation(lib):
    assert fwd(dtype=7) == DTYPE
    assert fwd(B=-1) == SHAPE
    assert fwd(Nk=-3) == SHAPE
    assert fwd(Hq=3, Hkv=2) == GQA
    assert fwd(Hq=2, Hkv=0) == GQA
    assert fwd(D=96) == HEADDIM
    assert fwd(D=32) == HEADDIM
    for s in (0.0, -1.0, math.inf, math.nan):
        assert fwd(scale=s) == SCALE
    assert fwd(q=None) == NULLPTR
    assert fwd(o=None) == NULLPTR
    assert fwd(k=None) == NULLPTR
    assert fwd(q=P + 8) == ALIGN
    assert fwd(v=P + 4) == ALIGN
    assert fwd(stats=P + 2) == ALIGN
    assert fwd(Nq=1 << 25, D=128) == TOO_LARGE
    assert fwd(B=1 << 12, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 10) == TOO_LARGE
    assert fwd(B=1 << 40, Hq=1 << 40, Hkv=1, Nq=1 << 40) == TOO_LARGE  # no int64 overflow


@pytest.mark.parametrize("dtype,es", [(ra.RA_BF16, 2), (ra.RA_F32, 4)])
@pytest.mark.parametrize("D", [64, 128])
def test_byte_offset_boundary(lib, dtype, es, D):
    """Every byte offset inside one head's matrix, a 256-row tile tail included, fits a signed
    32-bit int: (N + 256) * D * elem_size < 2^31 for N = Nq and N = Nk, else RA_ERR_TOO_LARGE.
    The size query returns 0 exactly where a call would be refused (no launch needed)."""
    n_max = (1 << 31) // (D * es) - 256 - 1          # the largest N the limit admits
    assert (n_max + 256) * D * es < (1 << 31) <= (n_max + 257) * D * es
    for nq, nk in ((n_max, 8), (8, n_max)):
        assert ra.ra_attn_bwd_workspace_bytes(1, 1, 1, nq, nk, D, dtype) > 0
    for nq, nk in ((n_max + 1, 8), (8, n_max + 1)):
        assert ra.ra_attn_bwd_workspace_bytes(1, 1, 1, nq, nk, D, dtype) == 0
        assert fwd(Nq=nq, Nk=nk, D=D, dtype=dtype, Hq=1) == TOO_LARGE
        assert ra.ra_attn_bwd_noalloc(P, P, P, P, P, None, P2, P2, P2, 1, 1, 1, nq, nk, D, 1,
                                      0.125, dtype, 0) == TOO_LARGE


def test_noalloc_rejects_beyond_its_array(lib):
    """ra_attn_bwd_noalloc keeps 36 bytes per query row (plus 256) in a 64 MiB array: one row
    more than fits is refused before anything is launched or resolved."""
    rows = ((64 << 20) - 256) // 36
    assert ra.ra_attn_bwd_workspace_bytes(1, 1, 1, rows, 8, 64, ra.RA_BF16) <= (64 << 20)
    assert ra.ra_attn_bwd_workspace_bytes(1, 1, 1, rows + 1, 8, 64, ra.RA_BF16) > (64 << 20)
    call = lambda B, Hq, Nq: ra.ra_attn_bwd_noalloc(P, P, P, P, P, None, P2, P2, P2, B, Hq, 1, Nq,
                                                    8, 64, 1, 0.125, ra.RA_BF16, 0)
    assert call(1, 1, rows + 1) == TOO_LARGE
    assert call(7, 1, rows // 7 + 1) == TOO_LARGE
    # nothing to compute needs no array: RA_OK without touching the GPU
    assert call(0, 1, rows + 1) == OK
    assert ra.ra_attn_bwd_noalloc(P, P, P, P, P, None, P2, P2, P2, 1, 1, 1, 8, 8, 64, 1, 0.125, 9,
                                  0) == DTYPE


def test_fwd_empty_problems_launch_nothing(lib):
    # nothing to compute: RA_OK without touching the (fake) pointers or the GPU
    assert fwd(B=0) == OK
    assert fwd(Nq=0) == OK
    assert fwd(Hq=0, Hkv=0) == OK
    assert fwd(B=0, q=None, k=None, v=None, o=None) == OK


def test_counted_needs_counters(lib):
    assert ra.ra_attn_fwd_counted(P, P, P, P2, None, 1, 2, 1, 8, 8, 64, 1, 0.125, ra.RA_BF16,
                                  None, 0) == NULLPTR


def test_workspace_size(lib):
    n = ra.ra_attn_bwd_workspace_bytes(4, 16, 16, 8192, 8192, 128, ra.RA_BF16)
    assert n >= 4 * 16 * 8192 * (2 * 4 + 3 * 4)
    assert ra.ra_attn_bwd_workspace_bytes(4, 16, 16, 8192, 8192, 96, ra.RA_BF16) == 0
    assert ra.ra_attn_bwd_workspace_bytes(1, 2, 1, 100, 100, 64, ra.RA_F32) < \
        ra.ra_attn_bwd_workspace_bytes(1, 2, 1, 200, 100, 64, ra.RA_F32)


def bwd(ws=P2, ws_bytes=1 << 30, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=64, scale=0.125,
        dtype=ra.RA_BF16, q=P, dq=P2, dk=P2, stats=None):
    return ra.ra_attn_bwd(q, P, P, P, P, stats, dq, dk, P2, ws, ws_bytes, B, Hq, Hkv, Nq, Nk,
                          D, 1, scale, dtype, 0)


def test_bwd_validation(lib):
    assert bwd(dtype=3) == DTYPE
    assert bwd(Hq=3, Hkv=2) == GQA
    assert bwd(D=80) == HEADDIM
    assert bwd(scale=-0.5) == SCALE
    assert bwd(q=None) == NULLPTR
    assert bwd(dk=None) == NULLPTR
    assert bwd(dq=P2 + 2) == ALIGN
    assert bwd(stats=P + 1) == ALIGN
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws_bytes=16) == WORKSPACE
    assert bwd(B=0) == OK


def test_bwd_phase_validation(lib):
    def dq_phase(dq=P2, o=P, ws=P2, ws_bytes=1 << 30, B=1, D=64, dk=None):
        return ra.ra_attn_bwd_dq(P, P, P, o, P, None, dq, ws, ws_bytes, B, 2, 1, 8, 8, D, 1,
                                 0.125, ra.RA_BF16, 0)

    def kv_phase(dk=P2, dv=P2, ws=P2, ws_bytes=1 << 30, B=1, D=64, scale=0.125):
        return ra.ra_attn_bwd_dkdv(P, P, P, P, None, dk, dv, ws, ws_bytes, B, 2, 1, 8, 8, D, 1,
                                   scale, ra.RA_BF16, 0)

    # each phase needs its own outputs, not the other phase's
    assert dq_phase(dq=None) == NULLPTR
    assert dq_phase(o=None) == NULLPTR
    assert kv_phase(dk=None) == NULLPTR
    assert kv_phase(dv=None) == NULLPTR
    assert dq_phase(ws=None) == WORKSPACE
    assert kv_phase(ws_bytes=8) == WORKSPACE
    assert dq_phase(D=96) == HEADDIM
    assert kv_phase(scale=0.0) == SCALE
    assert kv_phase(dv=P2 + 4) == ALIGN
    assert dq_phase(B=0) == OK
    assert kv_phase(B=0) == OK


def test_softmax_rows_validation(lib):
    assert ra.ra_softmax_rows(P, P, 4, 4, 9, 0) == DTYPE
    assert ra.ra_softmax_rows(P, P, -1, 4, ra.RA_F32, 0) == SHAPE
    assert ra.ra_softmax_rows(P, P, 1 << 31, 4, ra.RA_F32, 0) == TOO_LARGE
    assert ra.ra_softmax_rows(None, P, 4, 4, ra.RA_F32, 0) == NULLPTR
    assert ra.ra_softmax_rows(P + 2, P, 4, 4, ra.RA_F32, 0) == ALIGN
    assert ra.ra_softmax_rows(P, P, 0, 4, ra.RA_F32, 0) == OK
    assert ra.ra_softmax_rows(P, P, 4, 0, ra.RA_F32, 0) == OK


def test_softmax_rows_bwd_validation(lib):
    f = ra.ra_softmax_rows_bwd
    assert f(P, P, P2, 4, 4, 9, 0) == DTYPE
    assert f(P, P, P2, -1, 4, ra.RA_F32, 0) == SHAPE
    assert f(P, P, P2, 1 << 31, 4, ra.RA_F32, 0) == TOO_LARGE
    assert f(None, P, P2, 4, 4, ra.RA_F32, 0) == NULLPTR
    assert f(P, None, P2, 4, 4, ra.RA_F32, 0) == NULLPTR
    assert f(P, P, None, 4, 4, ra.RA_F32, 0) == NULLPTR
    assert f(P, P + 2, P2, 4, 4, ra.RA_F32, 0) == ALIGN
    assert f(P, P, P2 + 1, 4, 4, ra.RA_BF16, 0) == ALIGN
    assert f(P, P, P2, 0, 4, ra.RA_F32, 0) == OK
    assert f(None, None, None, 4, 0, ra.RA_F32, 0) == OK


def test_rope_validation(lib):
    f = ra.ra_rope_neox
    assert f(P, P2, None, 2, 8, 64, 10000.0, 0, 7, 0) == DTYPE
    assert f(P, P2, None, -1, 8, 64, 10000.0, 0, ra.RA_F32, 0) == SHAPE
    assert f(P, P2, None, 2, 8, 63, 10000.0, 0, ra.RA_F32, 0) == HEADDIM
    for th in (0.0, -1.0, math.inf, math.nan):
        assert f(P, P2, None, 2, 8, 64, th, 0, ra.RA_F32, 0) == SCALE
    assert f(P, P2, None, 2, 1 << 26, 64, 10000.0, 0, ra.RA_F32, 0) == TOO_LARGE
    assert f(None, P2, None, 2, 8, 64, 10000.0, 0, ra.RA_F32, 0) == NULLPTR
    assert f(P, None, None, 2, 8, 64, 10000.0, 0, ra.RA_F32, 0) == NULLPTR
    assert f(P + 2, P2, None, 2, 8, 64, 10000.0, 0, ra.RA_F32, 0) == ALIGN
    assert f(P, P2, P + 2, 2, 8, 64, 10000.0, 0, ra.RA_F32, 0) == ALIGN
    assert f(P, P2, None, 0, 8, 64, 10000.0, 0, ra.RA_F32, 0) == OK
    assert f(None, None, None, 2, 0, 64, 10000.0, 0, ra.RA_F32, 0) == OK


def fwd_rope(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, D=64, causal=1, scale=0.125, dtype=ra.RA_BF16,
             q=P, k=P, v=P, o=P2, q_rot=None, k_rot=P2, qp=None, kp=None, theta=10000.0):
    return ra.ra_attn_fwd_rope(q, k, v, o, None, q_rot, k_rot, qp, kp, theta, B, Hq, Hkv, Nq, Nk,
                               D, causal, scale, dtype, stream=0)


def test_fwd_rope_validation(lib):
    assert fwd_rope(dtype=7) == DTYPE
    assert fwd_rope(Hq=3, Hkv=2) == GQA
    assert fwd_rope(D=96) == HEADDIM
    assert fwd_rope(causal=5) == MASK
    for th in (0.0, -1.0, math.inf, math.nan):
        assert fwd_rope(theta=th) == SCALE
    assert fwd_rope(scale=0.0) == SCALE
    assert fwd_rope(q=None) == NULLPTR
    assert fwd_rope(o=None) == NULLPTR
    assert fwd_rope(k_rot=None) == NULLPTR
    assert fwd_rope(q_rot=P2 + 2) == ALIGN
    assert fwd_rope(k_rot=P2 + 8) == ALIGN
    assert fwd_rope(qp=P + 2) == ALIGN
    assert fwd_rope(kp=P + 1) == ALIGN
    assert fwd_rope(Nq=1 << 25, D=128) == TOO_LARGE
    assert fwd_rope(B=0) == OK
    assert fwd_rope(Nq=0, q=None, o=None, k_rot=None) == OK
    bad = ra.ra_attn_fwd_rope(P, P, P, P2, None, None, P2, None, None, 10000.0, 1, 2, 1, 8, 8, 64, 1,
                              0.125, ra.RA_BF16, P + 1, ra.RA_MASK_ADD, (8, 0, 0, 1), stream=0)
    assert bad == ALIGN          # the mask's checks apply (a bf16 additive mask: 2-byte aligned)
    bad = ra.ra_attn_fwd_rope(P, P, P, P2, None, None, P2, None, None, 10000.0, 1, 2, 1, 8, 8, 64, 1,
                              0.125, ra.RA_BF16, P, 9, (8, 0, 0, 1), stream=0)
    assert bad == MASK


def test_bwd_rope_validation(lib):
    def f(dtype=ra.RA_BF16, theta=10000.0, ws=P2, ws_bytes=1 << 30, dq=P2, qp=None, B=1, D=64):
        return ra.ra_attn_bwd_rope(P, P, P, P, P, None, dq, P2, P2, ws, ws_bytes, qp, None, theta,
                                   B, 2, 1, 8, 8, D, 1, 0.125, dtype, stream=0)
    assert f(dtype=5) == DTYPE
    assert f(theta=0.0) == SCALE
    assert f(theta=math.nan) == SCALE
    assert f(qp=P + 2) == ALIGN
    assert f(dq=None) == NULLPTR
    assert f(dq=P2 + 2) == ALIGN
    assert f(ws=None) == WORKSPACE
    assert f(D=80) == HEADDIM
    assert f(B=0) == OK


def test_product_path_has_no_fallback():
    # The binding must not reach the oracle or any CPU implementation.
    import rational_softmax_tiled_amd
    src = open(rational_softmax_tiled_amd.__file__).read()
    assert "oracle" not in src.replace("no CPU or PyTorch fallback", "")
    for name in os.listdir(os.path.join(ROOT, "rational_softmax_tiled_amd", "csrc")):
        text = open(os.path.join(ROOT, "rational_softmax_tiled_amd", "csrc", name)).read()
        assert "oracle" not in text.lower(), name


def mfwd(kind=ra.RA_MASK_BOOL, strides=(0, 0, 8, 1), data=P + 0x200000, causal=0, B=1, Hq=2, Nq=8,
         Nk=8, dtype=ra.RA_BF16):
    return ra.ra_attn_fwd_masked(P, P, P, P2, None, B, Hq, 1, Nq, Nk, 64, causal, 0.125, dtype, data,
                                 kind, strides, 0)


def test_causal_mode_validation(lib):
    assert fwd(causal=3) == MASK
    assert fwd(causal=-1) == MASK
    assert bwd(B=1, q=P) == bwd()   # causal 1 is valid
    assert ra.ra_attn_bwd(P, P, P, P, P, None, P2, P2, P2, P2, 1 << 30, 1, 2, 1, 8, 8, 64, 5, 0.125,
                          ra.RA_BF16, 0) == MASK
    assert mfwd(causal=9) == MASK
    # the mode is checked even when there is nothing to compute
    assert fwd(causal=4, B=0) == MASK


def test_mask_validation(lib):
    assert mfwd(kind=3) == MASK
    assert mfwd(kind=-1) == MASK
    assert mfwd(strides=(0, 0, -8, 1)) == MASK
    assert mfwd(strides=(-1, 0, 8, 1)) == MASK
    assert mfwd(data=None) == NULLPTR
    assert mfwd(kind=ra.RA_MASK_ADD, data=P + 1) == ALIGN              # bf16 elements
    assert mfwd(kind=ra.RA_MASK_ADD, data=P + 2, dtype=ra.RA_F32) == ALIGN
    assert mfwd(kind=ra.RA_MASK_BOOL, data=P + 1, B=0) == OK           # bytes: any address
    # one slice (plus tile tails) must stay below 2^31 bytes
    # (Nq + 64) * stride_q + (Nk + 128) * stride_k elements, Nq = Nk = 8
    assert mfwd(strides=(0, 0, 1 << 25, 1)) == TOO_LARGE
    assert mfwd(kind=ra.RA_MASK_ADD, strides=(0, 0, 1 << 24, 1)) == TOO_LARGE
    assert mfwd(strides=(0, 0, 1, 1 << 24)) == TOO_LARGE
    assert mfwd(strides=(1 << 62, 0, 8, 1), B=3) == TOO_LARGE          # no int64 overflow
    # no mask (NULL descriptor or kind NONE) behaves as ra_attn_fwd
    assert ra.ra_attn_fwd_masked(P, P, P, P2, None, 1, 3, 2, 8, 8, 64, 0, 0.125, ra.RA_BF16, None,
                                 ra.RA_MASK_NONE, (0, 0, 0, 0), 0) == GQA
    assert mfwd(kind=ra.RA_MASK_NONE, data=None, B=0) == OK
    assert mfwd(B=0) == OK and mfwd(Nq=0) == OK


def test_masked_bwd_validation(lib):
    def mbwd(kind=ra.RA_MASK_BOOL, strides=(8, 0, 0, 1), data=P + 0x200000, ws=P2, causal=2, B=1):
        return ra.ra_attn_bwd_masked(P, P, P, P, P, None, P2, P2, P2, ws, 1 << 30, B, 2, 1, 8, 8, 64,
                                     causal, 0.125, ra.RA_BF16, data, kind, strides, 0)
    assert mbwd(kind=7) == MASK
    assert mbwd(causal=3) == MASK
    assert mbwd(strides=(8, 0, 0, -1)) == MASK
    assert mbwd(data=None) == NULLPTR
    assert mbwd(ws=None) == WORKSPACE
    assert mbwd(B=0) == OK


def dec(B=1, Hq=8, Hkv=2, Nq=1, Nk=100, D=128, causal=2, dtype=ra.RA_BF16, ws=P2, ws_bytes=1 << 30,
        seqlens=None, stats=None, q=P, o=P2):
    return ra.ra_attn_decode(q, P, P, o, stats, seqlens, ws, ws_bytes, B, Hq, Hkv, Nq, Nk, D, causal,
                             0.1, dtype, 0)


def test_decode_validation(lib):
    assert dec(dtype=7) == DTYPE
    assert dec(Hq=8, Hkv=2, Nq=9) == SHAPE          # 4 * 9 = 36 query rows per K/V head > 32
    assert dec(Hq=64, Hkv=1, Nq=1) == SHAPE
    assert dec(Hq=3, Hkv=2) == GQA
    assert dec(causal=3) == MASK
    assert dec(D=96) == HEADDIM
    assert dec(q=None) == NULLPTR
    assert dec(o=P2 + 8) == ALIGN
    assert dec(stats=P + 2) == ALIGN
    assert dec(seqlens=P + 2) == ALIGN
    assert dec(ws=None) == WORKSPACE
    assert dec(ws_bytes=1000) == WORKSPACE
    assert dec(ws=P2 + 16) == ALIGN                 # 256-byte aligned workspace
    assert dec(B=0) == OK and dec(Nq=0) == OK


def test_decode_workspace_size(lib):
    f = ra.ra_attn_decode_workspace_bytes
    assert f(16, 32, 8, 1, 16384, 128, ra.RA_BF16) > 16 * 8 * 16384 * 4 * 4   # scores of 4 rows
    assert f(16, 32, 8, 1, 16384, 128, ra.RA_F32) == f(16, 32, 8, 1, 16384, 128, ra.RA_BF16)
    assert f(16, 32, 8, 1, 16384, 128, 7) == 0
    assert f(1, 8, 2, 9, 100, 128, ra.RA_BF16) == 0
    assert f(0, 8, 2, 1, 100, 128, ra.RA_BF16) == 0
    assert f(1, 8, 2, 1, 100, 64, ra.RA_BF16) < f(1, 8, 2, 1, 10000, 64, ra.RA_BF16)
    assert f(1, 8, 2, 1, 100, 64, ra.RA_BF16) % 256 == 0
