"""Attention with the NEOX rotary embedding fused in (ra_attn_fwd_rope, ra_attn_bwd_rope) through
the C ABI.

* The fused forward equals the unfused chain (ra_rope_neox on q and k, then ra_attn_fwd) bit for
  bit, the rotated rows included, over head dims, causal modes, grouped heads, ragged lengths,
  positions and theta.
* The rotated rows against the fp64 rotation: within one bf16 rounding plus the fp32 rotation.
* Every head of the grouped-query workload (B=4, Hq=32, Hkv=8, N=4096, D=128, causal) against the
  oracle of attention on rotated rows: O within the bf16 tolerance of the exact function, m and l
  within bounds derived from the bf16 rounding of the rotated rows (tests/parity.py).
* The backward against the oracle's gradient with respect to the unrotated rows (near ties of the
  row max within the same rounding bound accepted either way), on small cases and on every
  (batch, K/V head) group of the grouped-query workload, and, at that size, against the unfused
  chain (ra_attn_bwd on the rotated rows, then the inverse rotation).
"""
import numpy as np
import pytest

import oracle
import parity
import workloads as wl
from helpers import to_dev, to_np

pytestmark = pytest.mark.gpu

GQA = "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"


def _positions(kind, n, seed):
    if kind is None:
        return None
    return np.random.default_rng(seed).integers(0, 100000, size=n).astype(np.int32)


def _dev_pos(p):
    import torch
    return None if p is None else torch.as_tensor(p, dtype=torch.int32, device="cuda")


def _inputs(B, Hq, Hkv, Nq, Nk, D, seed, sigma=1.0, dtype="bf16"):
    rng = np.random.default_rng(seed)
    r = lambda *s, sg=1.0: wl.round_to_dtype(rng.standard_normal(s, dtype=np.float32) * np.float32(sg), dtype)
    return {"q": r(B, Hq, Nq, D, sg=sigma), "k": r(B, Hkv, Nk, D, sg=sigma), "v": r(B, Hkv, Nk, D),
            "do": r(B, Hq, Nq, D)}


def _code(ra, t):
    import torch
    return ra.RA_BF16 if t.dtype == torch.bfloat16 else ra.RA_F32


def fused_fwd(ra, qt, kt, vt, dims, causal, scale, theta, qp, kp, with_qrot=True):
    import torch
    B, Hq, Hkv, Nq, Nk, D = dims
    o = torch.empty_like(qt)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    q_rot = torch.empty_like(qt) if with_qrot else None
    k_rot = torch.empty_like(kt)
    st = ra.ra_attn_fwd_rope(qt, kt, vt, o, stats, q_rot, k_rot, _dev_pos(qp), _dev_pos(kp), theta,
                             B, Hq, Hkv, Nq, Nk, D, causal, scale, _code(ra, qt))
    assert st == 0, ra.ra_status_string(st)
    return o, stats, q_rot, k_rot


def chain_fwd(ra, qt, kt, vt, dims, causal, scale, theta, qp, kp):
    import torch
    B, Hq, Hkv, Nq, Nk, D = dims
    qr, kr = torch.empty_like(qt), torch.empty_like(kt)
    assert ra.ra_rope_neox(qt, qr, _dev_pos(qp), B * Hq, Nq, D, theta, False, _code(ra, qt)) == 0
    assert ra.ra_rope_neox(kt, kr, _dev_pos(kp), B * Hkv, Nk, D, theta, False, _code(ra, qt)) == 0
    o = torch.empty_like(qt)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    st = ra.ra_attn_fwd(qr, kr, vt, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, _code(ra, qt))
    assert st == 0, ra.ra_status_string(st)
    return o, stats, qr, kr


def fused_bwd(ra, q_rot, k_rot, vt, o, dot, stats, dims, causal, scale, theta, qp, kp):
    import torch
    B, Hq, Hkv, Nq, Nk, D = dims
    dq, dk, dv = torch.empty_like(q_rot), torch.empty_like(k_rot), torch.empty_like(vt)
    nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, _code(ra, q_rot))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    st = ra.ra_attn_bwd_rope(q_rot, k_rot, vt, o, dot, stats, dq, dk, dv, ws, nbytes, _dev_pos(qp),
                             _dev_pos(kp), theta, B, Hq, Hkv, Nq, Nk, D, causal, scale, _code(ra, q_rot))
    assert st == 0, ra.ra_status_string(st)
    return dq, dk, dv


def rotation_bound_check(gpu, x, theta, positions, what, dtype="bf16"):
    """|gpu - exact| <= e |exact| + 2^-19 n per element (n: the norm of its pair; e = 2^-8 for
    bf16, 2^-24 for fp32)."""
    ex = oracle.rope_neox(x, theta, positions)
    h = ex.shape[-1] // 2
    n = np.sqrt(ex[..., :h] ** 2 + ex[..., h:] ** 2)
    n = np.concatenate([n, n], axis=-1)
    e = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    excess = np.abs(gpu - ex) - (e * np.abs(ex) + 2.0 ** -19 * n)
    assert excess.max() <= 0, f"{what}: rotation beyond one bf16 rounding by {excess.max():.3e}"


CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, positions, theta, dtype)
    (1, 2, 1, 200, 200, 64, 1, None, 10000.0, "bf16"),
    (2, 4, 2, 333, 333, 128, 1, "random", 500000.0, "bf16"),
    (1, 4, 4, 70, 1000, 128, 2, "random", 10000.0, "bf16"),
    (1, 2, 2, 129, 77, 64, 0, None, 10000.0, "bf16"),
    (1, 8, 2, 1, 300, 128, 2, None, 10000.0, "bf16"),
    (1, 2, 1, 64, 64, 128, 1, "random", 100.0, "bf16"),
    (1, 2, 1, 100, 100, 64, 1, "random", 10000.0, "f32"),
    (1, 8, 2, 70, 130, 128, 2, None, 500000.0, "f32"),
    (1, 3, 3, 45, 33, 64, 0, None, 10000.0, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fused_forward_equals_the_unfused_chain(gpu_lib, case):
    import torch
    B, Hq, Hkv, Nq, Nk, D, causal, pk, theta, dt = case
    dims = (B, Hq, Hkv, Nq, Nk, D)
    inp = _inputs(B, Hq, Hkv, Nq, Nk, D, seed=Nq + Nk + D, dtype=dt)
    qp, kp = _positions(pk, Nq, 1), _positions(pk, Nk, 2)
    scale = float(np.float32(1 / np.sqrt(D)))
    qt, kt, vt = (to_dev(inp[n], dt) for n in ("q", "k", "v"))
    print(f"fused forward {case}", flush=True)
    o, stats, q_rot, k_rot = fused_fwd(gpu_lib, qt, kt, vt, dims, causal, scale, theta, qp, kp)
    o2 = fused_fwd(gpu_lib, qt, kt, vt, dims, causal, scale, theta, qp, kp, with_qrot=False)[0]
    ro, rstats, qr, kr = chain_fwd(gpu_lib, qt, kt, vt, dims, causal, scale, theta, qp, kp)
    torch.cuda.synchronize()
    assert torch.equal(q_rot, qr) and torch.equal(k_rot, kr)
    assert torch.equal(o, ro) and torch.equal(o2, ro)
    assert torch.equal(stats, rstats)
    rotation_bound_check(to_np(q_rot), inp["q"], theta, qp, "q_rot", dt)
    rotation_bound_check(to_np(k_rot), inp["k"], theta, kp, "k_rot", dt)
    if dt == "f32":   # fp32: the whole output against the exact function at fp32's bound
        oc = {0: False, 1: True, 2: "bottom_right"}[causal]
        res = parity.fwd_rope_all_heads(to_np(o), stats.cpu().numpy().astype(np.float64), inp, oc,
                                        scale, theta, qp, kp, dtype="f32")
        print(f"{case}: {res}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_no_keys_still_writes_the_rotated_queries(gpu_lib, dt):
    import torch
    inp = _inputs(1, 2, 1, 37, 0, 64, seed=3, dtype=dt)
    qt = to_dev(inp["q"], dt)
    kt = vt = torch.empty((1, 1, 0, 64), dtype=qt.dtype, device="cuda")
    o, stats, q_rot, _ = fused_fwd(gpu_lib, qt, kt, vt, (1, 2, 1, 37, 0, 64), 0, 0.125, 10000.0,
                                   None, None)
    torch.cuda.synchronize()
    assert (to_np(o) == 0).all()
    s = stats.cpu().numpy()
    assert np.isneginf(s[..., 0]).all() and (s[..., 1] == 0).all()
    rotation_bound_check(to_np(q_rot), inp["q"], 10000.0, None, "q_rot", dt)


def test_grouped_query_workload_every_head(gpu_lib):
    w = wl.WORKLOADS[GQA]
    inp = wl.make_unrotated_inputs(w)
    dims = (w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D)
    qt, kt, vt = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    print(f"fused forward {GQA}: {w.B * w.Hq} heads", flush=True)
    import torch
    o, stats, q_rot, k_rot = fused_fwd(gpu_lib, qt, kt, vt, dims, 1, w.scale, w.rope_theta, None, None)
    torch.cuda.synchronize()
    res = parity.fwd_rope_all_heads(to_np(o), stats.cpu().numpy().astype(np.float64), inp, True,
                                    w.scale, w.rope_theta)
    print(f"{GQA} fused forward: {res}")
    rotation_bound_check(to_np(q_rot), inp["q"], w.rope_theta, None, "q_rot")


BWD_CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, positions, theta, dtype)
    (1, 4, 2, 300, 300, 128, 1, "shifted", 10000.0, "bf16"),
    (2, 2, 1, 200, 520, 64, 2, "random", 500000.0, "bf16"),
    (1, 2, 2, 150, 90, 64, 0, None, 10000.0, "bf16"),
    (1, 2, 1, 96, 96, 64, 1, "shifted", 10000.0, "f32"),
    (1, 4, 2, 64, 150, 128, 2, "random", 500000.0, "f32"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_fused_backward_against_the_oracle(gpu_lib, case):
    import torch
    B, Hq, Hkv, Nq, Nk, D, causal, pk, theta, dt = case
    dims = (B, Hq, Hkv, Nq, Nk, D)
    inp = _inputs(B, Hq, Hkv, Nq, Nk, D, seed=7 * Nq + Nk, dtype=dt)
    if pk == "shifted":
        qp, kp = np.arange(Nq, dtype=np.int32) + 17, np.arange(Nk, dtype=np.int32) + 17
    else:
        qp, kp = _positions(pk, Nq, 5), _positions(pk, Nk, 6)
    scale = float(np.float32(1 / np.sqrt(D)))
    qt, kt, vt, dot = (to_dev(inp[n], dt) for n in ("q", "k", "v", "do"))
    print(f"fused backward {case}", flush=True)
    o, stats, q_rot, k_rot = fused_fwd(gpu_lib, qt, kt, vt, dims, causal, scale, theta, qp, kp)
    dq, dk, dv = fused_bwd(gpu_lib, q_rot, k_rot, vt, o, dot, stats, dims, causal, scale, theta, qp, kp)
    dq2, dk2, dv2 = fused_bwd(gpu_lib, q_rot, k_rot, vt, o, dot, None, dims, causal, scale, theta,
                              qp, kp)
    torch.cuda.synchronize()
    # without the saved statistics the backward recomputes them from the rotated rows
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    oc = {0: False, 1: True, 2: "bottom_right"}[causal]
    res = parity.bwd_all_groups(to_np(dq), to_np(dk), to_np(dv), inp, oc, scale, dt,
                                rope={"theta": theta, "q_positions": qp, "k_positions": kp})
    print(f"{case}: {res}")


def _pair_norm(x):
    h = x.shape[-1] // 2
    n = np.sqrt(x[..., :h] ** 2 + x[..., h:] ** 2)
    return np.concatenate([n, n], axis=-1)


def test_grouped_query_backward_against_the_unfused_chain(gpu_lib):
    """The fused epilogues rotate the fp32 accumulators back before the one bf16 rounding; the
    unfused chain rounds dQ and dK of the rotated rows, then rotates those back.  The two differ
    by at most two bf16 roundings of a pair's norm.  dV takes no rotation: bit for bit."""
    import torch
    w = wl.WORKLOADS[GQA]
    inp = wl.make_unrotated_inputs(w)
    dims = (w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D)
    qt, kt, vt, dot = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    print(f"fused backward {GQA}", flush=True)
    o, stats, q_rot, k_rot = fused_fwd(gpu_lib, qt, kt, vt, dims, 1, w.scale, w.rope_theta, None, None)
    dq, dk, dv = fused_bwd(gpu_lib, q_rot, k_rot, vt, o, dot, stats, dims, 1, w.scale, w.rope_theta,
                           None, None)
    dqr, dkr, dvr = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
    nbytes = gpu_lib.ra_attn_bwd_workspace_bytes(*dims, gpu_lib.RA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert gpu_lib.ra_attn_bwd(q_rot, k_rot, vt, o, dot, stats, dqr, dkr, dvr, ws, nbytes, *dims, 1,
                               w.scale, gpu_lib.RA_BF16) == 0
    for t, H, N in ((dqr, w.Hq, w.Nq), (dkr, w.Hkv, w.Nk)):
        assert gpu_lib.ra_rope_neox(t, t, None, w.B * H, N, w.D, w.rope_theta, True, gpu_lib.RA_BF16) == 0
    torch.cuda.synchronize()
    assert torch.equal(dv, dvr)
    for name, a, b in (("dq", dq, dqr), ("dk", dk, dkr)):
        a, b = to_np(a), to_np(b)
        excess = np.abs(a - b) - 1.01 * 2.0 ** -7 * _pair_norm(b) - 1e-30
        print(f"{name}: max |fused - chain| {np.abs(a - b).max():.3e}, max |chain| {np.abs(b).max():.3e}")
        assert excess.max() <= 0, f"{name}: beyond two bf16 roundings by {excess.max():.3e}"


def test_grouped_query_backward_every_group(gpu_lib):
    """The fused backward of the grouped-query workload against the oracle's gradient with
    respect to the unrotated rows, on every (batch, K/V head) group; near ties of the row max
    within the rounding bound of the rotated rows are taken either way (tests/parity.py)."""
    w = wl.WORKLOADS[GQA]
    inp = wl.make_unrotated_inputs(w)
    dims = (w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D)
    qt, kt, vt, dot = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    print(f"fused backward {GQA}: every group", flush=True)
    o, stats, q_rot, k_rot = fused_fwd(gpu_lib, qt, kt, vt, dims, 1, w.scale, w.rope_theta, None, None)
    dq, dk, dv = fused_bwd(gpu_lib, q_rot, k_rot, vt, o, dot, stats, dims, 1, w.scale, w.rope_theta,
                           None, None)
    import torch
    torch.cuda.synchronize()
    res = parity.bwd_all_groups(to_np(dq), to_np(dk), to_np(dv), inp, True, w.scale, "bf16",
                                rope={"theta": w.rope_theta, "q_positions": None, "k_positions": None})
    print(f"{GQA} fused backward: {res}")


MASK_CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, mask layout, dtype)
    (2, 8, 2, 200, 256, 128, 2, "keypad", "bf16"),          # key padding fast path
    (2, 4, 2, 130, 130, 64, 1, "keypad", "bf16"),           # Nk % 4 != 0: the general masked kernels
    (1, 4, 2, 100, 140, 128, 0, "head_bias", "bf16"),       # additive, per query head, -inf entries
    (1, 4, 2, 256, 256, 128, 1, "documents_mixed", "bf16"),  # additive 0 / -inf blocks read ahead as words
    (2, 2, 1, 200, 200, 64, 2, "documents_mixed", "bf16"),    # the same at D = 64, ragged tail
    (1, 2, 1, 77, 90, 64, 2, "full_bool", "f32"),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[str(c) for c in MASK_CASES])
def test_masked_rotary_attention_equals_the_unfused_chain(gpu_lib, case):
    """With an explicit mask: the fused forward equals the rotation passes followed by
    ra_attn_fwd_masked bit for bit, and O matches the oracle; the fused backward matches
    ra_attn_bwd_masked on the rotated rows followed by the inverse rotation (dV bit for bit; dQ
    and dK within two roundings of the dtype)."""
    import torch
    from test_mask_gpu import make_mask
    ra = gpu_lib
    B, Hq, Hkv, Nq, Nk, D, causal, layout, dt = case
    dims = (B, Hq, Hkv, Nq, Nk, D)
    theta = 10000.0
    inp = _inputs(B, Hq, Hkv, Nq, Nk, D, seed=Nq * 3 + Nk, dtype=dt)
    mask_np, t, kind, strides = make_mask(layout, B, Hq, Nq, Nk, dt, seed=Nq + Nk)
    scale = float(np.float32(1 / np.sqrt(D)))
    code = ra.RA_BF16 if dt == "bf16" else ra.RA_F32
    qt, kt, vt, dot = (to_dev(inp[n], dt) for n in ("q", "k", "v", "do"))
    print(f"masked rotary {case}", flush=True)
    o = torch.empty_like(qt)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    q_rot, k_rot = torch.empty_like(qt), torch.empty_like(kt)
    assert ra.ra_attn_fwd_rope(qt, kt, vt, o, stats, q_rot, k_rot, None, None, theta, *dims, causal,
                               scale, code, t, kind, strides) == 0
    qr, kr = torch.empty_like(qt), torch.empty_like(kt)
    assert ra.ra_rope_neox(qt, qr, None, B * Hq, Nq, D, theta, False, code) == 0
    assert ra.ra_rope_neox(kt, kr, None, B * Hkv, Nk, D, theta, False, code) == 0
    ro, rstats = torch.empty_like(qt), torch.empty_like(stats)
    assert ra.ra_attn_fwd_masked(qr, kr, vt, ro, rstats, *dims, causal, scale, code, t, kind,
                                 strides) == 0
    nbytes = ra.ra_attn_bwd_workspace_bytes(*dims, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
    assert ra.ra_attn_bwd_rope(q_rot, k_rot, vt, o, dot, stats, dq, dk, dv, ws, nbytes, None, None,
                               theta, *dims, causal, scale, code, t, kind, strides) == 0
    cq, ck, cv = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
    assert ra.ra_attn_bwd_masked(qr, kr, vt, ro, dot, rstats, cq, ck, cv, ws, nbytes, *dims, causal,
                                 scale, code, t, kind, strides) == 0
    for x, H, N in ((cq, Hq, Nq), (ck, Hkv, Nk)):
        assert ra.ra_rope_neox(x, x, None, B * H, N, D, theta, True, code) == 0
    torch.cuda.synchronize()
    assert torch.equal(q_rot, qr) and torch.equal(k_rot, kr)
    assert torch.equal(o, ro) and torch.equal(stats, rstats)
    assert torch.equal(dv, cv)
    e = 2.0 ** -8 if dt == "bf16" else 2.0 ** -23
    for name, a, b in (("dq", dq, cq), ("dk", dk, ck)):
        a, b = to_np(a), to_np(b)
        excess = np.abs(a - b) - 1.01 * 2 * e * _pair_norm(b)
        assert excess.max() <= 0, f"{name}: beyond two roundings by {excess.max():.3e}"
    oc = {0: False, 1: True, 2: "bottom_right"}[causal]
    ref = oracle.ra_attention_rope_fwd(inp["q"], inp["k"], inp["v"], oc, scale, theta,
                                       mask=mask_np)[0]
    from helpers import assert_close
    err = assert_close(to_np(o), ref, dt, "masked rotary O")
    print(f"{case}: O err {err:.3e}")
