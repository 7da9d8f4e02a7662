"""GPU parity of ra_attn_bwd (through the C ABI) against the fp64 oracle.

Tolerances (per tensor dQ, dK, dV): bf16 max|gpu - oracle| / max|oracle| <= 2e-2;
fp32 max-abs 1e-5, relative to max|oracle| when that exceeds 1.  The full-size workloads are
checked on every (batch, K/V head) group in test_full_parity_gpu.py.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, rel_to_max, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_fwd_bwd(ra, inp, causal, scale, dtype, use_stats=True):
    import torch
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    assert ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, code) == 0
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = ra.ra_attn_bwd(q, k, v, o, do, stats if use_stats else None, dq, dk, dv, ws, nbytes,
                        B, Hq, Hkv, Nq, Nk, D, causal, scale, code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv)


def rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    out = {
        "q": rng.standard_normal((B, Hq, Nq, D), dtype=np.float32) * np.float32(sigma),
        "k": rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32) * np.float32(sigma),
        "v": rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32),
        "do": rng.standard_normal((B, Hq, Nq, D), dtype=np.float32),
    }
    return {n: wl.round_to_dtype(a, dtype) for n, a in out.items()}


def check(grads, inp, causal, scale, dtype, groups=None, what=""):
    ref = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale,
                                  groups=groups)
    errs = []
    Hq, Hkv = inp["q"].shape[1], inp["k"].shape[1]
    rep = Hq // Hkv
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        if groups is not None:
            if name == "dq":
                idx = [(b, h) for b, gg in groups for h in range(gg * rep, (gg + 1) * rep)]
            else:
                idx = list(groups)
            bi = [x for x, _ in idx]
            hi = [y for _, y in idx]
            g, r = g[bi, hi], r[bi, hi]
        assert_close(g, r, dtype, f"{what} {name}", grad=True)
        errs.append(rel_to_max(g, r))
    return errs


SHAPES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, dtype)
    (1, 2, 1, 64, 64, 64, True, "f32"),
    (1, 2, 2, 37, 37, 64, False, "f32"),
    (2, 3, 1, 65, 65, 128, True, "f32"),
    (1, 4, 4, 130, 97, 128, False, "f32"),
    (1, 2, 1, 1, 1, 64, True, "bf16"),
    (2, 4, 2, 63, 63, 64, True, "bf16"),
    (1, 6, 3, 129, 129, 128, True, "bf16"),
    (3, 2, 2, 200, 200, 128, False, "bf16"),
    (1, 8, 1, 300, 300, 64, True, "bf16"),
    (2, 3, 3, 97, 250, 64, True, "bf16"),     # Nq < Nk
    (1, 4, 2, 250, 97, 128, True, "bf16"),    # Nq > Nk
    (1, 12, 4, 160, 160, 128, True, "bf16"),  # REP = 3
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_bwd_shapes(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, D, causal, dtype = shape
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed=Nq * 7 + Nk + D)
    scale = float(np.float32(1 / np.sqrt(D)))
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale, dtype)
    errs = check(grads, inp, causal, scale, dtype, what=str(shape))
    print(f"{shape}: rel-to-max errors dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")


def test_bwd_wide_scores(gpu_lib):
    """Score spread ~4 std: many entries off the support and near its edge."""
    inp = rand_inputs(1, 4, 2, 256, 256, 64, "bf16", seed=3, sigma=2.0)
    grads = run_fwd_bwd(gpu_lib, inp, True, 0.125, "bf16")
    check(grads, inp, True, 0.125, "bf16", what="wide")


def test_bwd_small_workload(gpu_lib):
    w = wl.WORKLOADS["bf16_causal_B2_H12_N128_D64"]
    rng_inp = rand_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, "bf16", seed=w.seed)
    grads = run_fwd_bwd(gpu_lib, rng_inp, True, w.scale, "bf16")
    check(grads, rng_inp, True, w.scale, "bf16", what=w.name)


def test_bwd_invariants(gpu_lib):
    inp = rand_inputs(2, 4, 2, 150, 150, 64, "f32", seed=11)
    dq, dk, dv = run_fwd_bwd(gpu_lib, inp, True, 0.125, "f32")
    # shift invariance: sum over keys of dK vanishes per K/V head
    assert np.abs(dk.sum(axis=2)).max() <= 1e-4 * np.abs(dk).sum(axis=2).max()
    # rows of P sum to one: sum_j dV_j = sum of dO over the group's query rows
    dsum = inp["do"].astype(np.float64).reshape(2, 2, 2, 150, 64).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), dsum, rtol=1e-4, atol=1e-4)
    # the loss depends on q.k only: <Q, dQ> = <K, dK>
    a = float(np.sum(inp["q"] * dq))
    b = float(np.sum(inp["k"] * dk))
    assert abs(a - b) <= 1e-4 * (abs(a) + abs(b) + 1)


def test_bwd_gqa_matches_summed_mha(gpu_lib):
    inp = rand_inputs(1, 8, 2, 96, 96, 128, "f32", seed=13)
    rep = 4
    mha = dict(inp)
    mha["k"] = np.repeat(inp["k"], rep, axis=1)
    mha["v"] = np.repeat(inp["v"], rep, axis=1)
    g1 = run_fwd_bwd(gpu_lib, inp, True, 0.0883883461356163, "f32")
    g2 = run_fwd_bwd(gpu_lib, mha, True, 0.0883883461356163, "f32")
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-6)
    np.testing.assert_allclose(g1[1], g2[1].reshape(1, 2, rep, 96, 128).sum(axis=2), atol=2e-5)
    np.testing.assert_allclose(g1[2], g2[2].reshape(1, 2, rep, 96, 128).sum(axis=2), atol=2e-5)


def test_bwd_without_stats_is_identical(gpu_lib):
    inp = rand_inputs(2, 4, 2, 100, 100, 128, "bf16", seed=17)
    a = run_fwd_bwd(gpu_lib, inp, True, 0.0883883461356163, "bf16", use_stats=True)
    b = run_fwd_bwd(gpu_lib, inp, True, 0.0883883461356163, "bf16", use_stats=False)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_deterministic(gpu_lib):
    inp = rand_inputs(1, 4, 4, 257, 257, 64, "bf16", seed=19)
    a = run_fwd_bwd(gpu_lib, inp, True, 0.125, "bf16")
    b = run_fwd_bwd(gpu_lib, inp, True, 0.125, "bf16")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_empty_sizes(gpu_lib):
    import torch
    ra = gpu_lib
    q = torch.randn(1, 2, 5, 64, device="cuda")
    k = torch.empty(1, 2, 0, 64, device="cuda")
    dq = torch.full_like(q, 3.0)
    st = ra.ra_attn_bwd(q, k, k, q, q, None, dq, k, k, None, 0, 1, 2, 2, 5, 0, 64, 1, 0.125, ra.RA_F32)
    assert st == 0
    torch.cuda.synchronize()
    assert (dq == 0).all()
    q0 = torch.empty(1, 2, 0, 64, device="cuda")
    k1 = torch.randn(1, 2, 7, 64, device="cuda")
    dk, dv = torch.full_like(k1, 3.0), torch.full_like(k1, 3.0)
    st = ra.ra_attn_bwd(q0, k1, k1, q0, q0, None, q0, dk, dv, None, 0, 1, 2, 2, 0, 7, 64, 1,
                        0.125, ra.RA_F32)
    assert st == 0
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()


def test_autograd_wrapper(gpu_lib):
    import torch
    inp = rand_inputs(1, 4, 2, 80, 80, 64, "f32", seed=21)
    q, k, v = (torch.from_numpy(inp[n]).cuda().requires_grad_() for n in ("q", "k", "v"))
    o = gpu_lib.ra_attention(q, k, v, is_causal=True)
    o.backward(torch.from_numpy(inp["do"]).cuda())
    ref_o = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], True, 0.125)[0]
    ref = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.125)
    assert_close(o.detach().cpu().numpy().astype(np.float64), ref_o, "f32", "o")
    for t, r, n in zip((q, k, v), ref, ("dq", "dk", "dv")):
        assert_close(t.grad.cpu().numpy().astype(np.float64), r, "f32", n, grad=True)


@pytest.mark.parametrize("dtype,use_stats", [("bf16", True), ("bf16", False), ("f32", True)])
def test_bwd_phases_equal_whole_call(gpu_lib, dtype, use_stats):
    """ra_attn_bwd_dq then ra_attn_bwd_dkdv reproduces ra_attn_bwd bit for bit."""
    import torch
    ra = gpu_lib
    B, Hq, Hkv, N, D = 2, 4, 2, 200, 128
    inp = rand_inputs(B, Hq, Hkv, N, N, D, dtype, seed=23)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    scale = 0.0883883461356163
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, N, 2), dtype=torch.float32, device="cuda")
    assert ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, N, N, D, True, scale, code) == 0
    st = stats if use_stats else None
    nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, N, N, D, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    whole = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    assert ra.ra_attn_bwd(q, k, v, o, do, st, *whole, ws, nbytes, B, Hq, Hkv, N, N, D, True,
                          scale, code) == 0
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert ra.ra_attn_bwd_dq(q, k, v, o, do, st, dq, ws2, nbytes, B, Hq, Hkv, N, N, D, True,
                             scale, code) == 0
    assert ra.ra_attn_bwd_dkdv(q, k, v, do, st, dk, dv, ws2, nbytes, B, Hq, Hkv, N, N, D, True,
                               scale, code) == 0
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), whole):
        assert torch.equal(x, y)
