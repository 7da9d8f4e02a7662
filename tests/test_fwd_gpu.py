"""GPU parity of ra_attn_fwd (through the C ABI) against the fp64 oracle.

Tolerances: fp32 inputs max-abs 1e-5 (absolute); bf16 inputs max|gpu - oracle| / max|oracle|
<= 2e-2.  The full-size workloads are checked on every head in test_full_parity_gpu.py.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import (ULP16, U32, assert_close, score_error_bound, to_dev, to_np,
                     zero_pattern_mismatches)

pytestmark = pytest.mark.gpu


def run_fwd(ra, inp, causal, scale, dtype, counted=False):
    import torch
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    if counted:
        cnt = torch.zeros(4, dtype=torch.int64, device="cuda")
        st = ra.ra_attn_fwd_counted(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, code, cnt)
    else:
        cnt = None
        st = ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    out = (to_np(o), stats.cpu().numpy().astype(np.float64))
    if counted:
        return out + (cnt.cpu().numpy(),)
    return out


def rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, D), dtype=np.float32) * np.float32(sigma)
    k = rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32) * np.float32(sigma)
    v = rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32)
    return {n: wl.round_to_dtype(a, dtype) for n, a in (("q", q), ("k", k), ("v", v))}


def check_against_oracle(o, stats, inp, causal, scale, dtype, heads=None, what=""):
    ro, rm, rl, _ = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale, heads=heads)
    if heads is None:
        sel = (slice(None),)
        g_o, r_o = o, ro
        g_m, r_m, g_l, r_l = stats[..., 0], rm, stats[..., 1], rl
    else:
        bi = [b for b, _ in heads]
        hi = [h for _, h in heads]
        g_o, r_o = o[bi, hi], ro[bi, hi]
        g_m, r_m, g_l, r_l = stats[bi, hi, :, 0], rm[bi, hi], stats[bi, hi, :, 1], rl[bi, hi]
    err = assert_close(g_o, r_o, dtype, what)
    # stats: m is the raw dot-product max, the oracle's the scaled one
    np.testing.assert_allclose(g_m * scale, r_m, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(g_l, r_l, rtol=(1e-5 if dtype == "f32" else 1e-2))
    return err


# ----------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["fp32_noncausal_B1_H2_N128_D64", "bf16_causal_B2_H12_N128_D64"])
def test_small_workloads_full(gpu_lib, name):
    w = wl.WORKLOADS[name]
    inp = wl.make_attention_inputs(w)
    o, stats = run_fwd(gpu_lib, inp, w.causal, w.scale, w.dtype)
    err = check_against_oracle(o, stats, inp, w.causal, w.scale, w.dtype, what=name)
    print(f"{name}: max abs err {err:.3e}")


# ----------------------------------------------------------------- edge shapes

EDGE = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, dtype)
    (1, 1, 1, 1, 1, 64, True, "bf16"),
    (1, 2, 1, 63, 63, 64, True, "bf16"),
    (2, 3, 1, 65, 65, 128, True, "bf16"),
    (1, 4, 2, 127, 127, 64, False, "bf16"),
    (3, 2, 2, 129, 129, 128, True, "bf16"),
    (1, 8, 1, 1000, 1000, 128, True, "bf16"),
    (2, 6, 2, 97, 300, 64, True, "bf16"),     # Nq < Nk, top-left causal
    (2, 6, 3, 300, 97, 128, True, "bf16"),    # Nq > Nk: late rows see every key
    (1, 5, 5, 77, 1, 64, True, "bf16"),       # a single key
    (1, 5, 5, 77, 1, 64, False, "f32"),
    (2, 3, 1, 65, 130, 64, False, "f32"),
    (1, 4, 4, 200, 200, 128, True, "f32"),
    (1, 2, 1, 33, 33, 128, True, "f32"),
    (1, 16, 2, 96, 96, 64, True, "bf16"),     # REP = 8: two workgroups per row block
    (1, 12, 4, 70, 70, 128, True, "bf16"),    # REP = 3: tasks straddle row blocks
]


@pytest.mark.parametrize("shape", EDGE, ids=[str(e) for e in EDGE])
def test_edge_shapes(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, D, causal, dtype = shape
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed=B * 1000 + Nq + Nk)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, stats = run_fwd(gpu_lib, inp, causal, scale, dtype)
    check_against_oracle(o, stats, inp, causal, scale, dtype, what=str(shape))


def test_zero_key_rows_give_zero_output(gpu_lib):
    import torch
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    stats = torch.zeros(1, 2, 5, 2, device="cuda")
    st = gpu_lib.ra_attn_fwd(q, k, k, o, stats, 1, 2, 2, 5, 0, 64, 1, 0.125, gpu_lib.RA_BF16)
    assert st == 0
    torch.cuda.synchronize()
    assert (o == 0).all()
    assert torch.isinf(stats[..., 0]).all() and (stats[..., 1] == 0).all()


# ----------------------------------------------------------------- semantic probes

def test_causality_probe(gpu_lib):
    """Row t must not see keys t+1...: perturbing them leaves rows <= t bit-identical."""
    B, H, N, D = 1, 2, 200, 64
    inp = rand_inputs(B, H, H, N, N, D, "bf16", seed=5)
    o1, _ = run_fwd(gpu_lib, inp, True, 0.125, "bf16")
    rng = np.random.default_rng(6)
    for t in (0, 31, 32, 63, 64, 150):
        inp2 = {n: a.copy() for n, a in inp.items()}
        for n in ("k", "v"):
            inp2[n][:, :, t + 1:] = wl.round_to_dtype(
                rng.standard_normal(inp2[n][:, :, t + 1:].shape).astype(np.float32), "bf16")
        o2, _ = run_fwd(gpu_lib, inp2, True, 0.125, "bf16")
        np.testing.assert_array_equal(o1[:, :, : t + 1], o2[:, :, : t + 1])
        assert not np.array_equal(o1[:, :, t + 1:], o2[:, :, t + 1:])


def test_gqa_equals_mha_on_repeated_kv_bitwise(gpu_lib):
    B, Hq, Hkv, N, D = 2, 8, 2, 150, 128
    inp = rand_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=7)
    rep = Hq // Hkv
    inp_mha = {"q": inp["q"], "k": np.repeat(inp["k"], rep, axis=1),
               "v": np.repeat(inp["v"], rep, axis=1)}
    o1, s1 = run_fwd(gpu_lib, inp, True, 0.0883883461356163, "bf16")
    o2, s2 = run_fwd(gpu_lib, inp_mha, True, 0.0883883461356163, "bf16")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_deterministic(gpu_lib):
    w = wl.WORKLOADS["bf16_causal_B2_H12_N128_D64"]
    inp = wl.make_attention_inputs(w)
    a = run_fwd(gpu_lib, inp, True, w.scale, "bf16")
    b = run_fwd(gpu_lib, inp, True, w.scale, "bf16")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_one_hot_rows_select_value_exactly(gpu_lib):
    B, H, N, D = 1, 2, 64, 64
    rng = np.random.default_rng(8)
    k = np.zeros((B, H, N, D), np.float32)
    k[0, :, np.arange(N), np.arange(N)] = 1.0
    target = rng.permutation(N)
    q = np.zeros((B, H, N, D), np.float32)
    q[0, :, np.arange(N), target] = 256.0          # score 32 at the target, 0 elsewhere
    v = wl.round_to_dtype(rng.standard_normal((B, H, N, D)).astype(np.float32), "bf16")
    o, stats = run_fwd(gpu_lib, {"q": q, "k": k, "v": v}, False, 0.125, "bf16")
    np.testing.assert_array_equal(o[0, 0], v[0, 0, target])
    assert (stats[..., 1] == 1.0).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_zero_support_pattern_via_identity_values(gpu_lib, causal, dtype, D):
    """With V = I (Nk = D keys) the output row is the probability row, so the set of exact
    zeros is observable; it must match the oracle's {u >= 1} except inside the band."""
    B, H, N = 2, 3, D
    rng = np.random.default_rng(9 + D)
    q = wl.round_to_dtype(rng.standard_normal((B, H, N, D)).astype(np.float32) * 2.5, dtype)
    k = wl.round_to_dtype(rng.standard_normal((B, H, N, D)).astype(np.float32) * 2.5, dtype)
    v = np.broadcast_to(np.eye(N, D, dtype=np.float32), (B, H, N, D)).copy()
    scale = float(np.float32(1 / np.sqrt(D)))
    o, _ = run_fwd(gpu_lib, {"q": q, "k": k, "v": v}, causal, scale, dtype)
    p_ora, _, _, _ = oracle.ra_attention_fwd(q, k, v, causal, scale)
    total_bad = total_mism = total_zero = 0
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T)
            allowed = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
            sm = np.where(allowed, s, -np.inf)
            m = sm.max(axis=1, keepdims=True)
            delta = np.where(allowed, m - s, np.inf)
            es = score_error_bound(q[b, h].astype(np.float64), k[b, h].astype(np.float64), scale)
            # phi = 0 on the GPU iff 1 + u = fma(s, -c, kd) >= 2 (c = scale / 16, kd = 1 + m c):
            # beside the score errors of s and m, the rounding of kd and of 1 + u (half an ulp
            # each, at most 2^-23 for values below 4) and the reciprocal's error (one ulp of 0.5,
            # 2^-22 in units of 1 + u) move the edge by at most 2^-21 in 1 + u, 16 * 2^-21 =
            # 8 * 2^-24 * 16 in Delta; kd < 4 needs a scaled row max below 48
            assert np.nanmax(m) < 48
            band = ULP16 + es + es[np.arange(N), sm.argmax(1)][:, None] + 8 * U32 * 16
            bad, mism = zero_pattern_mismatches(o[b, h], p_ora[b, h], delta, band)
            total_bad += bad
            total_mism += mism
            total_zero += int((p_ora[b, h] == 0).sum())
    print(f"zeros in oracle: {total_zero}, mismatches in band: {total_mism}, outside: {total_bad}")
    assert total_zero > 0
    assert total_bad == 0


def test_tile_skipping_structured_workload(gpu_lib):
    """Scores that fall off away from the diagonal: whole tiles leave the support and are
    skipped; the output still matches the oracle."""
    inp = wl.make_local_inputs(B=1, H=4, N=2048, D=64, amplitude=4.0)
    o, stats, cnt = run_fwd(gpu_lib, inp, True, 0.125, "bf16", counted=True)
    print(f"counters: wave tiles {cnt[0]}, skipped {cnt[1]}, wg tiles {cnt[2]}, wg skipped {cnt[3]}")
    assert cnt[1] > 0 and cnt[3] > 0
    assert cnt[1] <= cnt[0] and cnt[3] <= cnt[2]
    # every (wave, key tile) pair inside the causal range is counted, dropped or not: a wave owns
    # 32 query rows q0..q0+31 and sees the 64-key tiles below ceil((q0 + 32) / 64)
    assert cnt[0] == 4 * sum(-(-(q0 + 32) // 64) for q0 in range(0, 2048, 32))
    check_against_oracle(o, stats, inp, True, 0.125, "bf16", heads=[(0, 0), (0, 3)], what="local")
    # the counting variant computes the same bits as the plain one
    o2, s2 = run_fwd(gpu_lib, inp, True, 0.125, "bf16")
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(stats, s2)


def test_iid_workload_skips_nothing_in_range(gpu_lib):
    w = wl.WORKLOADS["bf16_causal_B2_H12_N128_D64"]
    inp = wl.make_attention_inputs(w)
    _, _, cnt = run_fwd(gpu_lib, inp, True, w.scale, "bf16", counted=True)
    assert cnt[0] > 0 and cnt[1] == 0
