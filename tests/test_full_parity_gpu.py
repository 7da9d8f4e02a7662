"""Full-size parity through the C ABI: every (batch, head) of the forward and every (batch, K/V
head) group of the backward of the measured workloads, in the launch configuration the bench
times, element by element against the fp64 oracle (tests/parity.py).  Also long key ranges past
the forward's 512 recorded tile maxima.

Tolerances: bf16 max|gpu - oracle| / max|oracle| <= 2e-2 per tensor; fp32 max-abs 1e-5 for O.
"""
import numpy as np
import pytest

import oracle
import parity
import workloads as wl
from helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

C3 = "bf16_causal_B8_H16_N2048_D64_sigma2"
C4 = "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"
C5 = "bf16_causal_B4_H16_N8192_D128_fwd_bwd"


def gpu_run(ra, inp, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, bwd):
    """Forward (and backward) over the whole launch; host float64 copies of the outputs."""
    import torch
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    st = ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, code)
    assert st == 0, ra.ra_status_string(st)
    out = {}
    if bwd:
        do = to_dev(inp["do"], dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = ra.ra_attn_bwd(q, k, v, o, do, stats, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                            causal, scale, code)
        assert st == 0, ra.ra_status_string(st)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    res = {n: to_np(t) for n, t in out.items()}
    res["o"] = to_np(o)
    res["stats"] = stats.cpu().numpy().astype(np.float64)
    for n, t in res.items():
        if n != "stats":
            assert np.isfinite(t).all(), n
    return res


def workload_inputs(name, with_do=False):
    w = wl.WORKLOADS[name]
    inp = wl.make_attention_inputs(w)
    if with_do and "do" not in inp:
        # the grouped-query workload has no upstream gradient of its own: a seeded N(0, 1) one
        inp["do"] = wl.round_to_dtype(
            np.random.default_rng(99).standard_normal(inp["q"].shape, dtype=np.float32), w.dtype)
    return w, inp


@pytest.mark.parametrize("name", [C3, C4, C5])
def test_forward_every_head(gpu_lib, name):
    w, inp = workload_inputs(name)
    print(f"forward {name}: {w.B * w.Hq} heads", flush=True)
    r = gpu_run(gpu_lib, inp, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, int(w.causal), w.scale, w.dtype,
                bwd=False)
    res = parity.fwd_all_heads(r["o"], r["stats"], inp, w.causal, w.scale, w.dtype)
    print(f"forward {name}: {res}")


@pytest.mark.parametrize("name,part,parts", [(C4, 0, 1), (C5, 0, 2), (C5, 1, 2)])
def test_backward_every_group(gpu_lib, name, part, parts):
    """Every (batch, K/V head) group; the larger workload's groups in two halves so that each
    test stays short."""
    w, inp = workload_inputs(name, with_do=True)
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    n = len(groups)
    groups = groups[part * n // parts:(part + 1) * n // parts]
    print(f"backward {name}: groups {groups[0]}..{groups[-1]}", flush=True)
    r = gpu_run(gpu_lib, inp, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, int(w.causal), w.scale, w.dtype,
                bwd=True)
    res = parity.bwd_all_groups(r["dq"], r["dk"], r["dv"], inp, w.causal, w.scale, w.dtype,
                                groups=groups)
    print(f"backward {name} part {part}: {res}")


# ----------------------------------------------------------------- past 512 key tiles
# The forward records a maximum for the first 512 key tiles of a workgroup (64 keys per bf16
# tile, 32 per fp32 tile) and tests later tiles for skipping by their position only.

LONG = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, dtype, sampled query rows or None for all)
    (1, 2, 1, 64, 33000, 64, 0, "bf16", None),
    (1, 4, 2, 70, 33000, 128, 2, "bf16", None),          # bottom-right: late rows see every key
    (1, 1, 1, 33000, 33000, 64, 1, "bf16", "sample"),    # top-left over the whole range
    (1, 2, 2, 40, 17000, 64, 0, "f32", None),
    (1, 2, 1, 50, 17000, 128, 2, "f32", None),
    (1, 1, 1, 17000, 17000, 64, 1, "f32", "sample"),
]


@pytest.mark.parametrize("case", LONG, ids=[str(c[:8]) for c in LONG])
def test_forward_past_512_key_tiles(gpu_lib, case):
    B, Hq, Hkv, Nq, Nk, D, causal, dtype, rows = case
    rng = np.random.default_rng(Nq + Nk + D)
    inp = {n: wl.round_to_dtype(rng.standard_normal(s, dtype=np.float32), dtype)
           for n, s in (("q", (B, Hq, Nq, D)), ("k", (B, Hkv, Nk, D)), ("v", (B, Hkv, Nk, D)))}
    scale = float(np.float32(1 / np.sqrt(D)))
    print(f"long forward {case}", flush=True)
    r = gpu_run(gpu_lib, inp, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, bwd=False)
    oc = {0: False, 1: "top_left", 2: "bottom_right"}[causal]
    if rows is None:
        res = parity.fwd_all_heads(r["o"], r["stats"], inp, oc, scale, dtype)
        print(f"{case}: {res}")
        return
    # every query row of a causal Nq = Nk launch is too many for the oracle: rows at the start,
    # around the 512th tile and at the end, each compared with the oracle on its own keys
    tile = 64 if dtype == "bf16" else 32
    pos = np.unique(np.concatenate([np.arange(0, 40), np.arange(512 * tile - 40, 512 * tile + 40),
                                    np.arange(Nq - 64, Nq)]))
    ro, rm, rl, _ = oracle.ra_attention_fwd(inp["q"][:, :, pos], inp["k"], inp["v"], oc, scale,
                                            q_positions=pos, nq_total=Nq)
    err = assert_close(r["o"][:, :, pos], ro, dtype, str(case))
    np.testing.assert_allclose(r["stats"][:, :, pos, 0] * scale, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(r["stats"][:, :, pos, 1], rl, rtol=(1e-5 if dtype == "f32" else 1e-2))
    print(f"{case}: {len(pos)} rows, err {err:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_long_key_range(gpu_lib, dtype):
    """The backward over a key range past 512 tiles (bottom-right: the rows see every key)."""
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 64, 33000 if dtype == "bf16" else 17000, 64
    rng = np.random.default_rng(5)
    inp = {n: wl.round_to_dtype(rng.standard_normal(s, dtype=np.float32), dtype)
           for n, s in (("q", (B, Hq, Nq, D)), ("k", (B, Hkv, Nk, D)), ("v", (B, Hkv, Nk, D)),
                        ("do", (B, Hq, Nq, D)))}
    scale = float(np.float32(1 / np.sqrt(D)))
    r = gpu_run(gpu_lib, inp, B, Hq, Hkv, Nq, Nk, D, 2, scale, dtype, bwd=True)
    res = parity.bwd_all_groups(r["dq"], r["dk"], r["dv"], inp, "bottom_right", scale, dtype)
    print(f"long backward {dtype}: {res}")
