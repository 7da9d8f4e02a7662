"""GPU parity of ra_attn_decode (split-KV decode, through the C ABI) against the fp64 oracle's
ra_attention_decode (pinned in test_oracle_pins.py by the prefill-continuation identity and a
brute force).  bf16: max|gpu - oracle| / max|oracle| <= 2e-2 on O, l within 1e-2 relative;
fp32: max|gpu - oracle| <= 1e-5 absolute on O, l within 1e-5 relative; both: stats m within
the score rounding.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

CAUSAL = {"none": 0, "top_left": 1, "bottom_right": 2}
ORACLE_CAUSAL = {"none": False, "top_left": "top_left", "bottom_right": "bottom_right"}


def rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed, sigma=1.0, dtype="bf16"):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, D), dtype=np.float32) * np.float32(sigma)
    k = rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32) * np.float32(sigma)
    v = rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32)
    return {n: wl.round_to_dtype(a, dtype) for n, a in (("q", q), ("k", k), ("v", v))}


def run_decode(ra, inp, lens, causal, scale, dtype="bf16"):
    import torch
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    sl = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    nbytes = ra.ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    print(f"decode {dtype} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} D={D} {causal}", flush=True)
    st = ra.ra_attn_decode(q, k, v, o, stats, sl, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                           CAUSAL[causal], scale, code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    return to_np(o), stats.cpu().numpy().astype(np.float64)


def check(o, stats, inp, lens, causal, scale, what, dtype="bf16"):
    ro, rm, rl, _ = oracle.ra_attention_decode(inp["q"], inp["k"], inp["v"], scale, seqlens=lens,
                                               causal=ORACLE_CAUSAL[causal])
    err = assert_close(o, ro, dtype, what)
    np.testing.assert_allclose(stats[..., 0] * scale, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(stats[..., 1], rl, rtol=1e-2 if dtype == "bf16" else 1e-5)
    return err


CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, lengths): "full" = no seqlens, "rand" = seeded in [0, Nk]
    (2, 32, 8, 1, 1, 128, "none", "full"),
    (3, 32, 8, 1, 31, 128, "bottom_right", "rand"),
    (2, 8, 8, 1, 33, 64, "none", "rand"),
    (4, 32, 8, 1, 1000, 128, "bottom_right", "rand"),
    (1, 8, 1, 4, 517, 128, "bottom_right", "rand"),     # R = 32 rows per K/V head
    (2, 12, 4, 3, 300, 64, "top_left", "rand"),         # R = 9
    (2, 2, 2, 16, 257, 128, "bottom_right", "full"),    # R = 16
    (1, 28, 4, 1, 2048, 128, "none", "full"),           # R = 7
    (2, 16, 16, 2, 700, 64, "bottom_right", "rand"),    # R = 2, no grouping
    (1, 8, 2, 1, 5000, 128, "none", "rand"),            # 79 chunks of 64 keys per group
    (1, 4, 1, 1, 40000, 64, "bottom_right", "full"),    # 625 chunks
    # the keys per wave follow the actual lengths: more than 64 batches (the lengths are read in
    # windows of 64), and lengths short enough that the chunk shrinks below its bound
    (130, 4, 2, 1, 96, 64, "bottom_right", "rand"),
    (8, 8, 2, 1, 16384, 128, "bottom_right", "rand"),   # chunk between 64 and 256 keys
    (96, 2, 1, 1, 4096, 64, "none", "rand"),            # both: 96 batches, chunk 96..384
]


# fp32 caches: every head dimension, group size and length regime of the bf16 cases.  Up to 16
# query rows per K/V head take 16-column products, more take 32-column ones: R = 18 and 20 below
# besides R = 32 from the bf16 list.
CASES_F32 = [CASES[i] for i in (0, 1, 2, 4, 5, 6, 9, 10, 11, 13)] + [
    (2, 12, 4, 6, 300, 64, "top_left", "rand"),         # R = 18
    (1, 4, 1, 5, 700, 128, "bottom_right", "rand"),     # R = 20
]


def _decode_case(gpu_lib, case, dtype):
    B, Hq, Hkv, Nq, Nk, D, causal, lmode = case
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=Nk + 13 * Nq, dtype=dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    if lmode == "full":
        lens = None
    else:
        lens = np.random.default_rng(Nk).integers(0, Nk + 1, size=B).astype(np.int32)
        lens[0] = Nk
        if B > 2:
            lens[-1] = 0
    o, stats = run_decode(gpu_lib, inp, lens, causal, scale, dtype)
    err = check(o, stats, inp, lens, causal, scale, str(case), dtype)
    assert np.isfinite(o).all()
    if lens is not None:
        for b in np.nonzero(lens == 0)[0]:
            assert (o[b] == 0).all() and (stats[b, ..., 0] == -np.inf).all()
    print(f"{dtype} {case}: max err {err:.2e}")


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_parity(gpu_lib, case):
    _decode_case(gpu_lib, case, "bf16")


@pytest.mark.parametrize("case", CASES_F32, ids=[str(c) for c in CASES_F32])
def test_decode_parity_f32(gpu_lib, case):
    _decode_case(gpu_lib, case, "f32")


def test_decode_f32_last_cache_ragged(gpu_lib):
    """fp32: the last (batch, K/V head) group's cache ends inside a 32-key block past its first
    block, with the memory behind that cache holding NaN: keys past a cache's end must not reach
    the output (the value rows there are read as zeros or meet phi = 0 with finite data)."""
    import torch
    B, Hq, Hkv, Nq, Nk, D = 2, 8, 2, 1, 100, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=21, dtype="f32")
    scale = float(np.float32(1 / np.sqrt(D)))
    q = to_dev(inp["q"], "f32")
    # K and V as views at the start of larger buffers whose tails are NaN
    kb = torch.full((B * Hkv * Nk * D + 64 * D,), float("nan"), device="cuda")
    vb = torch.full_like(kb, float("nan"))
    kb[:B * Hkv * Nk * D] = torch.from_numpy(inp["k"]).reshape(-1).cuda()
    vb[:B * Hkv * Nk * D] = torch.from_numpy(inp["v"]).reshape(-1).cuda()
    k = kb[:B * Hkv * Nk * D].view(B, Hkv, Nk, D)
    v = vb[:B * Hkv * Nk * D].view(B, Hkv, Nk, D)
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    nbytes = gpu_lib.ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, gpu_lib.RA_F32)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    st = gpu_lib.ra_attn_decode(q, k, v, o, stats, None, ws, nbytes, B, Hq, Hkv, Nq, Nk, D, 2,
                                scale, gpu_lib.RA_F32)
    assert st == 0, gpu_lib.ra_status_string(st)
    torch.cuda.synchronize()
    check(to_np(o), stats.cpu().numpy().astype(np.float64), inp, None, "bottom_right", scale,
          "NaN past the cache", "f32")


def test_decode_short_caches_and_causal_rows(gpu_lib):
    """Caches shorter than the query block: with bottom-right alignment the first Nq - len rows
    of such a sample have no key and give 0; top-left rows see keys j <= i."""
    B, Hq, Hkv, Nq, Nk, D = 4, 8, 2, 8, 40, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=3)
    lens = np.array([3, 8, 40, 1], np.int32)
    scale = float(np.float32(1 / np.sqrt(D)))
    for causal in ("bottom_right", "top_left"):
        o, stats = run_decode(gpu_lib, inp, lens, causal, scale)
        check(o, stats, inp, lens, causal, scale, causal)
    o, _ = run_decode(gpu_lib, inp, lens, "bottom_right", scale)
    assert (o[0, :, :5] == 0).all() and (o[3, :, :7] == 0).all()


@pytest.mark.parametrize("dtype,Hq,Nq", [("bf16", 32, 1), ("f32", 32, 1), ("f32", 32, 6)])
def test_decode_matches_tiled_forward(gpu_lib, dtype, Hq, Nq):
    """Without lengths the decode equals the tiled forward with bottom-right alignment (two
    independent kernels, both checked against the oracle).  The row maxima agree bit for bit
    where the scores are the same products summed in the same order (bf16; fp32 with more than
    16 rows per K/V head, 32-column products as in the forward); fp32 with 16 rows or fewer sums
    each score in another order (16-column products), within the fp32 score bound."""
    import torch
    B, Hkv, Nk, D = 2, 8, 3000, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=5, dtype=dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    od, sd = run_decode(gpu_lib, inp, None, "bottom_right", scale, dtype)
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    of = torch.empty_like(q)
    sf = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    code = gpu_lib.RA_BF16 if dtype == "bf16" else gpu_lib.RA_F32
    assert gpu_lib.ra_attn_fwd(q, k, v, of, sf, B, Hq, Hkv, Nq, Nk, D, 2, scale, code) == 0
    torch.cuda.synchronize()
    assert_close(od, to_np(of), dtype, "decode vs tiled forward")
    mf = sf.cpu().numpy()[..., 0]
    if dtype == "bf16" or (Hq // Hkv) * Nq > 16:
        np.testing.assert_array_equal(sd[..., 0], mf)   # same fp32 scores, same max
    else:
        # |fp32 dot - exact| <= gamma_D sum |q k|, and sum |q k| <= |q| |k| <= D * max|q| max|k|
        bound = 2 * D * 2.0 ** -24 * D * np.abs(inp["q"]).max() * np.abs(inp["k"]).max()
        assert np.abs(sd[..., 0] - mf).max() <= bound


def test_decode_deterministic(gpu_lib):
    B, Hq, Hkv, Nq, Nk, D = 3, 32, 8, 1, 4099, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=9)
    lens = np.array([4099, 2000, 17], np.int32)
    a = run_decode(gpu_lib, inp, lens, "bottom_right", 0.088)
    b = run_decode(gpu_lib, inp, lens, "bottom_right", 0.088)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_decode_binding(gpu_lib):
    import torch
    B, Hq, Hkv, Nq, Nk, D = 2, 16, 4, 2, 600, 64
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, seed=11)
    lens = np.array([600, 123], np.int32)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    o, stats = gpu_lib.attn_decode(q, k, v, seqlens=torch.from_numpy(lens).cuda(),
                                   causal="bottom_right", with_stats=True)
    torch.cuda.synchronize()
    check(to_np(o), stats.cpu().numpy().astype(np.float64), inp, lens, "bottom_right",
          1 / np.sqrt(D), "binding")
    o32, s32 = gpu_lib.attn_decode(q.float(), k.float(), v.float(), seqlens=torch.from_numpy(lens).cuda(),
                                   causal="bottom_right", with_stats=True)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    check(to_np(o32), s32.cpu().numpy().astype(np.float64), inp, lens, "bottom_right",
          1 / np.sqrt(D), "binding fp32", "f32")
    with pytest.raises(gpu_lib.RaError):
        qq = torch.zeros((B, Hq, 9, D), dtype=torch.bfloat16, device="cuda")
        gpu_lib.attn_decode(qq, k, v)                                   # 4 * 9 rows per K/V head


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_workload_full_size(gpu_lib, dtype):
    """The measured decode step, B=16 Hq=32 Hkv=8 Nq=1, caches of 16384 with per-sample lengths
    (bf16, and the same step with fp32 caches): every row against the oracle."""
    w = wl.decode_workload(dtype)
    inp = wl.make_attention_inputs(w)
    lens = wl.decode_seqlens(w)
    o, stats = run_decode(gpu_lib, inp, lens, "bottom_right", w.scale, dtype)
    err = check(o, stats, inp, lens, "bottom_right", w.scale, w.name, dtype)
    print(f"{w.name}: max err {err:.2e}, lengths {lens.tolist()}")
