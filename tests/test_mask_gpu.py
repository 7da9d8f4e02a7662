"""GPU parity of the explicit masks and causal alignments (ra_attn_fwd_masked, ra_attn_bwd_masked
and the causal modes of ra_attn_fwd / ra_attn_bwd, through the C ABI) against the fp64 oracle.

Tolerances as the other attention tests: fp32 max-abs 1e-5 (relative to max|oracle| when that
exceeds 1), bf16 max|gpu - oracle| / max|oracle| <= 2e-2, per output tensor.  The oracle's mask
and alignment readings are pinned in test_oracle_pins.py (key padding equals dropping keys,
brute-force bottom-right, a hand-derived additive example, central differences).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, rel_to_max, to_dev, to_np

pytestmark = pytest.mark.gpu

CAUSAL = {"none": 0, "top_left": 1, "bottom_right": 2}
ORACLE_CAUSAL = {"none": False, "top_left": "top_left", "bottom_right": "bottom_right"}


def rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    out = {
        "q": rng.standard_normal((B, Hq, Nq, D), dtype=np.float32) * np.float32(sigma),
        "k": rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32) * np.float32(sigma),
        "v": rng.standard_normal((B, Hkv, Nk, D), dtype=np.float32),
        "do": rng.standard_normal((B, Hq, Nq, D), dtype=np.float32),
    }
    return {n: wl.round_to_dtype(a, dtype) for n, a in out.items()}


def make_mask(layout, B, Hq, Nq, Nk, dtype, seed):
    """(oracle mask broadcastable to [B, Hq, Nq, Nk], device tensor, RA_MASK kind, strides).

    The device tensor is the mask in its natural layout; the strides address it as element
    (b, h, i, j) with zeros on broadcast dimensions."""
    import torch
    import rational_softmax_tiled_amd as ra
    rng = np.random.default_rng(seed)
    if layout == "keypad":                        # [B, Nk], CrossAttention key padding
        keep = rng.random((B, Nk)) < 0.75
        keep[:, 0] = True
        t = torch.from_numpy(keep).cuda()
        return keep[:, None, None, :], t, ra.RA_MASK_BOOL, (Nk, 0, 0, 1)
    if layout == "keypad_shared":                 # one [Nk] key padding row for every sample
        keep = rng.random(Nk) < 0.75
        keep[0] = True
        keep[-3:] = True                          # kept keys in the last (possibly partial) dword
        t = torch.from_numpy(keep).cuda()
        return keep[None, None, None, :], t, ra.RA_MASK_BOOL, (0, 0, 0, 1)
    if layout == "shared2d":                      # one [Nq, Nk] mask for every batch and head
        keep = rng.random((Nq, Nk)) < 0.6
        t = torch.from_numpy(keep).cuda()
        return keep, t, ra.RA_MASK_BOOL, (0, 0, Nk, 1)
    if layout == "full_bool":                     # [B, Hq, Nq, Nk]
        keep = rng.random((B, Hq, Nq, Nk)) < 0.7
        t = torch.from_numpy(keep).cuda()
        return keep, t, ra.RA_MASK_BOOL, (Hq * Nq * Nk, Nq * Nk, Nk, 1)
    if layout == "transposed":                    # a [Nk, Nq] array read transposed
        keep_t = rng.random((Nk, Nq)) < 0.7
        t = torch.from_numpy(keep_t).cuda()
        return keep_t.T, t, ra.RA_MASK_BOOL, (0, 0, 1, Nq)
    if layout in ("documents", "documents_add", "documents_mixed"):  # packed documents, [B, N, N]
        assert Nq == Nk
        ids = wl.document_ids(B, Nq, seed, 40, 200)
        keep = ids[:, :, None] == ids[:, None, :]
        if layout == "documents":
            t = torch.from_numpy(keep).cuda()
            return keep[:, None], t, ra.RA_MASK_BOOL, (Nq * Nk, 0, Nk, 1)
        bias = np.where(keep, 0.0, -np.inf)[:, None].astype(np.float32)   # the same as 0 / -inf
        if layout == "documents_mixed":
            # -0.0 on some kept entries (still no change), a real bias on a few (their blocks take
            # the values, the others stay 0 / -inf)
            u = rng.random(bias.shape)
            bias[(u < 0.05) & (bias == 0)] = -0.0
            bias[(u > 0.998) & (bias == 0)] = rng.normal(0, 1, size=int(((u > 0.998) & (bias == 0)).sum()))
    elif layout == "head_bias":                   # additive [1, Hq, Nq, Nk] with -inf entries
        bias = rng.normal(0, 2, size=(1, Hq, Nq, Nk)).astype(np.float32)
        bias[rng.random(bias.shape) < 0.1] = -np.inf
    elif layout == "alibi":                       # additive -slope_h |i - j|
        slopes = 2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq)
        dist = np.abs(np.arange(Nq)[:, None] - np.arange(Nk)[None, :])
        bias = (-slopes[:, None, None] * dist)[None].astype(np.float32)
    elif layout == "key_bias":                    # additive per (batch, key), broadcast over rows
        bias = rng.normal(0, 3, size=(B, 1, 1, Nk)).astype(np.float32)
    else:
        raise ValueError(layout)
    bias = wl.round_to_dtype(bias, dtype)
    t = to_dev(bias, dtype)
    st = t.stride()
    strides = tuple(0 if bias.shape[i] == 1 else st[i] for i in range(4))
    return bias.astype(np.float64), t, ra.RA_MASK_ADD, strides


def run(ra, inp, causal, scale, dtype, mask=None, use_stats=True, bwd=True):
    """Forward (and backward) through the C ABI; mask = (tensor, kind, strides) or None."""
    import torch
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    cc = CAUSAL[causal]
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    if mask is None:
        st = ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, cc, scale, code)
    else:
        st = ra.ra_attn_fwd_masked(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, cc, scale, code, *mask)
    assert st == 0, ra.ra_status_string(st)
    out = {"o": o, "stats": stats}
    if bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, code)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        sp = stats if use_stats else None
        if mask is None:
            st = ra.ra_attn_bwd(q, k, v, o, do, sp, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                                cc, scale, code)
        else:
            st = ra.ra_attn_bwd_masked(q, k, v, o, do, sp, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq,
                                       Nk, D, cc, scale, code, *mask)
        assert st == 0, ra.ra_status_string(st)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    res = {n: to_np(t) for n, t in out.items() if n != "stats"}
    res["stats"] = stats.cpu().numpy().astype(np.float64)
    return res


def check(res, inp, causal, scale, dtype, mask_np=None, what="", bwd=True):
    oc = ORACLE_CAUSAL[causal]
    ro, rm, rl, _ = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], oc, scale, mask=mask_np)
    errs = {"o": assert_close(res["o"], ro, dtype, f"{what} o")}
    # stats: m in raw units (max of q.k + mask / scale), the oracle's in scaled units
    np.testing.assert_allclose(res["stats"][..., 0] * scale, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(res["stats"][..., 1], rl, rtol=(1e-5 if dtype == "f32" else 1e-2))
    if bwd:
        ref = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], oc, scale,
                                      mask=mask_np)
        for name, r in zip(("dq", "dk", "dv"), ref):
            assert_close(res[name], r, dtype, f"{what} {name}", grad=True)
            errs[name] = rel_to_max(res[name], r)
    return errs


# ----------------------------------------------------------------- causal alignment, no mask

ALIGN_CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, dtype)
    (2, 4, 2, 97, 250, 128, "bottom_right", "bf16"),    # Nq < Nk: every row sees Nk - Nq more keys
    (1, 6, 3, 250, 97, 128, "bottom_right", "bf16"),    # Nq > Nk: the first 153 rows see nothing
    (1, 4, 4, 64, 64, 64, "bottom_right", "bf16"),      # square: the same as top-left
    (2, 2, 1, 1, 300, 64, "bottom_right", "bf16"),      # one query row sees every key
    (1, 2, 2, 130, 65, 64, "bottom_right", "f32"),
    (1, 3, 1, 33, 200, 128, "bottom_right", "f32"),
    (1, 8, 2, 320, 640, 128, "bottom_right", "bf16"),   # several tiles, fast kernels
]


@pytest.mark.parametrize("shape", ALIGN_CASES, ids=[str(c) for c in ALIGN_CASES])
def test_bottom_right_alignment(gpu_lib, shape):
    B, Hq, Hkv, Nq, Nk, D, causal, dtype = shape
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed=Nq * 7 + Nk)
    scale = float(np.float32(1 / np.sqrt(D)))
    res = run(gpu_lib, inp, causal, scale, dtype)
    check(res, inp, causal, scale, dtype, what=str(shape))
    dead = max(0, Nq - Nk)
    if dead:
        assert (res["o"][:, :, :dead] == 0).all() and (res["dq"][:, :, :dead] == 0).all()
        assert (res["stats"][:, :, :dead, 0] == -np.inf).all()
        assert (res["stats"][:, :, :dead, 1] == 0).all()
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), n


def test_bottom_right_square_equals_top_left(gpu_lib):
    inp = rand_inputs(2, 4, 2, 200, 200, 128, "bf16", seed=3)
    scale = float(np.float32(1 / np.sqrt(128)))
    a = run(gpu_lib, inp, "bottom_right", scale, "bf16")
    b = run(gpu_lib, inp, "top_left", scale, "bf16")
    for n in ("o", "stats", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[n], b[n])


# ----------------------------------------------------------------- explicit masks

MASK_CASES = [
    # (layout, B, Hq, Hkv, Nq, Nk, D, causal, dtype)
    ("keypad", 2, 4, 2, 96, 200, 64, "none", "bf16"),
    ("keypad", 3, 2, 1, 130, 130, 128, "top_left", "bf16"),
    ("keypad", 2, 2, 2, 65, 190, 64, "bottom_right", "f32"),
    # bf16 key padding with 4-byte aligned rows (Nk % 4 == 0) runs the forward whose K ring also
    # carries the mask bytes: scattered padding (partial tiles), GQA, both alignments, D = 128
    ("keypad", 2, 4, 2, 96, 200, 128, "bottom_right", "bf16"),
    ("keypad", 3, 8, 2, 150, 260, 128, "top_left", "bf16"),
    # a key padding row shared by the batch (batch stride 0): with Nk % 4 != 0 its dword copies
    # would end past the resource, so it takes the general masked kernels; Nk % 4 == 0 the fast path
    ("keypad_shared", 2, 4, 2, 100, 130, 128, "none", "bf16"),
    ("keypad_shared", 2, 4, 2, 130, 130, 64, "top_left", "bf16"),
    ("keypad_shared", 3, 2, 1, 90, 132, 128, "bottom_right", "bf16"),
    ("shared2d", 1, 4, 4, 127, 127, 128, "top_left", "bf16"),
    ("shared2d", 2, 2, 1, 50, 90, 64, "none", "f32"),
    ("full_bool", 2, 6, 3, 70, 150, 128, "none", "bf16"),
    ("full_bool", 1, 4, 2, 100, 64, 64, "bottom_right", "bf16"),
    ("full_bool", 1, 2, 2, 33, 97, 128, "top_left", "f32"),
    ("transposed", 1, 3, 1, 80, 140, 64, "none", "bf16"),
    ("transposed", 1, 2, 2, 61, 61, 128, "top_left", "f32"),
    ("head_bias", 2, 4, 2, 90, 90, 128, "top_left", "bf16"),
    ("head_bias", 1, 4, 1, 64, 129, 64, "none", "f32"),
    # bf16 bias rows of 4-element multiples: the 16-byte loads of a key block, ragged last block
    ("head_bias", 1, 4, 2, 100, 132, 128, "bottom_right", "bf16"),
    ("alibi", 1, 8, 2, 160, 160, 128, "top_left", "bf16"),
    ("alibi", 1, 4, 4, 50, 120, 64, "bottom_right", "f32"),
    ("key_bias", 3, 2, 1, 75, 140, 128, "none", "bf16"),
    # packed documents: whole tiles kept (run as unmasked ones), partial ones at the documents'
    # edges and tiles the mask drops entirely (no products in either pass)
    ("documents", 2, 4, 2, 300, 300, 128, "top_left", "bf16"),
    ("documents", 1, 4, 4, 260, 260, 64, "none", "bf16"),
    ("documents", 1, 2, 2, 200, 200, 128, "top_left", "f32"),
    ("documents_add", 2, 2, 1, 300, 300, 128, "top_left", "bf16"),
    ("documents_add", 1, 2, 2, 170, 170, 64, "none", "f32"),
    ("documents_mixed", 1, 4, 2, 300, 300, 128, "top_left", "bf16"),
    ("documents_mixed", 2, 2, 2, 256, 256, 64, "none", "bf16"),
    ("key_bias", 2, 2, 2, 40, 40, 64, "top_left", "f32"),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[str(c) for c in MASK_CASES])
def test_masked_parity(gpu_lib, case):
    layout, B, Hq, Hkv, Nq, Nk, D, causal, dtype = case
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed=Nq * 31 + Nk + D)
    scale = float(np.float32(1 / np.sqrt(D)))
    mask_np, t, kind, strides = make_mask(layout, B, Hq, Nq, Nk, dtype, seed=Nq + 5)
    res = run(gpu_lib, inp, causal, scale, dtype, mask=(t, kind, strides))
    errs = check(res, inp, causal, scale, dtype, mask_np=mask_np, what=str(case))
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), n
    print(f"{case}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("causal", ["none", "top_left", "bottom_right"])
def test_key_padding_lengths(gpu_lib, causal):
    """Key padding from per-sample lengths (contiguous kept prefixes, one empty sample): whole
    padded tiles are dropped in both forward passes, the tile holding the boundary is masked
    entry by entry; a sample with no key gives o = 0, dk = dv = 0."""
    import torch
    import rational_softmax_tiled_amd as ra
    B, Hq, Hkv, Nq, Nk, D = 3, 4, 2, 192, 200, 128
    lens = np.array([200, 70, 0])
    keep = np.arange(Nk)[None, :] < lens[:, None]
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=41)
    scale = float(np.float32(1 / np.sqrt(D)))
    mask = (torch.from_numpy(keep).cuda(), ra.RA_MASK_BOOL, (Nk, 0, 0, 1))
    res = run(gpu_lib, inp, causal, scale, "bf16", mask=mask)
    check(res, inp, causal, scale, "bf16", mask_np=keep[:, None, None, :], what=f"lengths {causal}")
    assert (res["o"][2] == 0).all() and (res["dk"][2] == 0).all() and (res["dv"][2] == 0).all()
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), n


@pytest.mark.parametrize("layout,Nq,Nk", [("head_bias", 100, 170),       # Nk % 4 != 0: per element
                                          ("documents_mixed", 160, 160)])  # packed additive runs
def test_masked_backward_without_stats_is_identical(gpu_lib, layout, Nq, Nk):
    """The backward's own pass 1 (no saved statistics: the forward kernel without an output)
    gives the same gradients as the saved statistics."""
    B, Hq, Hkv, D = 2, 4, 2, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=11)
    mask_np, t, kind, strides = make_mask(layout, B, Hq, Nq, Nk, "bf16", seed=12)
    scale = float(np.float32(1 / np.sqrt(D)))
    a = run(gpu_lib, inp, "bottom_right", scale, "bf16", mask=(t, kind, strides))
    b = run(gpu_lib, inp, "bottom_right", scale, "bf16", mask=(t, kind, strides), use_stats=False)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(a[n], b[n])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fully_masked_rows_give_zeros(gpu_lib, dtype):
    """Rows with no allowed key (a key padding mask that drops every key of one sample, a
    boolean row of zeros, bottom-right rows above the diagonal) give o = 0, dq = 0 and
    contribute nothing to dk, dv; nothing is NaN."""
    import torch
    import rational_softmax_tiled_amd as ra
    B, Hq, Hkv, Nq, Nk, D = 3, 4, 2, 90, 70, 128
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed=21)
    scale = float(np.float32(1 / np.sqrt(D)))
    keep = np.random.default_rng(22).random((B, Hq, Nq, Nk)) < 0.8
    keep[1] = False                 # sample 1: nothing to attend to
    keep[2, 3, 40] = False          # one row of one head
    t = torch.from_numpy(keep).cuda()
    mask = (t, ra.RA_MASK_BOOL, (Hq * Nq * Nk, Nq * Nk, Nk, 1))
    res = run(gpu_lib, inp, "bottom_right", scale, dtype, mask=mask)
    check(res, inp, "bottom_right", scale, dtype, mask_np=keep, what="fully masked rows")
    dead = ~keep.any(axis=-1)
    dead[:, :, :Nq - Nk] = True     # bottom-right: rows 0..19 have no key
    assert (res["o"][dead] == 0).all() and (res["dq"][dead] == 0).all()
    assert (res["stats"][dead][:, 0] == -np.inf).all() and (res["stats"][dead][:, 1] == 0).all()
    assert (res["dk"][1] == 0).all() and (res["dv"][1] == 0).all()
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), n


def test_mask_reads_the_query_head_not_the_kv_head(gpu_lib):
    """GQA with a different mask per query head: head h must read mask[:, h], not mask[:, g]."""
    import torch
    import rational_softmax_tiled_amd as ra
    B, Hq, Hkv, Nq, Nk, D = 1, 8, 2, 64, 96, 64
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, "f32", seed=31)
    keep = np.zeros((B, Hq, Nq, Nk), bool)
    for h in range(Hq):
        keep[0, h, :, h::Hq] = True      # head h sees keys h, h + 8, ...
    t = torch.from_numpy(keep).cuda()
    scale = 0.125
    res = run(gpu_lib, inp, "none", scale, "f32", mask=(t, ra.RA_MASK_BOOL, (0, Nq * Nk, Nk, 1)))
    check(res, inp, "none", scale, "f32", mask_np=keep, what="per-head masks")


def test_autograd_wrapper_with_masks(gpu_lib):
    import torch
    B, Hq, Hkv, Nq, Nk, D = 2, 4, 2, 77, 150, 64
    inp = rand_inputs(B, Hq, Hkv, Nq, Nk, D, "f32", seed=41)
    scale = float(np.float32(1 / np.sqrt(D)))
    keep = np.random.default_rng(42).random((B, Nk)) < 0.7
    keep[:, -1] = True
    bias = wl.round_to_dtype(np.random.default_rng(43).normal(0, 2, size=(Nq, Nk)).astype(np.float32), "f32")
    cases = [
        (dict(key_padding_mask=torch.from_numpy(keep).cuda().float()), keep[:, None, None, :], "bottom_right"),
        (dict(attn_mask=torch.from_numpy(bias).cuda()), bias.astype(np.float64), True),
        (dict(attn_mask=torch.from_numpy(keep[:, None, None, :]).cuda()), keep[:, None, None, :], False),
    ]
    for kw, mask_np, causal in cases:
        q, k, v = (torch.from_numpy(inp[n]).cuda().requires_grad_() for n in ("q", "k", "v"))
        o = gpu_lib.ra_attention(q, k, v, is_causal=causal, scale=scale, **kw)
        o.backward(torch.from_numpy(inp["do"]).cuda())
        oc = {True: "top_left", False: False}.get(causal, causal)
        ro = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], oc, scale, mask=mask_np)[0]
        rq, rk, rv = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], oc, scale,
                                             mask=mask_np)
        what = f"{list(kw)} causal={causal}"
        assert_close(o.detach().cpu().numpy().astype(np.float64), ro, "f32", what)
        for g, r in ((q.grad, rq), (k.grad, rk), (v.grad, rv)):
            assert_close(g.cpu().numpy().astype(np.float64), r, "f32", what, grad=True)
    with pytest.raises(ValueError):
        gpu_lib.ra_attention(q, k, v, attn_mask=torch.zeros(Nq, Nk, device="cuda", requires_grad=True))
    with pytest.raises(TypeError):
        gpu_lib.ra_attention(q, k, v, attn_mask=torch.zeros(Nq, Nk, device="cuda", dtype=torch.float64))


def test_padded_batch_full_size_sampled_heads(gpu_lib):
    """A padded batch at full size in the launch shape the bench times: B=4 Hq=16 N=4096 D=128,
    causal, key padding with per-sample lengths (4096, 3000, 2048, 1111); whole heads are
    checked against the oracle on a sample, every row for finiteness and the zero rule."""
    import torch
    import rational_softmax_tiled_amd as ra
    w = wl.padded_batch_workload()
    inp = wl.make_attention_inputs(w)
    lengths = wl.padded_batch_lengths(w)
    keep = wl.padded_batch_keep(w)
    t = torch.from_numpy(keep).cuda()
    mask = (t, ra.RA_MASK_BOOL, (w.Nk, 0, 0, 1))
    res = run(gpu_lib, inp, "top_left", w.scale, w.dtype, mask=mask)
    heads = [(0, 0), (1, 7), (3, w.Hq - 1)]
    ro, rm, rl, _ = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], True, w.scale, heads=heads,
                                            mask=keep[:, None, None, :])
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    assert_close(res["o"][bi, hi], ro[bi, hi], w.dtype, "padded batch o")
    groups = [(3, w.Hkv - 1)]
    rq, rk, rv = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], True, w.scale,
                                         groups=groups, mask=keep[:, None, None, :])
    assert_close(res["dq"][3, -1], rq[3, -1], w.dtype, "padded batch dq", grad=True)
    assert_close(res["dk"][3, -1], rk[3, -1], w.dtype, "padded batch dk", grad=True)
    assert_close(res["dv"][3, -1], rv[3, -1], w.dtype, "padded batch dv", grad=True)
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), n
    # keys past a sample's length take no part: their dk, dv are exactly zero
    for b, n in enumerate(lengths):
        assert (res["dk"][b, :, n:] == 0).all() and (res["dv"][b, :, n:] == 0).all()


# ----------------------------------------------------------------- masks that change nothing

@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_identity_masks_equal_the_unmasked_forward(gpu_lib, dtype, D):
    """An all-true boolean mask and an all-zero additive one leave every score as it is: the masked
    forward (whose tiles pass 1 finds unmasked then run as unmasked ones) gives the unmasked
    forward's bits."""
    import torch
    ra = gpu_lib
    B, Hq, Hkv, N = 2, 4, 2, 333
    inp = rand_inputs(B, Hq, Hkv, N, N, D, dtype, seed=41)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = run(ra, inp, "top_left", scale, dtype, bwd=False)
    ones = torch.ones((N, N), dtype=torch.bool, device="cuda")
    zeros = torch.zeros((N, N), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    for mask in ((ones, ra.RA_MASK_BOOL, (0, 0, N, 1)), (zeros, ra.RA_MASK_ADD, (0, 0, N, 1))):
        got = run(ra, inp, "top_left", scale, dtype, mask=mask, bwd=False)
        np.testing.assert_array_equal(got["o"], ref["o"])
        np.testing.assert_array_equal(got["stats"], ref["stats"])
