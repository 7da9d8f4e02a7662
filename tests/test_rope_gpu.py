"""GPU parity of ra_rope_neox (through the C ABI) against the fp64 oracle, and the grouped-query
workload with the rotation done on the device instead of the host.

Tolerance: fp32 max-abs 1e-5 (relative to max|oracle| when that exceeds 1); bf16
max|gpu - oracle| / max|oracle| <= 2e-2 (the output is one bf16 rounding of the rotated value).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, rel_to_max, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_rope(ra, x, dtype, theta=10000.0, positions=None, inverse=False, inplace=False):
    import torch
    xt = to_dev(x, dtype)
    y = xt if inplace else torch.empty_like(xt)
    pos = None if positions is None else torch.as_tensor(positions, dtype=torch.int32, device="cuda")
    N, D = x.shape[-2], x.shape[-1]
    mats = int(np.prod(x.shape[:-2]))
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    st = ra.ra_rope_neox(xt, y, pos, mats, N, D, theta, inverse, code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    return to_np(y)


SHAPES = [((2, 3, 17, 64), "f32"), ((1, 4, 300, 128), "f32"), ((2, 2, 129, 128), "bf16"),
          ((3, 5, 2), "f32"), ((1, 1, 1, 128), "bf16"), ((4, 8, 1000, 64), "bf16")]


@pytest.mark.parametrize("shape,dtype", SHAPES, ids=[f"{s}-{d}" for s, d in SHAPES])
@pytest.mark.parametrize("inverse", [False, True])
def test_parity(gpu_lib, shape, dtype, inverse):
    x = wl.round_to_dtype(np.random.default_rng(len(shape) + shape[-2]).standard_normal(shape, dtype=np.float32), dtype)
    y = run_rope(gpu_lib, x, dtype, inverse=inverse)
    assert_close(y, oracle.rope_neox(x, 10000.0, inverse=inverse), dtype, f"{shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_positions_and_theta(gpu_lib, dtype):
    rng = np.random.default_rng(41)
    x = wl.round_to_dtype(rng.standard_normal((2, 3, 50, 64), dtype=np.float32), dtype)
    pos = rng.integers(0, 200000, size=50)           # large positions: the phase needs fp64
    y = run_rope(gpu_lib, x, dtype, theta=500000.0, positions=pos)
    assert_close(y, oracle.rope_neox(x, 500000.0, positions=pos), dtype, "positions")


def test_in_place_and_round_trip(gpu_lib):
    x = np.random.default_rng(42).standard_normal((2, 4, 333, 128), dtype=np.float32)
    np.testing.assert_array_equal(run_rope(gpu_lib, x, "f32", inplace=True), run_rope(gpu_lib, x, "f32"))
    import torch
    xt = to_dev(x, "f32")
    y = gpu_lib.ra_rope(xt)
    back = gpu_lib.ra_rope(y, inverse=True)
    np.testing.assert_allclose(to_np(back), x, atol=2e-6)


def test_autograd_is_the_inverse_rotation(gpu_lib):
    import torch
    rng = np.random.default_rng(43)
    x = rng.standard_normal((2, 3, 40, 64), dtype=np.float32)
    dy = rng.standard_normal(x.shape, dtype=np.float32)
    xt = torch.from_numpy(x).cuda().requires_grad_()
    gpu_lib.ra_rope(xt).backward(torch.from_numpy(dy).cuda())
    assert_close(xt.grad.cpu().numpy().astype(np.float64), oracle.rope_neox(dy, 10000.0, inverse=True),
                 "f32", "grad")


def test_grouped_query_workload_with_device_rope(gpu_lib):
    """B=4, Hq=32, Hkv=8, N=4096, D=128, causal: Q and K drawn as for the host-RoPE workload but
    left unrotated; the device rotates them (bf16 in, bf16 out) and the attention runs on the
    result.  The oracle rotates the same unrotated values in fp64; one (batch, K/V-head) group
    of query rows is checked."""
    import torch
    ra = gpu_lib
    w = wl.WORKLOADS["bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"]
    rng = np.random.default_rng(w.seed)
    q = wl.round_to_dtype(rng.standard_normal((w.B, w.Hq, w.Nq, w.D), dtype=np.float32), "bf16")
    k = wl.round_to_dtype(rng.standard_normal((w.B, w.Hkv, w.Nk, w.D), dtype=np.float32), "bf16")
    v = wl.round_to_dtype(rng.standard_normal((w.B, w.Hkv, w.Nk, w.D), dtype=np.float32), "bf16")
    qt, kt, vt = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    for t, H in ((qt, w.Hq), (kt, w.Hkv)):
        assert ra.ra_rope_neox(t, t, None, w.B * H, w.Nq, w.D, 10000.0, False, ra.RA_BF16) == 0
    o = torch.empty_like(qt)
    assert ra.ra_attn_fwd(qt, kt, vt, o, None, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, True, w.scale,
                          ra.RA_BF16) == 0
    torch.cuda.synchronize()
    b, g = 2, 5
    rep = w.Hq // w.Hkv
    qs = oracle.rope_neox(q[b:b + 1, g * rep:(g + 1) * rep], 10000.0)
    ks = oracle.rope_neox(k[b:b + 1, g:g + 1], 10000.0)
    ref = oracle.ra_attention_fwd(qs, ks, v[b:b + 1, g:g + 1], True, w.scale)[0]
    got = to_np(o)[b:b + 1, g * rep:(g + 1) * rep]
    assert_close(got, ref, "bf16", "device rope + attention")
    print(f"rel-to-max error {rel_to_max(got, ref):.2e}")
