"""GPU parity of ra_softmax_rows_bwd (through the C ABI) against the fp64 oracle.

Tolerance (per output tensor): bf16 max|gpu - oracle| / max|oracle| <= 2e-2; fp32 max-abs
1e-5, relative to max|oracle| when that exceeds 1.  The oracle is pinned by central
differences in test_oracle_pins.py.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, rel_to_max, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_bwd(ra, x, dp, dtype, alias=None):
    import torch
    xt, gt = to_dev(x, dtype), to_dev(dp, dtype)
    dx = {"x": xt, "dp": gt}.get(alias) if alias else torch.empty_like(xt)
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    st = ra.ra_softmax_rows_bwd(xt, gt, dx, x.shape[0], x.shape[1], code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    return to_np(dx)


def upstream(shape, dtype, seed):
    g = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return wl.round_to_dtype(g, dtype)


def check(dx, x, dp, dtype, what):
    ref = oracle.ra_softmax_rows_bwd(x.astype(np.float64), dp.astype(np.float64))
    assert_close(dx, ref, dtype, what, grad=True)
    return rel_to_max(dx, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example(gpu_lib, dtype):
    x = np.array([[2.0, 1.0, 0.0], [5.0, 1.0, -10.0]], np.float32)
    dp = np.array([[1.0, -2.0, 0.5], [0.25, 1.0, -1.0]], np.float32)
    dx = run_bwd(gpu_lib, x, dp, dtype)
    check(dx, x, dp, dtype, "worked example")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [1, 3, 8, 255, 256, 1000, 1024, 2048, 4096, 8192, 8193, 20000])
def test_shapes(gpu_lib, dtype, cols):
    rows = 37
    x = wl.make_rows(rows, cols, sigma=4.0, seed=cols, dtype=dtype)
    dp = upstream(x.shape, dtype, seed=cols + 1)
    dx = run_bwd(gpu_lib, x, dp, dtype)
    err = check(dx, x, dp, dtype, f"cols={cols}")
    # shift invariance: dL/dx sums to zero over every row
    scale = np.abs(dx).sum(axis=1).max() + 1e-30
    assert np.abs(dx.sum(axis=1)).max() <= (1e-5 if dtype == "f32" else 2e-2) * scale
    print(f"cols={cols}: rel-to-max error {err:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masking_one_hot_and_empty_rows(gpu_lib, dtype):
    rng = np.random.default_rng(3)
    x = rng.normal(0, 6, size=(6, 300)).astype(np.float32)
    x[0, ::3] = -np.inf
    x[1, :] = -np.inf                      # fully masked -> zeros, not NaN
    x[2, 1:] = -np.inf                     # one live entry -> p = 1 -> zero gradient
    x[3, 100] = np.float32(64.0)           # one-hot: everything else beyond the support
    x[3, :100] = np.clip(x[3, :100], -30, 40)
    x[3, 101:] = np.clip(x[3, 101:], -30, 40)
    x[4, 7] = x[4].max() + 15.0            # one entry just inside the support of the max
    x[4, 9] = x[4, 7] - 15.5
    x = wl.round_to_dtype(x, dtype)
    dp = upstream(x.shape, dtype, seed=4)
    dx = run_bwd(gpu_lib, x, dp, dtype)
    assert np.isfinite(dx).all()
    assert (dx[0, ::3] == 0).all()
    assert (dx[1] == 0).all()
    assert (dx[2] == 0).all()
    assert (dx[3] == 0).all()
    check(dx, x, dp, dtype, "masking")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ties_take_the_lowest_index(gpu_lib, dtype):
    x = np.array([[3.0, 1.0, 3.0, 0.0, 3.0], [0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    dp = np.array([[1.0, 0.0, -1.0, 2.0, 0.5], [1.0, 2.0, 3.0, 4.0, 5.0]], np.float32)
    dx = run_bwd(gpu_lib, x, dp, dtype)
    check(dx, x, dp, dtype, "ties")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [4096, 5000])        # register path, streaming path
@pytest.mark.parametrize("alias", ["x", "dp"])
def test_in_place(gpu_lib, dtype, cols, alias):
    x = wl.make_rows(9, cols, dtype=dtype)
    dp = upstream(x.shape, dtype, seed=5)
    np.testing.assert_array_equal(run_bwd(gpu_lib, x, dp, dtype, alias=alias), run_bwd(gpu_lib, x, dp, dtype))


def test_autograd_wrapper(gpu_lib):
    import torch
    x = wl.make_rows(16, 777, sigma=3.0, seed=8, dtype="f32")
    dp = upstream(x.shape, "f32", seed=9)
    xt = torch.from_numpy(x).cuda().requires_grad_()
    p = gpu_lib.ra_softmax(xt, dim=-1)
    p.backward(torch.from_numpy(dp).cuda())
    ref = oracle.ra_softmax_rows_bwd(x.astype(np.float64), dp.astype(np.float64))
    assert_close(xt.grad.cpu().numpy().astype(np.float64), ref, "f32", "autograd", grad=True)
    # along another dimension: the same rows, transposed
    xt2 = torch.from_numpy(np.ascontiguousarray(x.T)).cuda().requires_grad_()
    gpu_lib.ra_softmax(xt2, dim=0).backward(torch.from_numpy(np.ascontiguousarray(dp.T)).cuda())
    assert_close(xt2.grad.cpu().numpy().T.astype(np.float64), ref, "f32", "autograd dim=0", grad=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bench_shape_sampled_rows(gpu_lib, dtype):
    """The measured shape [16384, 8192]; the oracle checks a sample of rows."""
    x = wl.make_rows(16384, 8192, sigma=4.0, seed=11, dtype=dtype)
    dp = upstream(x.shape, dtype, seed=12)
    dx = run_bwd(gpu_lib, x, dp, dtype)
    rows = np.random.default_rng(0).choice(16384, 64, replace=False)
    check(dx[rows], x[rows], dp[rows], dtype, "bench shape")
