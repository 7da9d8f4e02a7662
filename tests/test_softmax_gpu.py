"""GPU parity of ra_softmax_rows (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import ULP16, U32, assert_close, to_dev, to_np, zero_pattern_mismatches

pytestmark = pytest.mark.gpu


def run_rows(ra, x, dtype, inplace=False):
    import torch
    xt = to_dev(x, dtype)
    p = xt if inplace else torch.empty_like(xt)
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    st = ra.ra_softmax_rows(xt, p, x.shape[0], x.shape[1], code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    return to_np(p)


def check(p, x, dtype, what):
    ref, _, m, _ = oracle.ra_softmax_rows(x.astype(np.float64), return_stats=True)
    assert_close(p, ref, dtype, what)
    with np.errstate(invalid="ignore"):
        delta = np.where(np.isneginf(x), np.inf, m[:, None] - x)
    band = ULP16 + 8 * U32 * 16
    bad, mism = zero_pattern_mismatches(p, ref, delta, band)
    assert bad == 0, f"{what}: {bad} zero-pattern mismatches outside the band"
    return mism


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example(gpu_lib, dtype):
    x = np.array([[2.0, 1.0, 0.0], [5.0, 1.0, -10.0]], np.float32)
    p = run_rows(gpu_lib, x, dtype)
    check(p, x, dtype, "worked example")
    assert p[1, 2] > 0          # Delta = 15 is inside the support


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [1, 3, 8, 255, 256, 1000, 1024, 2048, 4096, 8192, 8193, 20000])
def test_shapes(gpu_lib, dtype, cols):
    rows = 37
    x = wl.make_rows(rows, cols, sigma=4.0, seed=cols, dtype=dtype)
    p = run_rows(gpu_lib, x, dtype)
    mism = check(p, x, dtype, f"cols={cols}")
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=(1e-5 if dtype == "f32" else 2e-2))
    print(f"cols={cols}: zero-pattern mismatches inside band: {mism}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masking_and_empty_rows(gpu_lib, dtype):
    rng = np.random.default_rng(3)
    x = rng.normal(0, 6, size=(6, 300)).astype(np.float32)
    x[0, ::3] = -np.inf
    x[1, :] = -np.inf                      # fully masked -> zeros, not NaN
    x[2, 1:] = -np.inf                     # one live entry -> p = 1
    x[3, 100] = np.float32(64.0)           # everything else beyond the support
    x[3, :100] = np.clip(x[3, :100], -30, 40)
    x[3, 101:] = np.clip(x[3, 101:], -30, 40)
    x = wl.round_to_dtype(x, dtype)
    p = run_rows(gpu_lib, x, dtype)
    assert np.isfinite(p).all()
    assert (p[0, ::3] == 0).all()
    assert (p[1] == 0).all()
    assert p[2, 0] == 1.0 and (p[2, 1:] == 0).all()
    assert p[3, 100] == 1.0 and (np.delete(p[3], 100) == 0).all()
    check(p, x, dtype, "masking")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place(gpu_lib, dtype):
    x = wl.make_rows(9, 4096, dtype=dtype)
    np.testing.assert_array_equal(run_rows(gpu_lib, x, dtype, inplace=True), run_rows(gpu_lib, x, dtype))
    x = wl.make_rows(9, 5000, dtype=dtype)     # streaming path
    np.testing.assert_array_equal(run_rows(gpu_lib, x, dtype, inplace=True), run_rows(gpu_lib, x, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bench_shape_sampled_rows(gpu_lib, dtype):
    """The measured shape [16384, 8192]; the oracle checks a sample of rows."""
    x = wl.make_rows(16384, 8192, sigma=4.0, seed=11, dtype=dtype)
    p = run_rows(gpu_lib, x, dtype)
    rows = np.random.default_rng(0).choice(16384, 64, replace=False)
    check(p[rows], x[rows], dtype, "bench shape")
