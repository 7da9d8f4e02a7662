"""Host-side checks of the seeded input generators (no GPU)."""
import numpy as np
import pytest

import workloads as wl


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # exact ties between two bf16 neighbours, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-30, -1e30], dtype=np.float32),
    ])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_rope_is_a_rotation_of_split_halves():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 17, 8)).astype(np.float32)
    y = wl.neox_rope(x, 10000.0)
    n0 = x[..., :4] ** 2 + x[..., 4:] ** 2
    n1 = y[..., :4] ** 2 + y[..., 4:] ** 2
    np.testing.assert_allclose(n0, n1, rtol=1e-5)
    np.testing.assert_array_equal(y[..., 0, :], x[..., 0, :])   # position 0 is not rotated


def test_inputs_are_seeded_and_representable():
    w = wl.WORKLOADS["bf16_causal_B2_H12_N128_D64"]
    a = wl.make_attention_inputs(w)
    b = wl.make_attention_inputs(w)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(a[key], b[key])
        assert a[key].dtype == np.float32
        np.testing.assert_array_equal(wl.round_to_dtype(a[key], "bf16"), a[key])
    assert a["q"].shape == (2, 12, 128, 64)
    assert w.scale == np.float32(0.125)


def test_workload_flop_counts():
    w = wl.WORKLOADS["bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"]
    assert w.counted_flops_fwd() == pytest.approx(549.76e9, rel=1e-4)
    w5 = wl.WORKLOADS["bf16_causal_B4_H16_N8192_D128_fwd_bwd"]
    assert w5.counted_flops_fwd_bwd() == pytest.approx(3848.3e9, rel=1e-4)


def test_document_ids_are_contiguous_runs_of_bounded_length():
    ids = wl.document_ids(3, 1000, seed=5, lo=40, hi=200)
    for row in ids:
        assert row[0] == 0 and (np.diff(row) >= 0).all() and (np.diff(row) <= 1).all()
        lengths = np.bincount(row)
        assert (lengths[:-1] >= 40).all() and (lengths <= 200).all()
    keep = wl.documents_keep()
    assert keep.shape == (4, 4096, 4096) and keep.dtype == bool
    assert (keep == keep.transpose(0, 2, 1)).all() and keep[:, np.arange(4096), np.arange(4096)].all()
