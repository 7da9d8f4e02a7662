"""The forward at the largest sizes the boundary admits: (N + 256) * D * elem_size < 2^31 bytes
per head's matrix (the kernels' 32-bit byte offsets, a tile tail included).  One case puts the
key count at its limit (bf16, D = 128: K and V are 2 GiB each, 131,072 key tiles, far past the
512 with a recorded maximum), the other the query count (fp32, D = 64).  Compared with the fp64
oracle (every row of the first, sampled rows of the second)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def n_max(D, es):
    return (1 << 31) // (D * es) - 256 - 1


def _run(ra, q, k, v, dims, causal, scale, dtype):
    import torch
    B, Hq, Hkv, Nq, Nk, D = dims
    qt, kt, vt = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o = torch.empty_like(qt)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    st = ra.ra_attn_fwd(qt, kt, vt, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, code)
    assert st == 0, ra.ra_status_string(st)
    torch.cuda.synchronize()
    out = to_np(o), stats.cpu().numpy().astype(np.float64)
    del qt, kt, vt, o, stats
    torch.cuda.empty_cache()
    return out


def test_largest_key_count_bf16(gpu_lib):
    D, Nq = 128, 16
    Nk = n_max(D, 2)
    rng = np.random.default_rng(77)
    print(f"drawing K, V of {Nk} keys", flush=True)
    q = wl.round_to_dtype(rng.standard_normal((1, 1, Nq, D), dtype=np.float32), "bf16")
    k = wl.round_to_dtype(rng.standard_normal((1, 1, Nk, D), dtype=np.float32), "bf16")
    v = wl.round_to_dtype(rng.standard_normal((1, 1, Nk, D), dtype=np.float32), "bf16")
    scale = float(np.float32(1 / np.sqrt(D)))
    print("forward", flush=True)
    o, stats = _run(gpu_lib, q, k, v, (1, 1, 1, Nq, Nk, D), 2, scale, "bf16")
    print("oracle", flush=True)
    ro, rm, rl, _ = oracle.ra_attention_fwd(q, k, v, "bottom_right", scale)
    err = assert_close(o, ro, "bf16", "O at the largest key count")
    np.testing.assert_allclose(stats[..., 0] * scale, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(stats[..., 1], rl, rtol=1e-2)
    print(f"Nk = {Nk}: rel-to-max err {err:.2e}")


def test_largest_query_count_f32(gpu_lib):
    D, Nk = 64, 40
    Nq = n_max(D, 4)
    rng = np.random.default_rng(78)
    print(f"drawing Q of {Nq} rows", flush=True)
    q = rng.standard_normal((1, 1, Nq, D), dtype=np.float32)
    k = rng.standard_normal((1, 1, Nk, D), dtype=np.float32)
    v = rng.standard_normal((1, 1, Nk, D), dtype=np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, stats = _run(gpu_lib, q, k, v, (1, 1, 1, Nq, Nk, D), 1, scale, "f32")
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(Nq // 2 - 32, Nq // 2 + 32),
                                     np.arange(Nq - 64, Nq)]))
    ro, rm, rl, _ = oracle.ra_attention_fwd(q[:, :, rows], k, v, True, scale, q_positions=rows,
                                            nq_total=Nq)
    err = assert_close(o[:, :, rows], ro, "f32", "O at the largest query count")
    np.testing.assert_allclose(stats[:, :, rows, 0] * scale, rm, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(stats[:, :, rows, 1], rl, rtol=1e-5)
    print(f"Nq = {Nq}: {len(rows)} rows, max abs err {err:.2e}")
