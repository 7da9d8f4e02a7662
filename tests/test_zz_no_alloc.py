"""ra_attn_bwd_noalloc (the backward with its per-row terms in an array inside the library, for
callers that cannot allocate) against ra_attn_bwd with a caller workspace, through the C ABI.

Both run the same kernels, so the gradients must agree bit for bit.  Two calls in a row, the
second smaller: the array keeps the first call's contents, which the second must not read.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import to_dev

pytestmark = pytest.mark.gpu


def rand_inputs(B, Hq, Hkv, N, D, dtype, seed):
    rng = np.random.default_rng(seed)
    out = {
        "q": rng.standard_normal((B, Hq, N, D), dtype=np.float32),
        "k": rng.standard_normal((B, Hkv, N, D), dtype=np.float32),
        "v": rng.standard_normal((B, Hkv, N, D), dtype=np.float32),
        "do": rng.standard_normal((B, Hq, N, D), dtype=np.float32),
    }
    return {n: wl.round_to_dtype(a, dtype) for n, a in out.items()}


def both_calls(ra, B, Hq, Hkv, N, D, dtype, causal, use_stats, seed):
    import torch
    inp = rand_inputs(B, Hq, Hkv, N, D, dtype, seed)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    scale = float(np.float32(1 / np.sqrt(D)))
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, N, 2), dtype=torch.float32, device="cuda")
    assert ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, N, N, D, causal, scale, code) == 0
    st = stats if use_stats else None
    nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, N, N, D, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    s = ra.ra_attn_bwd(q, k, v, o, do, st, *ref, ws, nbytes, B, Hq, Hkv, N, N, D, causal, scale, code)
    assert s == 0, ra.ra_status_string(s)
    got = [torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)]
    s = ra.ra_attn_bwd_noalloc(q, k, v, o, do, st, *got, B, Hq, Hkv, N, N, D, causal, scale, code)
    assert s == 0, ra.ra_status_string(s)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{name} differs from ra_attn_bwd"
        assert torch.isfinite(a.float()).all()


@pytest.mark.parametrize("use_stats", [True, False])
def test_noalloc_equals_workspace_call_twice(gpu_lib, use_stats):
    """A larger problem, then a smaller one, each checked against ra_attn_bwd."""
    print(f"noalloc: B=2 Hq=8 Hkv=2 N=700 D=128 bf16, stats={use_stats}", flush=True)
    both_calls(gpu_lib, 2, 8, 2, 700, 128, "bf16", 1, use_stats, seed=1)
    print(f"noalloc: B=1 Hq=2 Hkv=1 N=100 D=64 bf16, stats={use_stats}", flush=True)
    both_calls(gpu_lib, 1, 2, 1, 100, 64, "bf16", 1, use_stats, seed=2)


def test_noalloc_fp32_and_noncausal(gpu_lib):
    print("noalloc: B=1 Hq=4 Hkv=4 N=300 D=128 f32 non-causal", flush=True)
    both_calls(gpu_lib, 1, 4, 4, 300, 128, "f32", 0, True, seed=3)
    print("noalloc: B=2 Hq=2 Hkv=1 N=65 D=64 f32 causal", flush=True)
    both_calls(gpu_lib, 2, 2, 1, 65, 64, "f32", 1, False, seed=4)
