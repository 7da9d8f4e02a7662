"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on the library's stream).

The library allocates nothing and clears memory with fill kernels, never hipMemsetAsync, so its
launches can be captured.  Each graph is replayed several times, with new inputs copied into the
captured buffers and eager work between the replays, and every replay is compared bit for bit
with the eager calls on the same inputs.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import to_dev

pytestmark = pytest.mark.gpu


def _draw(shape_q, shape_k, seed):
    rng = np.random.default_rng(seed)
    r = lambda s: wl.round_to_dtype(rng.standard_normal(s, dtype=np.float32), "bf16")
    return r(shape_q), r(shape_k), r(shape_k), r(shape_q)


@pytest.mark.parametrize("dims", [(2, 12, 12, 128, 128, 64, 1), (1, 8, 2, 300, 300, 128, 2)])
def test_fwd_bwd_graph_replays_match_eager(gpu_lib, dims):
    import torch
    ra = gpu_lib
    B, Hq, Hkv, Nq, Nk, D, causal = dims
    scale = float(np.float32(1 / np.sqrt(D)))
    sq, sk = (B, Hq, Nq, D), (B, Hkv, Nk, D)
    q, k, v, do = (to_dev(a, "bf16") for a in _draw(sq, sk, 0))
    o, dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    nbytes = ra.ra_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, ra.RA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        assert ra.ra_attn_fwd(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, ra.RA_BF16) == 0
        assert ra.ra_attn_bwd(q, k, v, o, do, stats, dq, dk, dv, ws, nbytes, B, Hq, Hkv, Nq, Nk, D,
                              causal, scale, ra.RA_BF16) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        new = [to_dev(a, "bf16") for a in _draw(sq, sk, rep + 1)]
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, stats, dq, dk, dv)]
        o.zero_(); dq.zero_()                    # eager work between replays
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "stats", "dq", "dk", "dv"), got, (o, stats, dq, dk, dv)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_decode_graph_replays_match_eager(gpu_lib):
    import torch
    ra = gpu_lib
    B, Hq, Hkv, Nq, Nk, D = 4, 8, 2, 1, 1000, 128
    scale = float(np.float32(1 / np.sqrt(D)))
    q, k, v, _ = (to_dev(a, "bf16") for a in _draw((B, Hq, Nq, D), (B, Hkv, Nk, D), 10))
    lens = torch.tensor([1000, 1, 517, 0], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    stats = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device="cuda")
    nbytes = ra.ra_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, ra.RA_BF16)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        assert ra.ra_attn_decode(q, k, v, o, stats, lens, ws, nbytes, B, Hq, Hkv, Nq, Nk, D, 2, scale,
                                 ra.RA_BF16) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep, new_lens in enumerate(([999, 2, 64, 1000], [0, 0, 0, 0], [1000, 1000, 1000, 1000])):
        qn, kn, vn, _ = (to_dev(a, "bf16") for a in _draw((B, Hq, Nq, D), (B, Hkv, Nk, D), 20 + rep))
        q.copy_(qn); k.copy_(kn); v.copy_(vn)
        lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), stats.clone())
        o.fill_(7.0)
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], o) and torch.equal(got[1], stats), f"replay {rep} differs"
