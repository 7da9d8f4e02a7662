"""The whole-launch parity checker (tests/parity.py) on the CPU, with the oracle standing in for
the GPU: it accepts the gradient of either candidate at a near tie of the row max, requires the
lowest index at an exact tie of identical keys, and rejects planted mistakes."""
import numpy as np
import pytest

import oracle
import parity
import workloads as wl


def near_tie_problem(exact=False):
    """fp32 inputs, one group (Hq=2, Hkv=1), non-causal; in row 5 of head 0 keys 1 and 3 tie for
    the max within fp32 rounding (exact=True: key 3 is a copy of key 1)."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, N, D = 1, 2, 1, 12, 8
    q = rng.standard_normal((B, Hq, N, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    do = rng.standard_normal((B, Hq, N, D)).astype(np.float32)
    qi = q[0, 0, 5].astype(np.float64)
    k[0, 0, 1] = (8.0 * qi / (qi @ qi)).astype(np.float32)          # score 8 * scale: the max
    if exact:
        k[0, 0, 3] = k[0, 0, 1]
    else:
        w = rng.standard_normal(D)
        w -= (w @ qi) / (qi @ qi) * qi                                # q_i . w = 0
        k[0, 0, 3] = (k[0, 0, 1] + w).astype(np.float32)
    return {"q": q, "k": k, "v": v, "do": do}


def test_finds_the_planted_near_tie():
    inp = near_tie_problem()
    t = parity.near_tie_candidates(inp["q"][0, 0].astype(np.float64), inp["k"][0, 0].astype(np.float64),
                                   0.35, False, 12, 12)
    assert 5 in t and 3 in t[5][1] + [t[5][0]] and 1 in t[5][1] + [t[5][0]]


@pytest.mark.parametrize("flip", [False, True])
def test_accepts_either_side_of_a_near_tie(flip):
    inp = near_tie_problem()
    ref_default = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], False, 0.35)
    a = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], False, 0.35)[3]
    over = np.full(a.shape, -1)
    over[0, 0, 5] = 4 - a[0, 0, 5]                  # the other one of keys 1 and 3
    gpu = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], False, 0.35,
                                  argmax=over) if flip else ref_default
    dq, dk, dv = (x.astype(np.float32).astype(np.float64) for x in gpu)
    res = parity.bwd_all_groups(dq, dk, dv, inp, False, 0.35, "f32")
    assert res["near_tie_rows"] >= 1
    assert res["flipped_rows"] == (1 if flip else 0)


def test_requires_lowest_index_at_an_exact_tie():
    inp = near_tie_problem(exact=True)
    over = np.full((1, 2, 12), -1)
    over[0, 0, 5] = 3                               # the copy, not the lowest index 1
    gpu = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], False, 0.35, argmax=over)
    with pytest.raises(AssertionError):
        parity.bwd_all_groups(*gpu, inp, False, 0.35, "f32")
    ok = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], False, 0.35)
    parity.bwd_all_groups(*ok, inp, False, 0.35, "f32")


def test_rejects_planted_gradient_and_output_mistakes():
    inp = near_tie_problem()
    dq, dk, dv = oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], False, 0.35)
    bad = dk.copy()
    bad[0, 0, 7] += 1e-3
    with pytest.raises(AssertionError):
        parity.bwd_all_groups(dq, bad, dv, inp, False, 0.35, "f32")
    o, m, l, _ = oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], False, 0.35)
    stats = np.stack([m / 0.35, l], axis=-1)
    parity.fwd_all_heads(o, stats, inp, False, 0.35, "f32")
    o_bad = o.copy()
    o_bad[0, 1, 2, 3] += 2e-5                       # beyond the absolute fp32 bound
    with pytest.raises(AssertionError):
        parity.fwd_all_heads(o_bad, stats, inp, False, 0.35, "f32")


# ------------------------------------------------------------- attention on rotated rows

def _rope_problem():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, N, D = 1, 4, 2, 40, 16
    r = lambda *s: wl.round_to_dtype(rng.standard_normal(s, dtype=np.float32), "bf16")
    inp = {"q": r(B, Hq, N, D), "k": r(B, Hkv, N, D), "v": r(B, Hkv, N, D), "do": r(B, Hq, N, D)}
    rope = {"theta": 500.0, "q_positions": np.arange(N) + 3, "k_positions": np.arange(N) + 3}
    return inp, rope


def _rounded_rotation(inp, rope):
    """The arithmetic the GPU performs, on the oracle: rotated rows rounded to bf16."""
    qr = wl.round_to_dtype(oracle.rope_neox(inp["q"], rope["theta"], rope["q_positions"]), "bf16")
    kr = wl.round_to_dtype(oracle.rope_neox(inp["k"], rope["theta"], rope["k_positions"]), "bf16")
    return qr, kr


def test_rope_checker_accepts_rounded_rotated_rows():
    inp, rope = _rope_problem()
    qr, kr = _rounded_rotation(inp, rope)
    o, m, l, _ = oracle.ra_attention_fwd(qr, kr, inp["v"], True, 0.25)
    stats = np.stack([m / 0.25, l], axis=-1)
    parity.fwd_rope_all_heads(o, stats, inp, True, 0.25, rope["theta"], rope["q_positions"],
                              rope["k_positions"])
    dqr, dkr, dv = oracle.ra_attention_bwd(qr, kr, inp["v"], inp["do"], True, 0.25)
    dq = oracle.rope_neox(dqr, rope["theta"], rope["q_positions"], inverse=True)
    dk = oracle.rope_neox(dkr, rope["theta"], rope["k_positions"], inverse=True)
    parity.bwd_all_groups(dq, dk, dv, inp, True, 0.25, "bf16", rope=rope)


def test_rope_checker_rejects_planted_mistakes():
    inp, rope = _rope_problem()
    qr, kr = _rounded_rotation(inp, rope)
    # keys left unrotated: the output moves beyond the bf16 tolerance or the stats bounds
    o, m, l, _ = oracle.ra_attention_fwd(qr, inp["k"], inp["v"], True, 0.25)
    with pytest.raises(AssertionError):
        parity.fwd_rope_all_heads(o, np.stack([m / 0.25, l], axis=-1), inp, True, 0.25,
                                  rope["theta"], rope["q_positions"], rope["k_positions"])
    # gradients rotated forward instead of back
    dqr, dkr, dv = oracle.ra_attention_bwd(qr, kr, inp["v"], inp["do"], True, 0.25)
    dq = oracle.rope_neox(dqr, rope["theta"], rope["q_positions"])
    dk = oracle.rope_neox(dkr, rope["theta"], rope["k_positions"], inverse=True)
    with pytest.raises(AssertionError):
        parity.bwd_all_groups(dq, dk, dv, inp, True, 0.25, "bf16", rope=rope)
