"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

None of these compares the oracle with itself: each check uses hand-derived
values (tests/golden/), a second closed form, an invariant, a special case that
reduces to a library routine, or central finite differences.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- ra_softmax

def test_worked_example_exact_phi_and_p():
    rows = _read_rows("ra_softmax_worked_example.txt")
    x = np.zeros((2, 3))
    phi_exact = [[None] * 3 for _ in range(2)]
    for r, c, logit, num, den in rows:
        r, c = int(r), int(c)
        x[r, c] = float(logit)
        phi_exact[r][c] = Fraction(int(num), int(den))
    p, phi, m, l = oracle.ra_softmax_rows(x, return_stats=True)
    for r in range(2):
        tot = sum(phi_exact[r])
        assert float(tot) == pytest.approx(l[r], rel=1e-15)
        assert m[r] == x[r].max()
        for c in range(3):
            assert phi[r, c] == pytest.approx(float(phi_exact[r][c]), rel=1e-14, abs=0)
            assert p[r, c] == pytest.approx(float(phi_exact[r][c] / tot), rel=1e-14, abs=0)


def test_support_edge_values():
    for d, num, den in _read_rows("ra_softmax_support_edge.txt"):
        want = float(Fraction(int(num), int(den)))
        got = float(oracle.ra_phi(float(d)))
        if want == 0.0:
            assert got == 0.0, d
        else:
            assert got == pytest.approx(want, rel=1e-14, abs=0), d


def test_phi_positive_just_inside_support():
    d = np.nextafter(16.0, 0.0)
    assert oracle.ra_phi(d) > 0.0
    assert oracle.ra_phi(16.0) == 0.0


def test_artanh_closed_form():
    # q = (1-u)/(1+u) = exp(-2 artanh u), so phi = exp(-16 artanh(Delta/16)) on [0, 16).
    rng = np.random.default_rng(1)
    d = np.concatenate([rng.uniform(0, 16, 20000), [0.0, 1e-9, 15.999]])
    want = np.exp(-16.0 * np.arctanh(d / 16.0))
    got = oracle.ra_phi(d)
    np.testing.assert_allclose(got, want, rtol=2e-13, atol=0)


def test_exp_sandwich():
    # artanh(u) >= u gives phi <= exp(-Delta); the series bound gives
    # log(phi) + Delta >= -Delta^3 / (768 (1 - u^2)).
    d = np.linspace(0, 15.99, 5001)
    u = d / 16
    lp = np.log(oracle.ra_phi(d))
    assert np.all(lp <= -d + 1e-12)
    assert np.all(lp + d >= -d ** 3 / (768 * (1 - u * u)) - 1e-12)


def test_softmax_invariants():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 6, size=(64, 37))
    p, phi, m, l = oracle.ra_softmax_rows(x, return_stats=True)
    assert np.all(phi.max(axis=1) == 1.0)                 # phi at the max is exactly 1
    assert np.all(l >= 1.0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(p[x <= (m[:, None] - 16.0)] == 0.0)     # exact zeros off the support
    assert np.all(p[x > (m[:, None] - 16.0)] > 0.0)


def test_softmax_shift_invariance_exact():
    rng = np.random.default_rng(3)
    x = rng.integers(-30, 30, size=(40, 25)).astype(np.float64)
    c = rng.integers(-1000, 1000, size=(40, 1)).astype(np.float64)
    np.testing.assert_array_equal(oracle.ra_softmax_rows(x), oracle.ra_softmax_rows(x + c))


def test_softmax_masking():
    x = np.array([[3.0, -np.inf, 1.0, -np.inf],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [-np.inf, 7.0, -np.inf, -np.inf]])
    p = oracle.ra_softmax_rows(x)
    assert p[0, 1] == 0 and p[0, 3] == 0
    want = oracle.ra_softmax_rows(np.array([[3.0, 1.0]]))[0]
    np.testing.assert_allclose(p[0, [0, 2]], want, rtol=1e-15)
    assert np.all(p[1] == 0.0)                            # fully masked row -> zeros, no NaN
    np.testing.assert_array_equal(p[2], [0, 1, 0, 0])


def test_softmax_close_to_exp_softmax_for_small_spread():
    # For Delta <= delta the two softmaxes differ by a factor within exp(+-eps),
    # eps = delta^3 / (768 (1 - (delta/16)^2)).
    rng = np.random.default_rng(4)
    delta = 0.3
    x = rng.uniform(0, delta, size=(50, 17))
    e = np.exp(x - x.max(axis=1, keepdims=True))
    sm = e / e.sum(axis=1, keepdims=True)
    eps = delta ** 3 / (768 * (1 - (delta / 16) ** 2))
    ratio = oracle.ra_softmax_rows(x) / sm
    assert np.all(ratio <= np.exp(eps) + 1e-15) and np.all(ratio >= np.exp(-eps) - 1e-15)


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy(); xp[i] += h
        xm = x.copy(); xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_softmax_bwd_matches_central_differences():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 5, size=(4, 9))
    x[0, 3] = x[0].max() - 15.0    # an entry near the support edge
    dp = rng.normal(size=x.shape)
    g = oracle.ra_softmax_rows_bwd(x, dp)
    fd = _fd_grad(lambda z: float((oracle.ra_softmax_rows(z) * dp).sum()), x)
    np.testing.assert_allclose(g, fd, rtol=0, atol=2e-8)
    # shift invariance: every row of the gradient sums to zero
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-14)


# ------------------------------------------------------------- ra_attention

def _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.0):
    q = rng.normal(0, sigma, size=(B, Hq, Nq, D))
    k = rng.normal(0, sigma, size=(B, Hkv, Nk, D))
    v = rng.normal(0, 1, size=(B, Hkv, Nk, D))
    return q, k, v


def test_single_key_returns_value():
    rng = np.random.default_rng(6)
    q, k, v = _rand_qkv(rng, 2, 3, 1, 5, 1, 4)
    for causal in (False, True):
        o = oracle.ra_attention_fwd(q, k, v, causal, 0.5)[0]
        np.testing.assert_array_equal(o, np.broadcast_to(v[:, :1], o.shape))


def test_equal_scores_give_prefix_mean():
    rng = np.random.default_rng(7)
    q = np.zeros((1, 2, 6, 4))
    k = rng.normal(size=(1, 2, 6, 4))
    v = rng.normal(size=(1, 2, 6, 4))
    o = oracle.ra_attention_fwd(q, k, v, False, 0.5)[0]
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-15)
    oc = oracle.ra_attention_fwd(q, k, v, True, 0.5)[0]
    csum = np.cumsum(v, axis=2) / np.arange(1, 7)[None, None, :, None]
    np.testing.assert_allclose(oc, csum, atol=1e-15)


def test_one_hot_rows_select_value_exactly():
    # Every other score at least 16 below the max -> phi = (1, 0, ...), O = v_argmax exactly.
    B, H, N, D = 1, 2, 8, 8
    rng = np.random.default_rng(8)
    k = np.eye(N, D)[None, None].repeat(H, axis=1) * 1.0
    target = rng.permutation(N)
    q = np.zeros((B, H, N, D))
    q[0, :, np.arange(N), target] = 40.0          # scale 1 -> score 40 at key target[i], 0 elsewhere
    v = rng.normal(size=(B, H, N, D))
    o = oracle.ra_attention_fwd(q, k, v, False, 1.0)[0]
    np.testing.assert_array_equal(o[0, 0], v[0, 0, target])


def test_identity_values_expose_probabilities():
    rng = np.random.default_rng(9)
    N = 7
    q, k, _ = _rand_qkv(rng, 1, 1, 1, N, N, 5, sigma=2.0)
    v = np.eye(N)[None, None]
    for causal in (False, True):
        o = oracle.ra_attention_fwd(q, k, v, causal, 0.7)[0]
        s = 0.7 * q[0, 0] @ k[0, 0].T
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        np.testing.assert_allclose(o[0, 0], oracle.ra_softmax_rows(s), rtol=0, atol=1e-15)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(10)
    q, k, v = _rand_qkv(rng, 2, 6, 2, 9, 9, 4)
    rep = 3
    kr, vr = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    for causal in (False, True):
        o1 = oracle.ra_attention_fwd(q, k, v, causal, 0.5)[0]
        o2 = oracle.ra_attention_fwd(q, kr, vr, causal, 0.5)[0]
        np.testing.assert_array_equal(o1, o2)
        # head h must read K/V head h // rep (not h % Hkv)
        o3 = oracle.ra_attention_fwd(q, np.tile(k, (1, rep, 1, 1)), np.tile(v, (1, rep, 1, 1)),
                                     causal, 0.5)[0]
        assert not np.allclose(o1, o3)


def test_small_spread_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Nq, Nk, D = 2, 4, 2, 11, 11, 6
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D)
    scale = 0.37
    q = q * 0.02            # |s| <= 0.1 -> every Delta <= 0.2
    delta = 0.2
    for causal in (False, True):
        o = oracle.ra_attention_fwd(q, k, v, causal, scale)[0]
        s = scale * np.einsum("bhnd,bhmd->bhnm", q, np.repeat(k, 2, axis=1))
        assert np.abs(s).max() <= delta / 2
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.repeat(k, 2, axis=1)),
            torch.from_numpy(np.repeat(v, 2, axis=1)), is_causal=causal, scale=scale).numpy()
        eps = delta ** 3 / (768 * (1 - (delta / 16) ** 2))
        bound = (np.exp(2 * eps) - 1) * np.abs(v).max()
        assert np.abs(o - ref).max() <= bound
        assert np.abs(o - ref).max() > 0


def test_causality_future_keys_do_not_leak():
    rng = np.random.default_rng(12)
    q, k, v = _rand_qkv(rng, 1, 2, 2, 10, 10, 4)
    o = oracle.ra_attention_fwd(q, k, v, True, 0.5)[0]
    for t in range(9):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, t + 1:] = rng.normal(size=k2[:, :, t + 1:].shape)
        v2[:, :, t + 1:] = rng.normal(size=v2[:, :, t + 1:].shape)
        o2 = oracle.ra_attention_fwd(q, k2, v2, True, 0.5)[0]
        np.testing.assert_array_equal(o[:, :, :t + 1], o2[:, :, :t + 1])
        assert not np.allclose(o[:, :, t + 1], o2[:, :, t + 1])


def test_query_positions_select_rows():
    rng = np.random.default_rng(13)
    q, k, v = _rand_qkv(rng, 1, 2, 1, 12, 12, 4)
    full = oracle.ra_attention_fwd(q, k, v, True, 0.5)
    rows = np.array([0, 5, 11])
    part = oracle.ra_attention_fwd(q[:, :, rows], k, v, True, 0.5, q_positions=rows)
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[:, :, rows], b)


def test_attention_stats():
    rng = np.random.default_rng(14)
    q, k, v = _rand_qkv(rng, 1, 2, 2, 8, 8, 4, sigma=2.0)
    o, m, l, a = oracle.ra_attention_fwd(q, k, v, True, 0.5)
    for h in range(2):
        s = 0.5 * q[0, h] @ k[0, h].T
        for i in range(8):
            assert m[0, h, i] == s[i, : i + 1].max()
            assert a[0, h, i] == int(np.argmax(s[i, : i + 1]))
            assert l[0, h, i] >= 1.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 6, 3), (2, 2, 2, 4, 4, 2)])
def test_attention_bwd_matches_central_differences(causal, shape):
    B, Hq, Hkv, Nq, Nk, D = shape
    rng = np.random.default_rng(15)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    do = rng.normal(size=q.shape)
    scale = 0.8
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        return float((oracle.ra_attention_fwd(qq, kk, vv, causal, scale)[0] * do).sum())

    fq = _fd_grad(lambda z: loss(z, k, v), q)
    fk = _fd_grad(lambda z: loss(q, z, v), k)
    fv = _fd_grad(lambda z: loss(q, k, z), v)
    np.testing.assert_allclose(dq, fq, rtol=0, atol=3e-8)
    np.testing.assert_allclose(dk, fk, rtol=0, atol=3e-8)
    np.testing.assert_allclose(dv, fv, rtol=0, atol=3e-8)


def test_attention_bwd_wide_scores_near_support_edge():
    # Scores spread wide enough that some entries sit inside (12, 16) and some beyond 16.
    rng = np.random.default_rng(16)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 6, 6, 3, sigma=3.0)
    do = rng.normal(size=q.shape)
    s = q[0, 0] @ k[0, 0].T
    assert (s.max(1, keepdims=True) - s > 16).any() and ((s.max(1, keepdims=True) - s) > 8).sum() > 3
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, False, 1.0)

    def loss(qq, kk):
        return float((oracle.ra_attention_fwd(qq, kk, v, False, 1.0)[0] * do).sum())

    np.testing.assert_allclose(dq, _fd_grad(lambda z: loss(z, k), q), atol=3e-8, rtol=0)
    np.testing.assert_allclose(dk, _fd_grad(lambda z: loss(q, z), k), atol=3e-8, rtol=0)


def test_attention_bwd_invariants():
    rng = np.random.default_rng(17)
    B, Hq, Hkv, N, D = 2, 4, 2, 13, 5
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, N, N, D)
    do = rng.normal(size=q.shape)
    for causal in (False, True):
        dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, causal, 0.6)
        # shift invariance of every softmax row -> sum_j dK_j = 0 per K/V head
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # each row of P sums to one -> sum_j dV_j = sum over the group's query rows of dO
        dsum = do.reshape(B, Hkv, Hq // Hkv, N, D).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), dsum, atol=1e-12)
        # the loss depends on q_i . k_j only -> <Q, dQ> = <K, dK>
        assert np.sum(q * dq) == pytest.approx(np.sum(k * dk), rel=1e-10, abs=1e-12)


def test_bwd_max_path_term_is_needed():
    # Planted mistake (in the oracle, on the CPU): dropping the row-max term R
    # must break agreement with finite differences, so the FD pin sees it.
    import oracle.ra_oracle as ro
    rng = np.random.default_rng(18)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 5, 5, 3, sigma=1.5)
    do = rng.normal(size=q.shape)

    def loss(qq):
        return float((oracle.ra_attention_fwd(qq, k, v, False, 1.0)[0] * do).sum())

    fd = _fd_grad(loss, q)
    orig = ro._softmax_vjp

    def no_max_path(p, delta, dp, a):
        return orig(p, delta, dp, np.full_like(a, -1))

    ro._softmax_vjp = no_max_path
    try:
        dq_bad = oracle.ra_attention_bwd(q, k, v, do, False, 1.0)[0]
    finally:
        ro._softmax_vjp = orig
    assert np.abs(dq_bad - fd).max() > 1e-3


def test_argmax_override_is_the_gradient_from_the_other_side_of_a_tie():
    # Where key a' is the row max by a margin delta over key a, the override argmax = a must give
    # the gradient the default takes once a leads by delta instead (the function on a's side of
    # the tie, where it is smooth): equal up to O(delta), and visibly different from the default
    # gradient at the same point, which puts the row-max term on a'.
    rng = np.random.default_rng(19)
    B, H, N, D, i, a, a2 = 1, 1, 6, 4, 5, 1, 3
    q, k, v = _rand_qkv(rng, B, H, H, N, N, D, sigma=0.7)
    do = rng.normal(size=q.shape)
    qi = q[0, 0, i]
    w = rng.normal(size=D)
    w -= (w @ qi) / (qi @ qi) * qi                   # q_i . w = 0
    delta = 1e-9
    k[0, 0, a2] = 3.0 * qi / (qi @ qi)               # s_{i,a2} = 3, the max of row i
    k_a_below = k[0, 0, a2] + w - delta * qi / (qi @ qi)
    k_a_above = k[0, 0, a2] + w + delta * qi / (qi @ qi)
    x_below, x_above = k.copy(), k.copy()
    x_below[0, 0, a], x_above[0, 0, a] = k_a_below, k_a_above
    _, _, _, am = oracle.ra_attention_fwd(q, x_below, v, False, 1.0)
    assert am[0, 0, i] == a2
    assert oracle.ra_attention_fwd(q, x_above, v, False, 1.0)[3][0, 0, i] == a
    over = np.full((B, H, N), -1)
    over[0, 0, i] = a
    g_over = oracle.ra_attention_bwd(q, x_below, v, do, False, 1.0, argmax=over)
    g_above = oracle.ra_attention_bwd(q, x_above, v, do, False, 1.0)
    g_default = oracle.ra_attention_bwd(q, x_below, v, do, False, 1.0)
    for x, y, z in zip(g_over, g_above, g_default):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-7)
    assert np.abs(g_over[0] - g_default[0]).max() > 1e-3    # dQ of row i moves with the argmax
    assert np.abs(g_over[1] - g_default[1]).max() > 1e-3    # so do dK_a, dK_a2
    # an override equal to the default argmax changes nothing
    same = np.full((B, H, N), -1)
    same[0, 0, i] = a2
    for x, y in zip(oracle.ra_attention_bwd(q, x_below, v, do, False, 1.0, argmax=same), g_default):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------------------- masks and causal alignment

def test_key_padding_equals_dropping_keys():
    # A key that is masked out for a sample must act exactly as if it were absent.
    rng = np.random.default_rng(40)
    B, Hq, Hkv, Nq, Nk, D = 2, 4, 2, 5, 9, 4
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    do = rng.normal(size=q.shape)
    keep = np.ones((B, Nk), bool)
    keep[0, [1, 4, 8]] = False
    keep[1, [0, 2]] = False
    kpm = keep[:, None, None, :]
    o, m, l, a = oracle.ra_attention_fwd(q, k, v, False, 0.6, mask=kpm)
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, False, 0.6, mask=kpm)
    for b in range(B):
        kb, vb = k[b:b + 1][:, :, keep[b]], v[b:b + 1][:, :, keep[b]]
        o1, m1, l1, a1 = oracle.ra_attention_fwd(q[b:b + 1], kb, vb, False, 0.6)
        np.testing.assert_allclose(o[b:b + 1], o1, rtol=0, atol=1e-14)
        np.testing.assert_array_equal(m[b:b + 1], m1)
        np.testing.assert_array_equal(a[b:b + 1], np.nonzero(keep[b])[0][a1])
        dq1, dk1, dv1 = oracle.ra_attention_bwd(q[b:b + 1], kb, vb, do[b:b + 1], False, 0.6)
        np.testing.assert_allclose(dq[b:b + 1], dq1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk[b:b + 1][:, :, keep[b]], dk1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv[b:b + 1][:, :, keep[b]], dv1, rtol=0, atol=1e-14)
        assert (dk[b][:, ~keep[b]] == 0).all() and (dv[b][:, ~keep[b]] == 0).all()


def test_all_true_mask_and_zero_bias_change_nothing():
    rng = np.random.default_rng(41)
    q, k, v = _rand_qkv(rng, 1, 2, 1, 6, 7, 4, sigma=1.5)
    for causal in (False, "top_left", "bottom_right"):
        ref = oracle.ra_attention_fwd(q, k, v, causal, 0.5)
        for mask in (np.ones((6, 7), bool), np.zeros((1, 1, 6, 7))):
            got = oracle.ra_attention_fwd(q, k, v, causal, 0.5, mask=mask)
            for x, y in zip(ref, got):
                np.testing.assert_array_equal(x, y)


def test_additive_mask_worked_example():
    # Scores scale * q.k = [2, 1, 0] (q = 1, k = 2, 1, 0, scale 1) and V = I, so O = p.
    q = np.ones((1, 1, 1, 1))
    k = np.array([2.0, 1.0, 0.0]).reshape(1, 1, 3, 1)
    v = np.eye(3).reshape(1, 1, 3, 3)
    # bias (0, -7, +2) -> logits (2, -6, 2): the max 2 is tied at keys 0 and 2 (lowest: 0),
    # Delta = (0, 8, 0), u = (0, 1/2, 0), phi = (1, (1/3)^8, 1)
    o, m, l, a = oracle.ra_attention_fwd(q, k, v, False, 1.0, mask=np.array([0.0, -7.0, 2.0]))
    third8 = Fraction(1, 3) ** 8
    lsum = 2 + third8
    np.testing.assert_allclose(o[0, 0, 0], [float(1 / lsum), float(third8 / lsum), float(1 / lsum)],
                               rtol=1e-15, atol=0)
    assert m[0, 0, 0] == 2.0 and a[0, 0, 0] == 0 and l[0, 0, 0] == pytest.approx(float(lsum), abs=1e-15)
    # bias (0, -inf, 0) drops key 1: Delta = (0, -, 2), phi(2) = ((1 - 1/8) / (1 + 1/8))^8 = (7/9)^8
    o, m, l, a = oracle.ra_attention_fwd(q, k, v, False, 1.0, mask=np.array([0.0, -np.inf, 0.0]))
    p2 = Fraction(7, 9) ** 8
    np.testing.assert_allclose(o[0, 0, 0], [float(1 / (1 + p2)), 0.0, float(p2 / (1 + p2))],
                               rtol=1e-15, atol=0)
    assert o[0, 0, 0, 1] == 0.0 and a[0, 0, 0] == 0


def test_row_constant_bias_changes_nothing():
    # phi depends on Delta = max - s only, so a constant added to a whole row changes nothing
    rng = np.random.default_rng(42)
    q, k, v = _rand_qkv(rng, 2, 2, 1, 5, 6, 3, sigma=1.5)
    do = rng.normal(size=q.shape)
    bias = np.broadcast_to(rng.normal(0, 3, size=(2, 2, 5, 1)), (2, 2, 5, 6))
    ref_o = oracle.ra_attention_fwd(q, k, v, True, 0.7)[0]
    got_o = oracle.ra_attention_fwd(q, k, v, True, 0.7, mask=bias)[0]
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-13)
    for x, y in zip(oracle.ra_attention_bwd(q, k, v, do, True, 0.7),
                    oracle.ra_attention_bwd(q, k, v, do, True, 0.7, mask=bias)):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)


def test_bool_false_equals_minus_inf_bias():
    rng = np.random.default_rng(43)
    q, k, v = _rand_qkv(rng, 1, 3, 3, 6, 8, 4, sigma=1.5)
    do = rng.normal(size=q.shape)
    mb = rng.random((1, 3, 6, 8)) < 0.7
    mf = np.where(mb, 0.0, -np.inf)
    for x, y in zip(oracle.ra_attention_fwd(q, k, v, False, 0.5, mask=mb),
                    oracle.ra_attention_fwd(q, k, v, False, 0.5, mask=mf)):
        np.testing.assert_array_equal(x, y)
    for x, y in zip(oracle.ra_attention_bwd(q, k, v, do, False, 0.5, mask=mb),
                    oracle.ra_attention_bwd(q, k, v, do, False, 0.5, mask=mf)):
        np.testing.assert_array_equal(x, y)


def _brute_attention(q, k, v, scale, allowed):
    """One head, pure Python loops, straight from the definitions (tiny inputs only)."""
    Nq, Nk, D = len(q), len(k), len(v[0])
    out = []
    for i in range(Nq):
        s = {j: scale * sum(q[i][d] * k[j][d] for d in range(len(q[i]))) for j in range(Nk)
             if allowed(i, j)}
        if not s:
            out.append([0.0] * D)
            continue
        mx = max(s.values())
        phi = {}
        for j, x in s.items():
            u = (mx - x) / 16.0
            phi[j] = ((1 - u) / (1 + u)) ** 8 if u < 1 else 0.0
        tot = sum(phi.values())
        out.append([sum(phi[j] / tot * v[j][d] for j in phi) for d in range(D)])
    return np.array(out)


@pytest.mark.parametrize("Nq,Nk", [(3, 7), (7, 3), (5, 5), (1, 6), (6, 1)])
def test_bottom_right_causal_brute_force(Nq, Nk):
    rng = np.random.default_rng(44 + Nq * 10 + Nk)
    q, k, v = _rand_qkv(rng, 1, 1, 1, Nq, Nk, 3, sigma=1.5)
    o = oracle.ra_attention_fwd(q, k, v, "bottom_right", 0.9)[0]
    ref = _brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.9,
                           lambda i, j: j <= i + Nk - Nq)
    np.testing.assert_allclose(o[0, 0], ref, rtol=0, atol=1e-14)
    top = oracle.ra_attention_fwd(q, k, v, "top_left", 0.9)[0]
    ref_top = _brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.9,
                               lambda i, j: j <= i)
    np.testing.assert_allclose(top[0, 0], ref_top, rtol=0, atol=1e-14)
    if Nq == Nk:
        np.testing.assert_array_equal(o, top)
    else:
        assert not np.allclose(o, top)


def test_bottom_right_is_the_tail_of_a_square_problem():
    # Nq <= Nk: the queries continue a sequence whose first Nk - Nq queries are not asked for.
    rng = np.random.default_rng(45)
    q, k, v = _rand_qkv(rng, 2, 4, 2, 4, 10, 3, sigma=1.5)
    do = rng.normal(size=q.shape)
    qfull = np.concatenate([rng.normal(size=(2, 4, 6, 3)), q], axis=2)
    dofull = np.concatenate([np.zeros((2, 4, 6, 3)), do], axis=2)
    o = oracle.ra_attention_fwd(q, k, v, "bottom_right", 0.8)[0]
    np.testing.assert_array_equal(o, oracle.ra_attention_fwd(qfull, k, v, True, 0.8)[0][:, :, 6:])
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, "bottom_right", 0.8)
    fq, fk, fv = oracle.ra_attention_bwd(qfull, k, v, dofull, True, 0.8)
    np.testing.assert_allclose(dq, fq[:, :, 6:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, fk, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, fv, rtol=0, atol=1e-14)


def test_fully_masked_rows_are_zero_not_nan():
    rng = np.random.default_rng(46)
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 7, 4, 3
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    do = rng.normal(size=q.shape)
    mask = np.ones((B, Hq, Nq, Nk), bool)
    mask[0, 1, 5] = False                      # an explicit fully masked row
    # bottom-right with Nq > Nk: rows 0..2 have no key at all
    o, m, l, a = oracle.ra_attention_fwd(q, k, v, "bottom_right", 0.5, mask=mask)
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, "bottom_right", 0.5, mask=mask)
    dead = np.zeros((B, Hq, Nq), bool)
    dead[:, :, :Nq - Nk] = True
    dead[0, 1, 5] = True
    for x in (o, dq, dk, dv):
        assert np.isfinite(x).all()
    assert (o[dead] == 0).all() and (dq[dead] == 0).all()
    assert (m[dead] == -np.inf).all() and (l[dead] == 0).all() and (a[dead] == -1).all()
    assert (l[~dead] >= 1).all() and np.isfinite(m[~dead]).all()


def test_sampled_rows_with_bottom_right_offset():
    rng = np.random.default_rng(47)
    q, k, v = _rand_qkv(rng, 1, 2, 1, 9, 13, 4, sigma=1.5)
    mask = rng.random((1, 2, 9, 13)) < 0.8
    full = oracle.ra_attention_fwd(q, k, v, "bottom_right", 0.5, mask=mask)
    rows = np.array([0, 4, 8])
    part = oracle.ra_attention_fwd(q[:, :, rows], k, v, "bottom_right", 0.5, q_positions=rows,
                                   nq_total=9, mask=mask[:, :, rows])
    for x, y in zip(full, part):
        np.testing.assert_array_equal(x[:, :, rows], y)


@pytest.mark.parametrize("case", ["keypad_bottom_right", "bias_top_left", "bias_bool_none"])
def test_masked_attention_bwd_matches_central_differences(case):
    rng = np.random.default_rng(48)
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 4, 6, 3
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    do = rng.normal(size=q.shape)
    if case == "keypad_bottom_right":
        causal, mask = "bottom_right", np.array([True, False, True, True, False, True])[None, None, None]
    elif case == "bias_top_left":
        causal, mask = "top_left", rng.normal(0, 2, size=(1, 1, Nq, Nk))
    else:
        bias = rng.normal(0, 2, size=(B, Hq, Nq, Nk))
        bias[rng.random(bias.shape) < 0.25] = -np.inf
        causal, mask = False, bias
    scale = 0.8
    dq, dk, dv = oracle.ra_attention_bwd(q, k, v, do, causal, scale, mask=mask)

    def loss(qq, kk, vv):
        return float((oracle.ra_attention_fwd(qq, kk, vv, causal, scale, mask=mask)[0] * do).sum())

    np.testing.assert_allclose(dq, _fd_grad(lambda z: loss(z, k, v), q), rtol=0, atol=3e-8)
    np.testing.assert_allclose(dk, _fd_grad(lambda z: loss(q, z, v), k), rtol=0, atol=3e-8)
    np.testing.assert_allclose(dv, _fd_grad(lambda z: loss(q, k, z), v), rtol=0, atol=3e-8)


# ------------------------------------------------------------- decode against a cache

def test_decode_continues_the_prefill():
    # Decoding the last Nq queries of a sequence of length L against its cache equals the last
    # Nq rows of the causal (top-left) prefill of the whole sequence.
    rng = np.random.default_rng(50)
    B, Hq, Hkv, Nq, Nk, D = 3, 4, 2, 2, 12, 4
    lens = np.array([12, 7, 2])
    k = rng.normal(0, 1.5, size=(B, Hkv, Nk, D))
    v = rng.normal(size=(B, Hkv, Nk, D))
    qfull = rng.normal(0, 1.5, size=(B, Hq, Nk, D))
    q = np.stack([qfull[b, :, lens[b] - Nq:lens[b]] for b in range(B)])
    o, m, l, a = oracle.ra_attention_decode(q, k, v, 0.6, seqlens=lens, causal="bottom_right")
    for b in range(B):
        n = lens[b]
        pf = oracle.ra_attention_fwd(qfull[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                                     True, 0.6)
        for x, y in zip((o, m, l, a), pf):
            np.testing.assert_array_equal(x[b], y[0, :, n - Nq:n])


def test_decode_brute_force_and_edges():
    rng = np.random.default_rng(51)
    B, Hq, Hkv, Nq, Nk, D = 4, 2, 1, 3, 9, 3
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    lens = np.array([9, 4, 0, 1])
    for causal in (False, "top_left", "bottom_right"):
        o, m, l, a = oracle.ra_attention_decode(q, k, v, 0.7, seqlens=lens, causal=causal)
        for b in range(B):
            n = int(lens[b])
            def allowed(i, j, n=n):
                if j >= n:
                    return False
                if causal == "top_left":
                    return j <= i
                if causal == "bottom_right":
                    return j <= i + n - Nq
                return True
            for h in range(Hq):
                ref = _brute_attention(q[b, h].tolist(), k[b, h // 2].tolist(), v[b, h // 2].tolist(),
                                       0.7, allowed)
                np.testing.assert_allclose(o[b, h], ref, rtol=0, atol=1e-14)
        assert (o[2] == 0).all() and (m[2] == -np.inf).all() and (l[2] == 0).all()
    # no lengths: the whole cache, the same as the plain forward
    for x, y in zip(oracle.ra_attention_decode(q, k, v, 0.7, causal="bottom_right"),
                    oracle.ra_attention_fwd(q, k, v, "bottom_right", 0.7)):
        np.testing.assert_array_equal(x, y)
    with pytest.raises(ValueError):
        oracle.ra_attention_decode(q, k, v, 0.7, seqlens=np.array([1, 2, 3, 10]))


def test_decode_gqa_equals_mha_on_repeated_cache():
    rng = np.random.default_rng(52)
    q, k, v = _rand_qkv(rng, 2, 8, 2, 1, 20, 4, sigma=1.5)
    lens = np.array([20, 13])
    o1 = oracle.ra_attention_decode(q, k, v, 0.5, seqlens=lens)[0]
    o2 = oracle.ra_attention_decode(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.5,
                                    seqlens=lens)[0]
    np.testing.assert_array_equal(o1, o2)


def test_gqa_per_query_head_masks_match_brute_force():
    # GQA with a different boolean mask per query head: head h attends with its own mask row and
    # K/V head h // REP.
    rng = np.random.default_rng(53)
    B, Hq, Hkv, Nq, Nk, D = 1, 4, 2, 4, 7, 3
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    mask = rng.random((B, Hq, Nq, Nk)) < 0.6
    mask[..., 0] = True
    o = oracle.ra_attention_fwd(q, k, v, False, 0.7, mask=mask)[0]
    for h in range(Hq):
        ref = _brute_attention(q[0, h].tolist(), k[0, h // 2].tolist(), v[0, h // 2].tolist(), 0.7,
                               lambda i, j, h=h: bool(mask[0, h, i, j]))
        np.testing.assert_allclose(o[0, h], ref, rtol=0, atol=1e-14)


# Planted mistakes (in the oracle, on the CPU): each must make at least one pin fail.

def _planted(name, replacement):
    """Context: oracle.ra_oracle.<name> replaced by replacement(original) while inside."""
    import contextlib
    import oracle.ra_oracle as ro

    @contextlib.contextmanager
    def ctx():
        orig = getattr(ro, name)
        setattr(ro, name, replacement(orig))
        try:
            yield
        finally:
            setattr(ro, name, orig)
    return ctx()


def test_planted_flipped_bottom_right_offset_breaks_brute_force():
    flip = lambda orig: (lambda causal, Nq, Nk: (lambda off: -off if off else off)(orig(causal, Nq, Nk)))
    with _planted("causal_offset", flip):
        with pytest.raises(AssertionError):
            test_bottom_right_causal_brute_force(3, 7)
        with pytest.raises(AssertionError):
            test_bottom_right_causal_brute_force(7, 3)
    test_bottom_right_causal_brute_force(3, 7)     # restored


def test_planted_ignored_bias_breaks_additive_example():
    def ignore_bias(orig):
        def scores(qh, kg, scale, allowed, mask, b, h, shape):
            if mask is not None and mask.dtype != np.bool_:
                mask = None
            return orig(qh, kg, scale, allowed, mask, b, h, shape)
        return scores
    with _planted("_scores", ignore_bias):
        with pytest.raises(AssertionError):
            test_additive_mask_worked_example()
    test_additive_mask_worked_example()


def test_planted_mask_of_the_kv_head_breaks_per_head_masks():
    def kv_head(orig):
        def scores(qh, kg, scale, allowed, mask, b, h, shape):
            return orig(qh, kg, scale, allowed, mask, b, h // 2, shape)   # REP = 2 in the pin
        return scores
    with _planted("_scores", kv_head):
        with pytest.raises(AssertionError):
            test_gqa_per_query_head_masks_match_brute_force()
    test_gqa_per_query_head_masks_match_brute_force()


@pytest.mark.parametrize("mistake", ["prefix_off_by_one", "lengths_ignored"])
def test_planted_decode_mistakes_break_decode_pins(mistake):
    # A scratch decode that takes one key too few per sample, or ignores the lengths, must fail
    # the prefill-continuation and brute-force pins.
    def bad_decode(orig):
        def decode(q, k, v, scale, seqlens=None, causal=False):
            if mistake == "lengths_ignored":
                return orig(q, k, v, scale, seqlens=None, causal=causal)
            lens = np.full(q.shape[0], k.shape[2]) if seqlens is None else np.asarray(seqlens)
            return orig(q, k, v, scale, seqlens=np.maximum(lens - 1, 0), causal=causal)
        return decode
    import oracle as oracle_pkg
    import oracle.ra_oracle as ro
    orig = ro.ra_attention_decode
    bad = bad_decode(orig)
    ro.ra_attention_decode, oracle_pkg.ra_attention_decode = bad, bad
    try:
        with pytest.raises(AssertionError):
            test_decode_continues_the_prefill()
        with pytest.raises(AssertionError):
            test_decode_brute_force_and_edges()
    finally:
        ro.ra_attention_decode, oracle_pkg.ra_attention_decode = orig, orig
    test_decode_continues_the_prefill()


def test_planted_phi_exponent_error_breaks_golden():
    # Planted mistake: phi = q^7 instead of q^8 must fail the worked-example pin.
    import oracle.ra_oracle as ro
    orig = ro.ra_phi

    def wrong(delta):
        d = np.asarray(delta, dtype=np.float64)
        u = d / 16
        inside = u < 1
        uu = np.where(inside, u, 0)
        return np.where(inside, ((1 - uu) / (1 + uu)) ** 7, 0.0)

    ro.ra_phi = wrong
    try:
        with pytest.raises(AssertionError):
            test_worked_example_exact_phi_and_p()
    finally:
        ro.ra_phi = orig


# ------------------------------------------------------------- NEOX RoPE

def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(31)
    x = rng.normal(size=(2, 3, 7, 8))
    y = oracle.rope_neox(x, 10000.0)
    np.testing.assert_array_equal(y[..., 0, :], x[..., 0, :])
    half = 4
    np.testing.assert_allclose(y[..., :half] ** 2 + y[..., half:] ** 2,
                               x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-13)


def test_rope_inverse_undoes_forward():
    rng = np.random.default_rng(32)
    x = rng.normal(size=(3, 50, 16))
    y = oracle.rope_neox(oracle.rope_neox(x, 500.0), 500.0, inverse=True)
    np.testing.assert_allclose(y, x, atol=1e-13)


def test_rope_pairs_channel_j_with_j_plus_half():
    """Perturbing channel j moves only channels j and j + D/2 (not j + 1, the interleaved
    pairing the page warns against)."""
    D = 8
    x = np.zeros((1, 5, D))
    for j in range(D):
        e = x.copy()
        e[0, 3, j] = 1.0
        y = oracle.rope_neox(e, 10000.0)[0, 3]
        partner = (j + D // 2) % D
        moved = set(np.nonzero(np.abs(y) > 0)[0].tolist())
        assert moved <= {j, partner} and j in moved


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(33)
    q = rng.normal(size=(1, 16))
    k = rng.normal(size=(1, 16))
    def score(m, n):
        qm = oracle.rope_neox(q, 10000.0, positions=[m])
        kn = oracle.rope_neox(k, 10000.0, positions=[n])
        return float((qm * kn).sum())
    for m, n, s in ((5, 2, 17), (0, 9, 3), (100, 100, -40)):
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-10


def test_rope_first_frequency_turns_one_radian_per_position():
    """inv_freq_0 = 1: the pair (x_0, x_{D/2}) turns by exactly the position (in radians);
    the phase is read back with arctan2."""
    x = np.zeros((1, 6, 8))
    x[..., 0] = 1.0
    y = oracle.rope_neox(x, 10000.0)
    phase = np.unwrap(np.arctan2(y[0, :, 4], y[0, :, 0]))
    np.testing.assert_allclose(phase, np.arange(6), atol=1e-12)
    # the last pair turns at theta^(-2 (D/2-1) / D) radians per position
    x = np.zeros((1, 6, 8))
    x[..., 3] = 1.0
    y = oracle.rope_neox(x, 10000.0)
    phase = np.arctan2(y[0, :, 7], y[0, :, 3])
    np.testing.assert_allclose(phase, np.arange(6) * 10000.0 ** (-6 / 8), atol=1e-12)


def test_rope_matches_the_host_input_generator():
    """The fp32 host RoPE that builds the grouped-query inputs, written separately, agrees
    to fp32 accuracy."""
    rng = np.random.default_rng(34)
    x = rng.normal(size=(2, 64, 32)).astype(np.float32)
    np.testing.assert_allclose(wl.neox_rope(x, 10000.0), oracle.rope_neox(x, 10000.0), atol=2e-5)


# ------------------------------------------------------------- attention on rotated Q and K

@pytest.mark.parametrize("causal", [False, "bottom_right"])
def test_rope_attention_bwd_matches_central_differences(causal):
    """The gradients with respect to the unrotated q and k (positions given, distinct per side)
    against central differences of the composed forward."""
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 3, 5, 4
    rng = np.random.default_rng(35)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, Nq, Nk, D, sigma=1.5)
    do = rng.normal(size=q.shape)
    qp, kp = np.array([7, 2, 40]), np.array([3, 11, 0, 25, 9])
    args = (causal, 0.8, 100.0)
    dq, dk, dv = oracle.ra_attention_rope_bwd(q, k, v, do, *args, q_rope_positions=qp,
                                              k_rope_positions=kp)

    def loss(qq, kk, vv):
        o = oracle.ra_attention_rope_fwd(qq, kk, vv, *args, q_rope_positions=qp, k_rope_positions=kp)[0]
        return float((o * do).sum())

    np.testing.assert_allclose(dq, _fd_grad(lambda z: loss(z, k, v), q), rtol=0, atol=3e-8)
    np.testing.assert_allclose(dk, _fd_grad(lambda z: loss(q, z, v), k), rtol=0, atol=3e-8)
    np.testing.assert_allclose(dv, _fd_grad(lambda z: loss(q, k, z), v), rtol=0, atol=3e-8)


def test_rope_attention_at_position_zero_is_plain_attention():
    rng = np.random.default_rng(36)
    q, k, v = _rand_qkv(rng, 1, 2, 2, 4, 6, 8)
    zq, zk = np.zeros(4, int), np.zeros(6, int)
    o = oracle.ra_attention_rope_fwd(q, k, v, True, 0.5, 10000.0, zq, zk)[0]
    np.testing.assert_array_equal(o, oracle.ra_attention_fwd(q, k, v, True, 0.5)[0])


def test_rope_attention_depends_on_relative_positions_only():
    """The same shift of every query and key position leaves the output unchanged."""
    rng = np.random.default_rng(37)
    q, k, v = _rand_qkv(rng, 1, 2, 1, 5, 5, 8, sigma=2.0)
    base = oracle.ra_attention_rope_fwd(q, k, v, True, 0.6, 500.0)[0]
    shifted = oracle.ra_attention_rope_fwd(q, k, v, True, 0.6, 500.0, np.arange(5) + 1234,
                                           np.arange(5) + 1234)[0]
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-10)


def test_planted_forward_rotation_of_the_gradient_breaks_the_rope_pin():
    # Mapping dQ and dK back with the forward rotation instead of its transpose must fail.
    def no_inverse(orig):
        return lambda x, theta, positions=None, inverse=False: orig(x, theta, positions)
    with _planted("rope_neox", no_inverse):
        with pytest.raises(AssertionError):
            test_rope_attention_bwd_matches_central_differences(False)
    test_rope_attention_bwd_matches_central_differences(False)
