"""Plain fp64 CPU oracle for rational-softmax attention.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports it, and this module
imports nothing from the product path.

Everything here follows the definitions on the pages in their own order, in
float64, with the full score matrix materialised one (batch, head) at a time.
There is no tiling, fusion or reordering beyond what a definition states.

Sources
-------
* "Ra-Family: Rational Neural Architecture" (luminamoon.nn README), section 3
  "Rational Attention & Softmax", item ra_softmax: the shift Delta = x_max - x,
  u = Delta/16, q = (1-u)/(1+u), phi = q**8 for Delta < 16 and exactly 0 for
  Delta >= 16, and the denominator sum(phi) >= 1.  The same item gives the
  closed-form derivative d(phi)/du = -16 phi / (1-u^2) for u < 1 (the page's
  typeset formula lost its thin spaces; it is a product).
* Same page, section 3, item ra_attention: (Q, K, V) -> O without the
  [B, H, Nq, Nk] matrix; the functional form is a drop-in for
  scaled_dot_product_attention with is_causal.
* "nn -- neural-network layers on the grad tape", section "Layers",
  nn_gqa_attention: the unfused order scaled scores -> masked softmax ->
  weighted sum, which this oracle follows with ra_softmax in place of softmax.
* noeira "Primitives" page, section "Attention and transformers":
  RepeatKVHeads maps query head h to K/V head h // REP and its backward sums
  the REP copies; a fully masked row gives a zero context, not NaN.

Readings where the pages are silent (each is listed in the design notes):
* p = phi / sum(phi) is the normalisation of the "denominator" the page names.
* The row max is part of the function: the backward differentiates through it
  (term R below).  For the exp softmax that term vanishes; for phi it does not.
* Ties for the row max resolve to the lowest key index.
* Causal masking is top-left aligned by default (key j allowed for query i iff
  j <= i), as scaled_dot_product_attention's is_causal.  The pages do not say
  how the diagonal sits when Nq != Nk; the bottom-right alignment (query i
  takes keys j <= i + Nk - Nq, so the last query sees every key, the layout of
  queries that continue a key sequence) is offered as a second mode.
* An explicit mask follows scaled_dot_product_attention's attn_mask, for which
  ra_attention is the drop-in: a boolean mask takes part where it is True, a
  floating mask is added to the scaled scores before the row max.  The
  CrossAttention key padding mask of the "Primitives" page (1 = attend) is the
  boolean case broadcast over heads and query rows.  The mask is a constant:
  no gradient flows to it.
* Masked entries (-inf logits, or keys outside the causal set) are excluded
  from the max and from sum(phi), and get p = 0.  A row with no allowed entry
  gives p = 0 and O = 0 (the "Primitives" page, CrossAttention: a fully masked
  row produces a zero context, not NaN), and zero gradients.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SUPPORT_WIDTH",
    "causal_offset",
    "ra_phi",
    "ra_softmax_rows",
    "ra_softmax_rows_bwd",
    "ra_attention_fwd",
    "ra_attention_bwd",
    "ra_attention_decode",
    "ra_attention_rope_fwd",
    "ra_attention_rope_bwd",
    "rope_neox",
]

# Delta at which phi reaches exactly zero (the compact support edge, u = 1).
SUPPORT_WIDTH = 16.0


def ra_phi(delta):
    """phi(Delta) = ((1-u)/(1+u))**8 with u = Delta/16 for Delta < 16, else 0.

    Ra-Family page, section 3, ra_softmax.  ``delta`` must be >= 0 or +inf
    (+inf marks a masked entry and gives 0).
    """
    delta = np.asarray(delta, dtype=np.float64)
    u = delta / SUPPORT_WIDTH
    inside = u < 1.0
    u_in = np.where(inside, u, 0.0)
    q = (1.0 - u_in) / (1.0 + u_in)
    return np.where(inside, q ** 8, 0.0)


def _row_stats(x, allowed):
    """Row max over allowed entries, its lowest index, Delta and phi.

    Returns (m, a, delta, phi); rows with no allowed entry have m = -inf,
    a = -1, delta = +inf and phi = 0.
    """
    xm = np.where(allowed, x, -np.inf)
    m = xm.max(axis=-1)
    a = np.argmax(xm, axis=-1)  # numpy returns the first maximal index
    empty = ~allowed.any(axis=-1)
    a = np.where(empty, -1, a)
    with np.errstate(invalid="ignore"):
        delta = np.where(allowed, m[..., None] - x, np.inf)
    delta = np.where(empty[..., None], np.inf, delta)
    phi = ra_phi(delta)
    return m, a, delta, phi


def ra_softmax_rows(x, return_stats=False):
    """ra_softmax along the last axis of a 2-D array; -inf entries are masked.

    Ra-Family page, section 3, ra_softmax; p = phi / sum(phi).
    With ``return_stats`` also returns (phi, m, l) where l = sum(phi).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("ra_softmax_rows expects a 2-D array")
    allowed = ~np.isneginf(x)
    m, _, _, phi = _row_stats(x, allowed)
    l = phi.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[..., None] > 0, phi / l[..., None], 0.0)
    if return_stats:
        return p, phi, m, l
    return p


def _softmax_vjp(p, delta, dp, a):
    """Gradient of L through p = ra_softmax(s) for one block of rows.

    With c_i = sum_j p_ij dp_ij, the direct term is
    G_ij = p_ij (dp_ij - c_i) / (1 - u_ij^2) on the support (u < 1), else 0,
    which is the chain rule through phi with the page's closed form
    d(phi)/du = -16 phi/(1-u^2) and du/dDelta = 1/16, Delta = m - s.
    The row max m = s[a] carries R_i = -sum_j G_ij, added at the argmax.
    """
    u = delta / SUPPORT_WIDTH
    support = u < 1.0
    c = (p * dp).sum(axis=-1)
    u_in = np.where(support, u, 0.0)
    g = np.where(support, p * (dp - c[..., None]) / (1.0 - u_in * u_in), 0.0)
    r = -g.sum(axis=-1)
    ds = g.copy()
    rows = np.nonzero(a >= 0)[0]
    ds[rows, a[rows]] += r[rows]
    return ds


def ra_softmax_rows_bwd(x, dp):
    """Exact gradient dL/dx of ra_softmax_rows given dL/dp, max path included."""
    x = np.asarray(x, dtype=np.float64)
    dp = np.asarray(dp, dtype=np.float64)
    allowed = ~np.isneginf(x)
    m, a, delta, phi = _row_stats(x, allowed)
    l = phi.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[..., None] > 0, phi / l[..., None], 0.0)
    return _softmax_vjp(p, delta, dp, a)


def ra_attention_decode(q, k, v, scale, seqlens=None, causal=False):
    """Attention of a few query rows per head against a key/value cache.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D] hold the caches, of which sample b uses its first
    ``seqlens[b]`` keys (default all Nk).  ``causal``: False; True / "top_left" (query i takes
    keys j <= i); "bottom_right" (query i sits at position seqlens[b] - Nq + i of the sample's
    sequence and takes keys j <= seqlens[b] - Nq + i).  By definition this is ra_attention_fwd
    of each sample on its own cache prefix, so the bottom-right offset is seqlens[b] - Nq.
    Returns (O, m, l, a) as ra_attention_fwd.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, D, rep = _check_attention_shapes(q, k, v)
    lens = np.full(B, Nk, dtype=np.int64) if seqlens is None else np.asarray(seqlens, np.int64)
    if lens.shape != (B,) or (lens < 0).any() or (lens > Nk).any():
        raise ValueError("seqlens must hold B lengths in [0, Nk]")
    o = np.zeros((B, Hq, Nq, v.shape[3]))
    m = np.full((B, Hq, Nq), -np.inf)
    l = np.zeros((B, Hq, Nq))
    a = np.full((B, Hq, Nq), -1, dtype=np.int64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        ob, mb, lb, ab = ra_attention_fwd(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                                          causal, scale)
        o[b], m[b], l[b], a[b] = ob[0], mb[0], lb[0], ab[0]
    return o, m, l, a


def rope_neox(x, theta, positions=None, inverse=False):
    """Split-halves (NEOX) rotary position embedding along the last axis, positions on axis -2.

    "Primitives" page, section "Attention and transformers" (RoPE[SEQ, N_HEADS, HEAD_DIM,
    THETA]: channel j is paired with channel j + HEAD_DIM/2) and the nurl page, section
    "Layers" (nn_rope, NEOX half-split rotary).  The pages name the pairing and theta but not
    the frequency schedule; the reading used here is inv_freq_j = theta^(-2j/D), j < D/2, with
    angle = position * inv_freq_j, rotating each pair (x_j, x_{j+D/2}) counter-clockwise.
    ``positions`` defaults to 0..N-1; ``inverse`` rotates by the negative angle (the transpose,
    which maps output gradients to input gradients).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    N = x.shape[-2]
    if D % 2:
        raise ValueError("head dim must be even")
    half = D // 2
    pos = np.arange(N, dtype=np.float64) if positions is None else np.asarray(positions, np.float64)
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = pos[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    if inverse:
        sin = -sin
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def _check_attention_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D or v.shape[:3] != k.shape[:3]:
        raise ValueError("inconsistent q/k/v shapes")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, D, Hq // Hkv


CAUSAL_MODES = {False: None, 0: None, None: None, True: "top_left", 1: "top_left",
                "top_left": "top_left", 2: "bottom_right", "bottom_right": "bottom_right"}


def causal_offset(causal, Nq, Nk):
    """Diagonal offset of the causal set (key j allowed for query i iff j <= i + offset), or
    None without causal masking.  Top-left: 0; bottom-right: Nk - Nq."""
    if causal not in CAUSAL_MODES:
        raise ValueError(f"unknown causal mode {causal!r}")
    mode = CAUSAL_MODES[causal]
    if mode is None:
        return None
    return 0 if mode == "top_left" else Nk - Nq


def _allowed(Nq, Nk, causal, q_positions, nq_total=None):
    pos = np.arange(Nq) if q_positions is None else np.asarray(q_positions)
    off = causal_offset(causal, Nq if nq_total is None else nq_total, Nk)
    if off is None:
        return np.ones((len(pos), Nk), dtype=bool)
    return np.arange(Nk)[None, :] <= pos[:, None] + off


def _scores(qh, kg, scale, allowed, mask, b, h, shape):
    """Scaled scores of one (batch, head) and the entries that take part: the causal set, the
    True entries of a boolean mask, or the additive mask added to the scaled scores (its -inf
    entries drop out)."""
    s = scale * (qh @ kg.T)
    if mask is None:
        return s, allowed
    mb = np.broadcast_to(mask, shape)[b, h]
    if mb.dtype == np.bool_:
        return s, allowed & mb
    s = s + mb.astype(np.float64)
    return s, allowed & ~np.isneginf(s)


def ra_attention_fwd(q, k, v, causal, scale, q_positions=None, heads=None, mask=None,
                     nq_total=None):
    """O = ra_softmax(scale * Q K^T + mask) V with GQA and optional causal mask.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D]; query head h reads K/V head
    h // (Hq/Hkv).  ``causal``: False, True / "top_left" or "bottom_right".
    ``mask``: None, or an array broadcastable to [B, Hq, Nq, Nk]: boolean
    (True = attend) or floating (added to the scaled scores; -inf = masked).
    ``q_positions`` gives the absolute positions of the supplied query rows for
    the causal test (default 0..Nq-1) and ``nq_total`` the full query length
    (default Nq, used by the bottom-right offset), so a sample of rows can be
    checked on its own; a mask then covers the supplied rows only.  ``heads``
    restricts the work to a list of (b, h) pairs (other heads of the outputs
    stay zero / -inf).

    Returns (O, m, l, a): m is the row max of the scaled scores s, l the sum of
    phi, a the lowest key index attaining the max (-1 for an empty row).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, D, rep = _check_attention_shapes(q, k, v)
    allowed = _allowed(Nq, Nk, causal, q_positions, nq_total)
    mask = None if mask is None else np.asarray(mask)
    o = np.zeros((B, Hq, Nq, v.shape[3]))
    m = np.full((B, Hq, Nq), -np.inf)
    l = np.zeros((B, Hq, Nq))
    a = np.full((B, Hq, Nq), -1, dtype=np.int64)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    for b, h in todo:
        g = h // rep
        s, allowed_bh = _scores(q[b, h], k[b, g], scale, allowed, mask, b, h, (B, Hq, Nq, Nk))
        mb, ab, _, phi = _row_stats(s, allowed_bh)
        lb = phi.sum(axis=-1)
        with np.errstate(invalid="ignore", divide="ignore"):
            p = np.where(lb[:, None] > 0, phi / lb[:, None], 0.0)
        o[b, h] = p @ v[b, g]
        m[b, h], l[b, h], a[b, h] = mb, lb, ab
    return o, m, l, a


def ra_attention_bwd(q, k, v, do, causal, scale, groups=None, mask=None, argmax=None):
    """Gradients (dQ, dK, dV) of L = sum(O * dO) for ra_attention_fwd.

    Follows the chain rule in the forward's order: dP = dO V^T; the softmax
    vector-Jacobian product (direct closed-form term plus the row-max term);
    dQ = scale dS K; dK and dV are summed over the REP query heads that share
    a K/V head.  ``groups`` restricts the work to a list of (b, g) K/V groups
    (all their query heads are processed).  ``causal`` and ``mask`` as in
    ra_attention_fwd (the mask gets no gradient).

    ``argmax``: optional int array [B, Hq, Nq]; where an entry is >= 0 the
    row-max term R_i goes to that key instead of the lowest key attaining the
    max.  The function is not differentiable where two scores tie for the
    max; a parity check whose scores carry rounding error uses this to take
    the gradient on the side of the other near-tied candidate.  Delta is
    still measured from the true row max.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, D, rep = _check_attention_shapes(q, k, v)
    if do.shape != q.shape[:3] + v.shape[3:]:
        raise ValueError("dO must have the shape of O")
    allowed = _allowed(Nq, Nk, causal, None)
    mask = None if mask is None else np.asarray(mask)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else groups
    for b, g in todo:
        for h in range(g * rep, (g + 1) * rep):
            s, allowed_bh = _scores(q[b, h], k[b, g], scale, allowed, mask, b, h, (B, Hq, Nq, Nk))
            _, a, delta, phi = _row_stats(s, allowed_bh)
            if argmax is not None:
                a = np.where(argmax[b, h] >= 0, argmax[b, h], a)
            lb = phi.sum(axis=-1)
            with np.errstate(invalid="ignore", divide="ignore"):
                p = np.where(lb[:, None] > 0, phi / lb[:, None], 0.0)
            dp = do[b, h] @ v[b, g].T
            ds = _softmax_vjp(p, delta, dp, a)
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
            dv[b, g] += p.T @ do[b, h]
    return dq, dk, dv


def ra_attention_rope_fwd(q, k, v, causal, scale, theta, q_rope_positions=None,
                          k_rope_positions=None, mask=None):
    """Attention on rotated queries and keys: O = ra_attention(rope(Q), rope(K), V).

    The nurl page, section "Layers", applies nn_rope to the queries and keys of
    a head before the attention core; the "Primitives" page, section "Attention
    and transformers", gives the split-halves pairing.  The rotation positions
    (default 0..N-1) are independent of the causal test, which uses row and key
    indices as in ra_attention_fwd, and so does ``mask`` (as in ra_attention_fwd).  Returns
    (O, m, l, a) as ra_attention_fwd.
    """
    qr = rope_neox(q, theta, q_rope_positions)
    kr = rope_neox(k, theta, k_rope_positions)
    return ra_attention_fwd(qr, kr, v, causal, scale, mask=mask)


def ra_attention_rope_bwd(q, k, v, do, causal, scale, theta, q_rope_positions=None,
                          k_rope_positions=None, groups=None, argmax=None, mask=None):
    """Gradients (dQ, dK, dV) of L = sum(O * dO) for ra_attention_rope_fwd, with respect to the
    UNROTATED q and k: the attention gradients of the rotated inputs, each mapped back by the
    transpose of its rotation (the rotation by the negative angle).  ``groups``, ``argmax`` and
    ``mask`` as in ra_attention_bwd."""
    qr = rope_neox(q, theta, q_rope_positions)
    kr = rope_neox(k, theta, k_rope_positions)
    dqr, dkr, dv = ra_attention_bwd(qr, kr, v, do, causal, scale, groups=groups, argmax=argmax,
                                    mask=mask)
    return (rope_neox(dqr, theta, q_rope_positions, inverse=True),
            rope_neox(dkr, theta, k_rope_positions, inverse=True), dv)
