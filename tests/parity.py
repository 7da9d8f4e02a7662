"""Parity of whole full-size launches against the oracle: every (batch, head) of a forward and
every (batch, K/V head) group of a backward, element by element.

The oracle runs one head (forward) or one group (backward) at a time on host threads: heads are
independent, NumPy releases the GIL inside its matrix products and element-wise loops, and BLAS
is held to one thread per worker.

Tolerances (per output tensor, over the whole launch): bf16 max|gpu - oracle| / max|oracle|
<= 2e-2; fp32 max-abs 1e-5 (gradients: relative to max|oracle| when that exceeds 1).

Near ties of the row max (the reading of argmax ties): the backward puts the row-max term R_i at
the lowest key attaining the max.  Where the oracle's best score and another allowed score of a
row differ by less than the sum of their fp32 score error bounds, the GPU's fp32 scores may order
them the other way.  For such rows the checker accepts the gradient of either candidate: it
infers the GPU's choice per row from dQ (row-local) and compares every tensor with the oracle
run with that choice (the oracle's ``argmax`` override).  Two keys with bit-identical rows tie
exactly in both precisions, so the lowest index is required there.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import oracle
from helpers import U32

BF16_TOL = 2e-2
F32_TOL = 1e-5


def n_workers() -> int:
    """Host threads for the oracle: the cores granted to one GPU (16), or fewer if absent."""
    return max(1, min(16, os.cpu_count() or 1))


def _pool_map(fn, items):
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(1)
    except Exception:          # pragma: no cover
        limit = None
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=n_workers()) as ex:
            return list(ex.map(fn, items))
    finally:
        if limit is not None:
            limit.restore_original_limits()


class Tally:
    """Largest absolute error and largest |oracle| of one output tensor over many pieces."""

    def __init__(self, name, dtype, grad):
        self.name, self.dtype, self.grad = name, dtype, grad
        self.err = 0.0
        self.ref = 0.0
        self.where = None

    def add(self, gpu, ref, where):
        if gpu.size == 0:
            return
        e = float(np.abs(gpu - ref).max())
        if e > self.err:
            self.err, self.where = e, where
        self.ref = max(self.ref, float(np.abs(ref).max()))

    def check(self):
        if self.dtype == "bf16":
            r = self.err / (self.ref if self.ref > 0 else 1.0)
            assert r <= BF16_TOL, f"{self.name}: rel-to-max err {r:.3e} (worst at {self.where})"
            return r
        lim = F32_TOL * (max(1.0, self.ref) if self.grad else 1.0)
        assert self.err <= lim, f"{self.name}: max abs err {self.err:.3e} (worst at {self.where})"
        return self.err


def fwd_all_heads(o, stats, inp, causal, scale, dtype, heads=None):
    """Compare o [B, Hq, Nq, D] and stats [B, Hq, Nq, 2] (raw m, l) with the oracle on every
    (b, h) (or the given list).  Returns {name: error} (rel-to-max for bf16, abs for fp32)."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, Nq, D = q.shape
    rep = Hq // k.shape[1]
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)

    def one(bh):
        b, h = bh
        g = h // rep
        ro, rm, rl, _ = oracle.ra_attention_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1],
                                                v[b:b + 1, g:g + 1], causal, scale)
        eo = float(np.abs(o[b, h] - ro[0, 0]).max())
        mo = float(np.abs(ro[0, 0]).max())
        # m: the GPU stores the raw dot-product max, the oracle the scaled one
        gm, gl = stats[b, h, :, 0] * scale, stats[b, h, :, 1]
        fin = np.isfinite(rm[0, 0])
        assert (np.isfinite(gm) == fin).all(), f"m finiteness at {bh}"
        em = float(np.max(np.abs(gm[fin] - rm[0, 0][fin]) - 1e-5 * np.abs(rm[0, 0][fin]), initial=0.0))
        el = float(np.max(np.abs(gl - rl[0, 0]) / np.maximum(np.abs(rl[0, 0]), 1e-30), initial=0.0))
        return bh, eo, mo, em, el

    t = Tally("o", dtype, grad=False)
    em_max = el_max = 0.0
    for bh, eo, mo, em, el in _pool_map(one, todo):
        if eo > t.err:
            t.err, t.where = eo, bh
        t.ref = max(t.ref, mo)
        em_max, el_max = max(em_max, em), max(el_max, el)
    err = t.check()
    assert em_max <= 1e-4, f"row max m off by {em_max:.3e} beyond rtol 1e-5"
    assert el_max <= (1e-5 if dtype == "f32" else 1e-2), f"sum of phi rel err {el_max:.3e}"
    return {"o": err, "m": em_max, "l": el_max, "heads": len(todo)}


def fwd_rope_all_heads(o, stats, inp, causal, scale, theta, q_positions=None, k_positions=None,
                       heads=None, dtype="bf16"):
    """fwd_all_heads for attention on rotated rows: inp holds the UNROTATED q and k.  O is
    compared with the exact function (ra_attention_rope_fwd).  The GPU scores the rotated rows
    in the dtype, so m and l are held to bounds derived from rope_score_bound per row:
    |m~ - m| <= t_i = max_j b_ij over the allowed keys, and, with |delta Delta_ij| <= b_ij + t_i
    and |phi'| <= phi^(7/8) (phi decreasing in Delta),
    |l~ - l| <= sum_j (b_ij + t_i) phi(max(Delta_ij - b_ij - t_i, 0))^(7/8); each plus the fp32
    margins of fwd_all_heads."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    rep = Hq // k.shape[1]
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    off = oracle.causal_offset(causal, Nq, Nk)
    allowed = np.ones((Nq, Nk), bool) if off is None else \
        np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + off

    def one(bh):
        b, h = bh
        g = h // rep
        ro, rm, rl, _ = oracle.ra_attention_rope_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1],
                                                     v[b:b + 1, g:g + 1], causal, scale, theta,
                                                     q_positions, k_positions)
        qh = oracle.rope_neox(q[b, h].astype(np.float64), theta, q_positions)
        kg = oracle.rope_neox(k[b, g].astype(np.float64), theta, k_positions)
        bnd = np.where(allowed, rope_score_bound(qh, kg, scale, dtype), 0.0)
        t = bnd.max(axis=1)
        s = scale * (qh @ kg.T)
        m0 = rm[0, 0]
        fin = np.isfinite(m0)
        delta = np.where(allowed & fin[:, None], m0[:, None] - s, np.inf)
        w = bnd + t[:, None]
        lb = (w * oracle.ra_phi(np.maximum(delta - w, 0.0)) ** 0.875).sum(axis=1)
        gm, gl = stats[b, h, :, 0] * scale, stats[b, h, :, 1]
        assert (np.isfinite(gm) == fin).all(), f"m finiteness at {bh}"
        em = np.abs(gm[fin] - m0[fin]) - t[fin] - 1e-5 * np.abs(m0[fin])
        el = np.abs(gl - rl[0, 0]) - lb - 1e-5 * np.abs(rl[0, 0])
        return (bh, float(np.abs(o[b, h] - ro[0, 0]).max()), float(np.abs(ro[0, 0]).max()),
                float(np.max(em, initial=-np.inf)), float(np.max(el, initial=-np.inf)),
                float(t.max(initial=0.0)))

    tal = Tally("o", dtype, grad=False)
    em_max = el_max = -np.inf
    t_max = 0.0
    for bh, eo, mo, em, el, tm in _pool_map(one, todo):
        if eo > tal.err:
            tal.err, tal.where = eo, bh
        tal.ref = max(tal.ref, mo)
        em_max, el_max, t_max = max(em_max, em), max(el_max, el), max(t_max, tm)
    err = tal.check()
    assert em_max <= 1e-4, f"row max m beyond its rounding bound by {em_max:.3e}"
    assert el_max <= 0.0, f"sum of phi beyond its rounding bound by {el_max:.3e}"
    return {"o": err, "m_excess": em_max, "l_excess": el_max, "score_bound": t_max,
            "heads": len(todo)}


def score_error_bound(qh, kg, scale):
    """|fp32 score - exact score| <= gamma_D * scale * sum_d |q_d k_d| per (i, j)."""
    D = qh.shape[-1]
    gamma = D * U32 / (1 - D * U32)
    return gamma * scale * (np.abs(qh) @ np.abs(kg).T)


def rope_score_bound(qh, kg, scale, dtype="bf16"):
    """|GPU score - exact score| per (i, j) when the GPU multiplies rotated rows (qh, kg: the
    exactly rotated rows of one head).  Each rotated element is the fp32 rotation, within
    2^-20 times its pair's norm n, then rounded to the dtype (bf16: relative 2^-8; fp32: 2^-24),
    so |delta q_d| <= E_d = e |q_d| + 1.004 * 2^-20 n_d.  Then |q~.k~ - q.k| <= E_q.|k| + |q|.E_k
    + E_q.E_k, plus the fp32 dot product of the rotated rows, gamma_D (|q| + E_q).(|k| + E_k)."""
    D = qh.shape[-1]
    e = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    gamma = D * U32 / (1 - D * U32)

    def err(x):
        h = D // 2
        n = np.sqrt(x[:, :h] ** 2 + x[:, h:] ** 2)
        return e * np.abs(x) + 1.004 * 2.0 ** -20 * np.concatenate([n, n], axis=1)
    eq, ek = err(qh), err(kg)
    aq, ak = np.abs(qh), np.abs(kg)
    return scale * (eq @ ak.T + aq @ ek.T + eq @ ek.T + gamma * ((aq + eq) @ (ak + ek).T))


def near_tie_candidates(qh, kg, scale, causal, Nq, Nk, es=None):
    """Per row of one head: the other keys whose score may order before the oracle's argmax in
    fp32, as a dict row -> [keys] (keys with bit-identical rows to the argmax excluded).  ``es``:
    the per-entry score error bound (default: fp32 scoring of the given rows)."""
    s = scale * (qh @ kg.T)
    off = oracle.causal_offset(causal, Nq, Nk)
    allowed = np.ones((Nq, Nk), bool) if off is None else \
        np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + off
    xm = np.where(allowed, s, -np.inf)
    a = np.argmax(xm, axis=1)
    m = xm[np.arange(Nq), a]
    if es is None:
        es = score_error_bound(qh, kg, scale)
    near = allowed & (m[:, None] - s <= es + es[np.arange(Nq), a][:, None])
    near[np.arange(Nq), a] = False
    out = {}
    for i in np.nonzero(near.any(axis=1) & np.isfinite(m))[0]:
        cands = [int(j) for j in np.nonzero(near[i])[0] if not np.array_equal(kg[j], kg[a[i]])]
        if cands:
            out[int(i)] = (int(a[i]), cands)
    return out


def bwd_all_groups(dq, dk, dv, inp, causal, scale, dtype, groups=None, rope=None):
    """Compare dq [B, Hq, Nq, D], dk, dv [B, Hkv, Nk, D] with the oracle on every (b, g) group
    (or the given list), accepting either candidate at near ties of the row max.  ``rope``:
    None, or {"theta", "q_positions", "k_positions"}: q and k are unrotated, the oracle is
    ra_attention_rope_bwd and near ties are taken within rope_score_bound.  Returns
    {name: error, "near_tie_rows": n, "flipped_rows": n}."""
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    rep = Hq // Hkv
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else list(groups)

    def bwd(*args, argmax=None):
        if rope is None:
            return oracle.ra_attention_bwd(*args, argmax=argmax)
        return oracle.ra_attention_rope_bwd(*args, rope["theta"], rope["q_positions"],
                                            rope["k_positions"], argmax=argmax)

    def one(bg):
        b, g = bg
        hs = slice(g * rep, (g + 1) * rep)
        args = (q[b:b + 1, hs], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], do[b:b + 1, hs], causal, scale)
        kg = k[b, g].astype(np.float64)
        qg = [q[b, g * rep + r].astype(np.float64) for r in range(rep)]
        if rope is not None:
            kg = oracle.rope_neox(kg, rope["theta"], rope["k_positions"])
            qg = [oracle.rope_neox(x, rope["theta"], rope["q_positions"]) for x in qg]
        ties = {}
        for r in range(rep):
            es = None if rope is None else rope_score_bound(qg[r], kg, scale, dtype)
            ties[r] = near_tie_candidates(qg[r], kg, scale, causal, Nq, Nk, es)
        ref = bwd(*args)
        n_tie = sum(len(t) for t in ties.values())
        n_flip = 0
        if n_tie:
            # the GPU's choice per near-tie row, from dQ: the default or one of the alternatives
            choice = np.full((1, rep, Nq), -1)
            best = {(r, i): (np.abs(dq[b, g * rep + r, i] - ref[0][0, r, i]).max(), -1)
                    for r, t in ties.items() for i in t}
            depth = max(len(c) for t in ties.values() for _, c in t.values())
            for n in range(depth):
                over = np.full((1, rep, Nq), -1)
                for r, t in ties.items():
                    for i, (_, c) in t.items():
                        if n < len(c):
                            over[0, r, i] = c[n]
                alt = bwd(*args, argmax=over)
                for (r, i), (e, _) in list(best.items()):
                    if over[0, r, i] >= 0:
                        e2 = np.abs(dq[b, g * rep + r, i] - alt[0][0, r, i]).max()
                        if e2 < e:
                            best[(r, i)] = (e2, int(over[0, r, i]))
            for (r, i), (_, j) in best.items():
                choice[0, r, i] = j
            n_flip = int((choice >= 0).sum())
            if n_flip:
                ref = bwd(*args, argmax=choice)
        out = []
        for name, gpu, r in (("dq", dq[b, hs], ref[0][0]), ("dk", dk[b, g], ref[1][0, 0]),
                             ("dv", dv[b, g], ref[2][0, 0])):
            out.append((name, float(np.abs(gpu - r).max()), float(np.abs(r).max())))
        return bg, out, n_tie, n_flip

    tallies = {n: Tally(n, dtype, grad=True) for n in ("dq", "dk", "dv")}
    n_tie = n_flip = 0
    for bg, out, nt, nf in _pool_map(one, todo):
        n_tie += nt
        n_flip += nf
        for name, e, m in out:
            t = tallies[name]
            if e > t.err:
                t.err, t.where = e, bg
            t.ref = max(t.ref, m)
    res = {n: t.check() for n, t in tallies.items()}
    res.update(near_tie_rows=n_tie, flipped_rows=n_flip, groups=len(todo))
    return res
