"""Shared helpers of the GPU parity tests: device transfer, tolerances, band checks."""
import numpy as np

FLT_MIN = np.float32(np.finfo(np.float32).tiny)
ULP16 = 2.0 ** -19          # one fp32 ulp of 16
U32 = 2.0 ** -24            # fp32 unit roundoff


def to_dev(a, dtype: str):
    """float32 numpy array holding exact dtype values -> contiguous device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_to_max(gpu, ref):
    den = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (den if den > 0 else 1.0))


def assert_close(gpu, ref, dtype: str, what: str = "", grad=False, fp32_tol=1e-5, bf16_tol=2e-2):
    """fp32: max-abs error <= 1e-5, absolute for outputs (O, p, rotated inputs); for gradients
    (grad=True) relative to max|ref| when that exceeds 1, since the pages fix no gradient
    tolerance and gradient magnitudes grow with the problem.
    bf16: max|gpu - ref| / max|ref| <= 2e-2 (outputs and gradients)."""
    err_abs = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
    if dtype == "f32":
        scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0) if grad else 1.0
        assert err_abs <= fp32_tol * scale, f"{what}: max abs err {err_abs:.3e}"
    else:
        r = rel_to_max(gpu, ref) if gpu.size else 0.0
        assert r <= bf16_tol, f"{what}: rel-to-max err {r:.3e}"
    return err_abs


def score_error_bound(q, k, scale):
    """Bound on |fp32 score - exact score| per (i, j): gamma_D * scale * sum_d |q_d k_d|."""
    D = q.shape[-1]
    gamma = D * U32 / (1 - D * U32)
    return gamma * scale * (np.abs(q) @ np.abs(k).T)


def zero_pattern_mismatches(p_gpu, p_ora, delta_ora, band):
    """Entries where the GPU zero set and the oracle's differ, outside the allowed band:
    |Delta_oracle - 16| <= band (score and rounding error) or p_oracle below FLT_MIN
    (phi underflows in fp32 there)."""
    z_gpu = p_gpu == 0
    z_ora = p_ora == 0
    mism = z_gpu != z_ora
    allowed = (np.abs(delta_ora - 16.0) <= band) | (p_ora < 1.01 * FLT_MIN)
    bad = mism & ~allowed
    return int(bad.sum()), int(mism.sum())
