"""Helpers for the GPU parity tests: run the layer through the C-ABI and
compare with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np

# Float tolerances for bf16 storage with fp32 accumulation:
#   max_rel  = max_i |g_i - r_i| / max(|r_i|, rms(r))  <= 2e-2
#   mean_rel = sum |g - r| / sum |r|                      <= 2e-3
MAX_REL = 2e-2
MEAN_REL = 2e-3


def rel_errors(g, r):
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    r = np.asarray(r, dtype=np.float64).reshape(-1)
    if r.size == 0:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        err = float(np.abs(g).max())
        return err, err
    diff = np.abs(g - r)
    max_rel = float((diff / np.maximum(np.abs(r), rms)).max())
    mean_rel = float(diff.sum() / max(np.abs(r).sum(), 1e-300))
    return max_rel, mean_rel


def assert_close(name, g, r, max_tol=MAX_REL, mean_tol=MEAN_REL, report=None):
    mx, mn = rel_errors(g, r)
    if report is not None:
        report[name] = (mx, mn)
    assert np.all(np.isfinite(np.asarray(g, dtype=np.float64))), f"{name}: non-finite values"
    assert mx <= max_tol and mn <= mean_tol, f"{name}: max_rel={mx:.3e} (tol {max_tol}) mean_rel={mn:.3e} (tol {mean_tol})"


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def topk_margin(z32, K):
    """Per token: gap between the K-th and (K+1)-th largest logit (inf if K == E)."""
    s = -np.sort(-np.asarray(z32, dtype=np.float64), axis=1)
    if K >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, K - 1] - s[:, K]
