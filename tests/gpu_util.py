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


# Rounding flips.  a, b, y, dH and A' are stored in the activation dtype: the
# GPU rounds an fp32 value, the oracle an fp64 one.  Where the exact value
# lies within the fp32 arithmetic's error of a rounding midpoint, the two
# roundings may differ by one unit in the last place, and a weight gradient
# sums that stored value times a whole row of x (or dO) into its row.  The
# max check may therefore exceed the tolerance by at most the sum of those
# possible one-ulp flips; the mean check takes no allowance.
# fp32 error assumed for a value before it is stored, relative to it: the
# expert GEMMs sum at most a few thousand products in fp32 (about 2^-24 each,
# growing as the square root of the count), so 2^-16 leaves a wide margin
# while marking only about one stored value in a hundred as able to flip.
FLIP_REL = 2.0 ** -16


def storage_ulp(v, dtype):
    """One unit in the last place of the stored values v (bf16: 8 significant bits, fp32: 24)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - (bits - 1)), 0.0)


def flip_ulps(u, stored, dtype, rel=FLIP_REL):
    """One ulp where the unrounded u is within rel*|u| of a rounding midpoint, else 0."""
    u = np.asarray(u, dtype=np.float64)
    s = np.asarray(stored, dtype=np.float64)
    ulp = storage_ulp(s, dtype)
    to_mid = ulp / 2 - np.abs(u - s)
    return np.where(to_mid <= rel * np.abs(u), ulp, 0.0)


def dw_flip_allowance(flips, ids, rows, E, transpose=False, experts=None):
    """[E, h, d] (or [E, d, h] with transpose): sum over the assignments (t, k)
    of expert e of the outer product of flips[t, k] [h] with |rows[t]| [d]
    (only for the listed experts, if given; zero for the others)."""
    T, K, h = flips.shape
    d = rows.shape[1]
    out = np.zeros((E, d, h) if transpose else (E, h, d))
    ar = np.abs(np.asarray(rows, dtype=np.float64))
    for e in range(E) if experts is None else experts:
        t, k = np.nonzero(ids == e)
        if len(t) == 0:
            continue
        f = flips[t, k]
        out[e] = ar[t].T @ f if transpose else f.T @ ar[t]
    return out


def _deriv(f, a, step=1e-4):
    return (f(a + step) - f(a - step)) / (2 * step)


def stored_flip_bounds(fwd, bw, w, dtype, act="swiglu", saved="aby"):
    """How far the stored dA, dB and A' [T,K,h] of the GPU may sit from the
    oracle's under rounding flips: their own one-ulp flips, plus, to first
    order, the flips of the stored a, b (and y) that the backward computes
    them from (dB = dy SiLU(a), dA = dy b SiLU'(a), A' = w y)."""
    from oracle import moe_oracle as O
    a = fwd["a_s"]
    fa = flip_ulps(fwd["a_u"], a, dtype)
    dyv = np.abs(bw["dyv"])
    wk = np.abs(np.asarray(w, dtype=np.float64))[:, :, None]
    if act == "swiglu":
        b = fwd["b_s"]
        fb = flip_ulps(fwd["b_u"], b, dtype)
        g1 = np.abs(O.silu_grad(a))
        da = dyv * (np.abs(b * _deriv(O.silu_grad, a)) * fa + g1 * fb)
        db = dyv * g1 * fa + flip_ulps(bw["dh_b_u"], bw["dh_b"], dtype)
        y_from_h = np.abs(g1 * b) * fa + np.abs(O.silu(a)) * fb
    else:
        f, fd = O.ACTS[act]
        # a flip never changes the sign of a, so relu' does not move
        da = dyv * (np.abs(_deriv(fd, a)) * fa if act != "relu" else 0.0)
        db = None
        y_from_h = np.abs(fd(a)) * fa
    da = da + flip_ulps(bw["dh_a_u"], bw["dh_a"], dtype)
    fy = flip_ulps(fwd["y_u"], fwd["y_s"], dtype) if saved == "aby" else y_from_h
    ap = wk * fy + flip_ulps(bw["a_prime_u"], O.storage_rounder(dtype)(bw["a_prime_u"]), dtype)
    return dict(da=da, db=db, ap=ap)


def assert_close(name, g, r, max_tol=MAX_REL, mean_tol=MEAN_REL, report=None, allow=None):
    """allow: per-element absolute error granted to the max check only (rounding flips)."""
    if allow is not None:
        g64 = np.asarray(g, dtype=np.float64)
        r64 = np.asarray(r, dtype=np.float64)
        diff = np.abs(g64 - r64)
        shrink = np.minimum(diff, np.asarray(allow, dtype=np.float64))
        mx, _ = rel_errors(g64 - np.sign(g64 - r64) * shrink, r64)
        _, mn = rel_errors(g64, r64)
    else:
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
