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


# ---------------------------------------------------------------------------
# Rounding flips.  a, b, y, dH and A' are stored in the activation dtype: the
# GPU rounds an fp32 value, the oracle an fp64 one (exact for these inputs to
# far below the fp32 error).  Where the exact value lies closer to a rounding
# midpoint than the GPU's fp32 value lies to the exact one, the two roundings
# may differ by one unit in the last place; a weight gradient then sums that
# stored value times a whole row of x (or dO) into one of its rows.  The max
# check of a weight gradient may therefore exceed the tolerance by at most the
# sum of those possible one-ulp flips; the mean check takes no allowance.
#
# How far the GPU's fp32 value can sit from the exact one (the window):
#  * A dot product of n terms t_j accumulated in fp32 (the expert GEMMs: bf16
#    products are exact in fp32, the MFMA sums them in blocks and adds the
#    blocks to an fp32 accumulator) has first-order error sum_k delta_k s_k,
#    |delta_k| <= u = 2^-24, over the additions k with partial sums s_k.
#    With the delta_k mean-independent (the model of Higham and Mary's
#    probabilistic rounding-error analysis) Azuma's inequality bounds it by
#    LAMBDA * u * sqrt(sum_k s_k^2) except with probability 2 exp(-LAMBDA^2/2)
#    (3e-8 at LAMBDA = 6).  The terms here are products of independent
#    zero-mean inputs, so the partial sums are a random walk whose
#    sum_k s_k^2 is about n/2 * ||t||^2; the window takes n * ||t||^2:
#        window = LAMBDA * u * sqrt(n) * ||t||_2,   per output element,
#    computed from the same inputs as sqrt((rows^2) @ (W^2)^T).
#    test_tolerance_helpers.py checks it against emulated fp32 accumulation
#    (sequential, and in 16-product blocks) at n = 128 .. 14336: the largest
#    error seen is under a quarter of the window.
#  * Pointwise epilogue math (sigmoid through expf and a division, a few
#    products) adds at most POINTWISE_U units of u relative to the value.
#  * A value computed from a GEMM result carries that result's window times
#    the magnitude of its derivative with respect to it.
# At d = 6144 the window marks about 1.5% of stored values as able to flip.
# ---------------------------------------------------------------------------
U32 = 2.0 ** -24
LAMBDA = 6.0
POINTWISE_U = 16.0


def dot_window(rows, W):
    """fp32 error window of rows @ W^T: LAMBDA * u * sqrt(n) * ||rows_i * W_j||_2, [N, M]."""
    rows = np.asarray(rows, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    n = rows.shape[1]
    return LAMBDA * U32 * np.sqrt(n) * np.sqrt(np.square(rows) @ np.square(W).T)


def fp32_windows(x, dy, ids, w_gate, w_up, w_down, act="swiglu", only_experts=None, backward=True):
    """[T, K, h] windows of the GPU's fp32 a, b (x W^T over d) and dA' (dO W_down
    over d) at each assignment (t, k), zero where the expert is left out."""
    T, K = ids.shape
    E, h, d = np.shape(w_gate)
    wa = np.zeros((T, K, h))
    wb = np.zeros((T, K, h))
    wdap = np.zeros((T, K, h))
    for k in range(K):
        for e in range(E) if only_experts is None else only_experts:
            r = np.nonzero(ids[:, k] == e)[0]
            if len(r) == 0:
                continue
            wa[r, k] = dot_window(x[r], w_gate[e])
            if act == "swiglu":
                wb[r, k] = dot_window(x[r], w_up[e])
            if backward:
                wdap[r, k] = dot_window(dy[r], np.asarray(w_down[e]).T)
    return dict(a=wa, b=wb, dap=wdap)


def storage_ulp(v, dtype):
    """One unit in the last place of the stored values v (bf16: 8 significant bits, fp32: 24)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - (bits - 1)), 0.0)


def flip_ulps(u, stored, dtype, window):
    """The size of the other rounding where the exact value u lies within
    ``window`` (absolute, per element) of the rounding midpoint on its side
    of the stored value, else 0.  Below a power of two the binade below has
    half the ulp, and so does the midpoint's distance."""
    u = np.asarray(u, dtype=np.float64)
    s = np.asarray(stored, dtype=np.float64)
    ulp = storage_ulp(s, dtype)
    below = (np.abs(u) < np.abs(s)) & (ulp > 0) & (np.abs(s) == 2.0 ** np.floor(np.log2(np.where(s != 0, np.abs(s), 1.0))))
    ulp = np.where(below, ulp / 2, ulp)
    to_mid = ulp / 2 - np.abs(u - s)
    return np.where(to_mid <= np.asarray(window, dtype=np.float64), ulp, 0.0)


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


# share of the stored values that the windows mark as able to flip, per call
# of stored_flip_bounds (for the end-of-run summary)
FLIP_MARKED = []


def stored_flip_bounds(fwd, bw, w, dtype, act="swiglu", saved="aby", win=None):
    """How far the stored dA, dB and A' [T,K,h] of the GPU may sit from the
    oracle's under rounding flips: their own one-ulp flips, plus, to first
    order, the flips of the stored a, b (and y) that the backward computes
    them from (dB = dy SiLU(a), dA = dy b SiLU'(a), A' = w y).  ``win`` holds
    the fp32 windows of a, b and dA' (fp32_windows)."""
    from oracle import moe_oracle as O
    P = POINTWISE_U * U32
    a = fwd["a_s"]
    fa = flip_ulps(fwd["a_u"], a, dtype, win["a"])
    dyv = np.abs(bw["dyv"])
    wk = np.abs(np.asarray(w, dtype=np.float64))[:, :, None]
    if act == "swiglu":
        b = fwd["b_s"]
        fb = flip_ulps(fwd["b_u"], b, dtype, win["b"])
        g1 = np.abs(O.silu_grad(a))
        sa = np.abs(O.silu(a))
        w_da = wk * np.abs(b) * g1 * win["dap"] + P * np.abs(bw["dh_a_u"])
        w_db = wk * sa * win["dap"] + P * np.abs(bw["dh_b_u"])
        da = dyv * (np.abs(b * _deriv(O.silu_grad, a)) * fa + g1 * fb)
        db = dyv * g1 * fa + flip_ulps(bw["dh_b_u"], bw["dh_b"], dtype, w_db)
        y_from_h = g1 * np.abs(b) * fa + sa * fb
        au, bu = fwd["a_u"], fwd["b_u"]
        w_y = np.abs(O.silu_grad(au) * bu) * win["a"] + np.abs(O.silu(au)) * win["b"] + P * np.abs(fwd["y_u"])
        marked = [fa, fb]
    else:
        f, fd = O.ACTS[act]
        w_da = wk * np.abs(fd(a)) * win["dap"] + P * np.abs(bw["dh_a_u"])
        # a flip never changes the sign of a, so relu' does not move
        da = dyv * (np.abs(_deriv(fd, a)) * fa if act != "relu" else 0.0)
        db = None
        y_from_h = np.abs(fd(a)) * fa
        w_y = np.abs(fd(fwd["a_u"])) * win["a"] + P * np.abs(fwd["y_u"])
        marked = [fa]
    fda = flip_ulps(bw["dh_a_u"], bw["dh_a"], dtype, w_da)
    da = da + fda
    marked.append(fda)
    fy = flip_ulps(fwd["y_u"], fwd["y_s"], dtype, w_y) if saved == "aby" else y_from_h
    ap = wk * fy + flip_ulps(bw["a_prime_u"], O.storage_rounder(dtype)(bw["a_prime_u"]), dtype,
                             P * np.abs(bw["a_prime_u"]))
    live = np.abs(fwd["a_u"]) > 0   # assignments the oracle evaluated
    n = int(live.sum())
    if n and dtype == "bf16":       # (in fp32 storage every value is within the window: not a useful share)
        FLIP_MARKED.append(float(np.mean([np.count_nonzero(m[live]) / n for m in marked])))
    return dict(da=da, db=db, ap=ap)


# one record per max check that took an allowance: (name, elements that
# needed it, elements checked, largest share of the tolerance scale granted)
ALLOWANCE_LOG = []


def assert_close(name, g, r, max_tol=MAX_REL, mean_tol=MEAN_REL, report=None, allow=None):
    """allow: per-element absolute error granted to the max check only
    (rounding flips).  An element draws on it when its error is above the
    max tolerance without it; how many did, and the largest relative amount
    they were granted, go into the failure message and into ALLOWANCE_LOG."""
    g64 = np.asarray(g, dtype=np.float64)
    r64 = np.asarray(r, dtype=np.float64)
    note = ""
    if allow is not None:
        rf = r64.reshape(-1)
        diff = np.abs(g64 - r64).reshape(-1)
        rms = float(np.sqrt(np.mean(rf * rf))) if rf.size else 0.0
        scale = np.maximum(np.abs(rf), rms if rms > 0 else 1.0)
        granted = np.minimum(diff, np.asarray(allow, dtype=np.float64).reshape(-1))
        need = diff / scale > max_tol
        n_need = int(np.count_nonzero(need))
        largest = float((granted[need] / scale[need]).max()) if n_need else 0.0
        ALLOWANCE_LOG.append((name, n_need, int(diff.size), largest))
        note = f"; {n_need} of {diff.size} elements drew on the rounding-flip allowance (largest {largest:.2e})"
        mx = float(((diff - granted) / scale).max()) if diff.size else 0.0
        _, mn = rel_errors(g64, r64)
    else:
        mx, mn = rel_errors(g, r)
    if report is not None:
        report[name] = (mx, mn)
    assert np.all(np.isfinite(g64)), f"{name}: non-finite values"
    assert mx <= max_tol and mn <= mean_tol, \
        f"{name}: max_rel={mx:.3e} (tol {max_tol}) mean_rel={mn:.3e} (tol {mean_tol}){note}"


def allowance_summary():
    """One line for the end of a test run: how often the allowance was needed."""
    if not ALLOWANCE_LOG:
        return None
    checks = len(ALLOWANCE_LOG)
    drew = [x for x in ALLOWANCE_LOG if x[1] > 0]
    elems = sum(x[1] for x in ALLOWANCE_LOG)
    total = sum(x[2] for x in ALLOWANCE_LOG)
    largest = max((x[3] for x in ALLOWANCE_LOG), default=0.0)
    marked = f", {100 * np.mean(FLIP_MARKED):.2f}% of stored bf16 values marked able to flip" if FLIP_MARKED else ""
    return (f"rounding-flip allowance: {elems} of {total} gradient elements in {len(drew)} of {checks} "
            f"checks drew on it (largest {largest:.2e} of the max_rel scale){marked}")


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
