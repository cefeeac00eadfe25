"""CPU oracle for the dropless Mixture-of-Experts layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the GPU library (HIP
kernels, C-ABI, Python binding) and the GPU library shares none with it.

It is the plain definition of the layer, written in float64 with numpy:
per token, per chosen expert, an explicit SwiGLU feed-forward network, then a
weighted sum, plus explicit gradients.  Matrix products are computed with
numpy's ``@`` (one library primitive per step); rows that picked the same
expert are evaluated together only because each row's result is independent
of the others -- no blocking, fusion or reordering of any row's arithmetic.

Sources (the pages this implements):
  [MB]  "MoEBlaze: Breaking the Memory Wall for Efficient MoE Training on
        Modern GPUs" (paper-graph-ui analysis page): "Dispatch Data
        Structures: Specification and Roles", "Fused SwiGLU Kernel with
        Activation Checkpoint".
  [MBn] MoEBlaze reading notes (papercache.org): sec. 2.1 gating network,
        sec. 2.3 output aggregation, sec. 4.1 / Figure 2 worked example,
        sec. 5.2 Algorithm 1 (fused SwiGLU MoE training).
  [SM]  "SonicMoE: Accelerating MoE with IO and Tile-aware Optimizations"
        (paper-graph-ui analysis page), sec. 3.4.1 memory-efficient backward.
  [DM]  "Dropless MoE, in depth" (aicassindra.com), "A reference
        implementation".

Readings where the pages are silent or ambiguous (each is listed in the
design notes of the repository):
  * top-K ties go to the lower expert id; slots are ordered by descending
    logit, then ascending id.  The decision is taken on the logits the caller
    passes (float32 when they come from a float32 router).
  * the K chosen softmax probabilities are renormalised to sum to one [DM].
  * W_gate gets the SiLU, W_up is the linear branch, W_down projects back;
    every weight is stored [out, in] per expert.
  * storage precision: a, b (the saved pre-activations), y = SiLU(a)*b, dH,
    the layer output and dX are rounded to the storage type (bf16 or f32);
    y is formed from the unrounded a, b; the backward recomputes sigmoid and
    SiLU from the rounded a, b.  ``store=None`` gives the pure float64 layer.
  * the router score gradient dS is taken with respect to the renormalised
    weights w, and dX includes the router path.
  * dW_down uses the score-scaled activation A' = w * y held in the storage
    type, as SonicMoE sec. 3.4.1 defines it (dW2 = A'^T dO).

Parity status: every function below is pinned by tests/test_oracle_pins.py
(worked example, brute force, closed forms, special cases, finite
differences); no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage rounding (precision mirror)
# ---------------------------------------------------------------------------


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant bits,
    ties to even), returned as float64."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                    # v = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def storage_rounder(dtype: str):
    if dtype == "bf16":
        return round_bf16
    if dtype == "f32":
        return round_f32
    if dtype in (None, "f64"):
        return lambda v: np.asarray(v, dtype=np.float64)
    raise ValueError(dtype)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def silu(u):
    """SiLU(u) = u * sigmoid(u)  [MB, "Fused SwiGLU Kernel"; MBn sec. 5.1]."""
    return u * sigmoid(u)


def silu_grad(u):
    """d SiLU / du = sigma(u) + u*sigma(u)*(1 - sigma(u))  [MB, "Fused SwiGLU Kernel"]."""
    s = sigmoid(u)
    return s + u * s * (1.0 - s)


def relu(u):
    return np.maximum(u, 0.0)


def relu_grad(u):
    """d ReLU / du: 1 where u > 0, else 0 (0 at the kink)."""
    return (np.asarray(u) > 0.0).astype(np.float64)


# Expert feed-forward kinds.  "swiglu": y = SiLU(x W_gate^T) * (x W_up^T), the
# gated expert of MoEBlaze sec. 5 (Algorithm 1).  "silu" / "relu": the plain
# two-layer expert E_i(x) = W_2 sigma(W_1 x) of the MoEBlaze reading notes
# (sec. 2.2, expert FFNs) with sigma = SiLU or ReLU; W_1 is passed as w_gate
# and there is no w_up.
ACTS = {"silu": (silu, silu_grad), "relu": (relu, relu_grad)}


# ---------------------------------------------------------------------------
# a1: router logits   topk experts = TopK(softmax(W_g x)), W_g in R^{E x d}  [MBn sec. 2.1]
# ---------------------------------------------------------------------------


def router_logits(x, wg, bias=None) -> np.ndarray:
    """z[t, e] = sum_i x[t, i] * Wg[e, i] (+ b[e]), float64."""
    z = _f64(x) @ _f64(wg).T
    if bias is not None:
        z = z + _f64(bias)[None, :]
    return z


def softmax(z) -> np.ndarray:
    z = _f64(z)
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# a2: top-K selection and renormalised weights  [MBn sec. 2.1; DM reference]
# ---------------------------------------------------------------------------


def topk_select(z, K: int) -> np.ndarray:
    """ids[t, k]: the k-th largest logit of token t (ties -> lower expert id).

    Selection by K rounds of arg-max over the not-yet-chosen experts; the
    comparison is exact on whatever values are passed in.
    """
    z = np.array(z, dtype=np.float64, copy=True)
    T, E = z.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    ids = np.empty((T, K), dtype=np.int32)
    rows = np.arange(T)
    for k in range(K):
        j = np.argmax(z, axis=1)          # first maximal index = lowest id on ties
        ids[:, k] = j
        z[rows, j] = -np.inf
    return ids


def topk_weights(z, ids) -> np.ndarray:
    """w[t, k] = p[t, S_k] / sum_j p[t, S_j] with p = softmax(z[t, :])  [DM reference]."""
    p = softmax(z)
    ps = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return ps / ps.sum(axis=1, keepdims=True)


def route(z, K: int):
    ids = topk_select(z, K)
    return ids, topk_weights(z, ids)


# ---------------------------------------------------------------------------
# a3: the routing index  [MB, "Dispatch Data Structures"; MBn sec. 4.1, Fig. 2]
# ---------------------------------------------------------------------------


def build_index(ids, E: int):
    """Brute-force definition of the four index structures.

    expert_token_indices: for e = 0..E-1, for t = 0..T-1 in order, append t
        when e is one of token t's experts (stable by token within an expert).
    expert_token_offsets: exclusive prefix sum of the per-expert counts, with
        offsets[E] = T*K.
    token_expert_indices: the expert ids of token t at t*K .. t*K+K-1 (the
        flattened selection).
    token_index_map[t*K + k]: position of (t, ids[t, k]) in
        expert_token_indices.
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    eti = []
    for e in range(E):
        chosen = np.nonzero((ids == e).any(axis=1))[0]
        counts[e] = len(chosen)
        eti.append(chosen)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    eti = np.concatenate(eti) if eti else np.zeros(0, np.int64)
    tim = np.empty(T * K, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            seg = eti[offsets[e]:offsets[e + 1]]
            tim[t * K + k] = offsets[e] + int(np.searchsorted(seg, t))
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                expert_token_indices=eti.astype(np.int32),
                token_expert_indices=ids.reshape(-1).astype(np.int32),
                token_index_map=tim.astype(np.int32))


# ---------------------------------------------------------------------------
# a4 + a5: expert SwiGLU FFN and weighted combine
#   y = sum_i g_i(x) E_i(x)                               [MBn sec. 2.3]
#   SwiGLU(x; W1, W2) = SiLU(x W1) * (x W2)               [MB; MBn sec. 5.1]
#   Algorithm 1 forward: store A, B, Y_swi; Y_out = Y_swi W3  [MBn sec. 5.2]
# ---------------------------------------------------------------------------


def _rows_of(ids, k, e):
    return np.nonzero(ids[:, k] == e)[0]


def moe_forward(x, ids, w, w_gate, w_up, w_down, dtype="bf16", only_experts=None, act="swiglu"):
    """Forward pass.  Returns out [T,d] plus the per-assignment tensors
    a_s, b_s, y_s [T,K,h] (storage-rounded), a_u, b_u, y_u (the same before
    the storage rounding, for judging which stored values sit on a rounding
    boundary; nothing here uses them) and ye [T,K,d] (expert output).

    ``only_experts`` (for sampled checks) evaluates only the assignments of
    those experts; quantities of the other assignments stay zero.
    ``act``: "swiglu" (gated), or "silu" / "relu" (two-layer expert with
    W_1 = w_gate; w_up is unused and b_s stays zero)."""
    if act not in ("swiglu", *ACTS):
        raise ValueError(f"unknown activation {act!r}")
    st = storage_rounder(dtype)
    x = _f64(x)
    w = _f64(w)
    T, d = x.shape
    K = ids.shape[1]
    E, h, _ = np.shape(w_gate)
    a_s = np.zeros((T, K, h))
    b_s = np.zeros((T, K, h))
    y_s = np.zeros((T, K, h))
    a_u = np.zeros((T, K, h))
    b_u = np.zeros((T, K, h))
    y_u = np.zeros((T, K, h))
    ye = np.zeros((T, K, d))
    out = np.zeros((T, d))
    for k in range(K):                       # slot order of the weighted sum
        for e in range(E) if only_experts is None else only_experts:
            r = _rows_of(ids, k, e)
            if len(r) == 0:
                continue
            xe = x[r]
            a = xe @ _f64(w_gate[e]).T       # gate projection (W_1 of a plain expert)
            if act == "swiglu":
                b = xe @ _f64(w_up[e]).T     # up projection
                yu = silu(a) * b             # SiLU(a) * b from the unrounded a, b
                b_s[r, k] = st(b)
                b_u[r, k] = b
            else:
                yu = ACTS[act][0](a)         # sigma(a) from the unrounded a
            y = st(yu)
            yo = y @ _f64(w_down[e]).T       # down projection
            a_s[r, k] = st(a)
            a_u[r, k] = a
            y_s[r, k] = y
            y_u[r, k] = yu
            ye[r, k] = yo
            out[r] += w[r, k][:, None] * yo
    return dict(out=st(out), out_f64=out, a_s=a_s, b_s=b_s, y_s=y_s, a_u=a_u, b_u=b_u, y_u=y_u, ye=ye)


# ---------------------------------------------------------------------------
# a6 .. a10: backward for L = <dY, out>
#   Algorithm 1 backward (recompute SiLU(A) from stored A)   [MBn sec. 5.2]
#   grad_a = grad(out) * b * SiLU'(a); grad_x = grad_a W1^T + grad_b W2^T  [MB]
#   dS = <dO, Y>;  dA = s * dO W2^T                           [SM sec. 3.4.1]
# ---------------------------------------------------------------------------


def moe_backward(dy, x, wg, ids, w, w_gate, w_up, w_down, fwd, z, dtype="bf16", only_experts=None,
                 saved="aby", act="swiglu", router_only=False):
    """Backward pass.  ``z`` are the logits the weights were computed from.
    ``only_experts`` restricts the expert path to those experts (the weight
    gradients of those experts are then complete; dx, ds, dwg are not).
    ``router_only`` computes only what the router gradient needs (ds, ds_alt,
    dz, dwg): the score gradients of every assignment, without dH and the
    expert weight gradients (they stay zero), and dx then holds the router
    term alone; what is computed goes through the same arithmetic as in the
    full pass.

    ``saved`` names what the forward kept for the backward:
      "aby" -- a, b and y (MoEBlaze Algorithm 1 stores A, B and Y_swi);
      "ab"  -- only the pre-activations H = [a | b] (SonicMoE sec. 3.4.1,
               minimal cached set): the backward recomputes
               y = SiLU(a_s) * b_s from the stored a, b and uses it for
               <dA', y> and for A' = w * y.

    Returns dx [T,d], dwg [E,d], dw_gate/dw_up [E,h,d], dw_down [E,d,h],
    ds [T,K] (= dL/dw), ds_alt [T,K] (= <dA', y>), dz [T,E] (closed form),
    dz_long [T,E] (through the full softmax), dh_a/dh_b [T,K,h] as stored,
    and dh_a_u/dh_b_u/a_prime_u [T,K,h]: the same values and A' before the
    storage rounding, and dyv [T,K,h], the gradient reaching y (for judging
    which stored values sit on a rounding boundary and what a one-ulp change
    of them moves; nothing here uses them).
    """
    if saved not in ("aby", "ab"):
        raise ValueError(f"saved must be 'aby' or 'ab', not {saved!r}")
    st = storage_rounder(dtype)
    g_all = _f64(dy)
    x = _f64(x)
    w = _f64(w)
    T, d = x.shape
    K = ids.shape[1]
    E, h, _ = np.shape(w_gate)
    dx = np.zeros((T, d))
    dw_gate = np.zeros((E, h, d))
    dw_up = np.zeros((E, h, d))
    dw_down = np.zeros((E, d, h))
    ds = np.zeros((T, K))
    ds_alt = np.zeros((T, K))
    dh_a = np.zeros((T, K, h))
    dh_b = np.zeros((T, K, h))
    dh_a_u = np.zeros((T, K, h))
    dh_b_u = np.zeros((T, K, h))
    a_prime_u = np.zeros((T, K, h))
    dyv_all = np.zeros((T, K, h))
    for k in range(K):
        for e in range(E) if only_experts is None else only_experts:
            r = _rows_of(ids, k, e)
            if len(r) == 0:
                continue
            g = g_all[r]                               # dO rows of these tokens
            wd = _f64(w_down[e])
            da_p = g @ wd                              # dA' = dO W_down   (length h)
            a = fwd["a_s"][r, k]
            b = fwd["b_s"][r, k]
            # the y the backward sees: the stored one, or recomputed from H
            if saved == "aby":
                y_b = fwd["y_s"][r, k]
            else:
                y_b = silu(a) * b if act == "swiglu" else ACTS[act][0](a)
            ds[r, k] = np.einsum("rd,rd->r", g, fwd["ye"][r, k])      # <dO, Y>
            ds_alt[r, k] = np.einsum("rh,rh->r", da_p, y_b)           # <dA', y>
            dyv = w[r, k][:, None] * da_p              # gradient reaching y
            dyv_all[r, k] = dyv
            if router_only:
                continue
            if act == "swiglu":
                da_u = dyv * b * silu_grad(a)          # SiLU recomputed from stored a
                db_u = dyv * silu(a)
                db = st(db_u)
                dh_b[r, k] = db
                dh_b_u[r, k] = db_u
            else:
                da_u = dyv * ACTS[act][1](a)           # sigma' recomputed from stored a
                db = None
            da = st(da_u)
            dh_a[r, k] = da
            dh_a_u[r, k] = da_u
            # A' = w * y, held in the storage type (SonicMoE sec. 3.4.1: dW2 = A'^T dO)
            ap_u = w[r, k][:, None] * y_b
            a_prime_u[r, k] = ap_u
            a_prime = st(ap_u)
            dw_down[e] += g.T @ a_prime
            dw_gate[e] += da.T @ x[r]
            dx[r] += da @ _f64(w_gate[e])
            if db is not None:
                dw_up[e] += db.T @ x[r]
                dx[r] += db @ _f64(w_up[e])
    # the router gradient takes the dS the backward has: the plain <dO, Y>
    # with the stored y, or <dA', y> with y recomputed from H (H-only: the
    # forward's y is gone, SonicMoE sec. 3.4.1 forms dS from the recomputed y)
    ds_r = ds if saved == "aby" else ds_alt
    # the closed form is exact zero off the chosen set; it is pinned to the
    # long way (full softmax + renormalisation) by the oracle's own tests
    dz = router_backward_closed(w, ids, ds_r, E)
    dwg = dz.T @ x
    dx = dx + dz @ _f64(wg)
    return dict(dx=st(dx), dx_f64=dx, dwg=dwg, dw_gate=dw_gate, dw_up=dw_up,
                dw_down=dw_down, ds=ds, ds_alt=ds_alt, ds_router=ds_r, dz=dz,
                dz_long=router_backward_long(z, ids, ds_r), dh_a=dh_a, dh_b=dh_b, dh_a_u=dh_a_u,
                dh_b_u=dh_b_u, a_prime_u=a_prime_u, dyv=dyv_all)


def router_backward_long(z, ids, ds) -> np.ndarray:
    """dL/dz through the full softmax and the renormalisation, the long way.

    With p = softmax(z), P = sum_{j in S} p_j and w_k = p_{S_k} / P:
      dL/dp_e = (dS_e - sum_k w_k dS_k) / P   for e in S, 0 otherwise;
      dL/dz   = p * (dL/dp - <p, dL/dp>)       (softmax backward).
    """
    p = softmax(z)
    T, E = p.shape
    K = ids.shape[1]
    ids64 = ids.astype(np.int64)
    ps = np.take_along_axis(p, ids64, axis=1)
    P = ps.sum(axis=1, keepdims=True)
    wk = ps / P
    centre = (wk * ds).sum(axis=1, keepdims=True)
    dp = np.zeros((T, E))
    np.put_along_axis(dp, ids64, (ds - centre) / P, axis=1)
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def router_backward_closed(w, ids, ds, E: int) -> np.ndarray:
    """Closed form: dz[t, S_k] = w_k (dS_k - sum_j w_j dS_j); zero off the chosen set."""
    w = _f64(w)
    T, K = w.shape
    centre = (w * ds).sum(axis=1, keepdims=True)
    dz = np.zeros((T, E))
    np.put_along_axis(dz, ids.astype(np.int64), w * (ds - centre), axis=1)
    return dz


# ---------------------------------------------------------------------------
# the whole layer (router included), for the finite-difference checks
# ---------------------------------------------------------------------------


def layer_loss(x, wg, bias, w_gate, w_up, w_down, dy, ids, act="swiglu"):
    """L = <dY, out> of the pure float64 layer with the routing set ``ids``
    held fixed (the weights w still depend on the logits)."""
    z = router_logits(x, wg, bias)
    w = topk_weights(z, ids)
    f = moe_forward(x, ids, w, w_gate, w_up, w_down, dtype=None, act=act)
    return float((_f64(dy) * f["out_f64"]).sum())


def layer_grads(x, wg, bias, w_gate, w_up, w_down, dy, K, act="swiglu"):
    """Pure float64 forward + backward of the whole layer."""
    z = router_logits(x, wg, bias)
    ids, w = route(z, K)
    f = moe_forward(x, ids, w, w_gate, w_up, w_down, dtype=None, act=act)
    b = moe_backward(dy, x, wg, ids, w, w_gate, w_up, w_down, f, z, dtype=None, act=act)
    return z, ids, w, f, b
