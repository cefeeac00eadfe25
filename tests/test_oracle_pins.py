"""Pins for the CPU oracle (no GPU).

Each test ties an oracle function to something other than itself: values
printed on the pages, a second plain definition, brute force, closed forms,
special cases that reduce to a dense computation, or finite differences.
"""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from dropless_moe_dispatch_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_ids(rng, T, E, K):
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


# --------------------------------------------------------------------------
# index (a3)
# --------------------------------------------------------------------------

def test_figure2_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "moeblaze_figure2.json")))
    ids = np.array(g["assignments"], dtype=np.int32)
    ix = O.build_index(ids, g["E"])
    assert ix["expert_token_indices"].tolist() == g["printed"]["expert_token_indices"]
    assert ix["offsets"].tolist() == g["printed"]["expert_token_offsets"]
    assert ix["token_index_map"][0:2].tolist() == g["printed"]["token_index_map_token0"]
    for e, toks in g["printed"]["experts_tokens"].items():
        e = int(e)
        seg = ix["expert_token_indices"][ix["offsets"][e]:ix["offsets"][e + 1]]
        assert seg.tolist() == toks
    assert ix["token_expert_indices"].tolist() == g["derived"]["token_expert_indices"]
    assert ix["token_index_map"].tolist() == g["derived"]["token_index_map"]


def _rank_definition_index(ids, E):
    """Second plain definition, from what the index means rather than from
    how it is built (the "Dropless MoE, in depth" page, "A reference
    implementation", states the grouping as a stable sort of the flattened
    expert ids): assignment (t, k) of expert e sits at offsets[e] plus the
    number of earlier tokens that also chose e, and every position holds the
    token of the assignment placed there."""
    T, K = ids.shape
    counts = [sum(1 for t in range(T) if e in ids[t]) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    pos = [0] * (T * K)
    eti = [-1] * (T * K)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            p = offsets[e] + sum(1 for u in range(t) if e in ids[u])
            pos[t * K + k] = p
            eti[p] = t
    return counts, offsets, eti, pos


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (1, 8, 8), (7, 4, 2), (33, 8, 3), (64, 16, 16), (100, 32, 5)])
def test_index_matches_rank_definition(T, E, K):
    rng = np.random.default_rng(T * 131 + E * 7 + K)
    ids = _rand_ids(rng, T, E, K)
    ix = O.build_index(ids, E)
    counts, offsets, src_tok, pos = _rank_definition_index(ids, E)
    assert ix["counts"].tolist() == counts
    assert ix["offsets"].tolist() == offsets
    assert ix["expert_token_indices"].tolist() == src_tok
    assert ix["token_index_map"].tolist() == pos


@pytest.mark.parametrize("kind", ["gaussian", "one_expert_set", "zero_rows", "ties", "hot_expert", "all_equal"])
def test_index_invariants(kind):
    T, E, K = 200, 16, 4
    z = synth.structured_logits(T, E, K, kind, seed=3)
    ids = O.topk_select(z, K)
    ix = O.build_index(ids, E)
    off, eti, tim = ix["offsets"], ix["expert_token_indices"], ix["token_index_map"]
    assert off[0] == 0 and off[E] == T * K
    assert ix["counts"].sum() == T * K
    assert np.all(np.diff(off) == ix["counts"])
    # the reverse map is a bijection onto the T*K positions
    assert sorted(tim.tolist()) == list(range(T * K))
    for t in range(T):
        # expert ids per token are unique
        assert len(set(ids[t].tolist())) == K
        for k in range(K):
            p = tim[t * K + k]
            e = ids[t, k]
            assert eti[p] == t
            assert off[e] <= p < off[e + 1]
    for e in range(E):
        seg = eti[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)     # strictly increasing token ids (stable)
    # every token appears exactly K times
    assert np.all(np.bincount(eti, minlength=T) == K)


# --------------------------------------------------------------------------
# top-K and weights (a2)
# --------------------------------------------------------------------------

def _brute_topk(z, K):
    T, E = z.shape
    return np.array([sorted(range(E), key=lambda e: (-z[t, e], e))[:K] for t in range(T)], dtype=np.int32)


@pytest.mark.parametrize("kind", ["gaussian", "ties", "all_equal", "hot_expert"])
@pytest.mark.parametrize("E,K", [(8, 2), (8, 8), (16, 1), (64, 6)])
def test_topk_matches_full_sort(kind, E, K):
    z = synth.structured_logits(50, E, K, kind, seed=E + K)
    ids = O.topk_select(z, K)
    assert ids.tolist() == _brute_topk(z, K).tolist()


def test_topk_special_cases():
    z = synth.structured_logits(40, 8, 8, "gaussian", seed=5)
    ids, w = O.route(z, 8)
    # K = E: all experts in descending order; renormalisation is a no-op
    assert np.all(np.diff(np.take_along_axis(z, ids.astype(np.int64), 1), axis=1) <= 0)
    np.testing.assert_allclose(w, np.take_along_axis(O.softmax(z), ids.astype(np.int64), 1), rtol=1e-12)
    ids1, w1 = O.route(z, 1)
    assert np.all(w1 == 1.0)
    assert ids1[:, 0].tolist() == np.argmax(z, axis=1).tolist()


def test_topk_weights_closed_form():
    z = synth.structured_logits(64, 32, 4, "gaussian", seed=9).astype(np.float64) * 3
    ids, w = O.route(z, 4)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    zs = np.take_along_axis(z, ids.astype(np.int64), 1)
    ez = np.exp(zs - zs.max(axis=1, keepdims=True))
    np.testing.assert_allclose(w, ez / ez.sum(axis=1, keepdims=True), rtol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)   # slot order = descending weight


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def test_round_bf16_known_values():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -2.5, 1.0 + 2 ** -8 + 2 ** -20,
                  3.0e-3, 65504.0])
    r = O.round_bf16(v)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even
    assert r[2] == 1.0 + 2 ** -6            # tie -> even (up)
    assert r[3] == 1.0 + 2 ** -7            # representable
    assert r[4] == -2.5
    assert r[5] == 1.0 + 2 ** -7            # above the tie -> up
    # independent implementation: float32 bit-rounding of the input generator
    for x in v[[0, 4, 6, 7]]:
        assert O.round_bf16(np.array([x]))[0] == synth.round_to_bf16(np.array([x], np.float32))[0]
    rng = np.random.default_rng(0)
    f32 = (rng.standard_normal(10000) * 10).astype(np.float32)
    np.testing.assert_array_equal(O.round_bf16(f32.astype(np.float64)), synth.round_to_bf16(f32).astype(np.float64))


# --------------------------------------------------------------------------
# forward (a4, a5)
# --------------------------------------------------------------------------

def _small_layer(T=24, d=16, E=4, K=2, h=12, seed=0, scale_router=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / np.sqrt(d) * scale_router
    wgt = rng.standard_normal((E, h, d)) / np.sqrt(d)
    wup = rng.standard_normal((E, h, d)) / np.sqrt(d)
    wdn = rng.standard_normal((E, d, h)) / np.sqrt(h)
    dy = rng.standard_normal((T, d))
    return x, wg, wgt, wup, wdn, dy


def test_forward_reduces_to_dense_swiglu_when_single_expert():
    x, wg, wgt, wup, wdn, dy = _small_layer(E=1, K=1)
    z = O.router_logits(x, wg)
    ids, w = O.route(z, 1)
    assert np.all(w == 1.0)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype=None)
    a = x @ wgt[0].T
    b = x @ wup[0].T
    dense = ((a / (1 + np.exp(-a))) * b) @ wdn[0].T
    np.testing.assert_allclose(f["out"], dense, rtol=1e-12, atol=1e-12)


def test_forward_dense_mixture_when_k_equals_e():
    x, wg, wgt, wup, wdn, dy = _small_layer(E=3, K=3)
    z = O.router_logits(x, wg)
    ids, w = O.route(z, 3)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype=None)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    mix = sum(p[:, e:e + 1] * (((x @ wgt[e].T) / (1 + np.exp(-(x @ wgt[e].T)))) * (x @ wup[e].T)) @ wdn[e].T
              for e in range(3))
    np.testing.assert_allclose(f["out"], mix, rtol=1e-12, atol=1e-12)


def test_forward_linear_in_down_projection_and_token_equivariant():
    x, wg, wgt, wup, wdn, dy = _small_layer(T=30)
    z = O.router_logits(x, wg)
    ids, w = O.route(z, 2)
    f1 = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype=None)["out"]
    f2 = O.moe_forward(x, ids, w, wgt, wup, 2.0 * wdn, dtype=None)["out"]
    np.testing.assert_array_equal(f2, 2.0 * f1)
    perm = np.random.default_rng(1).permutation(30)
    fp = O.moe_forward(x[perm], ids[perm], w[perm], wgt, wup, wdn, dtype=None)["out"]
    np.testing.assert_allclose(fp, f1[perm], rtol=1e-13, atol=1e-13)
    # duplicating an expert and splitting its tokens between the copies leaves out unchanged
    wgt2 = np.concatenate([wgt, wgt[:1]])
    wup2 = np.concatenate([wup, wup[:1]])
    wdn2 = np.concatenate([wdn, wdn[:1]])
    ids2 = ids.copy()
    sel = (ids2 == 0) & (np.arange(30)[:, None] % 2 == 1)
    ids2[sel] = 4
    f3 = O.moe_forward(x, ids2, w, wgt2, wup2, wdn2, dtype=None)["out"]
    np.testing.assert_allclose(f3, f1, rtol=1e-13, atol=1e-13)


def test_silu_zero_and_gradient():
    assert O.silu(np.array([0.0]))[0] == 0.0
    u = np.linspace(-6, 6, 101)
    eps = 1e-6
    fd = (O.silu(u + eps) - O.silu(u - eps)) / (2 * eps)
    np.testing.assert_allclose(O.silu_grad(u), fd, rtol=1e-7, atol=1e-9)


def test_storage_rounding_mirror_points():
    x, wg, wgt, wup, wdn, dy = _small_layer()
    x = O.round_bf16(x)
    z = O.router_logits(x, wg)
    ids, w = O.route(z, 2)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype="bf16")
    for key in ("a_s", "b_s", "y_s", "out"):
        np.testing.assert_array_equal(f[key], O.round_bf16(f[key]))
    fp = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype=None)
    rel = np.abs(f["out"] - fp["out"]).max() / np.abs(fp["out"]).max()
    assert 0 < rel < 2e-2


# --------------------------------------------------------------------------
# backward (a6 .. a10)
# --------------------------------------------------------------------------

def _margin(z, K):
    s = -np.sort(-z, axis=1)
    return (s[:, K - 1] - s[:, K]).min() if K < z.shape[1] else np.inf


@pytest.mark.parametrize("E,K", [(4, 2), (5, 1), (3, 3)])
def test_backward_finite_differences(E, K):
    T, d, h = 16, 8, 8
    x, wg, wgt, wup, wdn, dy = _small_layer(T=T, d=d, E=E, K=K, h=h, seed=E * 10 + K, scale_router=3.0)
    bias = np.linspace(-0.3, 0.3, E)
    z, ids, w, f, b = O.layer_grads(x, wg, bias, wgt, wup, wdn, dy, K)
    assert _margin(z, K) > 1e-3
    eps = 1e-6
    rng = np.random.default_rng(42)
    params = dict(x=x, wg=wg, w_gate=wgt, w_up=wup, w_down=wdn)
    grads = dict(x=b["dx"], wg=b["dwg"], w_gate=b["dw_gate"], w_up=b["dw_up"], w_down=b["dw_down"])
    for name, P in params.items():
        for trial in range(3):
            V = rng.standard_normal(P.shape)
            args = dict(params)
            args[name] = P + eps * V
            lp = O.layer_loss(args["x"], args["wg"], bias, args["w_gate"], args["w_up"], args["w_down"], dy, ids)
            args[name] = P - eps * V
            lm = O.layer_loss(args["x"], args["wg"], bias, args["w_gate"], args["w_up"], args["w_down"], dy, ids)
            fd = (lp - lm) / (2 * eps)
            an = float((grads[name] * V).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_router_score_gradient_identities():
    x, wg, wgt, wup, wdn, dy = _small_layer(T=40, E=6, K=3, seed=3)
    z, ids, w, f, b = O.layer_grads(x, wg, None, wgt, wup, wdn, dy, 3)
    # <dO, Y> = <dA', y>  (score gradient over h instead of d)
    np.testing.assert_allclose(b["ds"], b["ds_alt"], rtol=1e-11, atol=1e-12)
    dz_closed = O.router_backward_closed(w, ids, b["ds"], 6)
    np.testing.assert_array_equal(b["dz"], dz_closed)
    np.testing.assert_allclose(b["dz_long"], dz_closed, rtol=1e-10, atol=1e-13)
    # zero off the chosen set, and shift invariance of the softmax
    mask = np.zeros_like(b["dz"], dtype=bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, axis=1)
    assert np.all(dz_closed[~mask] == 0.0)
    np.testing.assert_allclose(b["dz"].sum(axis=1), 0.0, atol=1e-13)


def test_zero_row_experts_get_exact_zero_weight_gradients():
    x, wg, wgt, wup, wdn, dy = _small_layer(T=20, E=6, K=2, seed=4)
    wg[4:] = -10.0 * np.abs(wg[4:])
    x = np.abs(x)
    bias = np.array([0, 0, 0, 0, -100.0, -100.0])
    z, ids, w, f, b = O.layer_grads(x, wg, bias, wgt, wup, wdn, dy, 2)
    assert not np.isin(ids, [4, 5]).any()
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(b[key][4:] == 0.0)
    assert np.all(b["dwg"][4:] == 0.0)


def test_backward_matches_explicit_per_token_loop():
    """Independent restatement of the backward for one token, written as
    plain per-assignment vector algebra (Algorithm 1 order)."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=6, E=4, K=2, seed=8)
    z, ids, w, f, b = O.layer_grads(x, wg, None, wgt, wup, wdn, dy, 2)
    t = 3
    dx_t = np.zeros(x.shape[1])
    for k in range(2):
        e = ids[t, k]
        a = wgt[e] @ x[t]
        bb = wup[e] @ x[t]
        s = 1 / (1 + np.exp(-a))
        y = a * s * bb
        grad_y = w[t, k] * (wdn[e].T @ dy[t])          # grad of Y_swi
        grad_a = grad_y * bb * (s + a * s * (1 - s))
        grad_b = grad_y * a * s
        dx_t += wgt[e].T @ grad_a + wup[e].T @ grad_b
        np.testing.assert_allclose(b["ds"][t, k], dy[t] @ (wdn[e] @ y), rtol=1e-12)
    dx_t += b["dz"][t] @ wg
    np.testing.assert_allclose(b["dx"][t], dx_t, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# H-only saved activations (SonicMoE sec. 3.4.1): y recomputed from a, b
# --------------------------------------------------------------------------

def test_h_only_backward_equals_stored_y_in_float64():
    """With no storage rounding the recomputed y is the forward's y, so the
    H-only backward must equal the stored-y backward -- which the finite
    difference test pins to the true gradient.  A wrong recompute (SiLU on
    the up branch, a missing factor) fails here."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=24, E=5, K=2, seed=11)
    z, ids, w, f, b = O.layer_grads(x, wg, None, wgt, wup, wdn, dy, 2)
    bh = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype=None, saved="ab")
    for key in ("dw_gate", "dw_up", "dw_down", "ds_alt"):
        np.testing.assert_allclose(bh[key], b[key], rtol=1e-12, atol=1e-13, err_msg=key)
    # the router path takes <dA', y> here, which equals <dO, Y> up to rounding
    for key in ("dx_f64", "dwg", "dz"):
        np.testing.assert_allclose(bh[key], b[key], rtol=1e-9, atol=1e-12, err_msg=key)


def test_h_only_backward_finite_differences_on_w_down():
    """dW_down of the H-only path against central differences directly (the
    one gradient that goes through A' = w * recomputed y)."""
    T, d, E, K, h = 12, 8, 4, 2, 8
    x, wg, wgt, wup, wdn, dy = _small_layer(T=T, d=d, E=E, K=K, h=h, seed=21, scale_router=3.0)
    z = O.router_logits(x, wg, None)
    ids, w = O.route(z, K)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype=None)
    bh = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype=None, saved="ab")
    eps = 1e-6
    V = np.random.default_rng(5).standard_normal(wdn.shape)
    lp = O.layer_loss(x, wg, None, wgt, wup, wdn + eps * V, dy, ids)
    lm = O.layer_loss(x, wg, None, wgt, wup, wdn - eps * V, dy, ids)
    fd = (lp - lm) / (2 * eps)
    an = float((bh["dw_down"] * V).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_h_only_differs_from_stored_y_by_y_rounding_only():
    """In bf16 storage the two readings differ only through the rounding of
    y: every gradient agrees to a few bf16 ulps of y, and the pieces that do
    not touch y (dH, dW_gate, dW_up, dX) are identical."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=32, E=4, K=2, seed=13)
    x, wg, wgt, wup, wdn, dy = (O.round_bf16(v) for v in (x, wg, wgt, wup, wdn, dy))
    z = O.router_logits(x, wg, None)
    ids, w = O.route(z.astype(np.float32).astype(np.float64), 2)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype="bf16")
    b = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype="bf16")
    bh = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype="bf16", saved="ab")
    for key in ("dh_a", "dh_b", "dw_gate", "dw_up"):
        np.testing.assert_array_equal(bh[key], b[key], err_msg=key)
    np.testing.assert_array_equal(bh["ds"], b["ds"])   # the plain definition does not move
    rel = np.abs(bh["dw_down"] - b["dw_down"]).max() / np.abs(b["dw_down"]).max()
    assert 0 < rel < 2 ** -6, rel
    rel = np.abs(bh["ds_alt"] - b["ds_alt"]).max() / np.abs(b["ds_alt"]).max()
    assert rel < 2 ** -6, rel


# --------------------------------------------------------------------------
# non-gated experts: E_i(x) = W_2 sigma(W_1 x), sigma = SiLU or ReLU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["silu", "relu"])
def test_non_gated_forward_reduces_to_dense_mlp_when_single_expert(act):
    x, wg, w1, _, w2, dy = _small_layer(E=1, K=1, seed=2)
    z = O.router_logits(x, wg)
    ids, w = O.route(z, 1)
    f = O.moe_forward(x, ids, w, w1, None, w2, dtype=None, act=act)
    a = x @ w1[0].T
    hid = a / (1 + np.exp(-a)) if act == "silu" else np.where(a > 0, a, 0.0)
    np.testing.assert_allclose(f["out"], hid @ w2[0].T, rtol=1e-12, atol=1e-12)
    assert np.all(f["b_s"] == 0.0)


@pytest.mark.parametrize("act", ["silu", "relu"])
@pytest.mark.parametrize("E,K", [(4, 2), (3, 3)])
def test_non_gated_backward_finite_differences(act, E, K):
    T, d, h = 16, 8, 8
    x, wg, w1, _, w2, dy = _small_layer(T=T, d=d, E=E, K=K, h=h, seed=E * 7 + K, scale_router=3.0)
    z, ids, w, f, b = O.layer_grads(x, wg, None, w1, None, w2, dy, K, act=act)
    assert _margin(z, K) > 1e-3
    if act == "relu":   # stay off the kink: every pre-activation clear of zero by >> eps
        assert np.abs(f["a_s"][f["a_s"] != 0]).min() > 1e-4
    eps = 1e-6
    rng = np.random.default_rng(7)
    params = dict(x=x, wg=wg, w1=w1, w2=w2)
    grads = dict(x=b["dx"], wg=b["dwg"], w1=b["dw_gate"], w2=b["dw_down"])
    for name, P in params.items():
        for _ in range(2):
            V = rng.standard_normal(P.shape)
            args = dict(params)
            args[name] = P + eps * V
            lp = O.layer_loss(args["x"], args["wg"], None, args["w1"], None, args["w2"], dy, ids, act=act)
            args[name] = P - eps * V
            lm = O.layer_loss(args["x"], args["wg"], None, args["w1"], None, args["w2"], dy, ids, act=act)
            fd = (lp - lm) / (2 * eps)
            an = float((grads[name] * V).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (act, name, fd, an)
    assert np.all(b["dw_up"] == 0.0)


def test_relu_expert_rows_with_negative_preactivation_are_inert():
    """ReLU: an assignment whose pre-activations are all negative adds
    nothing to out and passes no gradient to W_1 or x (only the router
    term remains)."""
    x, wg, w1, _, w2, dy = _small_layer(T=10, E=2, K=1, seed=9)
    w1 = np.abs(w1)
    x[3] = -np.abs(x[3])                      # token 3: a = x W1^T < 0 for both experts
    z, ids, w, f, b = O.layer_grads(x, wg, None, w1, None, w2, dy, 1, act="relu")
    assert np.all(f["a_s"][3] < 0)
    np.testing.assert_array_equal(f["out"][3], 0.0)
    np.testing.assert_array_equal(b["dh_a"][3], 0.0)
    np.testing.assert_allclose(b["dx"][3], b["dz"][3] @ wg, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("act", ["swiglu", "silu"])
def test_unrounded_intermediates_round_to_the_stored_ones(act):
    """The unrounded a, b, y, dA, dB and A' the oracle reports (for the
    parity tests' rounding-flip allowance) are the values its stored ones
    were rounded from, and dyv is w times dA' = dO W_down."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=20, E=4, K=2, seed=5)
    st = O.storage_rounder("bf16")
    xs, wgs, wgts, wups, wdns, dys = (st(v) for v in (x, wg, wgt, wup, wdn, dy))
    z = O.router_logits(xs, wgs, None)
    ids, w = O.route(z, 2)
    f = O.moe_forward(xs, ids, w, wgts, wups, wdns, dtype="bf16", act=act)
    b = O.moe_backward(dys, xs, wgs, ids, w, wgts, wups, wdns, f, z, dtype="bf16", act=act)
    for u, s_ in (("a_u", "a_s"), ("y_u", "y_s")) + ((("b_u", "b_s"),) if act == "swiglu" else ()):
        assert np.array_equal(st(f[u]), f[s_]), u
    assert np.array_equal(st(b["dh_a_u"]), b["dh_a"])
    if act == "swiglu":
        assert np.array_equal(st(b["dh_b_u"]), b["dh_b"])
    t, k = 3, 1
    e = ids[t, k]
    np.testing.assert_allclose(b["dyv"][t, k], w[t, k] * (dys[t] @ wdns[e]), rtol=1e-12)
    np.testing.assert_allclose(b["a_prime_u"][t, k], w[t, k] * f["y_s"][t, k], rtol=1e-12)


# --------------------------------------------------------------------------
# the restricted modes the full-size parity tests use
# --------------------------------------------------------------------------

@pytest.mark.parametrize("saved", ["aby", "ab"])
@pytest.mark.parametrize("act", ["swiglu", "silu"])
def test_only_experts_equals_the_full_run_on_those_experts(saved, act):
    """moe_forward / moe_backward restricted to experts [e] give, for e's
    assignments and e's weight gradients, exactly what the unrestricted run
    gives (the full-size tests check the largest experts this way), and
    zeros elsewhere."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=40, E=5, K=2, seed=31)
    x, wg, wgt, wup, wdn, dy = (O.round_bf16(v) for v in (x, wg, wgt, wup, wdn, dy))
    if act != "swiglu":
        wup = None
    z = O.router_logits(x, wg, None)
    ids, w = O.route(z, 2)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype="bf16", act=act)
    b = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype="bf16", saved=saved, act=act)
    for e in (1, 3):
        fe = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype="bf16", only_experts=[e], act=act)
        be = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, fe, z, dtype="bf16", only_experts=[e],
                            saved=saved, act=act)
        mine = ids == e
        assert mine.any()
        for key in ("a_s", "b_s", "y_s", "ye", "a_u", "y_u"):
            np.testing.assert_array_equal(fe[key][mine], f[key][mine], err_msg=key)
            assert np.all(fe[key][~mine] == 0.0), key
        for key in ("dh_a", "dh_b", "a_prime_u", "dyv"):
            np.testing.assert_array_equal(be[key][mine], b[key][mine], err_msg=key)
            assert np.all(be[key][~mine] == 0.0), key
        np.testing.assert_array_equal(be["ds"][mine], b["ds"][mine])
        np.testing.assert_array_equal(be["ds_alt"][mine], b["ds_alt"][mine])
        for key in ("dw_gate", "dw_up", "dw_down"):
            np.testing.assert_array_equal(be[key][e], b[key][e], err_msg=key)
            others = [j for j in range(5) if j != e]
            assert np.all(be[key][others] == 0.0), key


@pytest.mark.parametrize("saved", ["aby", "ab"])
def test_router_only_backward_equals_the_full_run(saved):
    """The router-only backward (score gradients, dz, dWg) matches the full
    backward bit for bit, and leaves the expert gradients at zero."""
    x, wg, wgt, wup, wdn, dy = _small_layer(T=30, E=6, K=3, seed=12)
    x, wg, wgt, wup, wdn, dy = (O.round_bf16(v) for v in (x, wg, wgt, wup, wdn, dy))
    z = O.router_logits(x, wg, None)
    ids, w = O.route(z, 3)
    f = O.moe_forward(x, ids, w, wgt, wup, wdn, dtype="bf16")
    b = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype="bf16", saved=saved)
    r = O.moe_backward(dy, x, wg, ids, w, wgt, wup, wdn, f, z, dtype="bf16", saved=saved, router_only=True)
    for key in ("ds", "ds_alt", "ds_router", "dz", "dwg"):
        np.testing.assert_array_equal(r[key], b[key], err_msg=key)
    np.testing.assert_array_equal(r["dx_f64"], b["dz"] @ wg)
    for key in ("dw_gate", "dw_up", "dw_down", "dh_a", "dh_b"):
        assert np.all(r[key] == 0.0), key
