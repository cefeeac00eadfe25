"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Small shapes (several 128-row tiles, ragged tails, edge cases) are compared
element by element; routing ids, counts, offsets and the index bit-exact,
floats within max_rel 2e-2 / mean_rel 2e-3.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dropless_moe_dispatch_amd import binding as B
from dropless_moe_dispatch_amd import layer as Lyr
from dropless_moe_dispatch_amd import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dw_flip_allowance, fp32_windows, stored_flip_bounds, to_np, topk_margin

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # fails loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# a2: top-K from given logits (bit-exact ids, weights to tolerance)
# ---------------------------------------------------------------------------
TOPK_CASES = [
    (1, 8, 3, "gaussian"), (257, 8, 2, "gaussian"), (300, 8, 8, "all_equal"), (1000, 128, 8, "gaussian"),
    (513, 64, 6, "ties"), (200, 16, 1, "ties"), (300, 1024, 32, "gaussian"), (100, 200, 5, "hot_expert"),
    (64, 33, 7, "zero_rows"), (128, 4, 4, "one_expert_set"),
]


@pytest.mark.parametrize("T,E,K,kind", TOPK_CASES)
def test_topk_from_logits_bitexact(T, E, K, kind):
    _say("topk", T, E, K, kind)
    z = synth.structured_logits(T, E, K, kind, seed=T + E)
    buf = Lyr.MoEBuffers(T, 128, E, K, 128, "bf16", backward=False)
    buf.logits.copy_(torch.from_numpy(z))
    Lyr.route(buf, None, None, None, logits_in=True)
    torch.cuda.synchronize()
    ids_ref, w_ref = O.route(z.astype(np.float64), K)
    ids = to_np(buf.topk_ids)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(to_np(buf.topk_w), w_ref, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# a3: index bit-exact
# ---------------------------------------------------------------------------
INDEX_CASES = [
    (1, 8, 3, "gaussian"), (255, 8, 2, "gaussian"), (256, 16, 4, "one_expert_set"), (1000, 128, 8, "gaussian"),
    (777, 64, 6, "zero_rows"), (4096, 1024, 32, "gaussian"), (3000, 32, 32, "all_equal"), (2000, 64, 4, "hot_expert"),
    # expert sets of four and eight 64-expert words, the last one ragged
    (600, 200, 6, "gaussian"), (900, 300, 5, "zero_rows"),
]


@pytest.mark.parametrize("backend", ["ballot", "dense"])
@pytest.mark.parametrize("T,E,K,kind", INDEX_CASES)
def test_index_bitexact(T, E, K, kind, backend):
    """Both index backends: the wave-ballot counting sort and MoEBlaze's
    literal three steps with a dense [E][T] map."""
    _say("index", backend, T, E, K, kind)
    z = synth.structured_logits(T, E, K, kind, seed=2 * T + E)
    ids_np = O.topk_select(z, K)
    buf = Lyr.MoEBuffers(T, 128, E, K, 128, "bf16", backward=False)
    buf.topk_ids.copy_(torch.from_numpy(ids_np))
    if backend == "ballot":
        B.moe_build_index(buf.shape, buf.topk_ids, buf.offsets, buf.eti, buf.tim, buf.ws_index)
    else:
        ws = torch.empty(B.workspace_bytes(buf.shape, B.MOE_WS_INDEX_DENSE), dtype=torch.uint8, device="cuda")
        B.moe_build_index_dense(buf.shape, buf.topk_ids, buf.offsets, buf.eti, buf.tim, ws)
    torch.cuda.synchronize()
    ix = O.build_index(ids_np, E)
    assert np.array_equal(to_np(buf.offsets), ix["offsets"])
    assert np.array_equal(to_np(buf.eti), ix["expert_token_indices"])
    assert np.array_equal(to_np(buf.tim), ix["token_index_map"])


# ---------------------------------------------------------------------------
# a1: router logits
# ---------------------------------------------------------------------------
ROUTER_CASES = [
    (300, 256, 8, "bf16"), (1000, 384, 128, "bf16"), (129, 128, 64, "f32"), (77, 512, 200, "bf16"),
    # the fused router (under 16384 tokens, d a multiple of 256) with 32, 64
    # and 96-128 expert columns, ragged token tails and a ring longer than the
    # slice; and the separate logits GEMM + top-K just past its bounds
    (3000, 1024, 64, "bf16"), (16351, 256, 100, "bf16"), (40, 256, 33, "bf16"), (100, 2048, 128, "bf16"),
    (16400, 256, 100, "bf16"), (40, 128, 33, "bf16"), (17000, 512, 4, "bf16"),
]


@pytest.mark.parametrize("T,d,E,dtype", ROUTER_CASES)
def test_router_logits(T, d, E, dtype):
    _say("router_logits", T, d, E, dtype)
    wl = synth.small_workload(T, d, E, 2, 128, dtype=dtype, seed=T, zipf_s=1.2)
    inp = synth.make_inputs(wl, tensors=("x", "wg"))
    buf = Lyr.MoEBuffers(T, d, E, 2, 128, dtype, backward=False)
    x = Lyr.to_device(inp["x"], dtype)
    wg = Lyr.to_device(inp["wg"], dtype)
    bias = torch.from_numpy(inp["bias"]).cuda()
    Lyr.route(buf, x, wg, bias)
    torch.cuda.synchronize()
    z = O.router_logits(inp["x"], inp["wg"], inp["bias"])
    err = np.abs(to_np(buf.logits) - z).max()
    assert err < 2e-5 * np.sqrt(d / 128), err


@pytest.mark.parametrize("kmax", [4, 32])
@pytest.mark.parametrize("T,d,E,dtype", ROUTER_CASES)
def test_route_from_x_selects_on_its_logits(T, d, E, dtype, kmax):
    """Routing from x (the fused router where it applies) gives the ids and
    weights that top-K from the logits it wrote gives, bit for bit, and the
    oracle's top-K of those logits (the selection is taken on the same fp32
    values on both sides)."""
    K = min(kmax, E)
    _say("route_from_x", T, d, E, K, dtype)
    wl = synth.small_workload(T, d, E, K, 128, dtype=dtype, seed=T + 7, zipf_s=1.2)
    inp = synth.make_inputs(wl, tensors=("x", "wg"))
    buf = Lyr.MoEBuffers(T, d, E, K, 128, dtype, backward=False)
    Lyr.route(buf, Lyr.to_device(inp["x"], dtype), Lyr.to_device(inp["wg"], dtype),
              torch.from_numpy(inp["bias"]).cuda())
    ref = Lyr.MoEBuffers(T, d, E, K, 128, dtype, backward=False)
    ref.logits.copy_(buf.logits)
    Lyr.route(ref, None, None, None, logits_in=True)
    torch.cuda.synchronize()
    assert torch.equal(buf.topk_ids, ref.topk_ids)
    assert torch.equal(buf.topk_w, ref.topk_w)
    ids_ref, w_ref = O.route(to_np(buf.logits).astype(np.float64), K)
    assert np.array_equal(to_np(buf.topk_ids), ids_ref)
    np.testing.assert_allclose(to_np(buf.topk_w), w_ref, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# whole layer, routing from given logits (deterministic ids on both sides)
# ---------------------------------------------------------------------------
LAYER_CASES = [
    # name, T, d, E, K, h, dtype, zipf
    ("ragged", 300, 256, 8, 2, 256, "bf16", None),
    ("multi_tile", 1000, 384, 16, 4, 384, "bf16", None),
    ("tiny_f32", 256, 128, 8, 2, 256, "f32", None),
    ("skewed", 700, 256, 32, 6, 256, "bf16", 1.2),
    ("fine", 513, 256, 64, 8, 128, "bf16", None),
    ("k1", 200, 128, 4, 1, 128, "bf16", None),
    ("k_eq_e", 130, 128, 4, 4, 128, "bf16", None),
    ("t1", 1, 128, 8, 3, 128, "bf16", None),
    ("f32_bwd", 300, 256, 16, 4, 256, "f32", None),
    # few dW tiles, many rows per expert: the dW GEMMs split each expert's
    # rows into 8 chunks and sum the partials
    ("split_k", 4096, 256, 2, 2, 256, "bf16", None),
    ("split_k_f32", 4096, 128, 2, 2, 128, "f32", None),
    # router weight gradient on MFMA: two 128-expert blocks (the second
    # ragged), and 16 or 32 slots per token (more entries per thread)
    ("experts_200", 600, 128, 200, 4, 128, "bf16", None),
    ("k16", 300, 128, 32, 16, 128, "bf16", None),
    ("k32", 130, 128, 64, 32, 128, "bf16", 1.2),
    # d = 4096, 2h = 8192: gate/up on the 256 x 256 tile and the dX fold on
    # the wide (two-pass) fold; more experts than assignments (most empty,
    # E > 128 in the separate top-K); fp32 with eight slots
    ("wide_fold", 200, 4096, 4, 2, 4096, "bf16", None),
    # d = 1024: the folds on the 128 x 256 tile over four column blocks
    # (four of the eight fold queues), rows ragged in every expert
    ("mid_fold", 700, 1024, 16, 4, 256, "bf16", None),
    ("many_empty", 50, 128, 256, 2, 128, "bf16", None),
    ("f32_k8", 200, 128, 16, 8, 128, "f32", 1.2),
    # the largest E (eight 128-expert blocks in dWg, almost every expert
    # empty) and the largest K with K = E
    ("experts_1024", 300, 128, 1024, 2, 128, "bf16", None),
    ("k_eq_e_32", 70, 128, 32, 32, 128, "bf16", None),
    # d = 6144: dH on the 128 x 256 tile (a long reduction), with h = 384 an
    # odd multiple of 128, so its last column block runs past h
    ("dh_mid_d6144", 200, 6144, 4, 2, 384, "bf16", None),
    # the skewed workload's tile choices at a small T: the dX fold on the
    # 256 x 256 tile with a reduction of 2h = 3072, six ranks per token, Zipf
    # skew (22 to 291 rows per expert, ragged in every 256-row block)
    ("wide_dx_k6", 300, 4096, 16, 6, 1536, "bf16", 1.2),
    # the large-d workload's tile choices: gate/up and the dW GEMMs on 256 x 256,
    # dH and down-combine on 128 x 256, the dX fold on 256 x 256 (reduction 4096)
    ("large_d_tiles", 200, 6144, 8, 4, 2048, "bf16", None),
]


def _gpu_layer(inp, wl, logits32=None, backward=True, saved="aby", combine="fold", dh_over_h=True):
    dt = wl.dtype
    buf = Lyr.MoEBuffers(wl.T, wl.d, wl.E, wl.K, wl.h, dt, backward=backward, saved=saved, combine=combine,
                         act=wl.act, dh_over_h=dh_over_h)
    dev = {k: (Lyr.to_device(inp[k], dt) if inp[k] is not None else None)
           for k in ("x", "wg", "w_gate", "w_up", "w_down", "dy") if k in inp}
    bias = torch.from_numpy(inp["bias"]).cuda() if inp.get("bias") is not None else None
    if logits32 is not None:
        buf.logits.copy_(torch.from_numpy(logits32))
    Lyr.forward(buf, dev["x"], dev["wg"], bias, dev["w_gate"], dev["w_up"], dev["w_down"],
                logits_in=logits32 is not None)
    buf.y_fwd = buf.y_swi.clone()       # an H-only backward writes A' over y_swi
    buf.h_fwd = buf.h_ab.clone() if buf.h_ab is not None else None   # the backward writes dH over h_ab
    if backward:
        Lyr.backward(buf, dev["dy"], dev["x"], dev["wg"], dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    return buf, dev


def _compare_layer(buf, inp, wl, z32, backward=True, report=None, w_rtol=2e-6, saved="aby"):
    T, K, E, h = wl.T, wl.K, wl.E, wl.h
    zz = z32.astype(np.float64)
    ids, w = O.route(zz, K)
    ix = O.build_index(ids, E)
    assert np.array_equal(to_np(buf.topk_ids), ids)
    np.testing.assert_allclose(to_np(buf.topk_w), w, rtol=w_rtol, atol=1e-7)
    assert np.array_equal(to_np(buf.offsets), ix["offsets"])
    assert np.array_equal(to_np(buf.eti), ix["expert_token_indices"])
    assert np.array_equal(to_np(buf.tim), ix["token_index_map"])
    gated = wl.act == "swiglu"
    f = O.moe_forward(inp["x"], ids, w, inp["w_gate"], inp["w_up"], inp["w_down"], dtype=wl.dtype, act=wl.act)
    pos = ix["token_index_map"].reshape(T, K)
    if getattr(buf, "h_fwd", None) is not None:   # H as the forward left it (the backward writes dH over it)
        hab = to_np(buf.h_fwd)[pos]     # [T,K,2h] (gated) or [T,K,h]
        assert_close("a", hab[..., :h], f["a_s"], report=report)
        if gated:
            assert_close("b", hab[..., h:], f["b_s"], report=report)
    if getattr(buf, "y_fwd", None) is not None:   # y as the forward left it (an H-only backward overwrites it)
        assert_close("y_swi", to_np(buf.y_fwd)[pos], f["y_s"], report=report)
    assert_close("out", to_np(buf.out), f["out"], report=report)
    if not backward:
        return
    bw = O.moe_backward(inp["dy"], inp["x"], inp["wg"], ids, w, inp["w_gate"], inp["w_up"], inp["w_down"], f, zz,
                        dtype=wl.dtype, saved=saved, act=wl.act)
    # the kernels form dS = <dA', y> with the y the backward sees
    assert_close("ds", to_np(buf.ds), bw["ds_alt"] if saved == "ab" else bw["ds"], report=report)
    assert_close("dx", to_np(buf.dx), bw["dx"], report=report)
    assert_close("dwg", to_np(buf.dwg), bw["dwg"], report=report)
    win = fp32_windows(inp["x"], inp["dy"], ids, inp["w_gate"], inp["w_up"], inp["w_down"], act=wl.act)
    fl = stored_flip_bounds(f, bw, w, wl.dtype, wl.act, saved, win)
    assert_close("dw_gate", to_np(buf.dw_gate), bw["dw_gate"], report=report,
                 allow=dw_flip_allowance(fl["da"], ids, inp["x"], E))
    if gated:
        assert_close("dw_up", to_np(buf.dw_up), bw["dw_up"], report=report,
                     allow=dw_flip_allowance(fl["db"], ids, inp["x"], E))
    assert_close("dw_down", to_np(buf.dw_down), bw["dw_down"], report=report,
                 allow=dw_flip_allowance(fl["ap"], ids, inp["dy"], E, transpose=True))
    if buf.dh_over_h:                   # h_ab now holds dH = [dA | dB], stored in the activation dtype
        dh = to_np(buf.h_ab)[pos]
        assert_close("dA", dh[..., :h], bw["dh_a"], report=report, allow=fl["da"])
        if gated:
            assert_close("dB", dh[..., h:], bw["dh_b"], report=report, allow=fl["db"])
    # experts without rows: exact zeros
    empty = np.nonzero(np.diff(ix["offsets"]) == 0)[0]
    for key in ("dw_gate", "dw_down", "dwg") + (("dw_up",) if gated else ()):
        assert np.all(to_np(getattr(buf, key))[empty] == 0.0), key


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_parity_from_logits(case):
    name, T, d, E, K, h, dtype, zipf = case
    _say("layer", case)
    wl = synth.small_workload(T, d, E, K, h, dtype=dtype, seed=sum(map(ord, name)), zipf_s=zipf)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    buf, _ = _gpu_layer(inp, wl, logits32=z32)
    assert buf.device_error_words() == [0, 0]
    _compare_layer(buf, inp, wl, z32)


# H-only is what the benchmark runs: every layer case, except the slowest
# oracle run (d = h = 4096), whose kernels the stored-y case above covers
H_ONLY_CASES = [c for c in LAYER_CASES if c[0] != "wide_fold"]


@pytest.mark.parametrize("case", H_ONLY_CASES, ids=[c[0] for c in H_ONLY_CASES])
def test_layer_parity_h_only(case):
    """H-only saving: the backward recomputes y from a, b (y_swi not passed)."""
    name, T, d, E, K, h, dtype, zipf = case
    _say("layer_h_only", case)
    wl = synth.small_workload(T, d, E, K, h, dtype=dtype, seed=sum(map(ord, name)) + 7, zipf_s=zipf)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    buf, _ = _gpu_layer(inp, wl, logits32=z32, saved="ab")
    assert buf.device_error_words() == [0, 0]
    _compare_layer(buf, inp, wl, z32, saved="ab")


def test_h_only_leaves_y_independent_gradients_unchanged():
    """dW_gate and dW_up do not depend on y: the two savings give them bit for bit."""
    T, d, E, K, h = 700, 256, 16, 4, 256
    _say("h_only_vs_aby", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=31)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    b1, _ = _gpu_layer(inp, wl, logits32=z32, saved="aby")
    b2, _ = _gpu_layer(inp, wl, logits32=z32, saved="ab")
    for key in ("out", "dw_gate", "dw_up"):
        assert torch.equal(getattr(b1, key), getattr(b2, key)), key
    assert not torch.equal(b1.dw_down, b2.dw_down)  # A' comes from a different y rounding


STAGED_CASES = [c for c in LAYER_CASES if c[0] in ("ragged", "multi_tile", "skewed", "t1", "tiny_f32", "k_eq_e")]


@pytest.mark.parametrize("case", STAGED_CASES, ids=[c[0] for c in STAGED_CASES])
def test_staged_combine_parity(case):
    """Staged-Y combine (ablation): same forward outputs within tolerance."""
    name, T, d, E, K, h, dtype, zipf = case
    _say("staged_combine", case)
    wl = synth.small_workload(T, d, E, K, h, dtype=dtype, seed=sum(map(ord, name)) + 3, zipf_s=zipf)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    buf, _ = _gpu_layer(inp, wl, logits32=z32, backward=False, combine="staged")
    _compare_layer(buf, inp, wl, z32, backward=False)


def test_staged_combine_repeatable_and_close_to_fold():
    T, d, E, K, h = 900, 256, 16, 4, 256
    _say("staged_vs_fold", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=41)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    a, _ = _gpu_layer(inp, wl, logits32=z32, backward=False, combine="staged")
    b, _ = _gpu_layer(inp, wl, logits32=z32, backward=False, combine="staged")
    c, _ = _gpu_layer(inp, wl, logits32=z32, backward=False, combine="fold")
    assert torch.equal(a.out, b.out)
    assert_close("staged_vs_fold", to_np(a.out), to_np(c.out))


PLAIN_CASES = [
    # name, T, d, E, K, h, dtype, act, saved
    ("silu_ragged", 300, 256, 8, 2, 256, "bf16", "silu", "aby"),
    ("relu_multi_tile", 1000, 384, 16, 4, 384, "bf16", "relu", "aby"),
    ("silu_h_only", 700, 256, 32, 6, 256, "bf16", "silu", "ab"),
    ("relu_h_only", 513, 256, 64, 8, 128, "bf16", "relu", "ab"),
    ("silu_f32", 256, 128, 8, 2, 256, "f32", "silu", "aby"),
    ("relu_k1", 200, 128, 4, 1, 128, "bf16", "relu", "aby"),
    ("silu_h_only_split_k", 8192, 256, 4, 1, 256, "bf16", "silu", "ab"),  # dW rows in 4 chunks
    # h = 4d as in MoEBlaze's shapes: the first layer and the dX fold (a
    # reduction of 4096) on the 256 x 256 tile, rows ragged in every expert
    ("silu_h4d_wide", 700, 1024, 8, 4, 4096, "bf16", "silu", "ab"),
]


@pytest.mark.parametrize("case", PLAIN_CASES, ids=[c[0] for c in PLAIN_CASES])
def test_layer_parity_plain_expert(case):
    """Plain two-layer experts W_2 sigma(W_1 x), sigma = SiLU or ReLU."""
    name, T, d, E, K, h, dtype, act, saved = case
    _say("layer_plain", case)
    wl = synth.small_workload(T, d, E, K, h, dtype=dtype, seed=sum(map(ord, name)), act=act)
    inp = synth.make_inputs(wl)
    assert inp["w_up"] is None
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    buf, _ = _gpu_layer(inp, wl, logits32=z32, saved=saved)
    assert buf.device_error_words() == [0, 0]
    _compare_layer(buf, inp, wl, z32, saved=saved)


@pytest.mark.parametrize("kind", ["one_expert_set", "zero_rows", "hot_expert"])
def test_layer_parity_structured_routing(kind):
    T, d, E, K, h = 600, 256, 16, 4, 128
    _say("layer_structured", kind)
    wl = synth.small_workload(T, d, E, K, h, seed=5)
    inp = synth.make_inputs(wl)
    z32 = synth.structured_logits(T, E, K, kind, seed=17)
    buf, _ = _gpu_layer(inp, wl, logits32=z32)
    assert buf.device_error_words() == [0, 0]
    _compare_layer(buf, inp, wl, z32)


def test_layer_router_end_to_end():
    """Router logits computed on the GPU: ids must agree with the oracle's
    decision on its own float32-rounded logits except at near ties."""
    T, d, E, K, h = 800, 512, 32, 4, 256
    _say("layer_e2e_router", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=23, zipf_s=1.2)
    inp = synth.make_inputs(wl)
    buf, _ = _gpu_layer(inp, wl)
    z = O.router_logits(inp["x"], inp["wg"], inp["bias"])
    zg = to_np(buf.logits)
    dz = np.abs(zg - z).max()
    assert dz < 1e-4
    ids_ref = O.topk_select(z.astype(np.float32), K)
    mism = np.nonzero((to_np(buf.topk_ids) != ids_ref).any(axis=1))[0]
    margin = topk_margin(z.astype(np.float32), K)
    assert np.all(margin[mism] <= 4 * dz), "routing differs away from a near tie"
    if len(mism) == 0:
        # the oracle keeps its own logits; the weights then differ only by the
        # logits' float32 accumulation error
        _compare_layer(buf, inp, wl, z.astype(np.float32), w_rtol=1e-4)


def test_bitwise_repeatable():
    T, d, E, K, h = 1000, 256, 16, 4, 256
    _say("repeat", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=3)
    inp = synth.make_inputs(wl)
    b1, _ = _gpu_layer(inp, wl)
    b2, _ = _gpu_layer(inp, wl)
    for key in ("topk_ids", "topk_w", "eti", "tim", "h_fwd", "h_ab", "y_fwd", "y_swi", "out", "dx", "dwg",
                "dw_gate", "dw_up", "dw_down", "ds"):
        assert torch.equal(getattr(b1, key), getattr(b2, key)), key


@pytest.mark.parametrize("saved", ["aby", "ab"])
def test_dh_over_saved_h_matches_the_workspace_dh(saved):
    """dH written over the saved H (the lean backward workspace) gives the
    same gradients, bit for bit, as dH in the workspace, and as dH in a
    caller buffer of its own; h_ab then holds dH in the first case and still
    holds H in the others."""
    T, d, E, K, h = 700, 1024, 16, 4, 512
    _say("dh_over_h", saved, T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=29, zipf_s=1.2)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    lean, _ = _gpu_layer(inp, wl, logits32=z32, saved=saved, dh_over_h=True)
    full, _ = _gpu_layer(inp, wl, logits32=z32, saved=saved, dh_over_h=False)
    assert lean.ws_main.numel() < full.ws_main.numel()
    assert lean.device_error_words() == [0, 0] and full.device_error_words() == [0, 0]
    for key in ("h_fwd", "y_fwd", "y_swi", "out", "dx", "dwg", "dw_gate", "dw_up", "dw_down", "ds"):
        assert torch.equal(getattr(lean, key), getattr(full, key)), key
    assert torch.equal(full.h_ab, full.h_fwd)
    assert not torch.equal(lean.h_ab, lean.h_fwd)
    _compare_layer(lean, inp, wl, z32, saved=saved)
    # dH in a buffer of its own (neither h_ab nor the workspace): the same dH
    # and gradients, with the saved H left as it was
    sep, dev = _gpu_layer(inp, wl, logits32=z32, saved=saved, dh_over_h=False)
    dh = torch.full_like(sep.h_ab, -7.0)
    for key in ("dx", "dwg", "dw_gate", "dw_up", "dw_down", "ds"):   # every output written again
        getattr(sep, key).fill_(float("nan"))
    honly = saved == "ab"
    B.moe_expert_bwd(sep.shape, dev["dy"], dev["x"], dev["wg"], dev["w_gate"], dev["w_up"], dev["w_down"],
                     sep.topk_ids, sep.topk_w, sep.offsets, sep.eti, sep.tim, sep.h_ab,
                     None if honly else sep.y_swi, sep.y_swi if honly else None, dh, sep.dx, sep.dwg, sep.dw_gate,
                     sep.dw_up, sep.dw_down, sep.ds, sep.ws_main)
    torch.cuda.synchronize()
    assert sep.device_error_words() == [0, 0]
    assert torch.equal(dh, lean.h_ab)
    assert torch.equal(sep.h_ab, sep.h_fwd)
    for key in ("dx", "dwg", "dw_gate", "dw_up", "dw_down", "ds"):
        assert torch.equal(getattr(sep, key), getattr(lean, key)), key


def test_bounded_wait_reports_and_finishes():
    """Error path of the ordered fold, forced from the host: with a wait limit
    of one poll, a contribution whose predecessor has not folded yet gives up,
    sets the workspace error word and its kernel still finishes.  Every token
    chooses every expert (K = E), so the rows of expert e wait on those of
    expert e - 1, whose tiles run at the same time.  The next call, with the
    normal limit, is clean and matches the oracle."""
    T, d, E, K, h = 512, 128, 4, 4, 128
    _say("bounded_wait", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=17)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    prev = B.set_spin_limit(1)
    try:
        bad, _ = _gpu_layer(inp, wl, logits32=z32)
        words = bad.device_error_words()
    finally:
        B.set_spin_limit(prev)
    assert words != [0, 0], "no wait ran out with a limit of one poll"
    good, _ = _gpu_layer(inp, wl, logits32=z32)
    assert good.device_error_words() == [0, 0]
    _compare_layer(good, inp, wl, z32)


def test_graph_capture_replays_match_eager():
    """The five entry points enqueue kernels only (no allocation, copy, memset
    or host wait, no routing-dependent launch size), so a forward + backward
    captures into one HIP graph.  Each replay, after eager work that
    overwrites every output, reproduces the eager results bit for bit."""
    T, d, E, K, h = 600, 256, 16, 4, 256
    _say("graph", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=23, zipf_s=1.2)
    inp = synth.make_inputs(wl)
    dev = {k: Lyr.to_device(inp[k], "bf16") for k in ("x", "wg", "w_gate", "w_up", "w_down", "dy")}
    bias = torch.from_numpy(inp["bias"]).cuda()
    buf = Lyr.MoEBuffers(T, d, E, K, h, "bf16", backward=True)
    keys = ("logits", "topk_ids", "topk_w", "offsets", "eti", "tim", "h_ab", "y_swi", "out", "dx", "dwg",
            "dw_gate", "dw_up", "dw_down", "ds")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def step():
        sp = torch.cuda.current_stream().cuda_stream
        Lyr.forward(buf, dev["x"], dev["wg"], bias, dev["w_gate"], dev["w_up"], dev["w_down"], stream=sp)
        Lyr.backward(buf, dev["dy"], dev["x"], dev["wg"], dev["w_gate"], dev["w_up"], dev["w_down"], stream=sp)

    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    assert buf.device_error_words() == [0, 0]
    ref = {k: getattr(buf, k).clone() for k in keys}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        for k in keys:                       # eager work between the replays
            getattr(buf, k).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert buf.device_error_words() == [0, 0], i
        for k in keys:
            assert torch.equal(getattr(buf, k), ref[k]), (i, k)


@pytest.mark.parametrize("act", ["swiglu", "silu"])
def test_forward_without_saving(act):
    """A forward that no backward follows may pass h_ab = NULL: nothing is
    stored but y_swi, and the output and y are those of the saving forward,
    bit for bit, and the oracle's."""
    T, d, E, K, h = 300, 256, 8, 2, 256
    _say("forward_no_save", act)
    wl = synth.small_workload(T, d, E, K, h, seed=31, act=act, backward=False)
    inp = synth.make_inputs(wl)
    z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
    dev = {k: Lyr.to_device(inp[k], "bf16") for k in ("x", "wg", "w_gate", "w_up", "w_down") if inp[k] is not None}
    outs = []
    for save in (True, False):
        buf = Lyr.MoEBuffers(T, d, E, K, h, "bf16", backward=False, act=act, save=save)
        assert (buf.h_ab is None) == (not save)
        buf.logits.copy_(torch.from_numpy(z32))
        Lyr.forward(buf, dev["x"], dev["wg"], None, dev["w_gate"], dev.get("w_up"), dev["w_down"], logits_in=True)
        torch.cuda.synchronize()
        assert buf.device_error_words() == [0]
        outs.append(buf)
    assert torch.equal(outs[0].out, outs[1].out)
    assert torch.equal(outs[0].y_swi, outs[1].y_swi)
    ids, w = O.route(z32.astype(np.float64), K)
    f = O.moe_forward(inp["x"], ids, w, inp["w_gate"], inp["w_up"], inp["w_down"], dtype="bf16", act=act)
    assert_close("out", to_np(outs[1].out), f["out"])


# ---------------------------------------------------------------------------
# forced tile choices (the tuning switches are read once per process, so each
# setting runs in a child process of its own)
# ---------------------------------------------------------------------------
FORCED_TILE_CASES = ["ragged", "multi_tile", "skewed", "mid_fold", "dh_mid_d6144", "f32_bwd", "k16"]


def run_cases_in_this_process(names):
    """Run the named layer cases (both savings) and report; used by the child processes."""
    byname = {c[0]: c for c in LAYER_CASES}
    B.lib()
    for name in names:
        for saved in ("aby", "ab"):
            _, T, d, E, K, h, dtype, zipf = byname[name]
            print("[child case]", name, saved, os.environ.get("MOE_DISPATCH_TILE"),
                  os.environ.get("MOE_DISPATCH_MID"), file=sys.stderr, flush=True)
            wl = synth.small_workload(T, d, E, K, h, dtype=dtype, seed=sum(map(ord, name)) + 11, zipf_s=zipf)
            inp = synth.make_inputs(wl)
            z32 = O.router_logits(inp["x"], inp["wg"], inp["bias"]).astype(np.float32)
            buf, _ = _gpu_layer(inp, wl, logits32=z32, saved=saved)
            assert buf.device_error_words() == [0, 0]
            _compare_layer(buf, inp, wl, z32, saved=saved)
    print("child ok", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("env", [{"MOE_DISPATCH_TILE": "256"}, {"MOE_DISPATCH_TILE": "128"},
                                 {"MOE_DISPATCH_MID": "1"}, {"MOE_DISPATCH_MID": "0"}],
                         ids=["tile256", "tile128", "mid_on", "mid_off"])
def test_layer_parity_under_forced_tiles(env):
    """Layer parity with every expert GEMM forced onto one tile (256 x 256 or
    128 x 128), or the 128 x 256 tile forced on or off, one child process per
    setting (the switches are read once per process)."""
    _say("forced tiles", env)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r); from tests.test_gpu_parity import run_cases_in_this_process as r; "
            "r(%r)" % (root, FORCED_TILE_CASES))
    child_env = dict(os.environ, **env)
    p = subprocess.run([sys.executable, "-c", code], env=child_env, cwd=root, capture_output=True, text=True,
                       timeout=540)
    assert p.returncode == 0 and "child ok" in p.stdout, (p.returncode, p.stdout[-2000:], p.stderr[-4000:])


# ---------------------------------------------------------------------------
# HIP graph replay under changed routing
# ---------------------------------------------------------------------------
def test_graph_replay_follows_changed_routing():
    """A forward + backward captured once, replayed after x and the router
    bias change in place: new routing each time (one replay with an expert
    emptied by the bias, one with a hot expert), so the counts, tile maps and
    fold order all differ from those at capture.  Every replay equals an
    eager run on the same inputs bit for bit, and matches the oracle."""
    T, d, E, K, h = 500, 256, 16, 4, 256
    _say("graph_routing", T, d, E, K, h)
    wl = synth.small_workload(T, d, E, K, h, seed=61)
    inp = synth.make_inputs(wl)
    dev = {k: Lyr.to_device(inp[k], "bf16") for k in ("x", "wg", "w_gate", "w_up", "w_down", "dy")}
    bias_dev = torch.zeros(E, dtype=torch.float32, device="cuda")
    keys = ("logits", "topk_ids", "topk_w", "offsets", "eti", "tim", "h_ab", "out", "dx", "dwg", "dw_gate", "dw_up",
            "dw_down", "ds")
    gbuf = Lyr.MoEBuffers(T, d, E, K, h, "bf16", backward=True, saved="ab")
    ebuf = Lyr.MoEBuffers(T, d, E, K, h, "bf16", backward=True, saved="ab")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def step(buf):
        sp = torch.cuda.current_stream().cuda_stream
        Lyr.forward(buf, dev["x"], dev["wg"], bias_dev, dev["w_gate"], dev["w_up"], dev["w_down"], stream=sp)
        Lyr.backward(buf, dev["dy"], dev["x"], dev["wg"], dev["w_gate"], dev["w_up"], dev["w_down"], stream=sp)

    with torch.cuda.stream(side):
        step(gbuf)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(gbuf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    variants = []
    for i in range(3):
        x = synth.round_to_bf16(rng.standard_normal((T, d)).astype(np.float32))
        b = np.zeros(E, np.float32)
        if i == 1:
            b[3] = -60.0          # expert 3 gets no rows
        if i == 2:
            b[9] = 8.0            # expert 9 is in nearly every token's set
        variants.append((x, b))
    seen_counts = []
    for i, (x, b) in enumerate(variants):
        dev["x"].copy_(torch.from_numpy(x))
        bias_dev.copy_(torch.from_numpy(b))
        for k in keys:                        # eager work between the replays
            getattr(gbuf, k).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(ebuf)
        torch.cuda.synchronize()
        assert gbuf.device_error_words() == [0, 0], i
        for k in keys:
            assert torch.equal(getattr(gbuf, k), getattr(ebuf, k)), (i, k)
        counts = np.diff(to_np(gbuf.offsets))
        seen_counts.append(counts)
        if i == 1:
            assert counts[3] == 0
        if i == 2:
            assert counts[9] > 0.9 * T
        # the oracle routes on its own logits; the ids must agree but at near ties
        inp_i = dict(inp, x=x, bias=b)
        z = O.router_logits(x, inp["wg"], b)
        dz = float(np.abs(to_np(gbuf.logits) - z).max())
        assert dz < 1e-4, dz
        z32 = z.astype(np.float32)
        mism = np.nonzero((to_np(gbuf.topk_ids) != O.topk_select(z32, K)).any(axis=1))[0]
        assert np.all(topk_margin(z32, K)[mism] <= 4 * dz), "routing differs away from a near tie"
        if len(mism) == 0:
            _compare_layer(gbuf, inp_i, wl, z32, w_rtol=1e-4, saved="ab")
    assert not np.array_equal(seen_counts[0], seen_counts[1]) and not np.array_equal(seen_counts[1], seen_counts[2])
