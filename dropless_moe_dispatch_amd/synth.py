"""Seeded synthetic inputs for the dropless MoE layer.

This module only draws random numbers and shapes them into inputs; it contains
none of the layer's arithmetic (no routing, no GEMM, no activation).  The same
bytes are handed to the GPU library and to the CPU oracle.

Generator: numpy's Philox-4x32 counter-based bit generator, one independent
key per tensor, so any tensor of a workload can be regenerated without drawing
the others.  Normal variates come from numpy's ``standard_normal`` in float32
and are scaled, then rounded to bfloat16 with round-to-nearest-even when the
workload is bf16 (the rounded values are kept as exactly representable
float32).

Workload shapes follow the five synthetic single-layer cases used to evaluate
the method (token-choice top-K routing with renormalised weights and SwiGLU
experts); ``x ~ N(0,1)``, router and expert weights ``~ N(0, 1/sqrt(fan_in))``
(standard deviation ``1/sqrt(fan_in)``: ``d`` for the router, gate and up
projections, ``h`` for the down projection), ``dY ~ N(0,1)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    K: int
    h: int
    dtype: str            # "f32" or "bf16"
    backward: bool
    zipf_s: Optional[float] = None
    seed: int = 0
    note: str = field(default="", compare=False)
    act: str = "swiglu"   # "swiglu" (gated expert) or "silu" / "relu" (plain two-layer expert)
    zipf_draw: int = 0    # which draw of the Zipf permutation stream ranks the experts


# The five evaluation workloads.  Index i (1-based) uses seed 1000 + i.
WORKLOADS = {
    1: Workload("tiny_fwd_f32", 256, 128, 8, 2, 256, "f32", False, seed=1001,
                note="tiny forward, fp32"),
    2: Workload("coarse_fwd_bf16", 4096, 4096, 8, 2, 14336, "bf16", False, seed=1002,
                note="coarse experts, forward, near-balanced load"),
    3: Workload("fine_fwdbwd_bf16", 16384, 2048, 128, 8, 768, "bf16", True, seed=1003,
                note="fine-grained experts, forward + backward"),
    4: Workload("large_d_fwdbwd_bf16", 32768, 6144, 64, 4, 2048, "bf16", True, seed=1004,
                note="large model dimension, forward + backward"),
    # The skewed workload names its outcome: a few experts above 10% of the
    # assignments and several under 16 rows.  The Zipf(1.2) offset (zipf_bias)
    # fixes the shape of the skew; which expert gets which popularity rank is
    # a seeded permutation, and draw 11 of its stream is the first whose
    # routing of this workload's tokens shows that outcome (3 experts above
    # 10%, 4 under 16 rows, the smallest with 11; draws 0-10 leave at most 2
    # under 16 rows).  tests/test_workloads_cpu.py recomputes this with the
    # oracle.  No draw empties an expert: the least popular one is offset by
    # -1.2 ln 64 = -5.0 against N(0,1) logits.
    5: Workload("skewed_fwdbwd_bf16", 16384, 4096, 64, 6, 1536, "bf16", True, zipf_s=1.2,
                seed=1005, note="Zipf(1.2) per-expert logit offset, forward + backward", zipf_draw=11),
    # MoEBlaze's own evaluation shapes (reading notes, Table 1: the printed
    # conf1, conf3, conf4 and conf7; T = batch x sequence, h = 4d) with the
    # plain two-layer SiLU expert of its Figure 3 comparison.
    6: Workload("moeblaze_conf1_silu", 32 * 2048, 512, 4, 1, 2048, "bf16", True, seed=1006, act="silu",
                note="MoEBlaze conf1: d=512, E=4, K=1, B=32, L=2048"),
    7: Workload("moeblaze_conf3_silu", 32 * 2048, 1024, 16, 4, 4096, "bf16", True, seed=1007, act="silu",
                note="MoEBlaze conf3: d=1024, E=16, K=4, B=32, L=2048"),
    8: Workload("moeblaze_conf4_silu", 32 * 1024, 2048, 16, 4, 8192, "bf16", True, seed=1008, act="silu",
                note="MoEBlaze conf4: d=2048, E=16, K=4, B=32, L=1024"),
    9: Workload("moeblaze_conf7_silu", 16 * 512, 2048, 8, 4, 8192, "bf16", True, seed=1009, act="silu",
                note="MoEBlaze conf7: d=2048, E=8, K=4, B=16, L=512"),
}

_TENSOR_KEYS = {"x": 1, "wg": 2, "w_gate": 3, "w_up": 4, "w_down": 5, "dy": 6,
                "zipf_perm": 7, "logits": 8}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((bits + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, tensor: str, draw: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=seed * 64 + _TENSOR_KEYS[tensor] + draw * (1 << 40)))


def normal(seed: int, tensor: str, shape, std: float, dtype: str, chunk: int = 1 << 26) -> np.ndarray:
    """N(0, std^2) samples of ``shape`` in float32, bf16-rounded when dtype == 'bf16'."""
    g = _rng(seed, tensor)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = g.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if dtype == "bf16":
            v = round_to_bf16(v)
        out[s:e] = v
    return out.reshape(shape)


def zipf_bias(seed: int, E: int, s: float, draw: int = 0) -> np.ndarray:
    """Per-expert logit offset b_e = -s * ln(r_e), r a seeded permutation of 1..E
    (draw ``draw`` of the permutation stream).

    Adding b to Gaussian logits multiplies expert e's odds by r_e^-s, i.e. a
    Zipf(s) popularity profile over a random ranking of the experts.
    """
    r = _rng(seed, "zipf_perm", draw).permutation(E).astype(np.float64) + 1.0
    return (-s * np.log(r)).astype(np.float32)


def make_inputs(wl: Workload, tensors=("x", "wg", "w_gate", "w_up", "w_down", "dy"), T: Optional[int] = None):
    """Generate the requested tensors of workload ``wl`` (float32 numpy arrays).

    ``T`` optionally truncates the token dimension (x and dy are the first T
    rows of the full-size tensors, weights are unchanged).
    """
    T_full = wl.T
    T = T_full if T is None else T
    out = {}
    for name in tensors:
        if name == "x":
            out[name] = normal(wl.seed, "x", (T_full, wl.d), 1.0, wl.dtype)[:T].copy() if T != T_full \
                else normal(wl.seed, "x", (T_full, wl.d), 1.0, wl.dtype)
        elif name == "dy":
            out[name] = normal(wl.seed, "dy", (T_full, wl.d), 1.0, wl.dtype)[:T].copy() if T != T_full \
                else normal(wl.seed, "dy", (T_full, wl.d), 1.0, wl.dtype)
        elif name == "wg":
            out[name] = normal(wl.seed, "wg", (wl.E, wl.d), 1.0 / np.sqrt(wl.d), wl.dtype)
        elif name == "w_gate":
            out[name] = normal(wl.seed, "w_gate", (wl.E, wl.h, wl.d), 1.0 / np.sqrt(wl.d), wl.dtype)
        elif name == "w_up":   # a plain two-layer expert has no up projection
            out[name] = normal(wl.seed, "w_up", (wl.E, wl.h, wl.d), 1.0 / np.sqrt(wl.d), wl.dtype) \
                if wl.act == "swiglu" else None
        elif name == "w_down":
            out[name] = normal(wl.seed, "w_down", (wl.E, wl.d, wl.h), 1.0 / np.sqrt(wl.h), wl.dtype)
        else:
            raise KeyError(name)
    out["bias"] = zipf_bias(wl.seed, wl.E, wl.zipf_s, wl.zipf_draw) if wl.zipf_s else None
    return out


def small_workload(T, d, E, K, h, dtype="bf16", seed=7, zipf_s=None, backward=True, name="small", act="swiglu"):
    return Workload(name, T, d, E, K, h, dtype, backward, zipf_s=zipf_s, seed=seed, act=act)


# ---------------------------------------------------------------------------
# Router-logit inputs with a prescribed structure, for exercising routing and
# the index on edge cases directly (logits are an input of the router stage).
# ---------------------------------------------------------------------------
def structured_logits(T: int, E: int, K: int, kind: str, seed: int = 11) -> np.ndarray:
    g = _rng(seed, "logits")
    z = g.standard_normal((T, E), dtype=np.float32)
    if kind == "gaussian":
        pass
    elif kind == "one_expert_set":
        # every token prefers experts 0..K-1: those experts get every token,
        # all others get none.
        z[:, :K] += np.float32(50.0)
    elif kind == "zero_rows":
        # the upper half of the experts is never chosen (when K <= E/2).
        z[:, E // 2:] -= np.float32(50.0)
    elif kind == "ties":
        # small integer logits: many exact ties, exercising the tie-break.
        z = np.floor(z * 1.5).astype(np.float32)
    elif kind == "all_equal":
        z[:] = np.float32(0.25)
    elif kind == "hot_expert":
        # one expert is in nearly every token's set (skew).
        z[:, E - 1] += np.float32(6.0)
    elif kind == "sparse_experts":
        # extreme imbalance: experts 0-2 are never chosen, experts 3, 4 and 5
        # by exactly 1, 5 and 15 tokens (seeded choice), experts 6 and 7 by
        # nearly every token (needs E >= 10 and K >= 4).
        z[:, 0:6] -= np.float32(50.0)
        for i, n in enumerate((1, 5, 15)):
            z[g.choice(T, size=n, replace=False), 3 + i] += np.float32(100.0)
        z[:, 6] += np.float32(5.0)
        z[:, 7] += np.float32(4.0)
    else:
        raise KeyError(kind)
    return np.ascontiguousarray(z)
