"""Device buffers and the call sequence of one MoE layer through the C-ABI.

torch is used for device memory and the stream only; every computation is a
library kernel.  ``MoEBuffers`` allocates every output and workspace once for
a shape (sizes do not depend on the routing); ``forward``/``backward`` enqueue
the five entry points in order on the current stream with no host sync.

Memory: the expert forward, the combine and the backward share one workspace
(the library allows it for calls ordered on one stream), and under H-only
saving the backward writes A' = w * y into the forward's y_swi buffer, which
is dead once the combine has read it.  So y_swi holds A' after a backward.
By default the backward also writes dH over the saved H (``dh_over_h``): the
dH kernel is the last reader of H, so the workspace needs no [T*K, 2h] dH
buffer, and h_ab holds dH after a backward.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@dataclass
class MoEBuffers:
    T: int
    d: int
    E: int
    K: int
    h: int
    dtype: str = "bf16"
    backward: bool = True
    device: str = "cuda"
    # what the forward keeps for the backward: "aby" = a, b and y (MoEBlaze
    # Algorithm 1); "ab" = only H = [a | b] (SonicMoE's minimal cached set):
    # y_swi is then a forward transient and the backward recomputes y
    saved: str = "aby"
    # forward combine: "fold" (the ordered, buffer-free combine) or "staged"
    # (the staged-Y ablation, which holds a [T*K, d] buffer in its workspace)
    combine: str = "fold"
    # expert kind: "swiglu" (gated) or "silu" / "relu" (plain two-layer
    # expert: W_1 in the w_gate slot, no w_up, h_ab holds a only)
    act: str = "swiglu"
    # keep a|b from the forward (always, when a backward follows); a forward
    # alone may save nothing (h_ab is then None and not written)
    save: bool = True
    # the backward writes dH over the saved H (h_ab), its last reader being
    # the dH kernel: no dH buffer in the workspace, and H is gone afterwards
    dh_over_h: bool = True

    def __post_init__(self):
        dev, td = self.device, torch_dtype(self.dtype)
        T, d, E, K, h = self.T, self.d, self.E, self.K, self.h
        self.shape = B.shape(T, d, E, K, h, self.dtype, self.act)
        hw = 2 * h if self.act == "swiglu" else h
        A = T * K
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty(T, E, dtype=f32, device=dev)
        self.topk_ids = torch.empty(T, K, dtype=i32, device=dev)
        self.topk_w = torch.empty(T, K, dtype=f32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.eti = torch.empty(A, dtype=i32, device=dev)
        self.tim = torch.empty(A, dtype=i32, device=dev)
        self.h_ab = torch.empty(A, hw, dtype=td, device=dev) if (self.save or self.backward) else None
        self.y_swi = torch.empty(A, h, dtype=td, device=dev)
        self.out = torch.empty(T, d, dtype=td, device=dev)
        self.ws_index = self._ws(B.MOE_WS_INDEX)
        if self.combine not in ("fold", "staged"):
            raise ValueError(f"combine must be 'fold' or 'staged', not {self.combine!r}")
        if self.saved not in ("aby", "ab"):
            raise ValueError(f"saved must be 'aby' or 'ab', not {self.saved!r}")
        # one workspace for the expert forward, the ordered combine and the
        # backward (H-only: A' goes to y_swi, so the smaller backward kind;
        # dH over H: the lean one, without a dH buffer)
        bwd_kind = B.MOE_WS_EXPERT_BWD_LEAN if self.dh_over_h else B.MOE_WS_EXPERT_BWD
        kinds = [B.MOE_WS_EXPERT_FWD] + ([B.MOE_WS_COMBINE] if self.combine == "fold" else []) \
            + ([bwd_kind] if self.backward else [])
        self.ws_main = self._ws(*kinds)
        self.ws_comb = self.ws_main if self.combine == "fold" else self._ws(B.MOE_WS_COMBINE_STAGED)
        if self.backward:
            self.dx = torch.empty(T, d, dtype=td, device=dev)
            self.dwg = torch.empty(E, d, dtype=f32, device=dev)
            self.dw_gate = torch.empty(E, h, d, dtype=f32, device=dev)
            self.dw_up = torch.empty(E, h, d, dtype=f32, device=dev) if self.act == "swiglu" else None
            self.dw_down = torch.empty(E, d, h, dtype=f32, device=dev)
            self.ds = torch.empty(T, K, dtype=f32, device=dev)

    def _ws(self, *kinds):
        sizes = [B.workspace_bytes(self.shape, k) for k in kinds]
        if min(sizes) == 0:
            raise B.MoeError("moe_workspace_bytes", B.MOE_ERR_INVALID_ARG)
        return torch.empty(max(sizes), dtype=torch.uint8, device=self.device)

    # -- accounting ---------------------------------------------------------
    def saved_for_backward_bytes(self) -> int:
        """Activations kept from the forward for the backward: a|b, y_swi
        (unless H-only), the top-K ids and weights, and the index arrays."""
        if self.h_ab is None:
            return 0
        ts = [self.h_ab, self.topk_ids, self.topk_w, self.offsets, self.eti, self.tim]
        if self.saved == "aby":
            ts.append(self.y_swi)
        return sum(t.numel() * t.element_size() for t in ts)

    def weight_grad_bytes(self) -> int:
        """The fp32 weight gradients (dWg, dW_gate, dW_up, dW_down)."""
        if not self.backward:
            return 0
        return sum(t.numel() * t.element_size() for t in (self.dwg, self.dw_gate, self.dw_up, self.dw_down)
                   if t is not None)

    def workspace_bytes(self) -> int:
        ws = [self.ws_index, self.ws_main] + ([self.ws_comb] if self.ws_comb is not self.ws_main else [])
        return sum(t.numel() for t in ws)

    def device_error_words(self):
        """Error words of the ordered folds (nonzero: a bounded wait ran
        out): the combine's (bytes 0-3 of its workspace), then the
        backward's (bytes 4-7).  Synchronises with the device."""
        w = ([self.ws_comb[0:4]] if self.combine == "fold" else []) + ([self.ws_main[4:8]] if self.backward else [])
        return [int(x.view(torch.int32).item()) for x in w]

    def check_device_errors(self):
        """Raise MoeDeviceError if a fold's bounded wait ran out: out (or dx)
        of that call is then invalid although the call returned MOE_OK."""
        words = self.device_error_words()
        if any(words):
            names = (["moe_combine"] if self.combine == "fold" else []) + (["moe_expert_bwd"] if self.backward else [])
            bad = [n for n, w in zip(names, words) if w]
            raise B.MoeDeviceError(f"ordered fold wait ran out in {', '.join(bad)}: its output is invalid")


def route(buf: MoEBuffers, x, wg, bias=None, logits_in: bool = False, stream=None):
    B.moe_route_topk(buf.shape, None if logits_in else x, wg, bias, buf.logits, buf.topk_ids, buf.topk_w, stream)


def forward(buf: MoEBuffers, x, wg, bias, w_gate, w_up, w_down, logits_in: bool = False, stream=None):
    s = buf.shape
    route(buf, x, wg, bias, logits_in, stream)
    B.moe_build_index(s, buf.topk_ids, buf.offsets, buf.eti, buf.tim, buf.ws_index, stream)
    B.moe_expert_fwd(s, x, buf.offsets, buf.eti, w_gate, w_up, buf.h_ab, buf.y_swi, buf.ws_main, stream)
    comb = B.moe_combine if buf.combine == "fold" else B.moe_combine_staged
    comb(s, buf.y_swi, w_down, buf.offsets, buf.eti, buf.tim, buf.topk_ids, buf.topk_w, buf.out, buf.ws_comb, stream)
    return buf.out


def backward(buf: MoEBuffers, dy, x, wg, w_gate, w_up, w_down, stream=None, want_ds: bool = True):
    """H-only saving: y_swi is not passed as y, and receives A' (it is dead
    after the forward's combine).  With ``dh_over_h`` dH is written over
    h_ab."""
    honly = buf.saved == "ab"
    B.moe_expert_bwd(buf.shape, dy, x, wg, w_gate, w_up, w_down, buf.topk_ids, buf.topk_w, buf.offsets, buf.eti,
                     buf.tim, buf.h_ab, None if honly else buf.y_swi, buf.y_swi if honly else None,
                     buf.h_ab if buf.dh_over_h else None, buf.dx, buf.dwg, buf.dw_gate, buf.dw_up, buf.dw_down,
                     buf.ds if want_ds else None, buf.ws_main, stream)
    return buf.dx


def to_device(arr, dtype: str, device="cuda"):
    """float32 numpy array (already representable in ``dtype``) -> device tensor."""
    t = torch.from_numpy(arr).to(device)
    return t.to(torch_dtype(dtype)) if dtype == "bf16" else t
