"""Microbenchmark of the routing-index construction on one MI355X.

Three ways to build the same arrays (expert_token_offsets,
expert_token_indices, token_index_map) from the top-K ids:
  ballot -- moe_build_index: wave-ballot token masks, a scan of the
            [E][chunk] counts, a conflict-free scatter (the default backend);
  dense  -- moe_build_index_dense: MoEBlaze's three steps taken literally,
            with a dense [E][T] token-expert map;
  sort   -- the sorting method the MoEBlaze page contrasts them with: a
            stable device sort of the flattened ids (torch.sort, stable=True),
            then the index recovered from the order.

Every case first checks that the three agree bit for bit, then times each
with HIP events (median of --reps launches after --warmup).  Prints one JSON
line per case.  Inputs: seeded top-K ids from Gaussian logits, optionally with
a Zipf(s) per-expert offset (skew).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CASES = [  # T, E, K, zipf
    (16384, 128, 8, None), (16384, 128, 8, 1.2), (32768, 64, 4, None), (16384, 64, 6, 1.2),
    (4096, 8, 2, None), (131072, 256, 8, None), (262144, 64, 4, None), (65536, 1024, 8, None),
]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args()
    import numpy as np
    import torch
    from dropless_moe_dispatch_amd import binding as B
    from dropless_moe_dispatch_amd import synth

    torch.cuda.set_device(0)
    for T, E, K, zipf in CASES:
        rng = np.random.default_rng(T * 31 + E)
        z = rng.standard_normal((T, E)).astype(np.float32)
        if zipf:
            z += synth.zipf_bias(E, E, zipf).astype(np.float32)
        ids = torch.from_numpy(np.argsort(-z, axis=1, kind="stable")[:, :K].astype(np.int32)).cuda()
        s = B.shape(T, 128, E, K, 128)
        A = T * K
        outs = {}
        for name in ("ballot", "dense", "sort"):
            outs[name] = (torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                          torch.empty(A, dtype=torch.int32, device="cuda"),
                          torch.empty(A, dtype=torch.int32, device="cuda"))
        ws_b = torch.empty(B.workspace_bytes(s, B.MOE_WS_INDEX), dtype=torch.uint8, device="cuda")
        ws_d = torch.empty(B.workspace_bytes(s, B.MOE_WS_INDEX_DENSE), dtype=torch.uint8, device="cuda")
        flat = ids.view(-1)

        def run_ballot():
            o = outs["ballot"]
            B.moe_build_index(s, ids, o[0], o[1], o[2], ws_b)

        def run_dense():
            o = outs["dense"]
            B.moe_build_index_dense(s, ids, o[0], o[1], o[2], ws_d)

        def run_sort():
            off, eti, tim = outs["sort"]
            _, order = torch.sort(flat, stable=True)
            eti.copy_((order // K).to(torch.int32))
            tim.index_copy_(0, order, torch.arange(A, dtype=torch.int32, device="cuda"))
            off[0] = 0
            off[1:].copy_(torch.cumsum(torch.bincount(flat, minlength=E), 0))

        runs = {"ballot": run_ballot, "dense": run_dense, "sort": run_sort}
        for f in runs.values():
            f()
        torch.cuda.synchronize()
        for name in ("dense", "sort"):
            for a, b in zip(outs["ballot"], outs[name]):
                assert torch.equal(a, b), (name, T, E, K, zipf)
        times = {}
        for name, f in runs.items():
            for _ in range(args.warmup):
                f()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.reps)]
            for e0, e1 in ev:
                e0.record()
                f()
                e1.record()
            torch.cuda.synchronize()
            times[name] = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3  # us
        nbytes = 4 * A + 8 * A + 4 * (E + 1)   # ids in, index out
        print(json.dumps({"T": T, "E": E, "K": K, "zipf": zipf, "us": {k: round(v, 1) for k, v in times.items()},
                          "ballot_GBs": round(nbytes / (times["ballot"] * 1e-6) / 1e9, 1),
                          "workspace_MB": {"ballot": round(ws_b.numel() / 1e6, 2), "dense": round(ws_d.numel() / 1e6, 2)},
                          "identical": True}), flush=True)


if __name__ == "__main__":
    main()
