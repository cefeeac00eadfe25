"""Benchmark: one dropless MoE layer, forward + backward, on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
router logits + top-K, counting-sort index, gathered gate/up GEMM with the
SwiGLU epilogue, down projection with the ordered combine, and the backward
(dH with SiLU recompute, router backward, dWg, dW_down, dW_gate/up, dX fold).
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line (see the keys below).  Per-kernel durations come from
HIP events recorded by the library around each of its launches, on the
launch stream, during the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3  # MI355X fp32 (MFMA and vector)
PEAK_HBM_GBS = 8000.0

METRIC = "MoE layer fwd+bwd tokens/s and TFLOP/s at 1 GPU; % bf16 MFMA peak; peak act MB"


def kernel_source_hash(csrc=None):
    """Hash of the HIP sources with their comments and blank lines taken out;
    counter data taken with other code is stale (a comment edit is not)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "dropless_moe_dispatch_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(csrc, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
            h.update(f.encode() + b"\0" + "\n".join(lines).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    (profiles/traffic_<workload>.json), if it was taken with these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("src_sha") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def kernel_flops(name, T, d, E, K, h, gated=True):
    """Model FLOP of one launch; a plain two-layer expert has one first-layer
    projection where the gated one has two (gate and up)."""
    A = T * K
    g = 2.0 if gated else 1.0
    return {
        "router_logits": 2.0 * T * d * E,
        "gate_up": 2.0 * g * A * d * h,
        "down_combine": 2.0 * A * d * h,
        "down_staged": 2.0 * A * d * h,
        "dh": 2.0 * A * d * h,
        "dw_down": 2.0 * A * d * h,
        "dw_gate_up": 2.0 * g * A * d * h,
        "dx_fold": 2.0 * g * A * d * h,
    }.get(name)


def kernel_bytes(name, T, d, E, K, h, eb, gated=True):
    """Algorithmic HBM bytes (operands once, outputs once): the memory-bound
    stages, and the two GEMMs with the fused combine, whose ordered fold moves
    (8K-6)·T·d (forward) and (8K-4)·T·d (dX) accumulator and output bytes."""
    A = T * K
    hw = 2 * h if gated else h
    return {
        "router_logits": eb * T * d + eb * E * d + 4 * T * E + (8 * A if E <= 128 else 0),
        "topk": 4 * T * E + 8 * A,
        "route": eb * T * d + eb * E * d + 4 * T * E + 8 * A,
        "index": 4 * A + 8 * A + 8 * E * ((T + 63) // 64),
        "router_bwd": 4 * T * d + eb * E * d + 16 * A,
        "dwg": eb * T * d + 4 * E * d + 8 * A,
        "down_combine": eb * A * h + eb * E * d * h + (8 * K - 6) * T * d,
        "dx_fold": eb * A * hw + eb * E * hw * d + (8 * K - 4) * T * d,
        "gather_sum": eb * A * d + eb * T * d + 8 * A,
    }.get(name)


def device_info():
    import torch
    info = {"rocm": getattr(torch.version, "hip", None)}
    try:
        p = torch.cuda.get_device_properties(0)
        info["gpu"] = getattr(p, "gcnArchName", None) or p.name
        info["cus"] = p.multi_processor_count
        clk = getattr(p, "clock_rate", None)
        if clk:
            info["max_clock_mhz"] = clk / 1000.0
    except Exception:  # pragma: no cover
        pass
    return info


NOMINAL_CLOCK_MHZ = 2400.0  # the clock the published MFMA peaks assume


class ClockSampler:
    """GFX clock under the benchmark's load: amdsmi's current-clock query
    (read-only), sampled every ``period`` seconds from a background thread
    while the same step runs for ``duration`` seconds after the timed steps;
    samples from the first ``settle`` seconds are dropped (the library's
    metrics lag by a fraction of a second).  Under sustained MFMA load the
    chip runs well below the clock the published peaks assume, so the
    fractions are also reported against the peak at the measured clock.
    Everything is None where amdsmi is unavailable."""

    def __init__(self, period=0.05, duration=1.5, settle=0.6):
        import threading
        self.period = period
        self.duration = duration
        self.settle = settle
        self.samples = []
        self.error = None
        self.handle = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            self.handle = self._pick(amdsmi.amdsmi_get_processor_handles())
            if self.handle is None:
                self.error = "no amdsmi handle matches the device"
        except Exception as e:  # pragma: no cover - depends on the host
            self.error = repr(e)[:160]

    def _pick(self, handles):
        if len(handles) == 1:
            return handles[0]
        import torch
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        for h in handles:
            try:
                bdf = self.amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                    return h
            except Exception:
                continue
        return None

    def _read(self):
        info = self.amdsmi.amdsmi_get_clock_info(self.handle, self.amdsmi.AmdSmiClkType.GFX)
        return float(info.get("clk", info.get("cur_clk")))

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                v = self._read()
            except Exception as e:  # pragma: no cover
                self.error = repr(e)[:160]
                return
            if time.perf_counter() - t0 >= self.settle:
                self.samples.append(v)
            time.sleep(self.period)

    def measure(self, step):
        """Run ``step`` back to back for ``duration`` seconds while sampling."""
        if self.handle is None:
            return
        import torch
        self.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < self.duration:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
        self.stop()

    def start(self):
        if self.handle is None:
            return
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"gfx_mhz_mean": None, "samples": 0, "source": "amdsmi", "error": self.error}
        return {"gfx_mhz_mean": round(float(sum(self.samples) / len(self.samples)), 1),
                "gfx_mhz_min": min(self.samples), "gfx_mhz_max": max(self.samples),
                "samples": len(self.samples),
                "source": f"amdsmi current GFX clock every {self.period * 1e3:g} ms while the same step runs "
                          f"for {self.duration:g} s after the timed steps (first {self.settle:g} s dropped)"}


def cpu_baseline(wl, inp, sample_tokens, saved="ab"):
    """The CPU oracle (float64 numpy) on the first ``sample_tokens`` tokens of
    the same workload, forward + backward."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    n = sample_tokens
    x, dy = inp["x"][:n], inp["dy"][:n]
    t0 = time.perf_counter()
    z = O.router_logits(x, inp["wg"], inp["bias"])
    ids, w = O.route(z.astype(np.float32).astype(np.float64), wl.K)
    O.build_index(ids, wl.E)
    f = O.moe_forward(x, ids, w, inp["w_gate"], inp["w_up"], inp["w_down"], dtype=wl.dtype, act=wl.act)
    if wl.backward:
        O.moe_backward(dy, x, inp["wg"], ids, w, inp["w_gate"], inp["w_up"], inp["w_down"], f, z, dtype=wl.dtype,
                       act=wl.act, saved=saved)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} tokens of the workload, router+index+forward" + ("+backward" if wl.backward else "")
                      + f", float64 numpy, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4,
                    help="1..9 (default 4: large-d fwd+bwd, the largest workload; 6..9: MoEBlaze's shapes, SiLU experts)")
    ap.add_argument("--cpu-sample", type=int, default=32, help="tokens for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--saved", default="ab", choices=("aby", "ab"),
                    help="saved for backward: H-only (a and b; y recomputed; default) or a, b and y")
    ap.add_argument("--combine", default="fold", choices=("fold", "staged"),
                    help="forward combine: the ordered fold (default) or the staged-Y ablation")
    ap.add_argument("--no-timing", action="store_true", help="do not record per-kernel events")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one HIP graph of the step instead of eager launches")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MB "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from dropless_moe_dispatch_amd import binding as B
    from dropless_moe_dispatch_amd import layer as L
    from dropless_moe_dispatch_amd import synth

    wl = synth.WORKLOADS[args.workload]
    T, d, E, K, h, dt = wl.T, wl.d, wl.E, wl.K, wl.h, wl.dtype
    torch.cuda.set_device(0)
    print(f"[bench] generating workload {wl.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl, tensors=("x", "wg", "w_gate", "w_up", "w_down") + (("dy",) if wl.backward else ()))
    dev = {k: (L.to_device(inp[k], dt) if inp[k] is not None else None)
           for k in ("x", "wg", "w_gate", "w_up", "w_down", "dy") if k in inp}
    bias = torch.from_numpy(inp["bias"]).cuda() if inp["bias"] is not None else None
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    # a forward-only workload saves nothing for a backward (h_ab not written)
    buf = L.MoEBuffers(T, d, E, K, h, dt, backward=wl.backward, saved=args.saved, combine=args.combine,
                       act=wl.act, save=wl.backward)

    def step():
        L.forward(buf, dev["x"], dev["wg"], bias, dev["w_gate"], dev["w_up"], dev["w_down"])
        if wl.backward:
            L.backward(buf, dev["dy"], dev["x"], dev["wg"], dev["w_gate"], dev["w_up"], dev["w_down"])

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        run()
        torch.cuda.synchronize()
    print("[bench] timed", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-kernel durations: the library's HIP events around each launch, on
    # the launch stream, over a second pass of the same steps (the events add
    # about 1% to a step, so the throughput above is taken without them)
    recs, ms_instr = [], None
    if not args.no_timing:
        print("[bench] per-kernel events", file=sys.stderr, flush=True)
        B.timing_enable(True)
        B.timing_read()
        ti0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ti1 = time.perf_counter()
        recs = B.timing_read()
        B.timing_enable(False)
        ms_instr = (ti1 - ti0) * 1e3 / args.steps
    # the clock the same step runs at (measured after the timed region, not inside it)
    clock = ClockSampler()
    if not args.no_timing:
        clock.measure(step)
    clk = clock.summary()
    # peak scale at the measured clock (the published peaks assume 2.4 GHz)
    cscale = clk["gfx_mhz_mean"] / NOMINAL_CLOCK_MHZ if clk.get("gfx_mhz_mean") else None
    peak_alloc = torch.cuda.max_memory_allocated()
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    errs = buf.device_error_words()
    buf.check_device_errors()   # a fold that gave up leaves out / dx invalid: no number is reported then

    ms = (t1 - t0) * 1e3 / args.steps
    gated = wl.act == "swiglu"
    # model FLOP (SonicMoE convention): gated 6 A d h forward + 12 backward;
    # a plain two-layer expert 4 + 8
    flops = ((18.0 if wl.backward else 6.0) if gated else (12.0 if wl.backward else 4.0)) * T * K * d * h
    tflops = flops / (ms * 1e-3) / 1e12
    per = {}
    for name, t in recs:
        per.setdefault(name, []).append(t)
    per_kernel = {k: {"avg_ms": float(np.mean(v)), "launches": len(v)} for k, v in per.items()}
    peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_MFMA_TFLOPS
    eb = 2 if dt == "bf16" else 4

    def floors(k):
        """The kernel's two roofline floors (ms): its model FLOP at the MFMA
        peak and its algorithmic bytes at the HBM peak (None where not
        defined); the larger one binds."""
        fl = kernel_flops(k, T, d, E, K, h, gated)
        by = kernel_bytes(k, T, d, E, K, h, eb, gated)
        f_mfma = fl / (peak * 1e12) * 1e3 if fl is not None else None
        f_hbm = by / (PEAK_HBM_GBS * 1e9) * 1e3 if by is not None else None
        if f_mfma is None and f_hbm is None:
            return None, None, None
        bound = "mfma" if f_hbm is None or (f_mfma is not None and f_mfma >= f_hbm) else "hbm"
        return f_mfma, f_hbm, bound

    roofline = None
    gemms = {k: v for k, v in per_kernel.items() if kernel_flops(k, T, d, E, K, h, gated) is not None and k != "router_logits"}
    if gemms:
        dom = max(gemms, key=lambda k: gemms[k]["avg_ms"] * gemms[k]["launches"])
        fl = kernel_flops(dom, T, d, E, K, h, gated)
        by = kernel_bytes(dom, T, d, E, K, h, eb, gated)
        f_mfma, f_hbm, bound = floors(dom)
        t = gemms[dom]["avg_ms"]
        if bound == "mfma":
            ach, pk, unit = fl / (t * 1e-3) / 1e12, peak, "TFLOP/s"
        else:
            ach, pk, unit = by / (t * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        roofline = {"bound": bound, "kernel": dom, "achieved": round(ach, 2), "peak": pk, "unit": unit,
                    "frac": round(ach / pk, 4), "traffic": committed_traffic(wl.name, dom),
                    "avg_launch_ms": round(t, 4), "algorithmic_flop_per_launch": fl,
                    "algorithmic_bytes_per_launch": by,
                    "floor_ms": {"mfma": round(f_mfma, 4) if f_mfma else None,
                                 "hbm": round(f_hbm, 4) if f_hbm else None},
                    "src_sha": kernel_source_hash(),
                    "peak_at_measured_clock": round(pk * cscale, 1) if (cscale and bound == "mfma") else None,
                    "frac_at_measured_clock": round(ach / (pk * cscale), 4) if (cscale and bound == "mfma") else None}
    kernels = {}
    for k, v in per_kernel.items():
        rec = {"avg_ms": round(v["avg_ms"], 4)}
        fl = kernel_flops(k, T, d, E, K, h, gated)
        if fl is not None:
            rec["tflops"] = round(fl / (v["avg_ms"] * 1e-3) / 1e12, 1)
            rec["mfma_peak_frac"] = round(rec["tflops"] / peak, 4)
        by = kernel_bytes(k, T, d, E, K, h, eb, gated)
        if by is not None:
            rec["gbs"] = round(by / (v["avg_ms"] * 1e-3) / 1e9, 1)
            rec["hbm_peak_frac"] = round(rec["gbs"] / PEAK_HBM_GBS, 4)
        f_mfma, f_hbm, bound = floors(k)
        if bound is not None:
            rec["bound"] = bound
            rec["floor_frac"] = round(max(x for x in (f_mfma, f_hbm) if x is not None) / v["avg_ms"], 4)
        kernels[k] = rec
    counts = np.diff(buf.offsets.cpu().numpy())
    cpu = cpu_baseline(wl, inp, args.cpu_sample, args.saved) if args.cpu_sample > 0 else None
    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_with_kernel_events": round(ms_instr, 4) if ms_instr else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded Philox normals, random-init weights)",
        "config": {"workload": wl.name, "T": T, "d": d, "E": E, "K": K, "h": h,
                   "backward": wl.backward, "zipf_s": wl.zipf_s, "seed": wl.seed, "act": wl.act, "saved": args.saved,
                   "combine": args.combine, "launch": "hip_graph" if args.graph else "eager"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / (PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_MFMA_TFLOPS), 4),
        "mfma_peak_frac_at_measured_clock": (
            round(tflops / ((PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_MFMA_TFLOPS) * cscale), 4) if cscale else None),
        "clock": clk,
        "model_flop_per_step": flops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_kernel_ms": {k: round(v["avg_ms"], 4) for k, v in per_kernel.items()},
        "kernels": kernels,
        "act_saved_MB": round(buf.saved_for_backward_bytes() / 1e6, 1),
        "workspace_MB": round(buf.workspace_bytes() / 1e6, 1),
        # device bytes at the peak beyond inputs, weights and weight gradients
        "peak_transient_MB": round((peak_alloc - base_alloc - buf.weight_grad_bytes()) / 1e6, 1),
        "avoided_TKd_buffer_MB": round(T * K * d * (2 if dt == "bf16" else 4) / 1e6, 1),
        "routing": {"max_rows": int(counts.max()), "min_rows": int(counts.min()),
                    "zero_row_experts": int((counts == 0).sum()),
                    "padded_row_frac": round(float((np.ceil(counts / 128) * 128).sum() / counts.sum() - 1), 4)},
        "device_errors": errs,
        "device": device_info(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
