#!/usr/bin/env python3
"""Throughput of the routed-expert forward of one MXFP4 Stable LatentMoE layer on one MI355X.

One step = moe_route_forward over one batch of seeded synthetic tokens (router, top-K, grouping by
expert, latent down-projection and shared gate/up, MXFP4 gate/up and down expert products,
gate-weighted combine, up-projection plus shared down-projection) with the inputs already resident
in HBM; the router and the x-side products run as one product over a combined weight copy, and
the step is timed on the caller's stream. Prints one JSON line.

Headline workload (the line's top-level fields): one GPU's TP8 share of a Kimi K3 layer at decode
size (64 tokens, hidden 7168, latent 3584, 896 experts top-16, expert intermediate 384, 2 shared
experts), HBM-bound. The line also carries a `prefill` object: the same layer at 8192 tokens with
Zipf-skewed routing, matrix-core bound, measured in the same run.

Order of the GPU work: the prefill leg (its own warm-up and timed steps), then the decode warm-up
and right after it the decode timed steps, so the headline is measured on a GPU that has been
running the layer for a while (the first few dozen decode steps after an idle period run 5-10%
slower) and its warm-up directly precedes it (decode steps right after the prefill leg, whose
traffic evicts the decode's cached state, ran up to 6% slower).
`--stage2 fp8` / `--stage1 mxfp4` time the layer with its quantised expert stages instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s per MI355X; HBM GB/s (decode), MFMA TFLOPS (prefill)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense BF16 matrix cores
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 matrix cores (the FP8 x FP4 down product's rate)
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense MXFP4 matrix cores (the A4W4 gate/up product's rate)
MX_BYTES_PER_VALUE = 17 / 32    # E2M1 nibble + one E8M0 byte per 32 values
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_KIND = ("beyond-L2 bytes per launch: FETCH_SIZE and WRITE_SIZE (separate rocprofv3 --pmc runs), "
                "each scaled by its reading for a 1 GiB device copy")
CPU_MIN_SECONDS = 10.0
CPU_MIN_SECONDS_PREFILL = 5.0


# Headers every kernel source includes: a change there changes the compiled kernel too.
SHARED_HEADERS = ("common.hpp", "kernels.hpp", "wave.hpp", "partials.hpp")


def source_hash(rel: str) -> str:
    """Hash of a kernel source file together with the shared headers beside it."""
    h = hashlib.sha256()
    path = os.path.join(ROOT, rel)
    for p in [path] + [os.path.join(os.path.dirname(path), n) for n in SHARED_HEADERS]:
        if os.path.exists(p):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family / model / stepping numbers (some hosts
    report only a generic model name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                        info[k] = v
                if not line.strip() and info:
                    break
    except OSError:
        pass
    name = info.get("model name", "unknown")
    ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({ids})" if ids else name


def algorithmic(shape, n_active: int) -> dict:
    """Bytes and FLOPs the layer must move / compute for one batch (intermediates excluded)."""
    s = shape
    T, K, E, Lt, I = s.T, s.K, s.E, s.Lt, s.I
    Hin = s.Hin
    expert_mx = 3 * Lt * I * MX_BYTES_PER_VALUE
    gateup_w = 2 * I * Lt * MX_BYTES_PER_VALUE
    dense_w = E * Hin * 2
    if s.has_latent:
        dense_w += 2 * Lt * s.H * 2 + 3 * s.S * s.Is * s.H * 2
    step_bytes = dense_w + n_active * expert_mx + T * Hin * 2 + T * (s.H if s.has_latent else Lt) * 2
    flops = 2 * T * E * Hin + 2 * T * K * 3 * I * Lt
    if s.has_latent:
        flops += 2 * 2 * T * s.H * Lt + 2 * 3 * T * s.S * s.Is * s.H
    return dict(
        step_bytes=step_bytes, step_flops=flops,
        # gate/up product: weights of active experts + z rows in + h rows out
        gateup_bytes=n_active * gateup_w + T * Lt * 2 + T * K * I * 2,
        gateup_flops=2 * T * K * 2 * I * Lt,
    )


def kernel_roof(nbytes: float, flops: float, mma_peak_tflops: float, seconds: float) -> dict:
    """A kernel against the higher of its two roofs: `nbytes` at the HBM peak, or `flops` at the
    given matrix-core peak. The bound is the roof with the longer lower-bound time; `achieved` and
    `frac` are in that roof's unit, and both lower bounds are reported (`roof_us`)."""
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mma = flops / (mma_peak_tflops * 1e12)
    if t_hbm >= t_mma:
        achieved = nbytes / seconds / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4))
    else:
        achieved = flops / seconds / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=mma_peak_tflops, unit="TFLOP/s",
                    frac=round(achieved / mma_peak_tflops, 4))
    roof["bytes_per_launch"] = round(nbytes)
    roof["flops_per_launch"] = round(flops)
    roof["roof_us"] = {"hbm": round(t_hbm * 1e6, 2), "mfma": round(t_mma * 1e6, 2)}
    return roof


def read_traffic(workload: str, kernel: str):
    """Beyond-L2 bytes per launch from committed PMC counters (FETCH_SIZE + WRITE_SIZE, each scaled
    by the counter's reading for a copy of known size), or None once that kernel's source has
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
        e = d[workload][kernel]
        if e.get("source_sha256_16") != source_hash(e["source"]):
            return None
        return float(e["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy(nbytes: int) -> None:
    """A plain device copy of known size, for scaling HBM counters (run under rocprofv3 --pmc)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reads": nbytes, "writes": nbytes}), flush=True)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Leg:
    """One workload on the GPU: packed layer, resident inputs, routing and output buffers."""

    def __init__(self, shape, fp8: bool, a4: bool, shared_stream: bool = False):
        import numpy as np
        import torch
        from mxfp4_latent_mixture_sigmoid_amd import MoELayer, abi
        from workload import make_inputs

        def dev(a):
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).cuda()

        self.shape, self.fp8, self.a4 = shape, fp8, a4
        log(f"workload {shape.name}: generating inputs")
        self.inp = make_inputs(shape)
        weights = {k: dev(v) for k, v in self.inp.items() if k in abi.WEIGHT_FIELDS and v is not None}
        self.layer = MoELayer(shape.H, shape.Lt, shape.E, shape.K, shape.I, shape.S, shape.Is, shape.has_latent,
                              weights, T_max=shape.T, stage2_fp8=fp8, stage1_a4=a4, shared_stream=shared_stream)
        torch.cuda.synchronize()
        del weights
        self.x = dev(self.inp["x"])
        self.bias = dev(self.inp["router_bias"]) if self.inp.get("router_bias") is not None else None
        self.routing = self.layer.alloc_routing(shape.T)
        self.out = torch.empty(shape.T, self.layer.H, dtype=torch.bfloat16, device="cuda")

    def step(self):
        self.layer.route_forward(self.x, self.shape.T, self.routing, out=self.out, logit_bias=self.bias)

    def make_graph(self):
        """The step captured as one HIP graph on this leg's buffers (moe_graph_create)."""
        return self.layer.graph(self.x, self.shape.T, self.routing, self.out, logit_bias=self.bias)

    def step_separate(self):
        self.layer.route(self.x, self.shape.T, self.routing, logit_bias=self.bias)
        self.layer.forward(self.x, self.shape.T, self.routing, out=self.out)

    def warm(self, n: int):
        import torch
        for _ in range(n):
            self.step()
        torch.cuda.synchronize()

    def timed(self, steps: int, fn=None):
        """(wall ms per step, GPU-event ms per step) over exactly `steps` back-to-back steps,
        bracketed by synchronisation on both sides."""
        import torch
        fn = fn or self.step
        stream = torch.cuda.current_stream()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps

    def kernels_us(self, steps: int) -> dict:
        """Per-kernel durations from HIP events recorded around each launch on the same stream."""
        from mxfp4_latent_mixture_sigmoid_amd import abi
        n_launch = 16 * steps
        abi.profile_begin(self.layer.handle, n_launch)
        for _ in range(steps):
            self.step()
        prof = abi.profile_end(self.layer.handle, n_launch)
        per = {}
        for name, ms in prof:
            per.setdefault(name, []).append(ms)
        return {k: round(1e3 * sum(v) / len(v), 3) for k, v in per.items()}

    def n_active(self) -> int:
        return int((self.routing["counts"].cpu() > 0).sum())

    def is_decode(self) -> bool:
        return self.shape.T * self.shape.K <= 4 * self.shape.E   # few tokens per expert: weight-stream bound

    def roofline(self, kernels_us: dict, n_active: int) -> dict:
        """The dominant kernel (the routed gate|up product) against the higher of its two roofs: its
        algorithmic bytes at the HBM peak, or its flops at the matrix-core peak of its operand type
        (BF16, or MXFP4 with the A4W4 first stage). Both lower bounds are reported."""
        s = self.shape
        alg = algorithmic(s, n_active)
        gateup_s = kernels_us["gateup"] * 1e-6
        gb = alg["gateup_bytes"]
        if self.a4:   # the gate/up product reads MX FP4 z (17/32 bytes per value) instead of BF16 z
            gb += s.T * s.Lt * (MX_BYTES_PER_VALUE - 2)
        flops = alg["gateup_flops"]
        peak = FP4_PEAK_TFLOPS if self.a4 else BF16_PEAK_TFLOPS
        roof = kernel_roof(gb, flops, peak, gateup_s)
        roof["kernel"] = "gateup"
        roof["kernel_us"] = kernels_us["gateup"]
        roof["traffic"] = None if self.a4 else read_traffic(s.name, "gateup")
        roof["traffic_kind"] = TRAFFIC_KIND
        return roof

    def step_roofline(self, ms_per_step: float, n_active: int) -> dict:
        """The whole step against the roof of its regime: HBM for decode, dense BF16 for prefill."""
        alg = algorithmic(self.shape, n_active)
        step_s = ms_per_step * 1e-3
        if self.is_decode():
            a = alg["step_bytes"] / step_s / 1e9
            return dict(bound="hbm", achieved=round(a, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(a / HBM_PEAK_GBPS, 4))
        a = alg["step_flops"] / step_s / 1e12
        return dict(bound="mfma", achieved=round(a, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(a / BF16_PEAK_TFLOPS, 4))

    def cpu_baseline(self, n_sample: int, min_seconds: float) -> dict:
        """The FP64 oracle's full forward on a seeded token sample of the same workload, repeated until
        at least min_seconds of host work are timed; tokens processed per second."""
        from oracle import oracle as O
        from workload import sample_tokens
        tok = sample_tokens(self.shape, n_sample)
        sub = dict(self.inp, x=self.inp["x"][tok])
        log(f"CPU oracle on {len(tok)} tokens of {self.shape.name}")
        passes, c0 = 0, time.perf_counter()
        while True:
            O.forward(sub, self.shape.K, want_intermediates=False, stage2_fp8=self.fp8, stage1_a4=self.a4)
            passes += 1
            csec = time.perf_counter() - c0
            if csec >= min_seconds:
                break
        return dict(value=round(passes * len(tok) / csec, 3), unit="tokens/s", cores=O.num_threads(),
                    kind="oracle", cpu_model=cpu_model(),
                    sample=f"{len(tok)} seeded tokens of {self.shape.name} (all {self.shape.T} tokens are "
                           f"independent), full forward in FP64, {passes} pass(es) in {csec:.1f} s")

    def close(self):
        self.layer.close()


def pct(v):
    v = sorted(v)
    q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]   # noqa: E731
    return {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5), "n": len(v)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tp8_decode_t64")
    ap.add_argument("--prefill-workload", default="tp8_prefill_t8192",
                    help="workload of the `prefill` object measured in the same run")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--cpu-sample", type=int, default=256,
                    help="tokens the CPU oracle evaluates (seeded sample; the whole batch if it is smaller)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--stage2", choices=("bf16", "fp8"), default="bf16",
                    help="arithmetic of the experts' down product: BF16 h (the layer as defined), or h "
                         "quantised to MX FP8 on the scaled FP8 x FP4 matrix-core instruction")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="steps timed one by one after a 1 GiB scratch write each (cache-cold distribution)")
    ap.add_argument("--stage1", choices=("bf16", "mxfp4"), default="bf16",
                    help="arithmetic of the experts' gate/up product: BF16 z (the layer as defined), or z "
                         "quantised to MX FP4 on the scaled FP4 x FP4 matrix-core instruction (A4W4)")
    ap.add_argument("--shared-stream", action="store_true",
                    help="run the shared experts' gate/up product on a second stream, concurrently with the "
                         "routing and the routed experts, instead of inside the x-side product")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer's TP8 share is measured on a single MI355X", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return 0

    from mxfp4_latent_mixture_sigmoid_amd import abi
    if not os.path.exists(abi.LIB_PATH):
        raise RuntimeError(f"{abi.LIB_PATH} is not built (run __graft_entry__.build() first)")
    from workload import SHAPES

    fp8, a4 = args.stage2 == "fp8", args.stage1 == "mxfp4"
    shape = SHAPES[args.workload]
    T = shape.T
    main_leg = Leg(shape, fp8, a4, args.shared_stream)
    pre_leg = None
    if not args.no_prefill and args.prefill_workload != args.workload:
        pre_leg = Leg(SHAPES[args.prefill_workload], fp8, a4, args.shared_stream)

    prefill = None
    if pre_leg is not None:
        ps = pre_leg.shape
        p_steps = max(1, min(args.steps, 20))
        log(f"prefill leg {ps.name}: warmup {args.warmup}, {p_steps} timed steps")
        pre_leg.warm(args.warmup)
        p_ms, p_gpu_ms = pre_leg.timed(p_steps)
        p_kernels = pre_leg.kernels_us(min(p_steps, 5))
        p_active = pre_leg.n_active()
        prefill = {
            "workload": ps.name, "tokens": ps.T, "routing": ps.routing, "active_experts": p_active,
            "steps": p_steps, "warmup": args.warmup,
            "ms_per_step": round(p_ms, 5), "gpu_ms_per_step": round(p_gpu_ms, 5),
            "value": round(ps.T / (p_ms * 1e-3), 1), "unit": "tokens/s",
            "step_roofline": pre_leg.step_roofline(p_ms, p_active),
            "roofline": pre_leg.roofline(p_kernels, p_active),
            "kernels_us": p_kernels,
        }
        log(f"prefill {p_ms:.4f} ms/step")

    log(f"warmup {args.warmup} ({shape.name})")
    main_leg.warm(args.warmup)
    log(f"timed {args.steps} steps ({shape.name})")
    ms_per_step, gpu_ms = main_leg.timed(args.steps)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # Per-step distribution: events between back-to-back steps, then steps timed one by one, each
    # after a 1 GiB scratch write outside the timed region (nothing of the layer left in the caches).
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        main_leg.step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    step_pct = pct([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    flushed_pct = None
    if args.flush_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fl = []
        for i in range(args.flush_steps):
            scratch.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            main_leg.step()
            b.record(stream)
            torch.cuda.synchronize()
            fl.append(a.elapsed_time(b))
        flushed_pct = pct(fl)
        del scratch

    # The same work as two calls (moe_route, then moe_forward) on the one stream, for reference.
    for _ in range(min(args.warmup, 5)):
        main_leg.step_separate()
    ms_separate, _ = main_leg.timed(args.steps, main_leg.step_separate)

    # The same step replayed from one captured HIP graph (moe_graph_create / moe_graph_launch).
    graph = main_leg.make_graph()
    for _ in range(min(args.warmup, 5)):
        graph.launch()
    ms_graph, gpu_ms_graph = main_leg.timed(args.steps, graph.launch)
    graph.close()
    log(f"graph replay: {ms_graph:.4f} ms/step")

    kernels_us = main_leg.kernels_us(args.steps)
    n_active = main_leg.n_active()
    roof = main_leg.roofline(kernels_us, n_active)
    down_roof = None
    if fp8:   # the FP8 x FP4 down product against its own roof
        down_s = kernels_us["down"] * 1e-6
        P = T * shape.K
        if main_leg.is_decode():
            b = n_active * shape.Lt * shape.I * MX_BYTES_PER_VALUE + P * shape.I * 33 / 32 + P * shape.Lt * 2
            down_roof = dict(bound="hbm", achieved=round(b / down_s / 1e9, 1), peak=HBM_PEAK_GBPS, unit="GB/s")
        else:
            f = 2 * P * shape.I * shape.Lt
            down_roof = dict(bound="mfma", achieved=round(f / down_s / 1e12, 2), peak=FP8_PEAK_TFLOPS,
                             unit="TFLOP/s")
        down_roof["frac"] = round(down_roof["achieved"] / down_roof["peak"], 4)
        down_roof["kernel"] = "down"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = main_leg.cpu_baseline(args.cpu_sample, CPU_MIN_SECONDS)
        if prefill is not None:
            prefill["cpu_baseline"] = pre_leg.cpu_baseline(args.cpu_sample, CPU_MIN_SECONDS_PREFILL)

    alg = algorithmic(shape, n_active)
    step_s = ms_per_step * 1e-3
    line = {
        "metric": METRIC,
        "value": round(T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(["bf16"] + (["mxfp4"] if a4 else []) + (["fp8"] if fp8 else [])),
        "data": "synthetic",
        "config": {"workload": shape.name, "tokens": T, "hidden": shape.H, "latent": shape.Lt,
                   "experts": shape.E, "top_k": shape.K, "inter": shape.I, "shared_experts": shape.S,
                   "shared_inter": shape.Is, "routing": shape.routing, "active_experts": n_active,
                   "stage1": args.stage1, "stage2": args.stage2,
                   "shared": "stream" if args.shared_stream else "fused"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_ms_per_step": round(gpu_ms, 5),
        "step_ms_percentiles": step_pct,
        "step_ms_percentiles_cache_flushed": flushed_pct,
        "ms_per_step_route_then_forward": round(ms_separate, 5),
        "ms_per_step_graph": round(ms_graph, 5),
        "gpu_ms_per_step_graph": round(gpu_ms_graph, 5),
        "step_hbm_gbps": round(alg["step_bytes"] / step_s / 1e9, 1),
        "step_tflops": round(alg["step_flops"] / step_s / 1e12, 2),
        # the whole step against both roofs (the full unsharded experts sit at the ridge between them)
        "step_fracs": {"hbm": round(alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBPS, 4),
                       "mfma": round(alg["step_flops"] / step_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        # the whole step against the roof of its regime (HBM for decode, dense BF16 for prefill)
        "step_roofline": main_leg.step_roofline(ms_per_step, n_active),
        "kernels_us": kernels_us,
        "legs_order": (["prefill", "decode warm-up", "decode timed"] if prefill is not None else
                       ["warm-up", "timed"]),
    }
    if down_roof:
        line["roofline_down"] = down_roof
    if prefill is not None:
        line["prefill"] = prefill
    print(json.dumps(line), flush=True)
    main_leg.close()
    if pre_leg is not None:
        pre_leg.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
